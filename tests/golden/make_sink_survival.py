"""Writes sink_survival_8b.json: for the 512-frame InternVL3-8B-like layer
stream, the first frame at which the float64 oracle (running free, from frame
0) evicts each planted sink from each KV head's compressed state, or null if
it never does.  Calls only the oracle and the seeded input generator.

    python tests/golden/make_sink_survival.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import framegen  # noqa: E402
from oracle import StateKVOracle  # noqa: E402


def main():
    spec = framegen.workload("internvl3_8b_layer")
    plan = framegen.sink_plan(spec)
    sinks = plan[1]
    orc = StateKVOracle(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.frame_tokens,
                        spec.state_budget)
    lost = {h: {int(s): None for s in sinks} for h in range(spec.n_kv_heads)}
    for n in range(spec.n_frames):
        res = orc.step(*framegen.frame(spec, n, plan))
        seen = sinks[sinks < (n + 1) * spec.frame_tokens]
        for h in range(spec.n_kv_heads):
            for s in seen[~np.isin(seen, res.kept_positions[h])]:
                if lost[h][int(s)] is None:
                    lost[h][int(s)] = n
        if n % 32 == 0:
            print("frame", n, flush=True)
    out = {
        "what": "first frame at which the free-running float64 oracle evicts each planted "
                "sink (null: kept through the last frame)",
        "workload": "internvl3_8b_layer",
        "n_frames": spec.n_frames,
        "sink_positions": [int(s) for s in sinks],
        "first_lost_frame": {str(h): {str(s): f for s, f in d.items()} for h, d in lost.items()},
        "written_by": "tests/golden/make_sink_survival.py",
    }
    with open(os.path.join(HERE, "sink_survival_8b.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
