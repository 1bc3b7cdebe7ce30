"""Writes two expected-value files for the 512-frame InternVL3-8B-like layer
stream, from one free-running run of the float64 oracle (from frame 0, never
fed anything the GPU computed).  Calls only the oracle and the seeded input
generator.

* sink_survival_8b.json: the first frame at which the oracle evicts each
  planted sink from each KV head's compressed state, or null if it never does;
* kept_sets_8b.json: the oracle's whole kept set C_n of every KV head after
  the sampled frames KEPT_FRAMES, each as a bitmap over positions
  [0, (n+1)T) (bit p set when position p is kept), packed most significant
  bit first, zlib-compressed, base64-encoded.

    python tests/golden/make_sink_survival.py
"""

import base64
import json
import os
import sys
import zlib

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import framegen  # noqa: E402
from oracle import StateKVOracle  # noqa: E402

# first eviction frame, then spread over the stream up to its last frame
KEPT_FRAMES = (16, 64, 128, 256, 384, 511)


def encode_set(positions, n_positions: int) -> str:
    bits = np.zeros(n_positions, dtype=np.uint8)
    bits[np.asarray(positions, dtype=np.int64)] = 1
    return base64.b64encode(zlib.compress(np.packbits(bits).tobytes(), 9)).decode("ascii")


def decode_set(text: str, n_positions: int) -> np.ndarray:
    """Sorted kept positions from one encoded bitmap."""
    raw = np.frombuffer(zlib.decompress(base64.b64decode(text)), dtype=np.uint8)
    return np.flatnonzero(np.unpackbits(raw)[:n_positions]).astype(np.int64)


def main():
    spec = framegen.workload("internvl3_8b_layer")
    T = spec.frame_tokens
    plan = framegen.sink_plan(spec)
    sinks = plan[1]
    orc = StateKVOracle(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, T, spec.state_budget)
    lost = {h: {int(s): None for s in sinks} for h in range(spec.n_kv_heads)}
    kept = {}
    for n in range(spec.n_frames):
        res = orc.step(*framegen.frame(spec, n, plan))
        seen = sinks[sinks < (n + 1) * T]
        for h in range(spec.n_kv_heads):
            for s in seen[~np.isin(seen, res.kept_positions[h])]:
                if lost[h][int(s)] is None:
                    lost[h][int(s)] = n
        if n in KEPT_FRAMES:
            kept[str(n)] = {str(h): encode_set(res.kept_positions[h], (n + 1) * T)
                            for h in range(spec.n_kv_heads)}
        if n % 32 == 0:
            print("frame", n, flush=True)
    sink_out = {
        "what": "first frame at which the free-running float64 oracle evicts each planted "
                "sink (null: kept through the last frame)",
        "workload": "internvl3_8b_layer",
        "n_frames": spec.n_frames,
        "sink_positions": [int(s) for s in sinks],
        "first_lost_frame": {str(h): {str(s): f for s, f in d.items()} for h, d in lost.items()},
        "written_by": "tests/golden/make_sink_survival.py",
    }
    with open(os.path.join(HERE, "sink_survival_8b.json"), "w") as f:
        json.dump(sink_out, f, indent=1)
    kept_out = {
        "what": "kept set of every KV head of the free-running float64 oracle after each "
                "listed frame: bitmap over positions [0, (n+1)T), np.packbits order, "
                "zlib, base64",
        "workload": "internvl3_8b_layer",
        "frame_tokens": T,
        "state_budget": spec.state_budget,
        "frames": kept,
        "written_by": "tests/golden/make_sink_survival.py",
    }
    with open(os.path.join(HERE, "kept_sets_8b.json"), "w") as f:
        json.dump(kept_out, f, indent=1)


if __name__ == "__main__":
    main()
