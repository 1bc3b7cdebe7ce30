"""The per-frame step recorded as a HIP graph (torch.cuda.CUDAGraph over the
library's launches on the capture stream): every replay, with eager work and
synchronisations between replays, must reproduce the eager run bit for bit.
The step's launches are plain kernels (no memset or copy nodes), so they can
be captured; the host-side frame logic runs at capture time, so a replay
re-runs the recorded frames from a restored state."""

import numpy as np
import pytest

import framegen
from gpu_util import snapshot, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import streaming_long_video_amd as skv  # noqa: E402


@pytest.mark.parametrize("flags", [0, "in_place"])
def test_graph_replays_match_the_eager_run(flags):
    spec = framegen.workload("tiny").replace(head_dim=128, frame_tokens=64, state_budget=256,
                                             n_frames=8)
    f = skv.STATEKV_FLAG_SLOT_STABLE if flags == "in_place" else 0
    T, Hq, d, N = spec.frame_tokens, spec.n_q_heads, spec.head_dim, spec.n_frames
    qs, ks, vs = framegen.stacked_frames(spec, workers=4)
    q_d = [to_dev(x) for x in qs]
    k_d = [to_dev(x) for x in ks]
    v_d = [to_dev(x) for x in vs]

    def make():
        return skv.Layer(spec.n_q_heads, spec.n_kv_heads, d, T, spec.state_budget,
                         detailed_capacity=N * T, flags=f)

    eager = make()
    ref = [eager.prefill(q_d[n], k_d[n], v_d[n]) for n in range(N)]
    ref_state = snapshot(eager)

    # frames 0..3 fill the state, 4..7 evict and are recorded; an even count, so
    # the row layout's two state buffers are where a restore leaves them
    first = 4
    layer = make()
    for n in range(first):
        layer.prefill(q_d[n], k_d[n], v_d[n])
    ckpt = layer.checkpoint()
    outs = [torch.empty((T, Hq, d), dtype=torch.float32, device="cuda") for _ in range(N - first)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i, n in enumerate(range(first, N)):
            layer.prefill(q_d[n], k_d[n], v_d[n], out=outs[i])
    for rep in range(3):
        layer.restore(ckpt)  # eager copies, then a synchronisation
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, n in enumerate(range(first, N)):
            assert torch.equal(outs[i].view(torch.int32), ref[n].view(torch.int32)), (rep, n)
        st = snapshot(layer)
        assert st.count == ref_state.count
        for h in range(spec.n_kv_heads):
            assert np.array_equal(st.pos[h], ref_state.pos[h]), (rep, h)
            assert np.array_equal(st.k[h], ref_state.k[h]) and np.array_equal(st.v[h], ref_state.v[h])
