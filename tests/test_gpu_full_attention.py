"""The quadratic full-attention baseline on the GPU against the dense causal
oracle routine (frame n's queries over every token up to the frame)."""

import numpy as np
import pytest

import framegen
from gpu_util import O_MAXABS, O_RELRMS, o_errors, to_dev
from oracle import full_causal_attention

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import streaming_long_video_amd as skv  # noqa: E402


@pytest.mark.parametrize("name,frames,splits", [
    ("tiny", 8, 0),
    ("internvl3_1b_layer", 12, 0),
    ("internvl3_1b_layer", 6, 1),
])
def test_full_attention_matches_dense_oracle(name, frames, splits):
    spec = framegen.workload(name).replace(n_frames=frames)
    qs, ks, vs = framegen.stacked_frames(spec, workers=8)
    T = spec.frame_tokens
    layer = skv.Layer(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, T, spec.state_budget,
                      detailed_capacity=frames * T, num_splits=splits)
    for n in range(frames):
        o = layer.full_attention(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
        if n in (0, 1, frames // 2, frames - 1):
            Kall = ks[: n + 1].reshape(-1, spec.n_kv_heads, spec.head_dim)
            Vall = vs[: n + 1].reshape(-1, spec.n_kv_heads, spec.head_dim)
            ref = full_causal_attention(qs[n], Kall, Vall, first_query=n * T)
            maxabs, relrms = o_errors(o, ref)
            assert maxabs <= O_MAXABS and relrms <= O_RELRMS, (n, maxabs, relrms)


def test_full_attention_and_statekv_agree_without_eviction():
    """B covers the whole history: the StateKV step and the quadratic baseline
    compute the same thing."""
    spec = framegen.workload("internvl3_1b_layer").replace(n_frames=4, state_budget=1024)
    qs, ks, vs = framegen.stacked_frames(spec, workers=4)
    mk = lambda: skv.Layer(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.frame_tokens,
                           spec.state_budget, detailed_capacity=4 * spec.frame_tokens)
    a, b = mk(), mk()
    for n in range(4):
        oa = a.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
        ob = b.full_attention(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
        d = np.abs(oa - ob).max()
        assert d <= 2e-3, (n, d)


def test_mixing_modes_is_rejected():
    spec = framegen.workload("tiny").replace(n_frames=2)
    qs, ks, vs = framegen.stacked_frames(spec)
    layer = skv.Layer(2, 1, 64, 16, 32, detailed_capacity=32)
    layer.prefill(to_dev(qs[0]), to_dev(ks[0]), to_dev(vs[0]))
    with pytest.raises(skv.StateKVError):
        layer.full_attention(to_dev(qs[1]), to_dev(ks[1]), to_dev(vs[1]))
