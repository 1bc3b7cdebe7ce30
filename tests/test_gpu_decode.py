"""Decoding attention over the detailed state on the GPU against the float64
oracle routine (text queries over every video token kept in D)."""

import numpy as np
import pytest

import framegen
from gpu_util import O_MAXABS, O_RELRMS, o_errors, to_dev
from oracle import decode_attention

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import streaming_long_video_amd as skv  # noqa: E402


def _check(layer, spec, ks, vs, n_q, seed, ring_keep=None):
    q = framegen.text_queries(spec, n_q, seed)
    o = layer.decode(to_dev(q)).cpu().numpy()
    K = ks.reshape(-1, *ks.shape[-2:])
    V = vs.reshape(-1, *vs.shape[-2:])
    if ring_keep is not None:
        K, V = K[-ring_keep:], V[-ring_keep:]
    ref = decode_attention(q, K, V)
    maxabs, relrms = o_errors(o, ref)
    print(f"decode M={n_q}: maxabs {maxabs:.3e} relrms {relrms:.3e}")
    assert maxabs <= O_MAXABS and relrms <= O_RELRMS, (maxabs, relrms)


@pytest.mark.parametrize("name,frames,n_q", [
    ("tiny", 3, 1),                    # d=64, G=2, 48 tokens: one ragged split per head
    ("tiny", 8, 16),                   # G * M = 32 rows
    ("internvl3_1b_layer", 12, 1),     # d=64, G=7
    ("internvl3_1b_layer", 12, 4),     # 28 rows
    ("internvl3_2b_28layers", 9, 2),   # d=128, G=6, 2304 tokens
])
def test_decode_after_statekv_prefill(name, frames, n_q):
    spec = framegen.workload(name).replace(n_frames=frames, n_layers=1)
    qs, ks, vs = framegen.stacked_frames(spec, workers=8)
    layer = skv.Layer(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.frame_tokens,
                      spec.state_budget, detailed_capacity=frames * spec.frame_tokens)
    for n in range(frames):
        layer.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
    _check(layer, spec, ks, vs, n_q, seed=frames)
    _check(layer, spec, ks, vs, 1, seed=frames + 1)  # again: the call changes no state


def test_decode_after_full_attention_and_over_a_ring():
    spec = framegen.workload("internvl3_1b_layer").replace(n_frames=6)
    qs, ks, vs = framegen.stacked_frames(spec, workers=6)
    T = spec.frame_tokens
    full = skv.Layer(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, T, spec.state_budget,
                     detailed_capacity=6 * T)
    ring = skv.Layer(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, T, spec.state_budget,
                     detailed_capacity=4 * T, flags=skv.STATEKV_FLAG_D_RING)
    for n in range(6):
        full.full_attention(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
        ring.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
    _check(full, spec, ks, vs, 2, seed=3)
    _check(ring, spec, ks, vs, 2, seed=4, ring_keep=4 * T)


def test_decode_at_the_8b_shape_after_512_frames():
    """The whole 8B-like stream (131072 tokens per KV head), one text token."""
    spec = framegen.workload("internvl3_8b_layer")
    qs, ks, vs = framegen.stacked_frames(spec, workers=16)
    layer = skv.Layer(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.frame_tokens,
                      spec.state_budget, detailed_capacity=spec.n_frames * spec.frame_tokens)
    for n in range(spec.n_frames):
        layer.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
    _check(layer, spec, ks, vs, 1, seed=11)
    _check(layer, spec, ks, vs, 4, seed=12)
