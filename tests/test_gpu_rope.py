"""In-library rotary embedding on the GPU against the oracle's float64
rotation rounded once to bf16, alone and inside the per-frame step and
decoding."""

import numpy as np
import pytest

import framegen
from gpu_util import O_MAXABS, O_RELRMS, SELECT_AGREEMENT, o_errors, snapshot, to_bits, to_dev
from oracle import StateKVOracle, decode_attention, rope_at_positions, round_to_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import streaming_long_video_amd as skv  # noqa: E402


def _ulp_compare(gpu_bits, ref_bits):
    """Fraction of identical bf16 patterns and the largest difference in units
    of the last place (same-sign patterns are ordered like their values)."""
    a = gpu_bits.astype(np.int64)
    b = ref_bits.astype(np.int64)
    same = float(np.mean(a == b))
    diff = np.abs(a - b)
    return same, int(diff.max()) if diff.size else 0


def _oracle_rotated(x_bits, positions, theta, scaling=1.0):
    return round_to_bf16(rope_at_positions(x_bits, positions, theta, scaling))


@pytest.mark.parametrize("d,theta,scaling,first", [
    (128, 1e6, 0.0, 77 * 256),        # 8B-like frame 77
    (128, 1e6, 4.0, 10 ** 6 + 5),     # large offset, linear scaling
    (64, 1e4, 0.0, 0),                # token 0 at position 0: identity
    (64, 1e6, 0.0, 131071),
])
def test_rope_kernel_matches_oracle(d, theta, scaling, first):
    spec = framegen.workload("internvl3_8b_layer" if d == 128 else "internvl3_1b_layer")
    spec = spec.replace(rotated=False, sinks=False)
    q, k, _ = framegen.frame(spec, 5)
    layer = skv.Layer(spec.n_q_heads, spec.n_kv_heads, d, spec.frame_tokens, 64,
                      detailed_capacity=spec.frame_tokens, rope_theta=theta,
                      rope_scaling=scaling)
    for x in (q, k):
        dev = to_dev(x)
        layer.rope(dev, first)
        got = to_bits(dev)
        pos = first + np.arange(x.shape[0])
        ref = _oracle_rotated(x, pos, theta, scaling if scaling > 0 else 1.0)
        same, worst = _ulp_compare(got, ref)
        print(f"d={d} first={first}: identical {same:.6f}, worst {worst} ulp")
        assert worst <= 1 and same >= 0.999, (same, worst)
        if first == 0:  # token 0 sits at position 0: no rotation
            np.testing.assert_array_equal(got[0], x[0])


def test_prefill_and_decode_with_library_rope():
    """1B-like stream, unrotated inputs, rope_theta = 1e6: every frame against
    the oracle fed the oracle's own rotation of the same inputs (from the GPU's
    state), the detailed cache against the oracle-rotated keys, then decoding
    of text queries rotated by statekv_rope."""
    spec = framegen.workload("internvl3_1b_layer").replace(n_frames=12, rotated=False,
                                                           sinks=False)
    T, theta = spec.frame_tokens, spec.rope_theta
    qs, ks, vs = framegen.stacked_frames(spec, workers=8)
    layer = skv.Layer(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, T, spec.state_budget,
                      detailed_capacity=spec.n_frames * T, rope_theta=theta)
    orc = StateKVOracle(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, T, spec.state_budget)
    match = total = 0
    k_rot_all = []
    for n in range(spec.n_frames):
        before = snapshot(layer)
        orc.load_state(n, before.pos, before.k, before.v)
        pos = n * T + np.arange(T)
        q_rot = _oracle_rotated(qs[n], pos, theta)
        k_rot = _oracle_rotated(ks[n], pos, theta)
        k_rot_all.append(k_rot)
        o = layer.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
        ref = orc.step(q_rot, k_rot, vs[n])
        maxabs, relrms = o_errors(o, ref.o)
        assert maxabs <= O_MAXABS and relrms <= O_RELRMS, (n, maxabs, relrms)
        after = snapshot(layer)
        for h in range(spec.n_kv_heads):
            kept = set(ref.kept_positions[h].tolist())
            match += len(kept.intersection(after.pos[h].tolist()))
            total += len(kept)
    assert match >= SELECT_AGREEMENT * total, (match, total)
    torch.cuda.synchronize()
    dc = layer.detailed_cache()
    L = dc["length"]
    d_keys = to_bits(dc["k"][:, :L])                       # [Hkv][L][d]
    ref_keys = np.transpose(np.concatenate(k_rot_all), (1, 0, 2))
    same, worst = _ulp_compare(d_keys, ref_keys)
    assert worst <= 1 and same >= 0.999, (same, worst)
    np.testing.assert_array_equal(to_bits(dc["v"][:, :L]),
                                  np.transpose(vs.reshape(-1, *vs.shape[-2:]), (1, 0, 2)))
    # decoding: text queries rotated in the library at positions N*T + i
    tq = framegen.text_queries(spec, 3, 0)
    tq_dev = to_dev(tq)
    layer.rope(tq_dev, spec.n_frames * T)
    o = layer.decode(tq_dev).cpu().numpy()
    tq_ref = _oracle_rotated(tq, spec.n_frames * T + np.arange(3), theta)
    ref = decode_attention(tq_ref, np.transpose(d_keys, (1, 0, 2)),
                           vs.reshape(-1, *vs.shape[-2:]))
    maxabs, relrms = o_errors(o, ref)
    assert maxabs <= O_MAXABS and relrms <= O_RELRMS, (maxabs, relrms)
