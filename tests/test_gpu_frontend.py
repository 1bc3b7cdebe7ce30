"""The frame front end (q, k, v = rope(X W_Q), rope(X W_K), X W_V) against the
float64 oracle's frame_front_end, rounded to bf16 by the oracle's rounding.

The GPU sums the bf16 products in fp32 (the oracle in float64), so a value
can land one bf16 unit away when the exact result sits near a rounding
boundary, and a value that nearly cancels in the rotation carries the fp32
sums' absolute error: every value must lie within one bf16 unit of the
oracle's rounded value plus 2e-5 (about 20x the fp32 accumulation error of
unit-variance sums over <= 3584 terms), and at least 99.5 % of them must be
bit-identical."""

import numpy as np
import pytest

import framegen
from gpu_util import to_bits, to_dev
from oracle import frame_front_end, round_to_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import streaming_long_video_amd as skv  # noqa: E402

ABS_EXTRA = 2e-5
IDENTICAL = 0.995


def _bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def _ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _compare(name, got_bits, ref64):
    want_bits = round_to_bf16(ref64)
    got, want = _bits_to_f64(got_bits), _bits_to_f64(want_bits)
    err = np.abs(got - ref64)
    bound = _ulp_bf16(ref64) + ABS_EXTRA
    same = float(np.mean(got_bits == want_bits))
    print(f"  {name}: identical {same * 100:.3f} %, worst err/bound {float((err / bound).max()):.3f}")
    assert (err <= bound).all(), (name, float((err / bound).max()))
    assert same >= IDENTICAL, (name, same)


@pytest.mark.parametrize("name,T,frame", [("tiny", 16, 3), ("internvl3_1b_layer", 256, 5),
                                          ("internvl3_8b_layer", 256, 301),
                                          ("internvl3_8b_layer", 100, 7),
                                          ("internvl3_2b_28layers", 256, 0)])
def test_front_end_matches_oracle(name, T, frame):
    spec = framegen.workload(name)
    if name == "internvl3_2b_28layers":
        spec = spec.for_layer(5)
    Hq, Hkv, d = spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    x = framegen.hidden_states(spec, frame)[:T]
    w = framegen.projection_weights(spec)
    first = spec.position_offset + frame * spec.frame_tokens
    print(f"front end {name}: T={T}, hidden={x.shape[1]}, frame {frame}", flush=True)
    q, k, v = skv.qkv_rope(to_dev(x), to_dev(w), Hq, Hkv, d, first, spec.rope_theta)
    torch.cuda.synchronize()
    wq, wk, wv = framegen.split_projection_weights(spec, w)
    rq, rk, rv = frame_front_end(x, wq, wk, wv, Hq, Hkv, d, first + np.arange(T),
                                 spec.rope_theta)
    _compare("q", to_bits(q), rq)
    _compare("k", to_bits(k), rk)
    _compare("v", to_bits(v), rv)


def test_front_end_unrotated_and_scaled():
    """rope_theta = 0 leaves q and k unrotated; a linear scaling divides the
    positions (both against the oracle)."""
    spec = framegen.workload("internvl3_1b_layer")
    Hq, Hkv, d = spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    x = framegen.hidden_states(spec, 2)
    w = framegen.projection_weights(spec)
    wq, wk, wv = framegen.split_projection_weights(spec, w)
    pos = 70000 + np.arange(x.shape[0])
    for theta, scaling in ((0.0, 1.0), (1e6, 4.0)):
        q, k, v = skv.qkv_rope(to_dev(x), to_dev(w), Hq, Hkv, d, int(pos[0]), theta, scaling)
        torch.cuda.synchronize()
        if theta == 0.0:
            from oracle import project_frame
            rq, rk, rv = project_frame(x, wq, wk, wv, Hq, Hkv, d)
        else:
            rq, rk, rv = frame_front_end(x, wq, wk, wv, Hq, Hkv, d, pos, theta, scaling)
        _compare("q", to_bits(q), rq)
        _compare("k", to_bits(k), rk)
        _compare("v", to_bits(v), rv)


def test_front_end_feeds_the_prefill_step():
    """The front end's outputs drive the StateKV step of a layer with
    rope_theta = 0; the step then equals the oracle step on the same bf16
    q, k, v (teacher forced from the GPU's state)."""
    from gpu_util import teacher_forced_frame
    from oracle import StateKVOracle

    spec = framegen.workload("internvl3_1b_layer")
    Hq, Hkv, d, T = spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.frame_tokens
    w_d = to_dev(framegen.projection_weights(spec))
    layer = skv.Layer(Hq, Hkv, d, T, spec.state_budget, detailed_capacity=8 * T)
    orc = StateKVOracle(Hq, Hkv, d, T, spec.state_budget)
    for n in range(6):
        x = framegen.hidden_states(spec, n)
        q, k, v = skv.qkv_rope(to_dev(x), w_d, Hq, Hkv, d, n * T, spec.rope_theta)
        r = teacher_forced_frame(orc, layer, n, to_bits(q), to_bits(k), to_bits(v))
        print(f"frame {n}: relrms {r.relrms:.2e} kept {r.kept_match}/{r.kept_total}")
        assert r.relrms <= 1e-3 and r.maxabs <= 2e-2 and r.score_err <= 1.0


def test_front_end_workspace_forms_agree():
    """statekv_qkv_rope through the C ABI with the caller's workspace and
    with none (the library's stream-ordered allocation): bit-identical q, k,
    v at the 8B shape (split hidden dimension) and the 1B shape (no split,
    no workspace needed), on two calls in a row."""
    from streaming_long_video_amd import _binding as B

    for name in ("internvl3_8b_layer", "internvl3_1b_layer"):
        spec = framegen.workload(name)
        Hq, Hkv, d, T = spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.frame_tokens
        x = to_dev(framegen.hidden_states(spec, 9))
        w = to_dev(framegen.projection_weights(spec))
        hidden = x.shape[1]
        need = B.statekv_qkv_rope_workspace_size(T, hidden, Hq, Hkv, d)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
        print(f"{name}: workspace {need} bytes", flush=True)
        outs = []
        for workspace, nbytes in ((ws.data_ptr(), need), (0, 0), (ws.data_ptr(), need), (0, 0)):
            q = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=x.device)
            k = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=x.device)
            v = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=x.device)
            B.statekv_qkv_rope(x.data_ptr(), w.data_ptr(), T, hidden, Hq, Hkv, d, 9 * T,
                               spec.rope_theta, 0.0, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                               workspace, nbytes, 0)
            outs.append((q, k, v))
        torch.cuda.synchronize()
        for other in outs[1:]:
            for a, b in zip(outs[0], other):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
