"""GPU parity of the App. A diagnostics (statekv_attention_mass) against the
oracle's attention_mass_diagnostics.

The layer keeps every token, so its step is full attention; the GPU's
importance is checked against the oracle's within the score tolerance, and
the diagnostics are checked against the oracle applied to the GPU's own
layer-wide importance (the per-head fp32 rows summed in head order, as the
kernel forms them): the kept sets bit for bit, the shares within fp32
summation error."""

import math

import numpy as np
import pytest

import framegen
from gpu_util import SCORE_ATOL, SCORE_RTOL, snapshot, to_dev
from oracle import StateKVOracle, attention_mass_diagnostics

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import streaming_long_video_amd as skv  # noqa: E402

BUDGETS = [1, 3, 16, 64, 100, 256, 1000, 4096]


def _unpack(words: np.ndarray, n: int) -> np.ndarray:
    w = words.astype(np.uint32)
    bits = (w[:, None] >> np.arange(32, dtype=np.uint32)[None, :]) & 1
    return bits.reshape(-1)[:n].astype(bool)


@pytest.mark.parametrize("shape", [(4, 2, 64, 32, 10, True), (28, 4, 128, 256, 6, True),
                                   (2, 1, 64, 16, 5, False)])
def test_attention_mass_matches_oracle(shape):
    Hq, Hkv, d, T, N, sinks = shape
    spec = framegen.FrameSpec(Hq, Hkv, d, T, N, N * T, 1e4, 9, sinks=sinks)
    qs, ks, vs = framegen.stacked_frames(spec, workers=8)
    layer = skv.Layer(Hq, Hkv, d, T, N * T, detailed_capacity=N * T)
    orc = StateKVOracle(Hq, Hkv, d, T, N * T)
    sets = None
    prev = [None] * len(BUDGETS)
    for n in range(N):
        layer.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
        out, sets = layer.attention_mass(BUDGETS, sets)
        torch.cuda.synchronize()
        ref = orc.step(qs[n], ks[n], vs[n])
        snap = snapshot(layer)
        L, c = snap.pool, snap.pool - T
        assert L == (n + 1) * T
        for h in range(Hkv):
            err = np.abs(snap.scores[h].astype(np.float64) - ref.scores[h])
            assert (err <= SCORE_ATOL + SCORE_RTOL * np.abs(ref.scores[h])).all(), (n, h)
        s32 = snap.scores[0].astype(np.float32).copy()
        for h in range(1, Hkv):
            s32 = (s32 + snap.scores[h].astype(np.float32)).astype(np.float32)
        s64 = s32.astype(np.float64)
        o = out.cpu().numpy()
        words = sets.cpu().numpy().view(np.uint32)
        for i, b in enumerate(BUDGETS):
            t, r, rc, kept = attention_mass_diagnostics(s64, c, b, prev[i])
            np.testing.assert_array_equal(_unpack(words[i], L), kept, err_msg=f"frame {n} b {b}")
            for gpu, exp in zip(o[i], (t, r, rc)):
                if math.isnan(exp):
                    assert math.isnan(gpu), (n, b, o[i], (t, r, rc))
                else:
                    assert abs(gpu - exp) <= 2e-6 + 1e-5 * abs(exp), (n, b, o[i], (t, r, rc))
            prev[i] = kept


def test_attention_mass_refuses_a_layer_that_evicted():
    """tiny: T = 16, B = 32.  Frames 0-2 attend over every token (frame 2's
    pool is all 48 tokens; its selection then drops 16), frame 3 no longer."""
    spec = framegen.workload("tiny")
    qs, ks, vs = framegen.stacked_frames(spec, workers=2)
    layer = skv.Layer(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.frame_tokens,
                      spec.state_budget, detailed_capacity=spec.n_frames * spec.frame_tokens)
    for n in range(4):
        layer.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
        if n < 3:
            layer.attention_mass([1, 8])
        else:
            with pytest.raises(skv.StateKVError):
                layer.attention_mass([1, 8])
