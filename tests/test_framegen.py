"""Pins of the synthetic frame generator (inputs only, no StateKV arithmetic)."""

import numpy as np
import pytest
import torch

import framegen
from framegen import generator as gen


def test_bf16_rounding_matches_torch_rne():
    """fp64 -> fp32 -> bf16 round-to-nearest-even agrees with torch's CPU casts."""
    rng = np.random.default_rng(123)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
        # exact halfway cases between bf16 neighbours (ties to even)
        (np.arange(1, 2000, dtype=np.float64) * 2 + 1) * 2.0 ** -8,
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40]),
    ])
    ours = framegen.f64_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).view(torch.int16)
    np.testing.assert_array_equal(ours.view(np.int16), ref.numpy())


def test_bf16_widening_is_exact():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    bits = bits[finite]
    f32 = framegen.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(f32, ref)
    np.testing.assert_array_equal(framegen.bf16_bits_to_f64(bits), ref.astype(np.float64))


def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 64))
    np.testing.assert_array_equal(gen.rope_rotate(x, np.zeros(5), 1e4), x)
    y = gen.rope_rotate(x, np.arange(5) * 997, 1e6)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-13)


def test_rope_matches_complex_rotation():
    """Pairs (x_i, x_{i+d/2}) behave as the complex number x_i + j x_{i+d/2}
    multiplied by exp(j * p * theta^(-2i/d))."""
    rng = np.random.default_rng(1)
    d, theta = 128, 1e6
    x = rng.standard_normal((7, 2, d))
    pos = rng.integers(0, 200000, 7)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    w = np.exp(1j * pos[:, None] * theta ** (-np.arange(0, d, 2) / d))
    zr = z * w[:, None, :]
    y = gen.rope_rotate(x, pos, theta)
    np.testing.assert_allclose(y[..., : d // 2], zr.real, atol=1e-12)
    np.testing.assert_allclose(y[..., d // 2:], zr.imag, atol=1e-12)


def test_rope_dot_depends_only_on_relative_position():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    a = (gen.rope_rotate(q, [1000], 1e4) * gen.rope_rotate(k, [700], 1e4)).sum()
    b = (gen.rope_rotate(q, [5300], 1e4) * gen.rope_rotate(k, [5000], 1e4)).sum()
    c = (gen.rope_rotate(q, [300], 1e4) * k).sum()
    np.testing.assert_allclose([a, b], [c, c], rtol=1e-10)


def test_frames_are_deterministic_and_distinct():
    spec = framegen.workload("internvl3_1b_layer")
    a = framegen.frame(spec, 5)
    b = framegen.frame(spec, 5)
    c = framegen.frame(spec, 6)
    for x, y in zip(a, b):
        assert x.dtype == np.uint16
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    assert a[0].shape == (256, 14, 64) and a[1].shape == (256, 2, 64)


def test_sink_plan_and_planted_keys():
    spec = framegen.workload("internvl3_1b_layer")
    u, pos = framegen.sink_plan(spec)
    assert pos.shape == (10,) and np.all(np.diff(pos) > 0)
    assert pos.min() >= 0 and pos.max() < 4 * spec.frame_tokens
    assert abs(np.linalg.norm(u) - 1.0) < 1e-12
    # keys at sink positions carry ~4 along u; others ~0; queries ~0.5
    along_sink, along_other, along_q = [], [], []
    for n in range(4):
        q, k, _ = gen.frame_f64(spec, n)
        p = n * spec.frame_tokens + np.arange(spec.frame_tokens)
        # undo the rotation to read the planted component independent of position
        proj = (k @ u)
        hit = np.isin(p, pos)
        along_sink.append(proj[hit].ravel())
        along_other.append(proj[~hit].ravel())
        along_q.append((q @ u).ravel())
    s = np.concatenate(along_sink)
    o = np.concatenate(along_other)
    assert s.size == 10 * spec.n_kv_heads
    assert abs(s.mean() - 4.0) < 1.0 and abs(o.mean()) < 0.05
    assert abs(np.concatenate(along_q).mean() - 0.5) < 0.05


def test_no_sinks_means_plain_gaussians():
    spec = framegen.workload("tiny")
    q, k, v = gen.frame_f64(spec, 0)
    assert abs(v.mean()) < 0.1 and abs(v.std() - 1) < 0.1
    # rotation keeps the per-token norms of Gaussians
    assert abs((q ** 2).sum(-1).mean() / 64 - 1) < 0.15


@pytest.mark.parametrize("name", sorted(framegen.WORKLOADS))
def test_workload_shapes(name):
    spec = framegen.workload(name)
    assert spec.n_q_heads % spec.n_kv_heads == 0
    assert spec.head_dim in (64, 128)
    if spec.n_layers > 1:
        assert spec.for_layer(5).seed == spec.layer_seed_base + 5
