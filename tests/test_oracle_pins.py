"""The CPU oracle checked against facts fixed outside it (CPU only)."""

import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import framegen
import oracle_pins
from oracle import StateKVOracle, decode_attention, full_causal_attention, select_top_b


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_full_causal_attention_matches_torch_sdpa():
    """The dense causal routine agrees with torch's float64 causal SDPA."""
    rng = np.random.default_rng(0)
    L, Hq, Hkv, d = 37, 6, 2, 16
    q = rng.standard_normal((L, Hq, d))
    k = rng.standard_normal((L, Hkv, d))
    v = rng.standard_normal((L, Hkv, d))
    ours = full_causal_attention(q, k, v)
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(ours, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-13)
    # rows of the last queries only (the per-frame form used for baselines)
    tail = full_causal_attention(q[-9:], k, v, first_query=L - 9)
    np.testing.assert_allclose(tail, ours[-9:], rtol=0, atol=1e-13)


def test_decode_attention_pins():
    """Decoding over D: torch's float64 SDPA without a mask; the closed forms
    of a single D token (output = its value) and of all-zero keys (uniform
    weights: output = mean of the values of the query's KV head); and the
    order of D's tokens does not matter."""
    rng = np.random.default_rng(1)
    L, M, Hq, Hkv, d = 53, 3, 6, 2, 16
    q = rng.standard_normal((M, Hq, d))
    k = rng.standard_normal((L, Hkv, d))
    v = rng.standard_normal((L, Hkv, d))
    ours = decode_attention(q, k, v)
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    np.testing.assert_allclose(ours, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-13)
    one = decode_attention(q, k[:1], v[:1])
    for g in range(Hq):
        np.testing.assert_allclose(one[:, g, :], np.broadcast_to(v[0, g // G], (M, d)),
                                   rtol=0, atol=1e-15)
    flat = decode_attention(q, np.zeros_like(k), v)
    for g in range(Hq):
        np.testing.assert_allclose(flat[:, g, :], np.broadcast_to(v[:, g // G].mean(0), (M, d)),
                                   rtol=0, atol=1e-13)
    perm = rng.permutation(L)
    np.testing.assert_allclose(decode_attention(q, k[perm], v[perm]), ours, rtol=0, atol=1e-13)


def _brute_force_select(scores, positions, budget):
    idx = sorted(range(len(scores)), key=lambda j: (-float(scores[j]), int(positions[j])))
    keep = idx[: min(budget, len(scores))]
    return sorted(keep, key=lambda j: int(positions[j]))


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 64).flatmap(lambda n: st.tuples(
    st.lists(st.integers(0, 6), min_size=n, max_size=n),
    st.integers(1, 70))))
def test_select_matches_brute_force(case):
    """Top-B by (score desc, position asc) on tie-heavy quantised scores."""
    vals, budget = case
    scores = np.array(vals, dtype=np.float32) / 4
    positions = np.arange(len(vals)) * 3 + 11
    got = select_top_b(scores, positions, budget)
    np.testing.assert_array_equal(got, _brute_force_select(scores, positions, budget))


def test_select_edge_cases():
    s = np.array([0.5, 0.5, 0.5, 0.5], dtype=np.float32)
    p = np.arange(4)
    np.testing.assert_array_equal(select_top_b(s, p, 1), [0])
    np.testing.assert_array_equal(select_top_b(s, p, 3), [0, 1, 2])
    np.testing.assert_array_equal(select_top_b(s, p, 4), [0, 1, 2, 3])
    np.testing.assert_array_equal(select_top_b(s, p, 9), [0, 1, 2, 3])
    s2 = np.array([0.0, 3.0, 1.0, 3.0, 2.0], dtype=np.float32)
    np.testing.assert_array_equal(select_top_b(s2, np.arange(5), 2), [1, 3])
    np.testing.assert_array_equal(select_top_b(s2, np.arange(5), 4), [1, 2, 3, 4])


def test_tiny_full_budget_equals_full_attention_on_bf16_frames():
    """The 2-head, d=64, T=16 workload with B=128 >= all history: the streaming
    oracle and the dense causal routine agree on every frame (bf16 inputs)."""
    spec = framegen.workload("tiny_full")
    orc = StateKVOracle(spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                        spec.frame_tokens, spec.state_budget)
    ks, vs = [], []
    for n, (q, k, v) in enumerate(framegen.frames(spec)):
        ks.append(k), vs.append(v)
        res = orc.step(q, k, v)
        ref = full_causal_attention(q, np.concatenate(ks), np.concatenate(vs),
                                    first_query=n * spec.frame_tokens)
        np.testing.assert_allclose(res.o, ref, rtol=0, atol=1e-12)
        assert res.kept_positions[0].shape[0] == (n + 1) * spec.frame_tokens


def test_warmup_sizes_and_no_eviction_before_full():
    spec = framegen.workload("tiny")
    orc = StateKVOracle(spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                        spec.frame_tokens, spec.state_budget)
    for n, (q, k, v) in enumerate(framegen.frames(spec)):
        res = orc.step(q, k, v)
        c = min(spec.state_budget, n * spec.frame_tokens)
        assert res.pool_positions[0].shape[0] == c + spec.frame_tokens
        assert res.kept_positions[0].shape[0] == min(spec.state_budget,
                                                     (n + 1) * spec.frame_tokens)
        np.testing.assert_allclose(res.scores[0].sum(),
                                   spec.n_q_heads * spec.frame_tokens, rtol=1e-13)


def test_planted_sinks_survive_in_the_1b_layer_stream():
    """Temporal sinks planted in frames 0-3 stay in every head's state for all
    64 frames (the pages' claim that importance-based memory keeps old anchor
    tokens that a recency window drops)."""
    spec = framegen.workload("internvl3_1b_layer")
    _, sinks = framegen.sink_plan(spec)
    orc = StateKVOracle(spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                        spec.frame_tokens, spec.state_budget)
    T = spec.frame_tokens
    old_kept = 0
    for n, (q, k, v) in enumerate(framegen.frames(spec)):
        res = orc.step(q, k, v)
        seen = sinks[sinks < (n + 1) * T]
        for h in range(spec.n_kv_heads):
            assert np.isin(seen, res.kept_positions[h]).all(), (n, h)
        if n == spec.n_frames - 1:
            old_kept = sum(int((kp < 4 * T).sum()) for kp in res.kept_positions)
    # a recency window of B tokens would hold nothing from frames 0-3 by now
    assert old_kept > 0


def test_shared_mode():
    """SHARED: one kept set per layer from scores summed over all query heads.
    With one KV head it equals the per-head mode; scores then sum to Hq*T."""
    spec = framegen.workload("tiny")
    a = StateKVOracle(2, 1, 64, 16, 32)
    b = StateKVOracle(2, 1, 64, 16, 32, shared=True)
    for q, k, v in framegen.frames(spec):
        ra, rb = a.step(q, k, v), b.step(q, k, v)
        np.testing.assert_array_equal(ra.kept_positions[0], rb.kept_positions[0])
        np.testing.assert_array_equal(ra.o, rb.o)
    rng = np.random.default_rng(0)
    c = StateKVOracle(4, 2, 8, 4, 6, shared=True)
    for n in range(4):
        r = c.step(rng.standard_normal((4, 4, 8)), rng.standard_normal((4, 2, 8)),
                   rng.standard_normal((4, 2, 8)))
        np.testing.assert_array_equal(r.kept_positions[0], r.kept_positions[1])
        np.testing.assert_allclose(np.sum(r.scores), 4 * 4, rtol=1e-13)


def test_ring_capacity():
    rng = np.random.default_rng(0)
    lin = StateKVOracle(2, 1, 8, 4, 4, detailed_capacity=8)
    ring = StateKVOracle(2, 1, 8, 4, 4, detailed_capacity=8, ring=True)
    frames = [(rng.standard_normal((4, 2, 8)), rng.standard_normal((4, 1, 8)),
               rng.standard_normal((4, 1, 8))) for _ in range(3)]
    for f in frames[:2]:
        lin.step(*f), ring.step(*f)
    with pytest.raises(ValueError):
        lin.step(*frames[2])
    ring.step(*frames[2])
    pos, k, _ = ring.detailed(0)
    np.testing.assert_array_equal(pos, np.arange(4, 12))
    np.testing.assert_array_equal(k, np.concatenate([frames[1][1], frames[2][1]])[:, 0])


def test_scale_default_is_inverse_sqrt_d():
    orc = StateKVOracle(2, 1, 64, 16, 32)
    assert orc.scale == 1 / math.sqrt(64)
