"""Checks that pin the CPU oracle to facts fixed outside itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with a value
worked out by hand, a closed form, an invariant, a library routine or brute
force.  The same checks run against deliberately broken copies of the oracle
(see test_oracle_mutations.py) to show that each plausible mistake is caught.
"""

from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle.statekv_oracle as so

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _frac(s: str) -> float:
    return float(Fraction(s))


def check_hand_example() -> None:
    """Three-frame example worked by hand with exact rationals (tests/golden)."""
    ex = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    orc = so.StateKVOracle(ex["n_q_heads"], ex["n_kv_heads"], ex["head_dim"],
                           ex["frame_tokens"], ex["state_budget"], scale=math.log(2.0))
    for fr, exp in zip(ex["frames"], ex["expected"]):
        q = np.array(fr["q"], dtype=np.float64)[:, None, :]
        k = np.array(fr["k"], dtype=np.float64)[:, None, :]
        v = np.array(fr["v"], dtype=np.float64)[:, None, :]
        res = orc.step(q, k, v)
        o_exp = np.array([[_frac(x) for x in row] for row in exp["o"]])
        np.testing.assert_allclose(res.o[:, 0, :], o_exp, rtol=0, atol=1e-14)
        np.testing.assert_array_equal(res.pool_positions[0], exp["pool_positions"])
        np.testing.assert_allclose(res.scores[0], [_frac(x) for x in exp["scores"]],
                                   rtol=0, atol=1e-14)
        np.testing.assert_array_equal(res.kept_positions[0], exp["kept_positions"])


def check_single_token_frame() -> None:
    """T = 1 with an empty state: the only visible key is the token itself, O = v."""
    rng = np.random.default_rng(7)
    orc = so.StateKVOracle(4, 2, 8, 1, 3)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    res = orc.step(q, k, v)
    for g in range(4):
        np.testing.assert_allclose(res.o[0, g], v[0, g // 2], rtol=0, atol=1e-15)
    for h in range(2):
        np.testing.assert_allclose(res.scores[h], [2.0], rtol=0, atol=1e-15)


def check_uniform_attention_closed_form() -> None:
    """All keys zero: every visible key gets weight 1/(number visible).

    Query t of frame n sees c + t + 1 keys, so O_t is the mean of those values,
    and a state key's importance is G * sum_t 1/(c+t+1); frame key t' gets
    G * sum_{t>=t'} 1/(c+t+1).  Pins the causal mask, the state visibility and
    the score definition (sum, not mean, over queries and the group's heads).
    """
    rng = np.random.default_rng(11)
    Hq, Hkv, d, T, B = 6, 2, 4, 5, 7
    G = Hq // Hkv
    orc = so.StateKVOracle(Hq, Hkv, d, T, B)
    for n in range(3):
        q = rng.standard_normal((T, Hq, d))
        k = np.zeros((T, Hkv, d))
        v = rng.standard_normal((T, Hkv, d))
        prev_pos = [orc.state(h)[0].copy() for h in range(Hkv)]
        prev_v = [None if orc.state(h)[2] is None else orc.state(h)[2].copy()
                  for h in range(Hkv)]
        res = orc.step(q, k, v)
        for h in range(Hkv):
            c = prev_pos[h].shape[0]
            pool_v = v[:, h, :] if c == 0 else np.concatenate([prev_v[h], v[:, h, :]])
            for t in range(T):
                mean = pool_v[: c + t + 1].mean(axis=0)
                for g in range(h * G, (h + 1) * G):
                    np.testing.assert_allclose(res.o[t, g], mean, rtol=0, atol=1e-13)
            expect = np.zeros(c + T)
            for t in range(T):
                expect[: c + t + 1] += G / (c + t + 1)
            np.testing.assert_allclose(res.scores[h], expect, rtol=0, atol=1e-13)


def check_gqa_head_mapping() -> None:
    """Query head g reads KV head floor(g/G): make KV head 1's keys zero and its
    values constant per head; heads G..2G-1 must output that constant."""
    rng = np.random.default_rng(5)
    Hq, Hkv, d, T = 6, 3, 8, 4
    G = Hq // Hkv
    orc = so.StateKVOracle(Hq, Hkv, d, T, 16)
    q = rng.standard_normal((T, Hq, d)) * 3
    k = rng.standard_normal((T, Hkv, d)) * 3
    v = rng.standard_normal((T, Hkv, d))
    for h in range(Hkv):
        v[:, h, :] = float(h + 1)
    res = orc.step(q, k, v)
    for g in range(Hq):
        np.testing.assert_allclose(res.o[:, g, :], float(g // G + 1), rtol=0, atol=1e-13)


def check_probability_invariants() -> None:
    """Rows of P sum to 1; each KV head's scores sum to G*T (every query spends
    a total weight of 1); the scores equal column sums of P built by explicit
    scalar loops with math.exp."""
    rng = np.random.default_rng(3)
    Hq, Hkv, d, T, B = 4, 2, 6, 3, 4
    G = Hq // Hkv
    orc = so.StateKVOracle(Hq, Hkv, d, T, B, scale=0.7)
    for n in range(3):
        q = rng.standard_normal((T, Hq, d))
        k = rng.standard_normal((T, Hkv, d))
        v = rng.standard_normal((T, Hkv, d))
        st = [orc.state(h) for h in range(Hkv)]
        st = [(p.copy(), None if kk is None else kk.copy()) for p, kk, _ in st]
        res = orc.step(q, k, v, keep_probs=True)
        for P in res.probs:
            np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        for h in range(Hkv):
            np.testing.assert_allclose(res.scores[h].sum(), G * T, rtol=1e-14)
            c = st[h][0].shape[0]
            pool_k = k[:, h, :] if c == 0 else np.concatenate([st[h][1], k[:, h, :]])
            col = [0.0] * (c + T)
            for g in range(h * G, (h + 1) * G):
                for t in range(T):
                    visible = list(range(c + t + 1))
                    logits = [0.7 * sum(q[t, g, e] * pool_k[j, e] for e in range(d))
                              for j in visible]
                    mx = max(logits)
                    w = [math.exp(z - mx) for z in logits]
                    tot = sum(w)
                    for j, wj in zip(visible, w):
                        col[j] += wj / tot
            np.testing.assert_allclose(res.scores[h], col, rtol=0, atol=1e-13)


def check_full_attention_equivalence(n_frames: int = 8) -> None:
    """B >= every history: nothing is evicted, so each frame's output equals
    dense causal self-attention over the whole video so far."""
    rng = np.random.default_rng(9)
    Hq, Hkv, d, T = 4, 2, 16, 8
    B = T * n_frames
    orc = so.StateKVOracle(Hq, Hkv, d, T, B)
    qs, ks, vs = [], [], []
    for n in range(n_frames):
        q = rng.standard_normal((T, Hq, d))
        k = rng.standard_normal((T, Hkv, d))
        v = rng.standard_normal((T, Hkv, d))
        qs.append(q), ks.append(k), vs.append(v)
        res = orc.step(q, k, v)
        ref = so.full_causal_attention(q, np.concatenate(ks), np.concatenate(vs),
                                       first_query=n * T)
        np.testing.assert_allclose(res.o, ref, rtol=0, atol=1e-12)


def check_selection_and_caches() -> None:
    """Eviction keeps exactly B tokens once the pool exceeds B; the kept set is
    the top-B by (score desc, position asc); every state row is bit-identical
    to the frame row it came from; the detailed state holds every frame row."""
    rng = np.random.default_rng(21)
    Hq, Hkv, d, T, B = 4, 2, 8, 5, 7
    orc = so.StateKVOracle(Hq, Hkv, d, T, B)
    all_k, all_v = [], []
    for n in range(6):
        q = rng.standard_normal((T, Hq, d)).astype(np.float32)
        k = rng.standard_normal((T, Hkv, d)).astype(np.float32)
        v = rng.standard_normal((T, Hkv, d)).astype(np.float32)
        all_k.append(k), all_v.append(v)
        res = orc.step(q, k, v)
        for h in range(Hkv):
            pool = res.pool_positions[h]
            assert res.kept_positions[h].shape[0] == min(B, (n + 1) * T)
            if pool.shape[0] > B:
                order = sorted(range(pool.shape[0]),
                               key=lambda j: (-res.scores[h][j], pool[j]))
                np.testing.assert_array_equal(res.kept_positions[h],
                                              np.sort(pool[order[:B]]))
            pos, ck, cv = orc.state(h)
            K = np.concatenate(all_k)[:, h, :]
            V = np.concatenate(all_v)[:, h, :]
            assert ck.dtype == np.float32
            np.testing.assert_array_equal(ck, K[pos])
            np.testing.assert_array_equal(cv, V[pos])
            dpos, dk, dv = orc.detailed(h)
            np.testing.assert_array_equal(dpos, np.arange((n + 1) * T))
            np.testing.assert_array_equal(dk, K)
            np.testing.assert_array_equal(dv, V)



def check_decode_attention() -> None:
    """Decoding over D: scalar Python loops with math.exp on a tiny case;
    closed forms (one D token -> its value; all-zero keys -> mean of the KV
    head's values); D token order does not matter; query head g reads KV head
    g // G."""
    rng = np.random.default_rng(7)
    L, M, Hq, Hkv, d = 6, 2, 4, 2, 3
    q = rng.standard_normal((M, Hq, d))
    k = rng.standard_normal((L, Hkv, d))
    v = rng.standard_normal((L, Hkv, d))
    s = 0.7
    out = so.decode_attention(q, k, v, scale=s)
    G = Hq // Hkv
    for m in range(M):
        for g in range(Hq):
            h = g // G
            z = [s * sum(q[m, g, i] * k[j, h, i] for i in range(d)) for j in range(L)]
            zmax = max(z)
            w = [math.exp(x - zmax) for x in z]
            tot = sum(w)
            for i in range(d):
                ref = sum(w[j] * v[j, h, i] for j in range(L)) / tot
                assert abs(out[m, g, i] - ref) <= 1e-12, (m, g, i)
    one = so.decode_attention(q, k[:1], v[:1])
    for g in range(Hq):
        assert np.allclose(one[:, g, :], v[0, g // G], rtol=0, atol=1e-15)
    flat = so.decode_attention(q, np.zeros_like(k), v)
    for g in range(Hq):
        assert np.allclose(flat[:, g, :], v[:, g // G].mean(0), rtol=0, atol=1e-13)
    perm = rng.permutation(L)
    assert np.allclose(so.decode_attention(q, k[perm], v[perm]), so.decode_attention(q, k, v),
                       rtol=0, atol=1e-13)


def check_rope_and_rounding() -> None:
    """RoPE: identity at position 0; a worked example (d = 4, theta = 100:
    the second pair turns by 0.1 rad per position); pair norms preserved;
    q.k after rotation depends only on the position difference; linear
    scaling divides the position.  bf16 rounding: hand-picked ties and
    near-ties."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 2, 8))
    assert np.allclose(so.rope_at_positions(x, np.zeros(3), 1e4), x, rtol=0, atol=0)
    e1 = np.zeros((1, 1, 4))
    e1[0, 0, 1] = 1.0
    r = so.rope_at_positions(e1, np.array([2]), 100.0)[0, 0]
    assert np.allclose(r, [0.0, math.cos(0.2), 0.0, math.sin(0.2)], rtol=0, atol=1e-15)
    pos = np.array([5, 1000, 123456])
    y = so.rope_at_positions(x, pos, 1e6)
    half = 4
    assert np.allclose(x[..., :half] ** 2 + x[..., half:] ** 2,
                       y[..., :half] ** 2 + y[..., half:] ** 2, rtol=1e-12, atol=0)
    q = rng.standard_normal((1, 1, 8))
    k = rng.standard_normal((1, 1, 8))
    dots = []
    for p0 in (0, 17, 4096):
        qr = so.rope_at_positions(q, np.array([p0 + 9]), 1e4)
        kr = so.rope_at_positions(k, np.array([p0]), 1e4)
        dots.append(float(np.sum(qr * kr)))
    assert max(dots) - min(dots) <= 1e-10, dots
    assert np.allclose(so.rope_at_positions(x, pos, 1e6, scaling=4.0),
                       so.rope_at_positions(x, pos / 4.0, 1e6), rtol=0, atol=1e-12)
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 3 * 2.0 ** -8,
                     -2.5, 3.0 * 2.0 ** -100, 0.0])
    want = np.array([1.0, 1.0 + 2.0 ** -7, 1.0 + 2.0 ** -6, -2.5, 3.0 * 2.0 ** -100, 0.0])
    got = (so.round_to_bf16(vals).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(got, want), got


def check_recency_window() -> None:
    """Recency rule: the kept set is the B largest positions (closed form); in
    a stream, after frame n the state holds exactly positions
    [max(0, (n+1)T - B), (n+1)T)."""
    pos = np.array([3, 9, 1, 7, 20, 11])
    assert list(so.select_most_recent(pos, 3)) == [1, 4, 5]
    assert list(so.select_most_recent(pos, 10)) == [0, 1, 2, 3, 4, 5]
    rng = np.random.default_rng(5)
    T, B = 4, 10
    orc = so.StateKVOracle(2, 1, 8, T, B, recency=True)
    for n in range(6):
        r = orc.step(rng.standard_normal((T, 2, 8)), rng.standard_normal((T, 1, 8)),
                     rng.standard_normal((T, 1, 8)))
        hi = (n + 1) * T
        assert list(r.kept_positions[0]) == list(range(max(0, hi - B), hi)), (n, r.kept_positions)

def check_attention_mass() -> None:
    """App. A diagnostics: a case worked by hand; closed forms (uniform
    importance gives min(b, c)/c for both shares, ties kept at the lower
    positions); the top-b share is the best share over every subset of b
    historical tokens (brute force); the recency share is that of the b most
    recent ones; the recall is 1 when the kept set stays in the pool and 0
    when the pool misses the only kept token."""
    # by hand: history [5, 1, 3, 0.5], frame [2, 4], b = 2: top-2 history
    # 5 + 3 of 9.5; the last two 3 + 0.5; the new set {5, 4}; the pool holds
    # positions 1, 2 and the frame, so only 4 of the 9 is recalled
    t, r, rc, kept = so.attention_mass_diagnostics([5, 1, 3, 0.5, 2, 4], 4, 2,
                                                   [False, True, True, False])
    assert abs(t - 8 / 9.5) < 1e-15 and abs(r - 3.5 / 9.5) < 1e-15, (t, r)
    assert kept.tolist() == [True, False, False, False, False, True], kept
    assert abs(rc - 4 / 9) < 1e-15, rc
    # no earlier frame: the shares are undefined, the pool is everything
    t, r, rc, kept = so.attention_mass_diagnostics([1.0, 2.0], 0, 1)
    assert math.isnan(t) and math.isnan(r) and rc == 1.0 and kept.tolist() == [False, True]
    # uniform importance
    for b in (1, 3, 7, 12):
        t, r, _, kept = so.attention_mass_diagnostics(np.ones(12), 9, b)
        assert abs(t - min(b, 9) / 9) < 1e-15 and abs(r - min(b, 9) / 9) < 1e-15, (b, t, r)
        assert kept.tolist() == [i < b for i in range(12)], kept
    # stable set -> recall 1; pool missing the single kept token -> 0
    s = np.array([9.0, 1, 1, 1, 0.5, 0.5])
    assert so.attention_mass_diagnostics(s, 4, 1, [True, False, False, False])[2] == 1.0
    assert so.attention_mass_diagnostics(s, 4, 1, [False, True, True, True])[2] == 0.0
    # brute force on small random histories
    rng = np.random.default_rng(11)
    for _ in range(30):
        c, T, b = int(rng.integers(1, 8)), int(rng.integers(1, 4)), int(rng.integers(1, 6))
        s = rng.exponential(size=c + T)
        t, r, _, kept = so.attention_mass_diagnostics(s, c, b, rng.random(c) < 0.5)
        hist = s[:c]
        best = max(sum(hist[list(S)]) for S in itertools.combinations(range(c), min(b, c)))
        assert abs(t - best / hist.sum()) < 1e-12, (t, best)
        assert abs(r - sum(hist[i] for i in range(c) if i >= c - b) / hist.sum()) < 1e-12
        inside, outside = s[kept], s[~kept]
        assert len(inside) == min(b, c + T)
        assert not len(outside) or inside.min() >= outside.max()


def check_shared_layer_ranking() -> None:
    """SHARED selection with two KV heads, worked by hand.

    Hq = Hkv = 2 (G = 1), d = 1, T = 3, B = 2, softmax scale ln 2 and every
    query q = 1, so the weight of key j is 2^k_j / (sum over visible keys).
    Keys [0, 0, 3] give importance [8/5, 3/5, 4/5] (query 2 weights the frame
    1:1:8); keys [0, 0, 1] give [7/4, 3/4, 1/2] (query 2 weights 1:1:2).  Per
    KV head the first keeps positions {0, 2}, the second {0, 1}; the layer sum
    [67/20, 27/20, 13/10] keeps {0, 1} for both heads, while either head alone
    or the head-wise maximum ([7/4, 3/4, 4/5]) would keep {0, 2} in one of the
    two head orders.  (rainbus method steps: importance is a sum over queries;
    the layer-wide set sums every query head of the layer.)"""
    a = [Fraction(8, 5), Fraction(3, 5), Fraction(4, 5)]
    b = [Fraction(7, 4), Fraction(3, 4), Fraction(1, 2)]
    for keys, want in (([[0, 0, 3], [0, 0, 1]], [a, b]), ([[0, 0, 1], [0, 0, 3]], [b, a])):
        q = np.ones((3, 2, 1))
        k = np.array(keys, dtype=np.float64).T[:, :, None]      # (T, Hkv, 1)
        v = np.arange(6, dtype=np.float64).reshape(3, 2, 1)
        per = so.StateKVOracle(2, 2, 1, 3, 2, scale=math.log(2.0))
        lay = so.StateKVOracle(2, 2, 1, 3, 2, scale=math.log(2.0), shared=True)
        rp, rl = per.step(q, k, v), lay.step(q, k, v)
        for h in range(2):
            np.testing.assert_allclose(rl.scores[h], [float(x) for x in want[h]], rtol=0,
                                       atol=1e-14)
            np.testing.assert_array_equal(rl.kept_positions[h], [0, 1])
            np.testing.assert_array_equal(rl.o[:, h], rp.o[:, h])
        np.testing.assert_array_equal(rp.kept_positions[keys.index([0, 0, 3])], [0, 2])
        np.testing.assert_array_equal(rp.kept_positions[keys.index([0, 0, 1])], [0, 1])


def check_noncausal_closed_form() -> None:
    """Frame tokens visible to every frame query (the non-causal variant), all
    keys zero: every query sees the whole pool [C ; frame] with equal weight,
    so O_t is the mean of the pool's values for every t and every candidate's
    importance is G*T/(c+T); with all importances tied the lower positions are
    kept, so the state holds positions 0..B-1 once it is full."""
    rng = np.random.default_rng(13)
    Hq, Hkv, d, T, B = 6, 2, 4, 5, 7
    G = Hq // Hkv
    orc = so.StateKVOracle(Hq, Hkv, d, T, B, causal=False)
    for n in range(3):
        q = rng.standard_normal((T, Hq, d))
        k = np.zeros((T, Hkv, d))
        v = rng.standard_normal((T, Hkv, d))
        prev = [orc.state(h) for h in range(Hkv)]
        prev = [(p.copy(), None if vv is None else vv.copy()) for p, _, vv in prev]
        res = orc.step(q, k, v)
        for h in range(Hkv):
            c = prev[h][0].shape[0]
            pool_v = v[:, h, :] if c == 0 else np.concatenate([prev[h][1], v[:, h, :]])
            for t in range(T):
                for g in range(h * G, (h + 1) * G):
                    np.testing.assert_allclose(res.o[t, g], pool_v.mean(axis=0), rtol=0,
                                               atol=1e-13)
            np.testing.assert_allclose(res.scores[h], np.full(c + T, G * T / (c + T)),
                                       rtol=0, atol=1e-13)
            np.testing.assert_array_equal(res.kept_positions[h],
                                          np.arange(min(B, (n + 1) * T)))


def check_front_end() -> None:
    """Q = X W_Q, K = X W_K, V = X W_V, then RoPE on q and k only.

    Worked by hand: hidden = 2, one head of d = 2, x = [1, 2]; W_Q = I gives
    q = [1, 2], W_K = [[0, 1], [1, 0]] gives k = [2, 1], W_V = [[1, 1],
    [1, -1]] gives v = [3, -1]; at position 3 with d = 2 the only pair turns by
    3 rad, so q becomes [cos 3 - 2 sin 3, sin 3 + 2 cos 3], k becomes
    [2 cos 3 - sin 3, 2 sin 3 + cos 3] and v stays.  Brute force with scalar
    loops on a random case; W_Q = I splits x into heads of d consecutive
    features; at position 0 the front end equals the plain projection."""
    x = np.array([[1.0, 2.0]])
    wq = np.eye(2)
    wk = np.array([[0.0, 1.0], [1.0, 0.0]])
    wv = np.array([[1.0, 1.0], [1.0, -1.0]])
    q, k, v = so.project_frame(x, wq, wk, wv, 1, 1, 2)
    assert np.array_equal(q[0, 0], [1.0, 2.0]) and np.array_equal(k[0, 0], [2.0, 1.0])
    assert np.array_equal(v[0, 0], [3.0, -1.0])
    c3, s3 = math.cos(3.0), math.sin(3.0)
    qr, kr, vr = so.frame_front_end(x, wq, wk, wv, 1, 1, 2, np.array([3]), 100.0)
    assert np.allclose(qr[0, 0], [c3 - 2 * s3, s3 + 2 * c3], rtol=0, atol=1e-15), qr
    assert np.allclose(kr[0, 0], [2 * c3 - s3, 2 * s3 + c3], rtol=0, atol=1e-15), kr
    assert np.array_equal(vr[0, 0], [3.0, -1.0])
    rng = np.random.default_rng(17)
    T, Hq, Hkv, d = 3, 2, 1, 4
    hidden = Hq * d
    x = rng.standard_normal((T, hidden))
    wq = rng.standard_normal((hidden, Hq * d))
    wk = rng.standard_normal((hidden, Hkv * d))
    wv = rng.standard_normal((hidden, Hkv * d))
    q, k, v = so.project_frame(x, wq, wk, wv, Hq, Hkv, d)
    for t in range(T):
        for g in range(Hq):
            for e in range(d):
                ref = sum(x[t, i] * wq[i, g * d + e] for i in range(hidden))
                assert abs(q[t, g, e] - ref) <= 1e-12, (t, g, e)
        for h in range(Hkv):
            for e in range(d):
                assert abs(k[t, h, e] - sum(x[t, i] * wk[i, h * d + e] for i in range(hidden))) <= 1e-12
                assert abs(v[t, h, e] - sum(x[t, i] * wv[i, h * d + e] for i in range(hidden))) <= 1e-12
    qi, _, _ = so.project_frame(x, np.eye(hidden), wk, wv, Hq, Hkv, d)
    for g in range(Hq):
        assert np.array_equal(qi[:, g, :], x[:, g * d:(g + 1) * d])
    q0, k0, v0 = so.frame_front_end(x, wq, wk, wv, Hq, Hkv, d, np.zeros(T), 1e6)
    assert np.allclose(q0, q, rtol=0, atol=1e-15) and np.allclose(k0, k, rtol=0, atol=1e-15)
    _, _, v9 = so.frame_front_end(x, wq, wk, wv, Hq, Hkv, d, np.arange(T) + 9, 1e4)
    assert np.array_equal(v9, v)


ALL_CHECKS = [
    check_hand_example,
    check_single_token_frame,
    check_uniform_attention_closed_form,
    check_gqa_head_mapping,
    check_probability_invariants,
    check_full_attention_equivalence,
    check_selection_and_caches,
    check_decode_attention,
    check_rope_and_rounding,
    check_recency_window,
    check_attention_mass,
    check_shared_layer_ranking,
    check_noncausal_closed_form,
    check_front_end,
]
