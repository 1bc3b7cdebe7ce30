"""Plant plausible mistakes in the oracle (on the CPU) and show the pins catch them.

Each mutant replaces one function of the oracle module for the duration of a
test; at least one of the pins in oracle_pins must then fail.
"""

import numpy as np
import pytest

import oracle.statekv_oracle as so
import oracle_pins

_orig_attention = so.frame_attention
_orig_scores = so.importance_scores
_orig_select = so.select_top_b
_orig_layer = so.layer_scores


def attention_causal_off_by_one(q, keys, values, n_state, scale, causal=True):
    T = q.shape[0]
    z = scale * (q @ keys.T)
    t = np.arange(T)
    cols = np.arange(keys.shape[0] - n_state)
    z[:, n_state:][cols[None, :] >= t[:, None]] = -np.inf   # hides the token itself
    z[:, n_state:][0, 0] = 0.0 if T else 0.0                # keep row 0 finite
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    P = e / e.sum(axis=1, keepdims=True)
    return P, P @ values


def attention_mask_on_state_too(q, keys, values, n_state, scale, causal=True):
    T = q.shape[0]
    z = scale * (q @ keys.T)
    # treat the whole pool as if it were the frame: state tokens become causal
    cols = np.arange(keys.shape[0])
    z[cols[None, :] > (np.arange(T)[:, None] + n_state // 2)] = -np.inf
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    P = e / e.sum(axis=1, keepdims=True)
    return P, P @ values


def attention_no_scale(q, keys, values, n_state, scale, causal=True):
    return _orig_attention(q, keys, values, n_state, 1.0, causal)


def attention_transposed_values(q, keys, values, n_state, scale, causal=True):
    P, _ = _orig_attention(q, keys, values, n_state, scale, causal)
    # uses the values of the reversed pool
    return P, P @ values[::-1]


def scores_mean_over_queries(P_heads):
    return _orig_scores(P_heads) / P_heads[0].shape[0]


def scores_first_head_only(P_heads):
    return P_heads[0].sum(axis=0)


def scores_row_sums_broadcast(P_heads):
    # sums the wrong axis, then spreads it over the pool
    s = sum(P.sum(axis=1).sum() for P in P_heads)
    return np.full(P_heads[0].shape[1], s / P_heads[0].shape[1])


def select_ties_to_higher_position(scores, positions, budget):
    return _orig_select(scores, -np.asarray(positions), budget)[::-1]


def select_smallest_scores(scores, positions, budget):
    return _orig_select(-np.asarray(scores), positions, budget)


def select_off_by_one_budget(scores, positions, budget):
    return _orig_select(scores, positions, max(1, budget - 1))


def attention_causal_always(q, keys, values, n_state, scale, causal=True):
    return _orig_attention(q, keys, values, n_state, scale, True)


def layer_first_head_only(per_head_scores):
    return np.asarray(per_head_scores[0], dtype=np.float64)


def layer_last_head_only(per_head_scores):
    return np.asarray(per_head_scores[-1], dtype=np.float64)


def layer_headwise_max(per_head_scores):
    return np.max(np.asarray(per_head_scores, dtype=np.float64), axis=0)


MUTANTS = [
    ("frame_attention", attention_causal_off_by_one),
    ("frame_attention", attention_mask_on_state_too),
    ("frame_attention", attention_no_scale),
    ("frame_attention", attention_transposed_values),
    ("importance_scores", scores_mean_over_queries),
    ("importance_scores", scores_first_head_only),
    ("importance_scores", scores_row_sums_broadcast),
    ("select_top_b", select_ties_to_higher_position),
    ("select_top_b", select_smallest_scores),
    ("select_top_b", select_off_by_one_budget),
    ("frame_attention", attention_causal_always),
    ("layer_scores", layer_first_head_only),
    ("layer_scores", layer_last_head_only),
    ("layer_scores", layer_headwise_max),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_pins_catch_mutant(monkeypatch, name, mutant):
    monkeypatch.setattr(so, name, mutant)
    failures = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            failures.append(check.__name__)
    assert failures, f"no pin caught the mutant {mutant.__name__}"


def test_gqa_mapping_mutant(monkeypatch):
    """A wrong query-head -> KV-head mapping (g % Hkv instead of g // G)."""
    orig_step = so.StateKVOracle.step

    def step(self, q, k, v, keep_probs=False):
        # permute query heads so head g is served by KV head g % Hkv
        perm = np.array([(g % self.Hkv) * self.G + g // self.Hkv for g in range(self.Hq)])
        res = orig_step(self, np.asarray(q)[:, perm, :], k, v, keep_probs)
        inv = np.argsort(perm)
        res.o = res.o[:, inv, :]
        return res

    monkeypatch.setattr(so.StateKVOracle, "step", step)
    with pytest.raises(AssertionError):
        oracle_pins.check_gqa_head_mapping()


_orig_decode = so.decode_attention


def decode_drops_last_token(q, d_keys, d_values, scale=None):
    return _orig_decode(q, np.asarray(d_keys)[:-1], np.asarray(d_values)[:-1], scale)


def decode_heads_modulo(q, d_keys, d_values, scale=None):
    q = np.asarray(q)
    Hq, Hkv = q.shape[1], np.asarray(d_keys).shape[1]
    G = Hq // Hkv
    perm = np.array([(g % Hkv) * G + g // Hkv for g in range(Hq)])
    return _orig_decode(q[:, perm, :], d_keys, d_values, scale)[:, np.argsort(perm), :]


def decode_unscaled(q, d_keys, d_values, scale=None):
    return _orig_decode(q, d_keys, d_values, 1.0)


def decode_causal(q, d_keys, d_values, scale=None):
    # as if query m stood at position m of the video
    M = np.asarray(q).shape[0]
    out = np.stack([_orig_decode(np.asarray(q)[m:m + 1], np.asarray(d_keys)[:m + 1],
                                 np.asarray(d_values)[:m + 1], scale)[0] for m in range(M)])
    return out


@pytest.mark.parametrize("mutant", [decode_drops_last_token, decode_heads_modulo,
                                     decode_unscaled, decode_causal],
                         ids=lambda f: f.__name__)
def test_decode_pin_catches_mutant(monkeypatch, mutant):
    monkeypatch.setattr(so, "decode_attention", mutant)
    with pytest.raises(AssertionError):
        oracle_pins.check_decode_attention()


_orig_rope = so.rope_at_positions
_orig_round = so.round_to_bf16


def rope_adjacent_pairs(x, positions, theta, scaling=1.0):
    # pairs (2i, 2i+1) instead of (i, i + d/2)
    x = so.decode_bf16(x)
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inv = np.argsort(perm)
    return _orig_rope(x[..., perm], positions, theta, scaling)[..., inv]


def rope_wrong_frequency(x, positions, theta, scaling=1.0):
    return _orig_rope(x, positions, theta ** 2, scaling)


def rope_sign_flipped(x, positions, theta, scaling=1.0):
    return _orig_rope(x, -np.asarray(positions, dtype=np.float64), theta, scaling)


def rope_scaling_multiplies(x, positions, theta, scaling=1.0):
    return _orig_rope(x, np.asarray(positions, dtype=np.float64) * scaling, theta, 1.0)


def round_truncates(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def round_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.sign(m) * np.floor(np.abs(m) * 256.0 + 0.5), e - 8)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("name,mutant", [
    ("rope_at_positions", rope_adjacent_pairs), ("rope_at_positions", rope_wrong_frequency),
    ("rope_at_positions", rope_sign_flipped), ("rope_at_positions", rope_scaling_multiplies),
    ("round_to_bf16", round_truncates), ("round_to_bf16", round_ties_away)],
    ids=lambda v: v if isinstance(v, str) else v.__name__)
def test_rope_pin_catches_mutant(monkeypatch, name, mutant):
    monkeypatch.setattr(so, name, mutant)
    with pytest.raises(AssertionError):
        oracle_pins.check_rope_and_rounding()


_orig_recent = so.select_most_recent


def recent_keeps_oldest(positions, budget):
    p = np.asarray(positions)
    return np.sort(np.argsort(p, kind="stable")[: min(budget, len(p))])


def recent_off_by_one(positions, budget):
    return _orig_recent(positions, max(1, budget - 1))


@pytest.mark.parametrize("mutant", [recent_keeps_oldest, recent_off_by_one],
                         ids=lambda f: f.__name__)
def test_recency_pin_catches_mutant(monkeypatch, mutant):
    monkeypatch.setattr(so, "select_most_recent", mutant)
    with pytest.raises(AssertionError):
        oracle_pins.check_recency_window()


_orig_mass = so.attention_mass_diagnostics


def mass_recency_takes_oldest(scores, n_history, budget, prev_kept=None):
    t, _, rc, kept = _orig_mass(scores, n_history, budget, prev_kept)
    h = np.asarray(scores, dtype=np.float64)[:n_history]
    r = h[: min(budget, n_history)].sum() / h.sum() if n_history else float("nan")
    return t, r, rc, kept


def mass_history_includes_frame(scores, n_history, budget, prev_kept=None):
    L = len(scores)
    t, r, _, _ = _orig_mass(scores, L, budget, None)
    _, _, rc, kept = _orig_mass(scores, n_history, budget, prev_kept)
    return t, r, rc, kept


def mass_recall_unweighted(scores, n_history, budget, prev_kept=None):
    t, r, _, kept = _orig_mass(scores, n_history, budget, prev_kept)
    pool = np.ones(len(kept), dtype=bool)
    if prev_kept is not None:
        pool[:n_history] = np.asarray(prev_kept, dtype=bool)[:n_history]
    return t, r, float((kept & pool).sum() / kept.sum()), kept


def mass_pool_without_frame(scores, n_history, budget, prev_kept=None):
    t, r, _, kept = _orig_mass(scores, n_history, budget, prev_kept)
    s = np.asarray(scores, dtype=np.float64)
    pool = np.zeros(len(kept), dtype=bool)
    pool[:n_history] = True if prev_kept is None else np.asarray(prev_kept, dtype=bool)
    return t, r, float(s[kept & pool].sum() / s[kept].sum()), kept


def mass_keeps_smallest(scores, n_history, budget, prev_kept=None):
    s = -np.asarray(scores, dtype=np.float64)
    t, r, rc, kept = _orig_mass(s, n_history, budget, prev_kept)
    return t, r, rc, kept


@pytest.mark.parametrize("mutant", [mass_recency_takes_oldest, mass_history_includes_frame,
                                    mass_recall_unweighted, mass_pool_without_frame,
                                    mass_keeps_smallest], ids=lambda f: f.__name__)
def test_attention_mass_pin_catches_mutant(monkeypatch, mutant):
    monkeypatch.setattr(so, "attention_mass_diagnostics", mutant)
    with pytest.raises(AssertionError):
        oracle_pins.check_attention_mass()


_orig_project = so.project_frame
_orig_front = so.frame_front_end


def project_k_v_swapped(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim):
    q, k, v = _orig_project(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim)
    return q, v, k


def project_weights_transposed(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim):
    x = so.decode_bf16(x)
    T = x.shape[0]
    q = (x @ so.decode_bf16(w_q).T).reshape(T, n_q_heads, head_dim)
    _, k, v = _orig_project(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim)
    return q, k, v


def project_heads_interleaved(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim):
    q, k, v = _orig_project(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim)
    T = q.shape[0]
    q = q.reshape(T, head_dim, n_q_heads).transpose(0, 2, 1)
    return q, k, v


def front_end_rotates_v(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim, positions, theta,
                        scaling=1.0):
    q, k, v = _orig_front(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim, positions, theta,
                          scaling)
    return q, k, so.rope_at_positions(v, positions, theta, scaling)


def front_end_keys_unrotated(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim, positions, theta,
                             scaling=1.0):
    q, _, v = _orig_front(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim, positions, theta,
                          scaling)
    _, k, _ = _orig_project(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim)
    return q, k, v


@pytest.mark.parametrize("name,mutant", [
    ("project_frame", project_k_v_swapped), ("project_frame", project_weights_transposed),
    ("project_frame", project_heads_interleaved), ("frame_front_end", front_end_rotates_v),
    ("frame_front_end", front_end_keys_unrotated)],
    ids=lambda v: v if isinstance(v, str) else v.__name__)
def test_front_end_pin_catches_mutant(monkeypatch, name, mutant):
    monkeypatch.setattr(so, name, mutant)
    with pytest.raises(AssertionError):
        oracle_pins.check_front_end()
