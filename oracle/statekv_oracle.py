"""Plain float64 CPU oracle of the StateKV per-layer video-prefill step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the build
entry point and the CPU-baseline leg of the benchmark may import or run this
module.  The GPU library never calls it, and it shares no code with the GPU
path: it decodes bfloat16 itself and uses numpy only.

What it computes (cited by page and section):

* rainbus summary, "方法步骤详情" (method steps): per transformer layer there is a
  detailed state holding every visual token seen so far and a compressed state
  of fixed capacity B.  For frame n the frame's queries attend, with a softmax,
  over the concatenation of the compressed memory and the frame's own keys;
  the frame's keys/values are then appended to the detailed state; finally the
  compressed state is refreshed by keeping the top-B of the candidate pool
  (previous compressed state plus every token of the frame), where a
  candidate's importance is the sum over queries of its attention weight.
* paperlayer summary, section 3.3: the same per-frame step (attend to the
  compressed memory plus the frame, append to the detailed state, keep the
  top-B candidates); virtual RoPE positions are kept even though the
  compressed state is physically shorter (the inputs arrive already rotated).
* paperlayer summary, App. A ("Protocol"): sinks are kept and pruned
  separately within each layer and KV head, from video-only attention of the
  current frame's queries.

Readings taken where the pages are silent (each one is listed in the design
notes of the repository):

* importance of candidate j for KV head h is the raw sum of softmax weights
  over the G query heads that share h and over the T queries of the frame
  (no mean, no decay, recomputed every frame);  ``shared=True`` sums over all
  query heads and keeps one position set for the whole layer;
* the frame's own keys are causal (query t sees frame tokens t' <= t); every
  compressed-state token is visible to every query;
* ties in importance are broken by the lower original position;
* while |C| + T <= B nothing is evicted;  the compressed state is kept in
  ascending position order and the candidate pool is [state ; frame];
* softmax scale s = 1/sqrt(d) on the logits unless given;
* query head g reads KV head floor(g / G).

Special case with a plain definition: when B is at least the number of history
tokens nothing is ever evicted and every frame's output equals dense causal
self-attention over the whole video (``full_causal_attention``, written
independently below).
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np


def decode_bf16(x) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 (exact); float arrays pass through."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# ----------------------------------------------------------------------------
# The four parts of the per-frame step, one function each
# ----------------------------------------------------------------------------

def frame_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                    n_state: int, scale: float, causal: bool = True):
    """Softmax attention of one query head's frame queries over [state ; frame].

    q: (T, d) queries of the frame; keys/values: (c + T, d) candidate pool whose
    first ``n_state`` rows are the compressed state and whose last T rows are
    the frame's own tokens in order.  Returns (P, O): P (T, c+T) row-normalised
    attention weights, O (T, d) = P @ values.  (rainbus method steps: softmax of
    the dot products of the queries with the concatenated keys, times values.)
    """
    T = q.shape[0]
    z = scale * (q @ keys.T)
    if causal:
        t = np.arange(T)
        frame_cols = np.arange(keys.shape[0] - n_state)
        hidden = frame_cols[None, :] > t[:, None]          # future frame tokens
        z[:, n_state:][hidden] = -np.inf
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    P = e / e.sum(axis=1, keepdims=True)
    return P, P @ values


def importance_scores(P_heads: List[np.ndarray]) -> np.ndarray:
    """sigma_j = sum over the given query heads and over all queries i of P_ij.

    (rainbus method steps: a candidate's importance is the sum over queries of
    its attention weight; paperlayer App. A: kept per layer and KV head, from
    the current frame's queries.)
    """
    sigma = np.zeros(P_heads[0].shape[1])
    for P in P_heads:
        sigma += P.sum(axis=0)
    return sigma


def layer_scores(per_head_scores: List[np.ndarray]) -> np.ndarray:
    """Importance for the layer-wide (SHARED) selection: the per-KV-head scores
    of one pool summed over every KV head, i.e. the sum over every query head
    of the layer and every frame query (reading of rainbus method steps, which
    defines importance as a sum over queries without fixing the heads; the
    default instead keeps one set per KV head, paperlayer App. A "Protocol").
    Every head's pool holds the same positions in the same order, so the
    entries align."""
    total = np.zeros_like(np.asarray(per_head_scores[0], dtype=np.float64))
    for s in per_head_scores:
        total = total + np.asarray(s, dtype=np.float64)
    return total


def select_top_b(scores: np.ndarray, positions: np.ndarray, budget: int) -> np.ndarray:
    """Indices (into the pool) of the top-``budget`` candidates, ascending position.

    Order: larger score first, then lower original position.  When the pool has
    at most ``budget`` candidates every one is kept.  (rainbus method steps and
    paperlayer section 3.3: keep the top-B of the previous state plus the frame.)
    """
    scores = np.asarray(scores)
    positions = np.asarray(positions)
    if scores.shape[0] <= budget:
        keep = np.arange(scores.shape[0])
    else:
        order = np.lexsort((positions, -scores))
        keep = order[:budget]
    return keep[np.argsort(positions[keep], kind="stable")]


# ----------------------------------------------------------------------------
# Streaming layer
# ----------------------------------------------------------------------------

def select_most_recent(positions: np.ndarray, budget: int) -> np.ndarray:
    """The recency rule StateKV is compared against: keep the ``budget``
    candidates with the largest original positions (a window over the most
    recent tokens; rainbus summary, core method: ReKV keeps the last R frames,
    StateKV selects by importance instead; paperlayer App. A.3 measures the gap
    between the two).  Returns pool indices in ascending position order."""
    positions = np.asarray(positions)
    keep = np.argsort(positions, kind="stable")[::-1][: min(budget, len(positions))]
    return np.sort(keep)


@dataclasses.dataclass
class FrameResult:
    o: np.ndarray                    # (T, Hq, d) float64 attention output
    scores: List[np.ndarray]         # per KV head: importance of each pool candidate
    pool_positions: List[np.ndarray] # per KV head: positions of the pool candidates
    kept_positions: List[np.ndarray] # per KV head: positions of C_n (ascending)
    probs: Optional[List[np.ndarray]] = None  # per query head: P (T, c+T) if requested


class StateKVOracle:
    """One layer of StateKV streaming prefill, float64, per KV head.

    Per KV head h it keeps the compressed state C^h (positions, keys, values,
    ascending position) and the detailed state D^h (every frame token).  Inputs
    are bfloat16 bit patterns (uint16) or float arrays, layouts Q [T][Hq][d],
    K/V [T][Hkv][d].  Stored rows keep their input representation so that
    cache contents can be compared bit for bit.
    """

    def __init__(self, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 frame_tokens: int, state_budget: int, scale: Optional[float] = None,
                 causal: bool = True, shared: bool = False, position_offset: int = 0,
                 detailed_capacity: Optional[int] = None, ring: bool = False,
                 recency: bool = False):
        if n_q_heads % n_kv_heads:
            raise ValueError("n_q_heads must be a multiple of n_kv_heads")
        self.Hq, self.Hkv, self.d = n_q_heads, n_kv_heads, head_dim
        self.G = n_q_heads // n_kv_heads
        self.T, self.B = frame_tokens, state_budget
        self.scale = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
        self.causal, self.shared = causal, shared
        self.offset = position_offset
        self.capacity = detailed_capacity
        self.ring = ring
        self.recency = recency  # keep the most recent B candidates instead
        self.n = 0
        self.c_pos = [np.zeros(0, dtype=np.int64) for _ in range(n_kv_heads)]
        self.c_k: List[Optional[np.ndarray]] = [None] * n_kv_heads
        self.c_v: List[Optional[np.ndarray]] = [None] * n_kv_heads
        self.d_pos: List[List[np.ndarray]] = [[] for _ in range(n_kv_heads)]
        self.d_k: List[List[np.ndarray]] = [[] for _ in range(n_kv_heads)]
        self.d_v: List[List[np.ndarray]] = [[] for _ in range(n_kv_heads)]

    # -- state access --------------------------------------------------------
    def state(self, h: int):
        """(positions, keys, values) of C^h in ascending position order."""
        if self.c_k[h] is None:
            return self.c_pos[h], None, None
        return self.c_pos[h], self.c_k[h], self.c_v[h]

    def load_state(self, frames_seen: int, positions, keys, values) -> None:
        """Replace C by the given per-head (positions, keys, values) lists.

        Used to run one oracle step from a state produced elsewhere (a
        teacher-forced comparison).  The detailed state is left untouched.
        """
        self.n = frames_seen
        for h in range(self.Hkv):
            pos = np.asarray(positions[h], dtype=np.int64)
            order = np.argsort(pos, kind="stable")
            self.c_pos[h] = pos[order]
            self.c_k[h] = np.asarray(keys[h])[order]
            self.c_v[h] = np.asarray(values[h])[order]

    def detailed(self, h: int):
        """(positions, keys, values) of D^h: every frame token, in arrival order.

        With ``ring`` and a capacity, only the last ``capacity`` tokens are held.
        """
        if not self.d_pos[h]:
            return np.zeros(0, dtype=np.int64), None, None
        pos = np.concatenate(self.d_pos[h])
        k = np.concatenate(self.d_k[h])
        v = np.concatenate(self.d_v[h])
        if self.ring and self.capacity is not None and pos.shape[0] > self.capacity:
            pos, k, v = pos[-self.capacity:], k[-self.capacity:], v[-self.capacity:]
        return pos, k, v

    # -- the per-frame step --------------------------------------------------
    def step(self, q, k, v, keep_probs: bool = False) -> FrameResult:
        T, Hq, Hkv, d, G = self.T, self.Hq, self.Hkv, self.d, self.G
        q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
        if q.shape != (T, Hq, d) or k.shape != (T, Hkv, d) or v.shape != (T, Hkv, d):
            raise ValueError("frame shapes do not match the layer")
        if (self.capacity is not None and not self.ring
                and (self.n + 1) * T > self.capacity):
            raise ValueError("detailed cache capacity exceeded")
        qf, kf, vf = decode_bf16(q), decode_bf16(k), decode_bf16(v)
        positions = self.offset + self.n * T + np.arange(T, dtype=np.int64)

        o = np.zeros((T, Hq, d))
        scores, pools, probs = [], [], []
        raw_k, raw_v = [], []
        for h in range(Hkv):
            # candidate pool [C^h_{n-1} ; frame n] in ascending position
            c = self.c_pos[h].shape[0]
            pool_pos = np.concatenate([self.c_pos[h], positions])
            if c:
                pk = np.concatenate([self.c_k[h], k[:, h, :]])
                pv = np.concatenate([self.c_v[h], v[:, h, :]])
            else:
                pk, pv = k[:, h, :].copy(), v[:, h, :].copy()
            keys, values = decode_bf16(pk), decode_bf16(pv)
            P_group = []
            for g in range(h * G, (h + 1) * G):
                P, o[:, g, :] = frame_attention(qf[:, g, :], keys, values, c,
                                                self.scale, self.causal)
                P_group.append(P)
            scores.append(importance_scores(P_group))
            pools.append(pool_pos)
            raw_k.append(pk)
            raw_v.append(pv)
            if keep_probs:
                probs.extend(P_group)

        # the frame joins the detailed state (every token, every head)
        for h in range(Hkv):
            self.d_pos[h].append(positions.copy())
            self.d_k[h].append(k[:, h, :].copy())
            self.d_v[h].append(v[:, h, :].copy())

        # the compressed state becomes the top-B of the pool
        if self.shared:
            keep_shared = select_top_b(layer_scores(scores), pools[0], self.B)
        kept = []
        for h in range(Hkv):
            if self.recency:
                keep = select_most_recent(pools[h], self.B)
            elif self.shared:
                keep = keep_shared
            else:
                keep = select_top_b(scores[h], pools[h], self.B)
            self.c_pos[h] = pools[h][keep]
            self.c_k[h] = raw_k[h][keep]
            self.c_v[h] = raw_v[h][keep]
            kept.append(self.c_pos[h].copy())
        self.n += 1
        return FrameResult(o, scores, pools, kept, probs if keep_probs else None)


# ----------------------------------------------------------------------------
# Independent reference: dense causal self-attention over the whole video
# ----------------------------------------------------------------------------

def full_causal_attention(q_all, k_all, v_all, scale: Optional[float] = None,
                          first_query: int = 0) -> np.ndarray:
    """Full causal self-attention: query at position p sees every key p' <= p.

    q_all: (M, Hq, d) queries for positions first_query .. first_query+M-1;
    k_all, v_all: (L, Hkv, d) keys/values for positions 0 .. L-1, with
    L >= first_query + M.  Query head g reads KV head floor(g / (Hq/Hkv)).
    Returns (M, Hq, d) float64.  This is the quadratic baseline the pages
    compare against (rainbus prerequisites: every position attends to all
    previous positions).
    """
    q = decode_bf16(q_all)
    k = decode_bf16(k_all)
    v = decode_bf16(v_all)
    M, Hq, d = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    qpos = first_query + np.arange(M)
    kpos = np.arange(L)
    visible = kpos[None, :] <= qpos[:, None]
    out = np.zeros((M, Hq, d))
    for g in range(Hq):
        h = g // G
        z = s * (q[:, g, :] @ k[:, h, :].T)
        z = np.where(visible, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        e = np.exp(z)
        out[:, g, :] = (e / e.sum(axis=1, keepdims=True)) @ v[:, h, :]
    return out



# ----------------------------------------------------------------------------
# Decoding over the detailed state
# ----------------------------------------------------------------------------

def decode_attention(q, d_keys, d_values, scale: Optional[float] = None) -> np.ndarray:
    """Attention of text-token queries over every token of the detailed state.

    Once all frames are in, text generation is ordinary autoregressive decoding
    conditioned on the detailed state D_N, which holds every original video
    token (gist.science/nl, "Het Proces", decoding item; rainbus summary,
    "核心方法" core method: standard text decoding over all video tokens after
    the incremental cache build).  The text comes after the video, so every D
    token is visible to every query; the queries' own text context (prompt and
    generated tokens) is the standard decoder's cache and is not part of this
    routine.

    q: (M, Hq, d) queries; d_keys, d_values: (L, Hkv, d) the detailed state in
    any token order (softmax attention does not depend on it).  Query head g
    reads KV head floor(g / (Hq/Hkv)).  Returns (M, Hq, d) float64.
    """
    q = decode_bf16(q)
    k = decode_bf16(d_keys)
    v = decode_bf16(d_values)
    M, Hq, d = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = np.zeros((M, Hq, d))
    for g in range(Hq):
        h = g // G
        z = s * (q[:, g, :] @ k[:, h, :].T)
        z = z - z.max(axis=1, keepdims=True)
        e = np.exp(z)
        out[:, g, :] = (e / e.sum(axis=1, keepdims=True)) @ v[:, h, :]
    return out


# ----------------------------------------------------------------------------
# Rotary position embedding at the tokens' original positions
# ----------------------------------------------------------------------------

def rope_at_positions(x, positions, theta: float, scaling: float = 1.0) -> np.ndarray:
    """Rotary position embedding of queries or keys at their original
    positions, in float64.

    The compressed state is physically shorter than the video but its tokens
    keep the positions they arrived with, and the same RoPE scaling serves
    cache building and text generation (paperlayer summary, section 3.3;
    rainbus summary, prerequisites, "RoPE缩放": scaling stretches positions
    past the trained length and must not change between the two phases).
    Readings: the half-split pairing (component i pairs with i + d/2) at
    frequency theta^(-2i/d); ``scaling`` divides the position (linear
    interpolation; the pages give no value, 1 = none).

    x: (T, H, d) values (bf16 bits or floats); positions: (T,).  Written as the
    complex product (x_i + j x_{i+d/2}) * exp(j * angle).
    """
    x = decode_bf16(x)
    d = x.shape[-1]
    half = d // 2
    freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = (np.asarray(positions, dtype=np.float64)[:, None] / float(scaling)) * freq[None, :]
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * ang)[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


def project_frame(x, w_q, w_k, w_v, n_q_heads: int, n_kv_heads: int, head_dim: int):
    """The frame's queries, keys and values from its visual-token hidden states.

    rainbus summary, method steps: for frame n, Q_n = X_n W_Q, K_n = X_n W_K,
    V_n = X_n W_V, where X_n holds the hidden states of the frame's visual
    tokens.  x: (T, hidden); w_q: (hidden, Hq*d); w_k, w_v: (hidden, Hkv*d)
    (bf16 bits or floats).  Output columns h*d .. h*d+d-1 form head h.  No
    bias (the pages write none).  Returns float64 q (T, Hq, d), k and v
    (T, Hkv, d), unrotated.
    """
    x = decode_bf16(x)
    T = x.shape[0]
    q = (x @ decode_bf16(w_q)).reshape(T, n_q_heads, head_dim)
    k = (x @ decode_bf16(w_k)).reshape(T, n_kv_heads, head_dim)
    v = (x @ decode_bf16(w_v)).reshape(T, n_kv_heads, head_dim)
    return q, k, v


def frame_front_end(x, w_q, w_k, w_v, n_q_heads: int, n_kv_heads: int, head_dim: int,
                    positions, theta: float, scaling: float = 1.0):
    """Projection then rotary embedding of q and k at the tokens' original
    positions (paperlayer section 3.3: positions stay virtual; rainbus
    prerequisites: one RoPE scaling for cache building and generation); v is
    not rotated.  Returns float64 (q, k, v) before any rounding."""
    q, k, v = project_frame(x, w_q, w_k, w_v, n_q_heads, n_kv_heads, head_dim)
    return (rope_at_positions(q, positions, theta, scaling),
            rope_at_positions(k, positions, theta, scaling), v)


def attention_mass_diagnostics(scores, n_history: int, budget: int, prev_kept=None):
    """The App. A measurements of one frame (paperlayer summary, App. A.1-A.3).

    ``scores``: importance of every token seen through this frame, in
    ascending position, aggregated over the layer's query heads and the
    frame's queries under attention over every available token (App. A
    "Protocol"); the first ``n_history`` tokens belong to earlier frames.
    ``prev_kept``: boolean mask over those earlier tokens, the set this
    function returned for the previous frame (None before it).

    Returns (topb_mass, recency_mass, recall, kept):

    * topb_mass (A.1, concentration): the share of the historical attention
      mass held by the ``budget`` largest historical importances;
    * recency_mass (A.3, recency retention): the share held by the ``budget``
      most recent historical tokens;
    * kept (A.2, the oracle state): the top-``budget`` of all tokens through
      this frame, ties to the lower position, as a boolean mask;
    * recall (A.2, weighted candidate-pool recall): the share of the kept
      set's importance that lies in the candidate pool, i.e. the previous
      frame's kept set plus this frame's tokens.

    NaN where a share has no mass to divide (no earlier frame).
    """
    scores = np.asarray(scores, dtype=np.float64)
    L, c = scores.shape[0], int(n_history)
    b = int(budget)
    hist = scores[:c]
    total = hist.sum()
    bb = min(b, c)
    if c == 0 or total <= 0.0:
        topb = recency = math.nan
    else:
        topb = np.sort(hist)[::-1][:bb].sum() / total
        recency = hist[c - bb:].sum() / total
    kept = np.zeros(L, dtype=bool)
    kept[select_top_b(scores, np.arange(L), b)] = True
    pool = np.ones(L, dtype=bool)
    if prev_kept is not None:
        pool[:c] = np.asarray(prev_kept, dtype=bool)[:c]
    kept_mass = scores[kept].sum()
    recall = scores[kept & pool].sum() / kept_mass if kept_mass > 0.0 else math.nan
    return float(topb), float(recency), float(recall), kept


def round_to_bf16(x) -> np.ndarray:
    """float64 -> nearest bfloat16 (8 significant bits, ties to even), as
    uint16 bit patterns.  Normal range only (finite values whose magnitude is
    zero or at least 2^-126)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                    # x = m 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(m * 256.0), e - 8)  # np.rint: ties to even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
