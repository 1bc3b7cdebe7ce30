"""Seeded synthetic video-frame tokens (queries, keys, values) in bfloat16.

What the tokens stand for
-------------------------
The pages (paperlayer.ai summary of "Linear Scaling Video VLMs for Long Video
Understanding", section 3.3; rainbus summary, method-steps section) describe a
frame-by-frame cache builder: frame n produces T visual tokens, whose per-layer
queries/keys/values come from a frozen backbone, with rotary position
embedding applied at each token's original ("virtual") position.  No weights
or videos are available here, so these tokens are synthetic:

* every element of Q, K and V is drawn iid N(0, 1) in float64;
* Q and K are rotated (rotary embedding, half-split pairing, inverse
  frequencies theta^(-2i/d), no scaling) at position p = offset + n*T + t;
* optionally, "temporal sinks" are planted: a few keys among the first four
  frames get a shared unit direction u (magnitude 4) added, and every query of
  every frame gets 0.5*u, so those keys stay salient for the whole stream
  (the pages' hypothesis of a small, slowly evolving set of long-range sink
  tokens; paperlayer section 3.1 and App. A.3);
* the result is rounded float64 -> float32 -> bfloat16, round-to-nearest-even
  at each step, and returned as uint16 bit patterns.

Random streams (numpy PCG64): ``default_rng(seed)`` draws the sink direction u
and then the sink positions; frame n uses ``default_rng([seed, n])`` and draws
Q (T, Hq, d), then K (T, Hkv, d), then V (T, Hkv, d).

Layouts are token-major, the natural output of a QKV projection:
Q ``[T][Hq][d]``, K and V ``[T][Hkv][d]``.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Iterator, Optional, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# bfloat16 helpers (bit patterns carried as uint16)
# ----------------------------------------------------------------------------

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 -> float32 -> bfloat16 (round-to-nearest-even each step).

    Returns the bfloat16 bit patterns as uint16.  Inputs must be finite.
    """
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


# ----------------------------------------------------------------------------
# Rotary embedding at original positions (input preparation, not the method)
# ----------------------------------------------------------------------------

def rope_rotate(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate the last axis of ``x`` (size d, even) at the given positions.

    ``x`` has shape (T, H, d) and ``positions`` shape (T,).  Pairs are
    (x_i, x_{i+d/2}) for i < d/2, rotated by the angle p * theta^(-2i/d).
    Computed in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("head_dim must be even for the rotary embedding")
    half = d // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    lo = x[..., :half]
    hi = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = lo * cos - hi * sin
    out[..., half:] = lo * sin + hi * cos
    return out


# ----------------------------------------------------------------------------
# Workload description
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class FrameSpec:
    """Shape and seeding of one synthetic layer stream."""

    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    frame_tokens: int
    n_frames: int
    state_budget: int
    rope_theta: float
    seed: int
    sinks: bool = False
    position_offset: int = 0
    sink_frames: int = 4
    sink_fraction: float = 0.01
    sink_magnitude: float = 4.0
    query_sink: float = 0.5
    n_layers: int = 1
    layer_seed_base: Optional[int] = None  # seed of layer l = layer_seed_base + l
    # False: queries and keys are left unrotated (for a consumer that applies
    # the rotary embedding itself); the draws are the same either way
    rotated: bool = True

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def for_layer(self, layer: int) -> "FrameSpec":
        """The single-layer spec of layer ``layer`` (its own seed)."""
        if self.layer_seed_base is None:
            if layer != 0:
                raise ValueError("single-layer workload")
            return self
        return dataclasses.replace(self, seed=self.layer_seed_base + layer,
                                   n_layers=1, layer_seed_base=None)

    def replace(self, **kw) -> "FrameSpec":
        return dataclasses.replace(self, **kw)


# Workloads shaped like the pages' InternVL3-class backbones: 256 visual tokens
# per frame (paperlayer App. A.3 equates 256 tokens with one frame), state
# budgets 1024-4096 (rainbus method steps; paperlayer section 4), up to 512
# frames at 1 FPS (rainbus reproducibility section).  Head shapes are those of
# the 1B / 2B / 8B backbones.
WORKLOADS: Dict[str, FrameSpec] = {
    # 2 query heads sharing 1 KV head, d=64, 8 frames of 16 tokens, B=32.
    "tiny": FrameSpec(2, 1, 64, 16, 8, 32, 1e4, 0, sinks=False),
    # B=128 >= all history: no eviction ever happens.
    "tiny_full": FrameSpec(2, 1, 64, 16, 8, 128, 1e4, 0, sinks=False),
    # InternVL3-1B-like layer.
    "internvl3_1b_layer": FrameSpec(14, 2, 64, 256, 64, 1024, 1e6, 1, sinks=True),
    # InternVL3-8B-like layer at scale: 512 frames = 131072 video tokens.
    "internvl3_8b_layer": FrameSpec(28, 4, 128, 256, 512, 4096, 1e6, 2, sinks=True),
    # InternVL3-2B-like full depth: 28 layers, seed of layer l = 3 + l.
    "internvl3_2b_28layers": FrameSpec(12, 2, 128, 256, 256, 2048, 1e6, 3, sinks=True,
                                       n_layers=28, layer_seed_base=3),
    # Crossover sweep at the 1B shape (budget and frame count are swept).
    "crossover_1b": FrameSpec(14, 2, 64, 256, 512, 1024, 1e6, 4, sinks=False),
}


def workload(name: str, **overrides) -> FrameSpec:
    spec = WORKLOADS[name]
    return spec.replace(**overrides) if overrides else spec


# ----------------------------------------------------------------------------
# Sinks and frames
# ----------------------------------------------------------------------------

def sink_plan(spec: FrameSpec) -> Tuple[np.ndarray, np.ndarray]:
    """(u, positions): the shared unit sink direction and the sorted sink positions.

    positions are global positions in [offset, offset + sink_frames*T); their
    count is round(sink_fraction * sink_frames * T).  Without sinks both are empty.
    """
    if not spec.sinks:
        return np.zeros(0), np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng(spec.seed)
    u = rng.standard_normal(spec.head_dim)
    u = u / np.linalg.norm(u)
    pool = spec.sink_frames * spec.frame_tokens
    k = int(round(spec.sink_fraction * pool))
    pos = np.sort(rng.choice(pool, size=k, replace=False)).astype(np.int64)
    return u, pos + spec.position_offset


def frame_f64(spec: FrameSpec, n: int,
              plan: Optional[Tuple[np.ndarray, np.ndarray]] = None):
    """Frame n before rounding: (q, k, v) float64, shapes (T,Hq,d), (T,Hkv,d)x2."""
    T, Hq, Hkv, d = spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    rng = np.random.default_rng([spec.seed, n])
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    positions = spec.position_offset + n * T + np.arange(T, dtype=np.int64)
    if spec.rotated:
        q = rope_rotate(q, positions, spec.rope_theta)
        k = rope_rotate(k, positions, spec.rope_theta)
    if spec.sinks:
        u, spos = plan if plan is not None else sink_plan(spec)
        q = q + spec.query_sink * u
        hit = np.isin(positions, spos)
        if hit.any():
            k[hit] += spec.sink_magnitude * u
    return q, k, v


def frame(spec: FrameSpec, n: int,
          plan: Optional[Tuple[np.ndarray, np.ndarray]] = None):
    """Frame n as bfloat16 bit patterns: (q, k, v) uint16, C-contiguous."""
    q, k, v = frame_f64(spec, n, plan)
    return f64_to_bf16_bits(q), f64_to_bf16_bits(k), f64_to_bf16_bits(v)


def text_queries(spec: FrameSpec, n_tokens: int, index: int = 0) -> np.ndarray:
    """Queries of n_tokens text tokens that follow the video, as bf16 bits,
    shape (n_tokens, Hq, d): N(0,1) values from ``default_rng([seed, -1,
    index])``, RoPE at positions offset + N*T + i, plus the same query-side
    sink component as the frames' queries."""
    T, Hq, d = spec.frame_tokens, spec.n_q_heads, spec.head_dim
    rng = np.random.default_rng([spec.seed, 2**31 - 1, index])
    q = rng.standard_normal((n_tokens, Hq, d))
    positions = spec.position_offset + spec.n_frames * T + np.arange(n_tokens, dtype=np.int64)
    if spec.rotated:
        q = rope_rotate(q, positions, spec.rope_theta)
    if spec.sinks:
        u, _ = sink_plan(spec)
        q = q + spec.query_sink * u
    return f64_to_bf16_bits(q)


def hidden_width(spec: FrameSpec) -> int:
    """Width of the visual-token hidden states entering the projection: the
    pages give no model widths, so it is taken as Hq * d (which is the width
    of the InternVL3-class backbones' language models)."""
    return spec.n_q_heads * spec.head_dim


def hidden_states(spec: FrameSpec, n: int) -> np.ndarray:
    """Hidden states X_n of frame n's T visual tokens, (T, hidden) bf16 bits:
    N(0, 1) draws from ``default_rng([seed, 2^31 - 2, n])``."""
    rng = np.random.default_rng([spec.seed, 2**31 - 2, n])
    return f64_to_bf16_bits(rng.standard_normal((spec.frame_tokens, hidden_width(spec))))


def projection_weights(spec: FrameSpec) -> np.ndarray:
    """The layer's projection weights packed output-major, bf16 bits of shape
    ((Hq + 2 Hkv) d, hidden): row r holds the weights of output feature r,
    rows ordered Q heads, K heads, V heads (d rows per head), so W_Q is the
    transpose of rows [0, Hq d).  N(0, 1/hidden) draws (unit-variance
    outputs for unit-variance inputs) from ``default_rng([seed, 2^31 - 3])``."""
    hid = hidden_width(spec)
    rows = (spec.n_q_heads + 2 * spec.n_kv_heads) * spec.head_dim
    rng = np.random.default_rng([spec.seed, 2**31 - 3])
    return f64_to_bf16_bits(rng.standard_normal((rows, hid)) / np.sqrt(hid))


def split_projection_weights(spec: FrameSpec, w: np.ndarray):
    """(W_Q, W_K, W_V) in the (hidden, out) orientation of Q = X W_Q, from
    the packed output-major rows of projection_weights."""
    qd, kd = spec.n_q_heads * spec.head_dim, spec.n_kv_heads * spec.head_dim
    return w[:qd].T, w[qd:qd + kd].T, w[qd + kd:].T


def frames(spec: FrameSpec, start: int = 0, stop: Optional[int] = None
           ) -> Iterator[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
    """Frames start..stop-1 (default: all) as bfloat16 bit patterns."""
    stop = spec.n_frames if stop is None else stop
    plan = sink_plan(spec)
    for n in range(start, stop):
        yield frame(spec, n, plan)


def _frame_job(args):
    spec, n = args
    return frame(spec, n)


def stacked_frames(spec: FrameSpec, start: int = 0, stop: Optional[int] = None,
                   workers: int = 1):
    """Frames start..stop-1 stacked: q (N,T,Hq,d), k and v (N,T,Hkv,d), uint16.

    With workers > 1 the frames are drawn in a process pool; every frame has
    its own random stream, so the result does not depend on the worker count.
    """
    stop = spec.n_frames if stop is None else stop
    n = stop - start
    T, Hq, Hkv, d = spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    q = np.empty((n, T, Hq, d), dtype=np.uint16)
    k = np.empty((n, T, Hkv, d), dtype=np.uint16)
    v = np.empty((n, T, Hkv, d), dtype=np.uint16)
    jobs = [(spec, i) for i in range(start, stop)]
    if workers > 1 and n > 1:
        import multiprocessing as mp
        # spawned, never forked: a caller that already initialised the GPU
        # (or runs under a profiler that did) must not hand its state down
        with mp.get_context("spawn").Pool(min(workers, n)) as pool:
            for i, (a, b, c) in enumerate(pool.imap(_frame_job, jobs, chunksize=4)):
                q[i], k[i], v[i] = a, b, c
    else:
        plan = sink_plan(spec)
        for i, (_, m) in enumerate(jobs):
            q[i], k[i], v[i] = frame(spec, m, plan)
    return q, k, v
