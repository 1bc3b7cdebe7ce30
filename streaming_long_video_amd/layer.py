"""Torch-facing wrapper of one StateKV layer.

torch supplies device memory (the workspace and the frame tensors) and the
HIP stream; the computation is entirely the library's.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _binding as B


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


class Layer:
    """One transformer layer's StateKV caches on the current GPU.

    q: [T][Hq][d] bf16, k/v: [T][Hkv][d] bf16 (RoPE already applied at the
    tokens' original positions), output: [T][Hq][d] float32.
    """

    def __init__(self, n_q_heads: int, n_kv_heads: int, head_dim: int, frame_tokens: int,
                 state_budget: int, detailed_capacity: int, position_offset: int = 0,
                 softmax_scale: float = 0.0, flags: int = 0, num_splits: int = 0,
                 rope_theta: float = 0.0, rope_scaling: float = 0.0,
                 device: Optional[torch.device] = None):
        self.cfg = B.make_config(n_q_heads, n_kv_heads, head_dim, frame_tokens, state_budget,
                                 detailed_capacity, position_offset, softmax_scale, flags,
                                 num_splits, rope_theta, rope_scaling)
        self.Hq, self.Hkv, self.d = n_q_heads, n_kv_heads, head_dim
        self.T, self.B = frame_tokens, state_budget
        self.capacity = detailed_capacity
        self.position_offset = position_offset
        self.flags = flags
        nbytes = B.statekv_workspace_bytes(self.cfg)
        dev = torch.device("cuda") if device is None else torch.device(device)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.handle = B.statekv_init_layer(self.cfg, self.workspace.data_ptr(), nbytes)
        self.workspace_bytes = nbytes

    # -- per-frame calls -------------------------------------------------------
    def _check_frame(self, q, k, v, out, out_dtype=torch.float32):
        T, Hq, Hkv, d = self.T, self.Hq, self.Hkv, self.d
        for name, x, shape in (("q", q, (T, Hq, d)), ("k", k, (T, Hkv, d)),
                               ("v", v, (T, Hkv, d))):
            if x.dtype != torch.bfloat16 or tuple(x.shape) != shape or not x.is_contiguous():
                raise ValueError(f"{name} must be a contiguous bfloat16 tensor of shape {shape}")
            if x.device != self.workspace.device:
                raise ValueError(f"{name} is not on the layer's device")
        if out is None:
            out = torch.empty((T, Hq, d), dtype=out_dtype, device=self.workspace.device)
        elif (out.dtype != out_dtype or tuple(out.shape) != (T, Hq, d)
              or not out.is_contiguous()):
            raise ValueError(f"out must be a contiguous {out_dtype} tensor of shape (T, Hq, d)")
        return out

    def prefill(self, q, k, v, out=None, stream=None):
        """StateKV step for the next frame; returns the attention output (fp32,
        or bf16 for a layer made with STATEKV_FLAG_OUT_BF16)."""
        bf16_out = bool(self.flags & B.STATEKV_FLAG_OUT_BF16)
        out = self._check_frame(q, k, v, out, torch.bfloat16 if bf16_out else torch.float32)
        B.statekv_prefill_frame(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                out.data_ptr(), _stream_ptr(stream))
        return out

    def full_attention(self, q, k, v, out=None, stream=None):
        """Quadratic baseline: append the frame to D, attend over all of D."""
        out = self._check_frame(q, k, v, out)
        B.statekv_full_attention_frame(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       out.data_ptr(), _stream_ptr(stream))
        return out

    def rope(self, x, first_position: int, stream=None):
        """Rotate x [n][heads][d] (bf16, in place) at positions first_position + i
        with the layer's RoPE parameters; returns x."""
        if x.dtype != torch.bfloat16 or x.dim() != 3 or x.shape[2] != self.d \
                or not x.is_contiguous() or x.device != self.workspace.device:
            raise ValueError("x must be a contiguous bfloat16 (n, heads, d) tensor on the "
                             "layer's device")
        B.statekv_rope(self.handle, x.data_ptr(), x.shape[0], x.shape[1], int(first_position),
                       _stream_ptr(stream))
        return x

    def decode(self, q, out=None, stream=None):
        """Decoding attention of text queries q [M][Hq][d] (bf16) over every
        token of the detailed cache; returns fp32 [M][Hq][d]."""
        if q.dtype != torch.bfloat16 or q.dim() != 3 or tuple(q.shape[1:]) != (self.Hq, self.d) \
                or not q.is_contiguous() or q.device != self.workspace.device:
            raise ValueError(f"q must be a contiguous bfloat16 tensor of shape (M, {self.Hq}, "
                             f"{self.d}) on the layer's device")
        M = q.shape[0]
        if out is None:
            out = torch.empty((M, self.Hq, self.d), dtype=torch.float32, device=q.device)
        elif (out.dtype != torch.float32 or tuple(out.shape) != (M, self.Hq, self.d)
              or not out.is_contiguous()):
            raise ValueError("out must be a contiguous float32 tensor of shape (M, Hq, d)")
        B.statekv_decode_attention(self.handle, q.data_ptr(), M, out.data_ptr(),
                                   _stream_ptr(stream))
        return out

    def launch_plan(self, pool: int) -> dict:
        """Split and tile counts of the prefill step at a pool of `pool` candidates."""
        return B.statekv_launch_plan_for(self.handle, pool)

    def attention_mass(self, budgets, sets=None, out=None, stream=None):
        """App. A diagnostics of the last frame for a layer that has kept every
        token (see statekv_attention_mass).  ``sets`` (int32 tensor of
        len(budgets) x words, kept between calls; allocated zeroed when None)
        carries each budget's kept set to the next call.  Returns (out, sets):
        out is float32 [len(budgets)][3] = (top-b historical mass share,
        recency share, weighted candidate-pool recall)."""
        nb = len(budgets)
        dev = self.workspace.device
        words = B.statekv_mass_set_words(self.handle)
        if sets is None:
            sets = torch.zeros((nb, words), dtype=torch.int32, device=dev)
        elif (sets.dtype != torch.int32 or tuple(sets.shape) != (nb, words)
              or not sets.is_contiguous() or sets.device != dev):
            raise ValueError(f"sets must be a contiguous int32 tensor of shape ({nb}, {words})")
        if out is None:
            out = torch.empty((nb, 3), dtype=torch.float32, device=dev)
        elif out.dtype != torch.float32 or tuple(out.shape) != (nb, 3) or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 tensor of shape (len(budgets), 3)")
        B.statekv_attention_mass(self.handle, budgets, sets.data_ptr(), out.data_ptr(),
                                 _stream_ptr(stream))
        return out, sets

    # -- views -----------------------------------------------------------------
    def _ws_slice(self, ptr: int, nbytes: int, dtype, shape):
        off = ptr - self.workspace.data_ptr()
        assert 0 <= off and off + nbytes <= self.workspace_bytes
        return self.workspace[off:off + nbytes].view(dtype).view(shape)

    def state(self):
        """C_n as workspace views: dict(k, v, pos, count, scores, pool, frames_seen);
        k and v are None when the layer keeps C as positions into D."""
        v = B.statekv_state(self.handle)
        Hkv, Bc, d = v.n_kv_heads, v.capacity, v.head_dim
        rows = Hkv * Bc * d * 2
        return {
            "k": self._ws_slice(v.k, rows, torch.bfloat16, (Hkv, Bc, d)) if v.k else None,
            "v": self._ws_slice(v.v, rows, torch.bfloat16, (Hkv, Bc, d)) if v.v else None,
            "pos": self._ws_slice(v.pos, Hkv * Bc * 8, torch.int64, (Hkv, Bc)),
            "scores": self._ws_slice(v.last_scores, Hkv * v.scores_stride * 4, torch.float32,
                                     (Hkv, v.scores_stride)),
            "count": v.count,
            "pool": v.last_pool,
            "frames_seen": v.frames_seen,
        }

    def detailed_cache(self):
        """D_n as workspace views: dict(k, v, length, start)."""
        v = B.statekv_detailed_cache(self.handle)
        Hkv, cap, d = v.n_kv_heads, v.capacity, v.head_dim
        rows = Hkv * cap * d * 2
        return {
            "k": self._ws_slice(v.k, rows, torch.bfloat16, (Hkv, cap, d)),
            "v": self._ws_slice(v.v, rows, torch.bfloat16, (Hkv, cap, d)),
            "length": v.length,
            "start": v.start,
        }

    def reset(self):
        B.statekv_reset_layer(self.handle)

    def checkpoint(self):
        """Copies of the layer's resumable state: C rows with positions, the
        held D rows, frames seen (see restore)."""
        torch.cuda.synchronize(self.workspace.device)
        st, dc = self.state(), self.detailed_cache()
        c, L = st["count"], dc["length"]
        return {
            "frames_seen": st["frames_seen"], "count": c,
            "pos": st["pos"][:, :c].clone(),
            "k": None if st["k"] is None else st["k"][:, :c].clone(),
            "v": None if st["v"] is None else st["v"][:, :c].clone(),
            "d_k": dc["k"][:, :L].clone(), "d_v": dc["v"][:, :L].clone(),
        }

    def restore(self, ckpt):
        """Write a checkpoint into this layer's workspace (same configuration)
        and continue from its next frame."""
        B.statekv_reset_layer(self.handle)
        st, dc = self.state(), self.detailed_cache()
        c, L = ckpt["count"], ckpt["d_k"].shape[1]
        st["pos"][:, :c].copy_(ckpt["pos"])
        if st["k"] is not None:
            st["k"][:, :c].copy_(ckpt["k"])
            st["v"][:, :c].copy_(ckpt["v"])
        dc["k"][:, :L].copy_(ckpt["d_k"])
        dc["v"][:, :L].copy_(ckpt["d_v"])
        torch.cuda.synchronize(self.workspace.device)
        B.statekv_restore_layer(self.handle, ckpt["frames_seen"], c)

    def close(self):
        if getattr(self, "handle", None):
            B.statekv_free_layer(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def qkv_rope(x: torch.Tensor, w: torch.Tensor, n_q_heads: int, n_kv_heads: int, head_dim: int,
             first_position: int, rope_theta: float, rope_scaling: float = 0.0,
             out=None, workspace=None, stream=None):
    """The library's frame front end: q, k, v = rope(X W_Q), rope(X W_K), X W_V.
    x: [T][hidden] bf16; w: [(Hq + 2 Hkv) d][hidden] bf16 (output-major, rows
    Q heads, K heads, V heads).  Returns (q, k, v) bf16 [T][H][d] tensors.
    workspace: a uint8 device tensor of at least
    qkv_rope_workspace_bytes(...) bytes for the hidden-dimension splits' partial
    sums; taken from torch's allocator when None."""
    T, hidden = x.shape
    rows = (n_q_heads + 2 * n_kv_heads) * head_dim
    for name, t, shape in (("x", x, (T, hidden)), ("w", w, (rows, hidden))):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor of shape {shape}")
    if w.device != x.device:
        raise ValueError("x and w must be on one device")
    if out is None:
        out = (torch.empty((T, n_q_heads, head_dim), dtype=torch.bfloat16, device=x.device),
               torch.empty((T, n_kv_heads, head_dim), dtype=torch.bfloat16, device=x.device),
               torch.empty((T, n_kv_heads, head_dim), dtype=torch.bfloat16, device=x.device))
    q, k, v = out
    if workspace is None:
        need = B.statekv_qkv_rope_workspace_size(T, hidden, n_q_heads, n_kv_heads, head_dim)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
            if stream is not None:
                workspace.record_stream(stream)  # not reused before the launch stream passes it
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (workspace.data_ptr(), workspace.numel())
    B.statekv_qkv_rope(x.data_ptr(), w.data_ptr(), T, hidden, n_q_heads, n_kv_heads, head_dim,
                       int(first_position), float(rope_theta), float(rope_scaling),
                       q.data_ptr(), k.data_ptr(), v.data_ptr(), ws_ptr, ws_bytes,
                       _stream_ptr(stream))
    return q, k, v


def qkv_rope_workspace_bytes(T: int, hidden: int, n_q_heads: int, n_kv_heads: int,
                             head_dim: int) -> int:
    """Bytes of the front end's workspace for these sizes (0: it does not split)."""
    return B.statekv_qkv_rope_workspace_size(T, hidden, n_q_heads, n_kv_heads, head_dim)


def select_topb(scores: torch.Tensor, budget: int, stream=None) -> torch.Tensor:
    """The library's top-B select on a float32 device vector (ascending indices)."""
    if scores.dtype != torch.float32 or scores.dim() != 1 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous 1-D float32 tensor")
    n = scores.shape[0]
    out = torch.empty(min(n, budget), dtype=torch.int32, device=scores.device)
    B.statekv_select_topb(scores.data_ptr(), n, budget, out.data_ptr(), _stream_ptr(stream))
    return out
