"""Helpers for the GPU parity tests: device copies, views, error metrics, a
teacher-forced oracle comparison loop."""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

from oracle import select_most_recent, select_top_b

# Acceptance bounds for the attention output (fp32 O against the float64
# oracle, both fed identical bf16 inputs).
O_MAXABS = 2e-2
O_RELRMS = 1e-3
# fp32 scores against float64 scores: each probability carries ~1e-6
# relative error (fp32 logits from bf16 products, the exp2 instruction, the
# row log-sum-exp) and the fixed-order fp32 sums over <= 1792 positive terms
# add about as much; the bound sits ~10x above that (observed max about
# 0.04 of it at the 8B shape)
SCORE_RTOL = 1e-5
SCORE_ATOL = 1e-6
# free-running selected-set agreement
SELECT_AGREEMENT = 0.995


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> contiguous cuda bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def o_errors(o_gpu: np.ndarray, o_ref: np.ndarray):
    d = o_gpu.astype(np.float64) - o_ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(o_ref))


@dataclasses.dataclass
class StateSnapshot:
    count: int
    pos: List[np.ndarray]
    k: List[np.ndarray]
    v: List[np.ndarray]
    scores: List[np.ndarray]
    pool: int


def snapshot(layer) -> StateSnapshot:
    torch.cuda.synchronize()
    st = layer.state()
    c, pool = st["count"], st["pool"]
    pos = st["pos"][:, :c].cpu().numpy()
    if st["k"] is None:  # C kept as positions into D: read its rows from D
        dc = layer.detailed_cache()
        dk, dv = to_bits(dc["k"]), to_bits(dc["v"])
        base = layer.position_offset
        k = np.stack([dk[h][pos[h] - base] for h in range(pos.shape[0])])
        v = np.stack([dv[h][pos[h] - base] for h in range(pos.shape[0])])
    else:
        k = to_bits(st["k"][:, :c])
        v = to_bits(st["v"][:, :c])
    sc = st["scores"][:, :pool].cpu().numpy()
    H = pos.shape[0]
    return StateSnapshot(c, [pos[h] for h in range(H)], [k[h] for h in range(H)],
                         [v[h] for h in range(H)], [sc[h] for h in range(H)], pool)


# layer flags the helpers look at (values of include/statekv.h)
FLAG_SELECT_SHARED = 1 << 0
FLAG_SELECT_RECENT = 1 << 4
FLAG_SLOT_STABLE = 1 << 5


def expected_in_place_rows(prev_rows, kept_positions, frame_positions, budget):
    """Row layout of C after the in-place (slot-stable) update: rows whose
    position is kept stay put; the freed rows -- rows whose position was
    dropped, in row order, then the unused rows len(prev_rows)..budget-1 --
    take the kept frame tokens in frame order."""
    kept = set(int(p) for p in kept_positions)
    c = len(prev_rows)
    new_len = min(budget, c + len(frame_positions))
    rows = [int(p) for p in prev_rows] + [None] * (new_len - c)
    free = [r for r in range(c) if rows[r] not in kept] + list(range(c, new_len))
    incoming = [int(p) for p in frame_positions if int(p) in kept]
    assert len(free) == len(incoming), (len(free), len(incoming))
    for r, p in zip(free, incoming):
        rows[r] = p
    return np.array(rows, dtype=np.int64)


@dataclasses.dataclass
class FrameReport:
    n: int
    maxabs: float
    relrms: float
    score_err: float
    kept_match: int
    kept_total: int


def teacher_forced_frame(orc, layer, n, q, k, v, o_gpu_dev=None) -> FrameReport:
    """Run GPU frame n and the oracle step from the GPU's C_{n-1}; compare.

    Besides the errors against the oracle, the GPU's kept set must be exactly
    the oracle's selection rule applied to the GPU's own fp32 scores (per-head
    rule; the recency rule on positions), and the state rows must be in
    ascending position, or with SLOT_STABLE in the in-place layout."""
    flags = getattr(layer, "flags", 0)
    before = snapshot(layer)
    orc.load_state(n, before.pos, before.k, before.v)
    q_d, k_d, v_d = to_dev(q), to_dev(k), to_dev(v)
    o = layer.prefill(q_d, k_d, v_d, out=o_gpu_dev)
    after = snapshot(layer)
    ref = orc.step(q, k, v)
    maxabs, relrms = o_errors(o.cpu().numpy(), ref.o)
    frame_pos = layer.position_offset + n * q.shape[0] + np.arange(q.shape[0], dtype=np.int64)
    score_err = 0.0
    match = total = 0
    shared_rule = None
    if flags & FLAG_SELECT_SHARED and not flags & FLAG_SELECT_RECENT:
        # the layer-wide importance is the fp32 sum of the per-head rows in
        # head order (every head holds the same rows, so one pool serves)
        tot = after.scores[0].astype(np.float32)
        for h in range(1, len(ref.scores)):
            tot = (tot + after.scores[h].astype(np.float32)).astype(np.float32)
        pool0 = np.concatenate([before.pos[0], frame_pos])
        shared_rule = pool0[select_top_b(tot.astype(np.float64), pool0, layer.B)]
    for h in range(len(ref.scores)):
        np.testing.assert_array_equal(ref.pool_positions[h].shape[0], after.pool)
        # the GPU's pool is [its state rows as held ; frame]; the oracle's ascends
        gpu_pool = np.concatenate([before.pos[h], frame_pos])
        order = np.argsort(gpu_pool, kind="stable")
        np.testing.assert_array_equal(gpu_pool[order], ref.pool_positions[h])
        s_ref = ref.scores[h]
        s_gpu = after.scores[h].astype(np.float64)[order]
        score_err = max(score_err, float((np.abs(s_gpu - s_ref) /
                                          (SCORE_ATOL + SCORE_RTOL * np.abs(s_ref))).max()))
        kept_ref = set(ref.kept_positions[h].tolist())
        kept_gpu = after.pos[h].tolist()
        assert len(kept_gpu) == len(kept_ref)
        if flags & FLAG_SELECT_RECENT:
            rule = gpu_pool[select_most_recent(gpu_pool, layer.B)]
        elif not flags & FLAG_SELECT_SHARED:
            rule = gpu_pool[select_top_b(after.scores[h].astype(np.float64), gpu_pool, layer.B)]
        else:
            rule = shared_rule
        if rule is not None:
            assert sorted(kept_gpu) == sorted(rule.tolist()), (n, h, "selection rule")
        if flags & FLAG_SLOT_STABLE:
            np.testing.assert_array_equal(
                after.pos[h], expected_in_place_rows(before.pos[h], kept_gpu, frame_pos, layer.B))
        else:
            assert kept_gpu == sorted(kept_gpu), "state positions must ascend"
        match += len(kept_ref.intersection(kept_gpu))
        total += len(kept_ref)
    return FrameReport(n, maxabs, relrms, score_err, match, total)


def check_caches_bitwise(layer, frames_k, frames_v, n_frames: Optional[int] = None):
    """Every state row equals the detailed-cache row at its position, and the
    detailed cache equals the concatenated input frames (bit for bit)."""
    torch.cuda.synchronize()
    st = layer.state()
    dc = layer.detailed_cache()
    c = st["count"]
    L = dc["length"]
    dk = to_bits(dc["k"][:, :L])
    dv = to_bits(dc["v"][:, :L])
    K = np.concatenate(frames_k) if isinstance(frames_k, list) else frames_k
    V = np.concatenate(frames_v) if isinstance(frames_v, list) else frames_v
    K = K.reshape(-1, *K.shape[-2:])[:L]
    V = V.reshape(-1, *V.shape[-2:])[:L]
    np.testing.assert_array_equal(dk, np.transpose(K, (1, 0, 2)))
    np.testing.assert_array_equal(dv, np.transpose(V, (1, 0, 2)))
    pos = st["pos"][:, :c].cpu().numpy()
    in_place = getattr(layer, "flags", 0) & FLAG_SLOT_STABLE
    for h in range(pos.shape[0]):
        assert np.all(np.diff(np.sort(pos[h]) if in_place else pos[h]) > 0)
    if st["k"] is None:  # C kept as positions into D: nothing else to compare
        return
    ck = to_bits(st["k"][:, :c])
    cv = to_bits(st["v"][:, :c])
    for h in range(pos.shape[0]):
        np.testing.assert_array_equal(ck[h], dk[h][pos[h]])
        np.testing.assert_array_equal(cv[h], dv[h][pos[h]])
