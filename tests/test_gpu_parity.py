"""GPU parity: the HIP path (through the C ABI) against the float64 oracle."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import framegen
from gpu_util import (O_MAXABS, O_RELRMS, SELECT_AGREEMENT, check_caches_bitwise, o_errors,
                      snapshot, teacher_forced_frame, to_dev)
from oracle import StateKVOracle, full_causal_attention

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import streaming_long_video_amd as skv  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _layer(spec, **kw):
    cfg = dict(n_q_heads=spec.n_q_heads, n_kv_heads=spec.n_kv_heads, head_dim=spec.head_dim,
               frame_tokens=spec.frame_tokens, state_budget=spec.state_budget,
               detailed_capacity=spec.n_frames * spec.frame_tokens)
    cfg.update(kw)
    return skv.Layer(**cfg)


def _oracle(spec, **kw):
    return StateKVOracle(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.frame_tokens,
                         spec.state_budget, **kw)


def _run_teacher_forced(spec, layer=None, orc_kw=None, frames=None):
    layer = layer or _layer(spec)
    orc = _oracle(spec, **(orc_kw or {}))
    qs, ks, vs = frames if frames is not None else framegen.stacked_frames(spec, workers=8)
    reports = []
    for n in range(qs.shape[0]):
        reports.append(teacher_forced_frame(orc, layer, n, qs[n], ks[n], vs[n]))
    return layer, reports, (qs, ks, vs)


def _assert_reports(reports, exact_select=True):
    worst = max(reports, key=lambda r: r.relrms)
    print(f"worst frame {worst.n}: maxabs {worst.maxabs:.3e} relrms {worst.relrms:.3e}; "
          f"max score err {max(r.score_err for r in reports):.3f} x tol")
    for r in reports:
        assert r.maxabs <= O_MAXABS, r
        assert r.relrms <= O_RELRMS, r
        assert r.score_err <= 1.0, r
    match = sum(r.kept_match for r in reports)
    total = sum(r.kept_total for r in reports)
    if exact_select:
        assert match == total, (match, total)
    assert match >= SELECT_AGREEMENT * total


def test_hand_example_on_gpu():
    """The three-frame example worked by hand, embedded in d=64 with zero padding."""
    ex = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    layer = skv.Layer(1, 1, 64, 2, 2, detailed_capacity=6, softmax_scale=math.log(2.0))
    for fr, exp in zip(ex["frames"], ex["expected"]):
        pad = lambda x: np.pad(np.array(x, dtype=np.float32)[:, None, :], ((0, 0), (0, 0), (0, 62)))
        q, k, v = (torch.from_numpy(pad(fr[n])).cuda().to(torch.bfloat16) for n in "qkv")
        o = layer.prefill(q, k, v).cpu().numpy()[:, 0, :2]
        o_exp = np.array([[float(Fraction(x)) for x in row] for row in exp["o"]])
        np.testing.assert_allclose(o, o_exp, rtol=0, atol=2e-3)
        snap = snapshot(layer)
        np.testing.assert_allclose(snap.scores[0], [float(Fraction(x)) for x in exp["scores"]],
                                   rtol=1e-5, atol=1e-6)
        np.testing.assert_array_equal(snap.pos[0], exp["kept_positions"])


@pytest.mark.parametrize("name", ["tiny", "tiny_full"])
def test_tiny_workload(name):
    """2 query heads / 1 KV head, d=64, T=16, 8 frames, B=32 (evictions) and
    B=128 (no eviction: equals full causal attention)."""
    spec = framegen.workload(name)
    layer, reports, (qs, ks, vs) = _run_teacher_forced(spec)
    _assert_reports(reports)
    check_caches_bitwise(layer, ks, vs)
    if name == "tiny_full":
        # free-running GPU run == dense causal attention over the whole video
        layer2 = _layer(spec)
        for n in range(spec.n_frames):
            o = layer2.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
            ref = full_causal_attention(qs[n], ks[: n + 1].reshape(-1, 1, 64),
                                        vs[: n + 1].reshape(-1, 1, 64),
                                        first_query=n * spec.frame_tokens)
            maxabs, relrms = o_errors(o, ref)
            assert maxabs <= O_MAXABS and relrms <= O_RELRMS, (n, maxabs, relrms)


def test_1b_layer_free_running_and_teacher_forced():
    """InternVL3-1B-like layer, 64 frames, B=1024, planted sinks."""
    spec = framegen.workload("internvl3_1b_layer")
    frames = framegen.stacked_frames(spec, workers=8)
    qs, ks, vs = frames
    layer, reports, _ = _run_teacher_forced(spec, frames=frames)
    _assert_reports(reports, exact_select=False)
    check_caches_bitwise(layer, ks, vs)
    # free-running: GPU and oracle each follow their own trajectory
    layer2 = _layer(spec)
    orc = _oracle(spec)
    _, sinks = framegen.sink_plan(spec)
    match = total = 0
    for n in range(spec.n_frames):
        layer2.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
        ref = orc.step(qs[n], ks[n], vs[n])
        snap = snapshot(layer2)
        for h in range(spec.n_kv_heads):
            kept = set(ref.kept_positions[h].tolist())
            match += len(kept.intersection(snap.pos[h].tolist()))
            total += len(kept)
            seen = sinks[sinks < (n + 1) * spec.frame_tokens]
            assert np.isin(seen, snap.pos[h]).all(), (n, h)
    print(f"free-running selected-set agreement {match / total:.6f}")
    assert match >= SELECT_AGREEMENT * total


@pytest.mark.parametrize("layer_index", [0, 27])
@pytest.mark.parametrize("in_place", [False, True])
def test_2b_layer_shape(layer_index, in_place):
    """One layer of the InternVL3-2B-like 28-layer stream (Hq=12, Hkv=2, d=128,
    B=2048, its own seed), 12 frames, the last four evicting; teacher-forced."""
    spec = framegen.workload("internvl3_2b_28layers").for_layer(layer_index).replace(n_frames=12)
    layer = _layer(spec, flags=skv.STATEKV_FLAG_SLOT_STABLE if in_place else 0)
    layer, reports, (qs, ks, vs) = _run_teacher_forced(spec, layer=layer)
    _assert_reports(reports, exact_select=False)
    check_caches_bitwise(layer, ks, vs)


@pytest.mark.parametrize("flags", ["c_in_d", "c_in_d_shared"])
def test_state_kept_as_positions_into_d(flags):
    """C_IN_D: the state holds positions only and attention reads its rows
    from D.  1B-like layer, 24 frames: teacher-forced against the oracle (the
    state's rows read back from D), then bit-identical outputs to the default
    layout on the same stream."""
    spec = framegen.workload("internvl3_1b_layer").replace(n_frames=24)
    frames = framegen.stacked_frames(spec, workers=8)
    qs, ks, vs = frames
    f = skv.STATEKV_FLAG_C_IN_D
    shared = flags.endswith("shared")
    if shared:
        f |= skv.STATEKV_FLAG_SELECT_SHARED
    layer, reports, _ = _run_teacher_forced(spec, layer=_layer(spec, flags=f),
                                            orc_kw=dict(shared=shared), frames=frames)
    _assert_reports(reports, exact_select=False)
    assert layer.state()["k"] is None
    check_caches_bitwise(layer, ks, vs)
    a = _layer(spec, flags=f)
    b = _layer(spec, flags=f & ~skv.STATEKV_FLAG_C_IN_D)
    for n in range(spec.n_frames):
        oa = a.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
        ob = b.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
        np.testing.assert_array_equal(oa, ob)
        np.testing.assert_array_equal(snapshot(a).pos[0], snapshot(b).pos[0])


@pytest.mark.parametrize("flags", [0, "ring", "c_in_d", "in_place", "in_place_c_in_d"])
def test_checkpoint_and_restore(flags):
    """A layer checkpointed after 6 frames (C rows and positions, D, frames
    seen) and restored into a fresh layer continues bit-identically."""
    spec = framegen.workload("internvl3_1b_layer").replace(n_frames=12)
    qs, ks, vs = framegen.stacked_frames(spec, workers=8)
    f = {0: 0, "ring": skv.STATEKV_FLAG_D_RING, "c_in_d": skv.STATEKV_FLAG_C_IN_D,
         "in_place": skv.STATEKV_FLAG_SLOT_STABLE,
         "in_place_c_in_d": skv.STATEKV_FLAG_SLOT_STABLE | skv.STATEKV_FLAG_C_IN_D}[flags]
    cap = (8 if flags == "ring" else 12) * spec.frame_tokens
    a = _layer(spec, flags=f, detailed_capacity=cap)
    b = _layer(spec, flags=f, detailed_capacity=cap)
    for n in range(6):
        a.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
    b.restore(a.checkpoint())
    for n in range(6, 12):
        oa = a.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
        ob = b.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
        np.testing.assert_array_equal(oa, ob)
    sa, sb = snapshot(a), snapshot(b)
    for h in range(spec.n_kv_heads):
        np.testing.assert_array_equal(sa.pos[h], sb.pos[h])
        np.testing.assert_array_equal(sa.k[h], sb.k[h])


def test_recency_window_mode():
    """SELECT_RECENT keeps the B most recent candidates (the comparison rule
    of the pages' App. A.3): teacher-forced against the oracle's recency mode;
    the state after frame n holds positions [(n+1)T - B, (n+1)T)."""
    spec = framegen.workload("internvl3_1b_layer").replace(n_frames=10)
    frames = framegen.stacked_frames(spec, workers=8)
    layer = _layer(spec, flags=skv.STATEKV_FLAG_SELECT_RECENT)
    layer, reports, _ = _run_teacher_forced(spec, layer=layer, orc_kw=dict(recency=True),
                                            frames=frames)
    _assert_reports(reports, exact_select=True)
    snap = snapshot(layer)
    hi = spec.n_frames * spec.frame_tokens
    for h in range(spec.n_kv_heads):
        np.testing.assert_array_equal(snap.pos[h], np.arange(hi - spec.state_budget, hi))


def test_shared_selection_mode():
    """SHARED: one kept set per layer from the importance summed over all query
    heads; every KV head holds the same positions.  1B-like layer (Hkv = 2),
    24 frames: teacher-forced against the oracle's shared mode, then free
    running."""
    spec = framegen.workload("internvl3_1b_layer").replace(n_frames=24)
    frames = framegen.stacked_frames(spec, workers=8)
    qs, ks, vs = frames
    layer = _layer(spec, flags=skv.STATEKV_FLAG_SELECT_SHARED)
    layer, reports, _ = _run_teacher_forced(spec, layer=layer, orc_kw=dict(shared=True),
                                            frames=frames)
    _assert_reports(reports, exact_select=False)
    snap = snapshot(layer)
    np.testing.assert_array_equal(snap.pos[0], snap.pos[1])
    check_caches_bitwise(layer, ks, vs)
    layer2 = _layer(spec, flags=skv.STATEKV_FLAG_SELECT_SHARED)
    orc = _oracle(spec, shared=True)
    match = total = 0
    for n in range(spec.n_frames):
        layer2.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
        ref = orc.step(qs[n], ks[n], vs[n])
        snap = snapshot(layer2)
        kept = set(ref.kept_positions[0].tolist())
        match += len(kept.intersection(snap.pos[0].tolist()))
        total += len(kept)
        np.testing.assert_array_equal(snap.pos[0], snap.pos[1])
    assert match >= SELECT_AGREEMENT * total, (match, total)


@pytest.mark.parametrize("mode", ["plain", "shared", "c_in_d", "recent"])
def test_in_place_state_update(mode):
    """SLOT_STABLE: kept state rows stay where they are and the kept frame
    tokens fill the freed rows.  1B-like layer, 24 frames: teacher-forced
    against the oracle (the helper checks the exact row layout and the
    selection rule on the GPU's own scores), then free running beside the
    default layout on the same stream (same outputs up to the summation order
    of the state rows, same kept sets up to near-ties)."""
    spec = framegen.workload("internvl3_1b_layer").replace(n_frames=24)
    frames = framegen.stacked_frames(spec, workers=8)
    qs, ks, vs = frames
    extra = {"plain": 0, "shared": skv.STATEKV_FLAG_SELECT_SHARED,
             "c_in_d": skv.STATEKV_FLAG_C_IN_D, "recent": skv.STATEKV_FLAG_SELECT_RECENT}[mode]
    f = skv.STATEKV_FLAG_SLOT_STABLE | extra
    orc_kw = dict(shared=mode == "shared", recency=mode == "recent")
    layer, reports, _ = _run_teacher_forced(spec, layer=_layer(spec, flags=f), orc_kw=orc_kw,
                                            frames=frames)
    _assert_reports(reports, exact_select=mode == "recent")
    check_caches_bitwise(layer, ks, vs)
    a = _layer(spec, flags=f)
    b = _layer(spec, flags=extra)
    match = total = 0
    for n in range(spec.n_frames):
        oa = a.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
        ob = b.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
        maxabs, relrms = o_errors(oa, ob.astype(np.float64))
        assert maxabs <= O_MAXABS and relrms <= O_RELRMS, (n, maxabs, relrms)
        sa, sb = snapshot(a), snapshot(b)
        for h in range(spec.n_kv_heads):
            match += len(set(sa.pos[h].tolist()).intersection(sb.pos[h].tolist()))
            total += len(sb.pos[h])
    print(f"in-place vs row layout, kept-set agreement {match / total:.6f}")
    assert match >= SELECT_AGREEMENT * total, (match, total)


def test_in_place_ties_go_to_lower_positions():
    """Keys drawn from four vectors make whole groups of state tokens tie
    exactly (identical logits, identical column sums); with the in-place
    layout the state rows are out of position order, so the kept members of
    a tied group must be found by position.  Teacher-forced: the kept set is
    the oracle's rule on the GPU's own scores and the oracle's kept set."""
    Hq, Hkv, d, T, B, N = 4, 1, 64, 32, 48, 12
    spec = framegen.FrameSpec(Hq, Hkv, d, T, N, B, 1e4, 5, sinks=False)
    qs, ks, vs = framegen.stacked_frames(spec, workers=4)
    rng = np.random.default_rng(123)
    basis = framegen.f64_to_bf16_bits(rng.standard_normal((4, d)))
    ks = basis[rng.integers(0, 4, size=(N, T, Hkv))]
    layer = _layer(spec, flags=skv.STATEKV_FLAG_SLOT_STABLE)
    orc = _oracle(spec)
    tied_frames = 0
    for n in range(N):
        r = teacher_forced_frame(orc, layer, n, qs[n], ks[n], vs[n])
        assert r.kept_match == r.kept_total, r
        assert r.maxabs <= O_MAXABS and r.relrms <= O_RELRMS, r
        after = snapshot(layer)
        if after.pool > B:
            s = np.sort(after.scores[0])[::-1]
            tied_frames += int(s[B - 1] == s[B])  # a tie straddles the boundary
    print(f"frames with a tie across the budget boundary: {tied_frames}")
    assert tied_frames >= 3


@pytest.mark.parametrize("shape", [
    # (Hq, Hkv, d, T, B, frames): ragged T, B not a tile multiple, G=1, G=16, T=1
    (6, 2, 128, 17, 50, 6),
    (3, 3, 64, 100, 130, 4),
    (16, 1, 64, 40, 64, 4),
    (4, 2, 128, 1, 3, 7),
    (12, 2, 128, 256, 2048, 12),
    (8, 4, 64, 33, 1, 4),
])
@pytest.mark.parametrize("in_place", [False, True])
def test_ragged_and_edge_shapes(shape, in_place):
    Hq, Hkv, d, T, B, N = shape
    spec = framegen.FrameSpec(Hq, Hkv, d, T, N, B, 1e4, 11, sinks=False)
    layer = _layer(spec, flags=skv.STATEKV_FLAG_SLOT_STABLE if in_place else 0)
    layer, reports, (qs, ks, vs) = _run_teacher_forced(spec, layer=layer)
    _assert_reports(reports, exact_select=False)
    check_caches_bitwise(layer, ks, vs)


@pytest.mark.parametrize("d,shared", [(64, False), (128, True)])
def test_in_place_large_frame(d, shared):
    """T = 4096 (the largest frame): the in-place move lists no longer fit in
    LDS beside the pool's keys (B = 24000) and go through the selection rows;
    with d = 128 and SHARED the moves of every head are copied by one
    workgroup.  Seven frames, the last two evicting; teacher-forced."""
    Hkv = 2 if shared else 1
    spec = framegen.FrameSpec(Hkv, Hkv, d, 4096, 7, 24000, 1e4, 17, sinks=False)
    f = skv.STATEKV_FLAG_SLOT_STABLE | (skv.STATEKV_FLAG_SELECT_SHARED if shared else 0)
    layer = _layer(spec, flags=f)
    layer, reports, (qs, ks, vs) = _run_teacher_forced(spec, layer=layer,
                                                       orc_kw=dict(shared=shared))
    _assert_reports(reports, exact_select=False)
    check_caches_bitwise(layer, ks, vs)


@pytest.mark.parametrize("in_place", [False, True])
def test_largest_pool(in_place):
    """B + T = 32768, the largest pool the select keeps in LDS (T = 4096, B =
    28672): nine frames, the last two evicting; teacher-forced."""
    spec = framegen.FrameSpec(1, 1, 64, 4096, 9, 28672, 1e4, 23, sinks=False)
    layer = _layer(spec, flags=skv.STATEKV_FLAG_SLOT_STABLE if in_place else 0)
    layer, reports, (qs, ks, vs) = _run_teacher_forced(spec, layer=layer)
    _assert_reports(reports, exact_select=False)
    check_caches_bitwise(layer, ks, vs)


@pytest.mark.parametrize("in_place,splits", [(False, 3), (True, 3), (False, 1)])
def test_bf16_output_is_the_rounded_fp32_output(in_place, splits):
    """STATEKV_FLAG_OUT_BF16: O as bf16 equals the fp32 output of an otherwise
    identical layer rounded to nearest even, bit for bit, through warm-up and
    eviction, from the split sum and (one split) from the output pass itself;
    the state evolves identically; the quadratic baseline refuses the layer."""
    spec = framegen.workload("tiny").replace(frame_tokens=64, state_budget=256, n_frames=6)
    base = skv.STATEKV_FLAG_SLOT_STABLE if in_place else 0
    a = _layer(spec, flags=base, num_splits=splits)
    b = _layer(spec, flags=base | skv.STATEKV_FLAG_OUT_BF16, num_splits=splits)
    qs, ks, vs = framegen.stacked_frames(spec, workers=4)
    for n in range(spec.n_frames):
        o32 = a.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
        o16 = b.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
        assert o16.dtype == torch.bfloat16
        assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16)), n
    pool = spec.state_budget + spec.frame_tokens
    assert a.launch_plan(pool)["out_splits"] == splits
    sa, sb = snapshot(a), snapshot(b)
    assert np.array_equal(sa.pos, sb.pos)
    c = _layer(spec, flags=skv.STATEKV_FLAG_OUT_BF16)
    with pytest.raises(skv.StateKVError):
        c.full_attention(to_dev(qs[0]), to_dev(ks[0]), to_dev(vs[0]))


def test_launch_plan_introspection():
    """The plan the step runs at the 8B shape: 9 output splits, 18 statistics
    splits, 7 row tiles, 68 key tiles at the full pool; at a one-frame pool
    no split is emptier than a tile; pools outside [1, B+T] are refused."""
    layer = skv.Layer(28, 4, 128, 256, 4096, detailed_capacity=4096)
    assert layer.launch_plan(4352) == {"out_splits": 9, "stat_splits": 18, "row_tiles": 7,
                                       "key_tiles": 68}
    small = layer.launch_plan(256)
    assert small["key_tiles"] == 4 and small["out_splits"] <= 4 and small["stat_splits"] <= 4
    for bad in (0, 4353):
        with pytest.raises(skv.StateKVError):
            layer.launch_plan(bad)


@pytest.mark.parametrize("splits", [1, 2, 5])
def test_explicit_split_counts(splits):
    spec = framegen.workload("tiny").replace(n_q_heads=4, n_kv_heads=2, frame_tokens=48,
                                             state_budget=100, n_frames=5)
    layer = _layer(spec, num_splits=splits)
    _, reports, _ = _run_teacher_forced(spec, layer=layer)
    _assert_reports(reports, exact_select=False)


def test_noncausal_frame_flag():
    spec = framegen.workload("tiny").replace(n_frames=4)
    layer = _layer(spec, flags=skv.STATEKV_FLAG_NONCAUSAL_FRAME)
    _, reports, _ = _run_teacher_forced(spec, layer=layer, orc_kw=dict(causal=False))
    _assert_reports(reports, exact_select=False)


def test_ring_detailed_cache_wraps():
    spec = framegen.workload("tiny").replace(n_frames=5)
    layer = skv.Layer(2, 1, 64, 16, 32, detailed_capacity=40, flags=skv.STATEKV_FLAG_D_RING)
    qs, ks, vs = framegen.stacked_frames(spec)
    for n in range(5):
        layer.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
    torch.cuda.synchronize()
    dc = layer.detailed_cache()
    assert dc["length"] == 40 and dc["start"] == 80 - 40
    from gpu_util import to_bits
    dk = to_bits(dc["k"])[0]
    allk = ks.reshape(-1, 1, 64)[:, 0]
    for p in range(40, 80):
        np.testing.assert_array_equal(dk[p % 40], allk[p])


def test_capacity_error_leaves_layer_unchanged():
    spec = framegen.workload("tiny").replace(n_frames=3)
    layer = skv.Layer(2, 1, 64, 16, 32, detailed_capacity=32)
    qs, ks, vs = framegen.stacked_frames(spec)
    for n in range(2):
        layer.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n]))
    before = snapshot(layer)
    with pytest.raises(skv.StateKVError) as e:
        layer.prefill(to_dev(qs[2]), to_dev(ks[2]), to_dev(vs[2]))
    assert e.value.status == -4
    after = snapshot(layer)
    assert layer.state()["frames_seen"] == 2
    for h in range(1):
        np.testing.assert_array_equal(before.pos[h], after.pos[h])


def test_bitwise_determinism():
    spec = framegen.workload("internvl3_1b_layer").replace(n_frames=8)
    qs, ks, vs = framegen.stacked_frames(spec, workers=8)
    outs = []
    for _ in range(2):
        layer = _layer(spec)
        os_ = [layer.prefill(to_dev(qs[n]), to_dev(ks[n]), to_dev(vs[n])).cpu().numpy()
               for n in range(spec.n_frames)]
        snap = snapshot(layer)
        outs.append((np.stack(os_), snap))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    for h in range(spec.n_kv_heads):
        np.testing.assert_array_equal(outs[0][1].scores[h], outs[1][1].scores[h])
        np.testing.assert_array_equal(outs[0][1].k[h], outs[1][1].k[h])
        np.testing.assert_array_equal(outs[0][1].pos[h], outs[1][1].pos[h])
