"""Host logic and the C-ABI surface, on the CPU (no kernel is launched)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "statekv.h")
CSRC = os.path.join(ROOT, "streaming_long_video_amd", "csrc")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(statekv_\w+)\(", text, re.M)))


def test_plan_with_gxx_and_sanitizers(tmp_path):
    exe = tmp_path / "plan_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "cpp", "plan_check.cpp"), os.path.join(CSRC, "plan.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


skv = pytest.importorskip("streaming_long_video_amd")
B = skv._binding


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def _cfg(**kw):
    base = dict(n_q_heads=28, n_kv_heads=4, head_dim=128, frame_tokens=256, state_budget=4096,
                detailed_capacity=131072)
    base.update(kw)
    return B.make_config(**base)


def test_workspace_bytes_and_validation():
    n = B.statekv_workspace_bytes(_cfg())
    # two compressed states (K, V, positions), the detailed cache and scratch
    assert n >= 2 * (2 * 4 * 4096 * 128 * 2 + 4 * 4096 * 8) + 2 * 4 * 131072 * 128 * 2
    for bad, status in [(dict(head_dim=96), -2), (dict(n_kv_heads=5), -1),
                        (dict(detailed_capacity=10), -1), (dict(state_budget=0), -1),
                        (dict(flags=1 << 9), -1),
                        (dict(state_budget=32600), -2), (dict(frame_tokens=5000), -2)]:
        with pytest.raises(B.StateKVError) as e:
            B.statekv_workspace_bytes(_cfg(**bad))
        assert e.value.status == status, bad
    # every defined flag is accepted (SELECT_SHARED, D_RING, NONCAUSAL_FRAME)
    assert B.statekv_workspace_bytes(_cfg(flags=0b111)) >= n
    # C kept as positions into D: no K/V copies of C, and it needs a linear D
    assert B.statekv_workspace_bytes(_cfg(flags=B.STATEKV_FLAG_C_IN_D)) <= n - 4 * 4096 * 128 * 2 * 2
    with pytest.raises(B.StateKVError) as e:
        B.statekv_workspace_bytes(_cfg(flags=B.STATEKV_FLAG_C_IN_D | B.STATEKV_FLAG_D_RING))
    assert e.value.status == -2
    # in-place update: one compressed state instead of two
    m = B.statekv_workspace_bytes(_cfg(flags=B.STATEKV_FLAG_SLOT_STABLE))
    assert m <= n - 4 * 4096 * (128 * 2 * 2 + 8)
    assert B.statekv_workspace_bytes(_cfg(flags=0b1110111)) > 0  # all but C_IN_D
    # bf16 output: same workspace, and the next bit is undefined
    assert B.statekv_workspace_bytes(_cfg(flags=B.STATEKV_FLAG_OUT_BF16)) == n
    with pytest.raises(B.StateKVError) as e:
        B.statekv_workspace_bytes(_cfg(flags=1 << 7))
    assert e.value.status == -1


def test_in_place_layout_rule():
    """The row layout the GPU tests expect from the in-place update: a worked
    case, then invariants on random cases (kept rows unmoved, the rows hold
    exactly the kept set, frame tokens enter freed rows in frame order)."""
    from gpu_util import expected_in_place_rows
    # rows hold positions 5, 1, 9, 3; frame 10..13; keep {1, 3, 11, 13}; B = 4
    rows = expected_in_place_rows([5, 1, 9, 3], [1, 3, 11, 13], [10, 11, 12, 13], 4)
    assert rows.tolist() == [11, 1, 13, 3]
    # filling up: rows 0..1 live, B = 5, frame of 4, keep {0, 2, 3, 4, 5}
    rows = expected_in_place_rows([0, 1], [0, 2, 3, 4, 5], [2, 3, 4, 5], 5)
    assert rows.tolist() == [0, 2, 3, 4, 5]
    rng = np.random.default_rng(0)
    for _ in range(200):
        c, T, Bud = int(rng.integers(0, 12)), int(rng.integers(1, 8)), int(rng.integers(1, 14))
        c = min(c, Bud)
        prev = rng.permutation(50)[:c]
        frame = 50 + np.arange(T)
        pool = np.concatenate([prev, frame])
        keep = rng.permutation(pool)[: min(Bud, c + T)]
        if c + T > Bud and len(keep) < Bud:
            continue
        rows = expected_in_place_rows(prev, keep, frame, Bud)
        assert sorted(rows.tolist()) == sorted(keep.tolist())
        for r in range(c):
            if prev[r] in keep:
                assert rows[r] == prev[r]
        incoming = [p for p in rows.tolist() if p >= 50]
        freed = [r for r in range(len(rows)) if rows[r] >= 50]
        assert incoming == sorted(incoming) and freed == sorted(freed)


def test_init_views_and_argument_errors_are_host_side():
    cfg = _cfg()
    nbytes = B.statekv_workspace_bytes(cfg)
    fake = 1 << 40  # never dereferenced: init and views are host only
    with pytest.raises(B.StateKVError) as e:
        B.statekv_init_layer(cfg, fake, nbytes - 1)
    assert e.value.status == -3
    with pytest.raises(B.StateKVError) as e:
        B.statekv_init_layer(cfg, fake + 16, nbytes)
    assert e.value.status == -3
    h = B.statekv_init_layer(cfg, fake, nbytes)
    st = B.statekv_state(h)
    assert st.count == 0 and st.frames_seen == 0 and st.capacity == 4096 and st.last_pool == 0
    assert fake <= st.k < fake + nbytes and fake <= st.pos < fake + nbytes
    dc = B.statekv_detailed_cache(h)
    assert dc.length == 0 and dc.capacity == 131072 and dc.start == 0
    with pytest.raises(B.StateKVError) as e:
        B.statekv_prefill_frame(h, 0, 0, 0, 0)
    assert e.value.status == -1
    with pytest.raises(B.StateKVError) as e:
        B.statekv_prefill_frame(h, fake + 2, fake, fake, fake)
    assert e.value.status == -1
    B.statekv_reset_layer(h)
    B.statekv_free_layer(h)


def test_ring_layout_rejects_full_attention_before_any_launch():
    cfg = _cfg(flags=B.STATEKV_FLAG_D_RING)
    nbytes = B.statekv_workspace_bytes(cfg)
    fake = 1 << 40
    h = B.statekv_init_layer(cfg, fake, nbytes)
    with pytest.raises(B.StateKVError) as e:
        B.statekv_full_attention_frame(h, fake, fake, fake, fake)
    assert e.value.status == -2
    B.statekv_free_layer(h)


def test_decode_argument_errors_are_host_side():
    cfg = _cfg()  # G = 7
    nbytes = B.statekv_workspace_bytes(cfg)
    fake = 1 << 40
    h = B.statekv_init_layer(cfg, fake, nbytes)
    for args, status in [((0, 1, fake), -1), ((fake, 0, fake), -1), ((fake + 2, 1, fake), -1),
                         ((fake, 5, fake), -2),   # 7 * 5 > 32 rows
                         ((fake, 1, fake), -1)]:  # no frame in D yet
        with pytest.raises(B.StateKVError) as e:
            B.statekv_decode_attention(h, *args)
        assert e.value.status == status, args
    B.statekv_free_layer(h)


def test_rope_configuration_and_argument_errors():
    for bad in (dict(rope_theta=-1.0), dict(rope_theta=1.0), dict(rope_theta=float("inf")),
                dict(rope_scaling=float("nan"))):
        with pytest.raises(B.StateKVError) as e:
            B.statekv_workspace_bytes(_cfg(**bad))
        assert e.value.status == -1, bad
    plain = B.statekv_workspace_bytes(_cfg())
    # the rotated frame copies: T*Hq*d + T*Hkv*d bf16
    assert B.statekv_workspace_bytes(_cfg(rope_theta=1e6)) >= plain + 256 * 32 * 128 * 2
    fake = 1 << 40
    h = B.statekv_init_layer(_cfg(), fake, plain)
    with pytest.raises(B.StateKVError) as e:  # the layer has no RoPE configuration
        B.statekv_rope(h, fake, 1, 1, 0)
    assert e.value.status == -1
    B.statekv_free_layer(h)
    cfg = _cfg(rope_theta=1e6)
    h = B.statekv_init_layer(cfg, fake, B.statekv_workspace_bytes(cfg))
    for args in ((0, 1, 1, 0), (fake + 2, 1, 1, 0), (fake, 0, 1, 0), (fake, 1, 0, 0),
                 (fake, 1, 1, -1)):
        with pytest.raises(B.StateKVError) as e:
            B.statekv_rope(h, *args)
        assert e.value.status == -1, args
    B.statekv_free_layer(h)


def test_restore_argument_errors_are_host_side():
    cfg = _cfg()  # T = 256, B = 4096, capacity 131072
    nbytes = B.statekv_workspace_bytes(cfg)
    h = B.statekv_init_layer(cfg, 1 << 40, nbytes)
    for args, status in [((-1, 0), -1), ((3, 700), -1), ((20, 4095), -1), ((513, 4096), -4)]:
        with pytest.raises(B.StateKVError) as e:
            B.statekv_restore_layer(h, *args)
        assert e.value.status == status, args
    B.statekv_restore_layer(h, 3, 768)
    st = B.statekv_state(h)
    assert st.frames_seen == 3 and st.count == 768 and st.last_pool == 0
    B.statekv_restore_layer(h, 40, 4096)
    assert B.statekv_state(h).count == 4096
    B.statekv_free_layer(h)


def test_attention_mass_argument_errors_are_host_side():
    """The App. A diagnostics need a frame that saw every token; bad budget
    lists and pointers are refused before anything is launched."""
    cfg = _cfg()  # T = 256, B = 4096
    nbytes = B.statekv_workspace_bytes(cfg)
    h = B.statekv_init_layer(cfg, 1 << 40, nbytes)
    assert B.statekv_mass_set_words(h) == (4096 + 256 + 31) // 32
    fake = 1 << 41
    cases = [([], -1), ([0], -1), (list(range(1, 66)), -1),
             ([1, 4], -1)]  # the last: no frame processed yet
    for budgets, status in cases:
        with pytest.raises(B.StateKVError) as e:
            B.statekv_attention_mass(h, budgets, fake, fake)
        assert e.value.status == status, budgets
    with pytest.raises(B.StateKVError) as e:
        B.statekv_attention_mass(h, [1], 0, fake)
    assert e.value.status == -1
    B.statekv_restore_layer(h, 3, 768)  # restored: the last frame's scores are gone
    with pytest.raises(B.StateKVError) as e:
        B.statekv_attention_mass(h, [1], fake, fake)
    assert e.value.status == -1
    B.statekv_free_layer(h)


def test_select_argument_errors():
    with pytest.raises(B.StateKVError):
        B.statekv_select_topb(0, 10, 5, 0)
    with pytest.raises(B.StateKVError) as e:
        B.statekv_select_topb(1 << 40, 40000, 5, 1 << 40)
    assert e.value.status == -2
    with pytest.raises(B.StateKVError):
        B.statekv_select_topb(1 << 40, 0, 5, 1 << 40)


def test_front_end_argument_errors_are_host_side():
    """statekv_qkv_rope rejects bad arguments before any launch (fake,
    16-byte aligned device addresses: nothing is dereferenced)."""
    a = 1 << 40
    good = dict(x=a, w=a, n_tokens=256, hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128,
                first_position=0, rope_theta=1e6, rope_scaling=1.0, q=a, k=a, v=a)
    bad = [(dict(x=0), -1), (dict(q=a + 2), -1), (dict(n_tokens=0), -1), (dict(hidden=-64), -1),
           (dict(n_q_heads=27), -1), (dict(first_position=-1), -1), (dict(rope_theta=-1.0), -1),
           (dict(rope_theta=1.0), -1), (dict(rope_theta=float("inf")), -1),
           (dict(rope_scaling=float("nan")), -1), (dict(head_dim=96), -2),
           (dict(hidden=3584 + 32), -2), (dict(n_tokens=(1 << 20) + 1), -2)]
    for change, status in bad:
        args = dict(good, **change)
        with pytest.raises(B.StateKVError) as e:
            B.statekv_qkv_rope(**args)
        assert e.value.status == status, change
    # a caller's workspace that is too small or not 256-byte aligned
    need = B.statekv_qkv_rope_workspace_size(256, 3584, 28, 4, 128)
    for change in (dict(workspace=a, workspace_bytes=need - 1),
                   dict(workspace=a + 16, workspace_bytes=need)):
        with pytest.raises(B.StateKVError) as e:
            B.statekv_qkv_rope(**dict(good, **change))
        assert e.value.status == -3, change


def test_front_end_workspace_size():
    """The splits' partial sums (S x feature tiles x T x 128 fp32) and the
    rotation table (T x d/2 (cos, sin) doubles), with S chosen so the
    tiles x S workgroups fit one per CU, each split covers at least 8 chunks
    of 64 hidden features and S <= 8; no workspace without a split."""
    size = B.statekv_qkv_rope_workspace_size
    # 8B shape: 2 token tiles x 36 heads = 72 tiles, S = min(256 // 72, 56 // 8) = 3
    assert size(256, 3584, 28, 4, 128) == 3 * 36 * 256 * 128 * 4 + 256 * 64 * 16
    # ragged T = 100: one token tile, S = min(256 // 36, 7) = 7
    assert size(100, 3584, 28, 4, 128) == 7 * 36 * 100 * 128 * 4 + 100 * 64 * 16
    # many chunks, few tiles: S capped at 8
    assert size(64, 8192, 4, 2, 64) == 8 * 4 * 64 * 128 * 4 + 64 * 32 * 16
    # 1B shape: hidden 896 is 14 chunks, too few to split
    assert size(256, 896, 14, 2, 64) == 0
    assert size(16, 128, 2, 1, 64) == 0
    for args, status in (((0, 3584, 28, 4, 128), -1), ((256, 3584, 27, 4, 128), -1),
                         ((256, 3584, 28, 4, 96), -2), ((256, 3600, 28, 4, 128), -2)):
        with pytest.raises(B.StateKVError) as e:
            size(*args)
        assert e.value.status == status, args


def test_status_strings():
    assert B.statekv_status_string(0) == "ok"
    assert "capacity" in B.statekv_status_string(-4)
    assert B.statekv_status_string(12345) == "unknown status"
