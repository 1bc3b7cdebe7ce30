"""Benchmark of the StateKV per-layer video-prefill step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one frame through one layer: attention over [C_{n-1} ; frame]
with importance scores, top-B select, the state update C_n and the append to
D (every row of the hot path).  By default C is updated in place (kept rows
stay, kept frame tokens fill the freed rows; --state-layout rows rewrites C_n
in position order with a separate gather launch).  Default workload: the
InternVL3-8B-like layer (Hq=28, Hkv=4, d=128, T=256, B=4096) over the pages'
512-frame stream, D preallocated for all of it (131072 tokens).  The first
ceil(B/T) = 16 frames fill the state (no eviction, smaller pools) and are
never timed; then W more untimed frames, then K timed frames, every one at
the full pool of B + T = 4352 candidates (defaults: W=0, K=496, i.e. frames
16..511).  All frames are generated on the host (seeded, synthetic) and
staged in HBM before the timed region.

Prints ONE JSON line: frames/s per layer over the K timed frames (no
per-launch instrumentation inside them); the per-kernel breakdown (launch
durations from HIP events that the dispatch itself timestamps on the launch
stream) over the 32 frames right after the timed region, and the per-frame
distribution (median, p5, p95) over the 64 frames after those, all at the
same pool size; a roofline entry for the dominant kernel whose flops are
those of that pool; the state update's algorithmic HBM rate; and the float64
CPU oracle timed on a bounded sample of the same stream.

Other measurements (not the headline line):
    --mode crossover   StateKV vs quadratic full attention, 1B shape,
                       B in {1024, 2048, 4096}, N in {2, 4, ..., 512}, and
                       the frames where time and FLOPs cross over
    --mode depth28     28 independent 2B-shaped layers, layer-major per
                       frame, per-frame latency at frames 1, 9, 65, 256
    --mode decode      decoding attention over the detailed state after the
                       512-frame 8B stream (1 and 4 text tokens): time per
                       call and HBM bandwidth of the decode kernel
    --mode mass        App. A diagnostics (top-b historical mass, recency
                       mass, candidate-pool recall) of a layer that keeps
                       every token, averaged over --mass-frames frames
    --mode frontend    the frame front end (q/k/v projection + RoPE) at the
                       workload's shape, weights read from HBM
    --mode rope        the library's standalone RoPE launch on one frame's
                       queries and keys (in place)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE = "internvl3_8b_layer"
DOMINANT = "attn_out"        # the longest kernel of the step (attention pass 2)


def _fail_multi_gpu(n):
    print(json.dumps({"error": f"--gpus {n}: this benchmark runs on one GPU only; the "
                               "StateKV step of a layer is measured on a single MI355X "
                               "(per-KV-head selection shards by KV head without "
                               "communication; layers pipeline across GPUs)."}))
    sys.exit(2)


# ----------------------------------------------------------------------------
# algorithmic work per kernel launch
# ----------------------------------------------------------------------------

def visible_pairs(T: int, c: int, causal: bool = True) -> float:
    """(query, key) pairs of one query head: every state key, the frame triangle."""
    return T * c + (T * (T + 1) / 2 if causal else T * T)


def attn_out_flops(Hq, d, T, c) -> float:
    """Pass 2: QK^T (2d per pair) and PV (2d per pair) on MFMA."""
    return 4.0 * Hq * d * visible_pairs(T, c)


def attn_stats_flops(Hq, d, T, c) -> float:
    """Pass 1: QK^T only."""
    return 2.0 * Hq * d * visible_pairs(T, c)


def useful_attention_flops(Hq, d, T, c) -> float:
    """What the step needs once: QK^T + PV over the visible pairs."""
    return 4.0 * Hq * d * visible_pairs(T, c)


def layout_flags(args) -> int:
    """Layer flags of --state-layout (C rewritten in position order, kept as
    positions into D, updated in place, or both)."""
    import streaming_long_video_amd as skv

    return {"rows": 0, "positions": skv.STATEKV_FLAG_C_IN_D,
            "inplace": skv.STATEKV_FLAG_SLOT_STABLE,
            "inplace-positions": skv.STATEKV_FLAG_SLOT_STABLE | skv.STATEKV_FLAG_C_IN_D,
            }[args.state_layout]


def gen_workers(args) -> int:
    """Processes that generate the synthetic frames (spawned, so nothing this
    process has set up on the GPU is inherited; profiled runs still pass
    --gen-workers 1 to keep the profiler's process tree small)."""
    if args.gen_workers > 0:
        return args.gen_workers
    return min(16, os.cpu_count() or 1)


def gather_bytes(Hkv, d, T, B, c, rows=True) -> float:
    """C_n gather + D append, bytes that must cross HBM once.

    Per kept row: read K and V (2*d*2 bytes) from C_{n-1} or the frame, write
    them to C_n (not when C is kept as positions into D); read the selection
    index (4 B) and the old position (8 B), write the position (8 B).  Append:
    read the frame's K and V rows, write them to D."""
    newc = min(B, c + T)
    row = 2 * d * 2
    gather = Hkv * newc * ((2 * row if rows else 0) + 4 + 8 + 8)
    append = Hkv * T * 2 * row
    return float(gather + append)


def state_update_bytes(Hkv, d, T, B, moved_rows, in_place) -> float:
    """Algorithmic bytes of the state update (select, C_n, D append) at the
    steady state, as the scope table counts them: read the pool's importance
    (Hkv*(B+T) floats); write the selection (kept indices, or in place the
    move lists of 2T+1 words per head); move the kept rows (in place only the
    kept frame tokens: read and write their K and V rows; with the rewritten
    state every kept row plus its position); append the frame to D (read and
    write its K and V rows).  Split partials (score row tiles, O splits) are
    the attention's implementation traffic and are reported separately."""
    row = 2 * d * 2
    sigma = Hkv * (B + T) * 4
    sel = Hkv * ((2 * T + 1) if in_place else B) * 4
    if in_place:
        moves = moved_rows * 2 * row
    else:
        moves = Hkv * B * (2 * row + 8 + 8 + 4)
    append = Hkv * T * 2 * row
    return float(sigma + sel + moves + append)


def split_partial_bytes(Hq, Hkv, d, T, plan) -> dict:
    """Bytes the split-K attention writes and reads back beyond the algorithm:
    per-split row statistics (one log-sum-exp per row), per-row-tile score
    partials, per-split O."""
    stat = plan["stat_splits"] * Hq * T * 4
    pool_words = plan["key_tiles"] * 64
    score = Hkv * plan["row_tiles"] * pool_words * 4
    S = plan["out_splits"]
    opart = S * T * Hq * d * 4 if S > 1 else 0
    return {"stat_partials_written": float(stat), "score_partials_written": float(score),
            "o_partials_written": float(opart)}


# ----------------------------------------------------------------------------
# CPU baseline: the float64 oracle on host cores
# ----------------------------------------------------------------------------

def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, qs, ks, vs, warm: int, budget_s: float):
    """The oracle as it stands, one process, numpy's BLAS threads, on a bounded
    sample of the same stream (frames after the state has filled)."""
    from threadpoolctl import threadpool_info

    from oracle import StateKVOracle

    orc = StateKVOracle(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.frame_tokens,
                        spec.state_budget)
    for n in range(warm):
        orc.step(qs[n], ks[n], vs[n])
    t0 = time.perf_counter()
    done = 0
    n = warm
    while n < qs.shape[0] and (done < 3 or time.perf_counter() - t0 < budget_s):
        orc.step(qs[n], ks[n], vs[n])
        n += 1
        done += 1
    dt = time.perf_counter() - t0
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    return {
        "value": done / dt,
        "unit": "frames/s per layer",
        "cores": int(threads),
        "host_cores": len(os.sched_getaffinity(0)),
        "processes": 1,
        "cpu_model": _cpu_model(),
        "numpy": np.__version__,
        "blas": [{"library": p.get("internal_api"), "version": p.get("version"),
                  "threads": p.get("num_threads")} for p in blas],
        "kind": "oracle",
        "sample": (f"float64 numpy oracle, frames {warm}..{warm + done - 1} of the same "
                   f"stream (state full) after it ran frames 0..{warm - 1} untimed; "
                   f"{dt:.1f} s in one process"),
    }


# ----------------------------------------------------------------------------
# traffic counters taken with rocprofv3 (committed under profiles/)
# ----------------------------------------------------------------------------

def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when it is missing or was taken on other kernel sources."""
    from streaming_long_video_amd.profiling import source_hash

    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get("kernels", {}).get(kernel)
    if not entry or data.get("source_hash") != source_hash():
        return None
    return entry.get("bytes_per_launch")


# ----------------------------------------------------------------------------
# headline: one layer, 512-frame stream
# ----------------------------------------------------------------------------

def _pct(x, q):
    return float(np.percentile(np.asarray(x, dtype=np.float64), q))


def run_headline(args):
    import torch

    import framegen
    import streaming_long_video_amd as skv

    spec = framegen.workload(args.workload)
    if spec.n_layers != 1:
        raise SystemExit("the headline mode runs single-layer workloads")
    T, Hq, Hkv, d, Bs = (spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                         spec.state_budget)
    # frames 0..fill-1 fill the state (c < B, no eviction): never timed
    fill = -(-Bs // T)
    W, K = args.warmup, args.steps
    KB = args.breakdown_steps  # every kernel timed with HIP events
    KD = args.dist_steps       # one HIP event per frame boundary
    first = fill + W           # first timed frame
    N = first + K + KB + KD
    cap_frames = max(spec.n_frames, N)  # D sized for the whole stream
    t_gen = time.perf_counter()
    qs, ks, vs = framegen.stacked_frames(spec, 0, N, workers=gen_workers(args))
    t_gen = time.perf_counter() - t_gen

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    q_all, k_all, v_all = up(qs), up(ks), up(vs)
    flags = layout_flags(args)
    in_place = args.state_layout.startswith("inplace")
    layer = skv.Layer(Hq, Hkv, d, T, Bs, detailed_capacity=cap_frames * T,
                      num_splits=args.splits, flags=flags)
    out = torch.empty((T, Hq, d), dtype=torch.float32, device=dev)
    for n in range(first):
        layer.prefill(q_all[n], k_all[n], v_all[n], out=out)
    if args.copy_probe_mib > 0:
        # a plain device copy of known size: its FETCH_SIZE / WRITE_SIZE
        # counters scale the kernels' counters to bytes (outside the timed region)
        n_el = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n_el, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        del src, dst
    torch.cuda.synchronize()
    c_steady = layer.state()["count"]
    if c_steady != Bs:
        raise SystemExit(f"state not full before the timed region ({c_steady} of {Bs})")
    pool = c_steady + T

    all_mask = (1 << len(skv.STATEKV_KERNELS)) - 1
    mask = {"none": 0, "dominant": 1 << skv.STATEKV_KERNELS.index(DOMINANT),
            "all": all_mask}[args.events]
    skv.statekv_profile_start(layer.handle, mask, K * len(skv.STATEKV_KERNELS))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        layer.prefill(q_all[first + i], k_all[first + i], v_all[first + i], out=out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = skv.statekv_profile_stop(layer.handle)
    kernels_us = {k: (ms / cnt * 1e3 if cnt else None) for k, (ms, cnt) in prof.items()}

    # per-kernel launch durations on the frames right after the timed region
    # (events around every launch cost a little time, so they stay out of it);
    # every one of these frames runs at the same pool size as the timed ones
    n0 = first + K
    breakdown_us = {}
    moved_rows = None
    if KB > 0:
        skv.statekv_profile_start(layer.handle, all_mask, KB * len(skv.STATEKV_KERNELS))
        for i in range(KB):
            layer.prefill(q_all[n0 + i], k_all[n0 + i], v_all[n0 + i], out=out)
        torch.cuda.synchronize()
        bd = skv.statekv_profile_stop(layer.handle)
        breakdown_us = {k: ms / cnt * 1e3 for k, (ms, cnt) in bd.items() if cnt}
        # rows the last of these frames moved: its kept frame tokens, all heads
        st = layer.state()
        last0 = (n0 + KB - 1) * T + layer.position_offset
        moved_rows = int((st["pos"][:, :st["count"]] >= last0).sum().item())
    # per-frame wall time distribution: one event per frame boundary
    n1 = n0 + KB
    frame_us = None
    if KD > 0:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(KD + 1)]
        ev[0].record()
        for i in range(KD):
            layer.prefill(q_all[n1 + i], k_all[n1 + i], v_all[n1 + i], out=out)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(KD)]
        frame_us = {"mean": float(np.mean(per)), "median": _pct(per, 50),
                    "p5": _pct(per, 5), "p95": _pct(per, 95),
                    "frames": f"{n1}..{n1 + KD - 1}",
                    "how": "HIP events recorded between consecutive frames on the launch stream"}
    if layer.state()["pool"] != pool:
        raise SystemExit("the pool size changed during the measured frames")

    plan = layer.launch_plan(pool)
    result = {
        "metric": "video-prefill frames/s per layer + % bf16 MFMA peak (8B shape, B=4096, T=256)",
        "value": K / elapsed,
        "unit": "frames/s per layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, RoPE at original positions, "
                "10 planted temporal-sink keys in frames 0-3)",
        "config": {"workload": args.workload, "state_layout": args.state_layout,
                   "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": d, "frame_tokens": T, "state_budget": Bs,
                   "stream_frames": spec.n_frames, "frames_run": N,
                   "detailed_capacity": cap_frames * T,
                   "fill_frames_untimed": fill, "timed_frames": f"{first}..{first + K - 1}",
                   "timed_pool": pool},
    }
    if frame_us:
        result["per_frame_us"] = frame_us
    # the dominant kernel: its algorithmic flops at the pool of the frames whose
    # launch durations are used (HIP events the dispatch itself timestamps on
    # the launch stream): the timed region when it was instrumented, else the
    # breakdown frames that follow it
    flops = attn_out_flops(Hq, d, T, c_steady)
    att = kernels_us.get("attn_out") or breakdown_us.get("attn_out")
    att_src = ("timed region" if kernels_us.get("attn_out") else
               f"frames {n0}..{n0 + KB - 1}, right after the timed region")
    if att:
        achieved = flops / (att * 1e-6) / 1e12
        result["roofline"] = {
            "kernel": "attn_out (attention pass 2: QK^T recompute, P, PV, column sums)",
            "bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / PEAK_MFMA_TFLOPS,
            "traffic": measured_traffic("attn_out"),
            "flops_per_launch": flops, "pool": pool, "avg_launch_us": att,
            "avg_launch_us_from": "HIP events on the launch stream, " + att_src,
        }
    if breakdown_us.get("attn_stats") and breakdown_us.get("attn_out"):
        useful = useful_attention_flops(Hq, d, T, c_steady)
        t_att = (breakdown_us["attn_stats"] + breakdown_us["attn_out"]) * 1e-6
        result["attention"] = {
            "useful_gflop": useful / 1e9,
            "useful_tflops": useful / t_att / 1e12,
            "useful_frac_of_peak": useful / t_att / 1e12 / PEAK_MFMA_TFLOPS,
            "executed_frac_of_peak": 1.5 * useful / t_att / 1e12 / PEAK_MFMA_TFLOPS,
        }
    upd_us = (breakdown_us.get("select") or 0.0) + (breakdown_us.get("gather") or 0.0)
    if upd_us and moved_rows is not None:
        ub = state_update_bytes(Hkv, d, T, Bs, moved_rows, in_place)
        result["state_update"] = {
            "launches": ["select"] + ([] if in_place else ["gather"]),
            "algorithmic_bytes": ub, "us": upd_us,
            "achieved_gbs": ub / (upd_us * 1e-6) / 1e9,
            "frac_of_hbm_peak": ub / (upd_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "moved_rows_last_frame": moved_rows,
            "counts": "importance read, selection written, kept rows moved, D append "
                      "(read + write); not the attention's split partials",
        }
    result["split_partials"] = dict(split_partial_bytes(Hq, Hkv, d, T, plan), plan=plan)
    result["kernels_us"] = {k: v for k, v in breakdown_us.items()}
    result["kernels_us_frames"] = f"{n0}..{n0 + KB - 1}" if KB > 0 else None
    result["dominant_kernel"] = DOMINANT
    result["event_mode"] = args.events
    result["input_generation_s"] = t_gen
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, qs, ks, vs, fill, args.cpu_seconds)
    print(json.dumps(result), flush=True)


# ----------------------------------------------------------------------------
# crossover sweep: StateKV vs quadratic full attention at the 1B shape
# ----------------------------------------------------------------------------

def run_crossover(args):
    """StateKV against quadratic full attention at the 1B shape: per-frame time
    of every frame n < 512 for each budget (HIP events between frames), the
    marginal and cumulative time at N in {2, 4, ..., 512}, and the first frame
    from which full attention's per-frame time stays above StateKV's (the time
    crossover) beside the FLOP crossover."""
    import torch

    import framegen
    import streaming_long_video_amd as skv

    spec = framegen.workload("crossover_1b")
    T, Hq, Hkv, d = spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    Ns = [2, 4, 8, 16, 32, 64, 128, 256, 512]
    Nmax = max(Ns)
    qs, ks, vs = framegen.stacked_frames(spec, 0, Nmax, workers=gen_workers(args))
    dev = torch.device("cuda", 0)

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    q_all, k_all, v_all = up(qs), up(ks), up(vs)
    out = torch.empty((T, Hq, d), dtype=torch.float32, device=dev)

    def per_frame(call):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(Nmax + 1)]
        ev[0].record()
        for n in range(Nmax):
            call(n)
            ev[n + 1].record()
        torch.cuda.synchronize()
        return np.array([ev[n].elapsed_time(ev[n + 1]) for n in range(Nmax)])

    def first_stays_above(a, b):
        """first n from which a[m] > b[m] for every m >= n (None if never)"""
        above = a > b
        for n in range(len(a)):
            if above[n:].all():
                return n
        return None

    # untimed warm-up of both methods (the first launch of each kernel loads
    # its code object, about a millisecond), through the first evictions
    warm_frames = 2048 // T + 2
    for call in ("full_attention", "prefill"):
        layer = skv.Layer(Hq, Hkv, d, T, 1024, detailed_capacity=warm_frames * T,
                          num_splits=args.splits, flags=layout_flags(args))
        for n in range(warm_frames):
            getattr(layer, call)(q_all[n], k_all[n], v_all[n], out=out)
        torch.cuda.synchronize()
        layer.close()

    # quadratic full attention: frame n attends over all n*T earlier tokens
    layer = skv.Layer(Hq, Hkv, d, T, 1024, detailed_capacity=Nmax * T)
    full = per_frame(lambda n: layer.full_attention(q_all[n], k_all[n], v_all[n], out=out))
    layer.close()
    full_flops = np.array([useful_attention_flops(Hq, d, T, n * T) for n in range(Nmax)])
    rows, crossings = [], {}
    for B in (1024, 2048, 4096):
        layer = skv.Layer(Hq, Hkv, d, T, B, detailed_capacity=Nmax * T, num_splits=args.splits,
                          flags=layout_flags(args))
        per = per_frame(lambda n: layer.prefill(q_all[n], k_all[n], v_all[n], out=out))
        layer.close()
        flops = np.array([useful_attention_flops(Hq, d, T, min(B, n * T)) for n in range(Nmax)])
        crossings[str(B)] = {
            "time_frame": first_stays_above(full, per),
            "flop_frame": first_stays_above(full_flops, flops),
        }
        for N in Ns:
            steady = per[min(B // T + 1, N - 1):N]
            rows.append({"method": "statekv", "B": B, "N": N,
                         "ms_per_frame_steady": float(np.mean(steady)),
                         "ms_last_frame": float(per[N - 1]),
                         "ms_cumulative": float(per[:N].sum()),
                         "gflop_last_frame": float(flops[N - 1]) / 1e9,
                         "gflop_cumulative": float(flops[:N].sum()) / 1e9})
    for N in Ns:
        rows.append({"method": "full_attention", "N": N,
                     "ms_last_frame": float(full[N - 1]),
                     "ms_cumulative": float(full[:N].sum()),
                     "gflop_last_frame": float(full_flops[N - 1]) / 1e9,
                     "gflop_cumulative": float(full_flops[:N].sum()) / 1e9})
    print(json.dumps({"mode": "crossover", "workload": "crossover_1b",
                      "splits": args.splits or "auto", "state_layout": args.state_layout,
                      "timing": "HIP events between consecutive frames on the launch stream",
                      "crossover": crossings, "rows": rows}), flush=True)


# ----------------------------------------------------------------------------
# decoding over the detailed state after the whole 8B-like stream
# ----------------------------------------------------------------------------

def run_decode(args):
    import torch

    import framegen
    import streaming_long_video_amd as skv

    spec = framegen.workload(args.workload)
    T, Hq, Hkv, d, Bs, N = (spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                            spec.state_budget, spec.n_frames)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    layer = skv.Layer(Hq, Hkv, d, T, Bs, detailed_capacity=N * T)
    chunk = 64
    for n0 in range(0, N, chunk):
        qs, ks, vs = framegen.stacked_frames(spec, n0, min(N, n0 + chunk),
                                             workers=gen_workers(args))
        up = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        q_d, k_d, v_d = up(qs), up(ks), up(vs)
        for i in range(q_d.shape[0]):
            layer.prefill(q_d[i], k_d[i], v_d[i])
    torch.cuda.synchronize()
    out = {}
    for M in args.decode_queries:
        q = torch.from_numpy(framegen.text_queries(spec, M, 0).view(np.int16)).to(dev)
        q = q.view(torch.bfloat16)
        o = torch.empty((M, Hq, d), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            layer.decode(q, out=o)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            layer.decode(q, out=o)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        skv.statekv_profile_start(layer.handle, (1 << len(skv.STATEKV_KERNELS)) - 1,
                                  64 * len(skv.STATEKV_KERNELS))
        for _ in range(64):
            layer.decode(q, out=o)
        torch.cuda.synchronize()
        prof = skv.statekv_profile_stop(layer.handle)
        us = {k: ms / cnt * 1e3 for k, (ms, cnt) in prof.items() if cnt}
        nbytes = 2.0 * Hkv * N * T * d * 2  # K and V of every D token
        out[f"M={M}"] = {
            "us_per_step": dt * 1e6, "decode_kernel_us": us.get("decode"),
            "combine_us": us.get("split_sum"),
            "d_bytes": nbytes,
            "decode_kernel_gbs": nbytes / (us["decode"] * 1e-6) / 1e9 if us.get("decode") else None,
            "frac_of_hbm_peak": (nbytes / (us["decode"] * 1e-6) / 1e9 / PEAK_HBM_GBS
                                 if us.get("decode") else None),
        }
    print(json.dumps({"mode": "decode", "workload": args.workload, "frames": N,
                      "tokens_per_kv_head": N * T, "results": out}), flush=True)


# ----------------------------------------------------------------------------
# App. A diagnostics on the synthetic stream
# ----------------------------------------------------------------------------

MASS_BUDGETS = [1, 4, 16, 64, 256, 1024, 4096]


def run_mass(args):
    """A layer of the workload's shape that keeps every token (budget = the
    whole history) over --mass-frames frames; after each frame the App. A
    diagnostics: top-b historical mass share (A.1), recency share (A.3) and
    weighted candidate-pool recall (A.2), averaged over frames 1.. ."""
    import torch

    import framegen
    import streaming_long_video_amd as skv

    spec = framegen.workload(args.workload)
    T, Hq, Hkv, d = spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    N = args.mass_frames
    spec = spec.replace(n_frames=N, state_budget=N * T)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    layer = skv.Layer(Hq, Hkv, d, T, N * T, detailed_capacity=N * T)
    qs, ks, vs = framegen.stacked_frames(spec, 0, N, workers=gen_workers(args))
    up = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    q_d, k_d, v_d = up(qs), up(ks), up(vs)
    sets, rows = None, []
    for n in range(N):
        layer.prefill(q_d[n], k_d[n], v_d[n])
        out, sets = layer.attention_mass(MASS_BUDGETS, sets)
        if n >= 1:
            rows.append(out.cpu().numpy().astype(np.float64))
    a = np.stack(rows)  # [frames][budget][3]
    res = {}
    for i, b in enumerate(MASS_BUDGETS):
        res[str(b)] = {"topb_mass": float(np.nanmean(a[:, i, 0])),
                       "recency_mass": float(np.nanmean(a[:, i, 1])),
                       "pool_recall": float(np.nanmean(a[:, i, 2]))}
    print(json.dumps({"mode": "mass", "workload": args.workload, "frames": N,
                      "data": "synthetic (seeded N(0,1) bf16 Q/K/V, RoPE at original positions, "
                              "planted temporal-sink keys in frames 0-3)",
                      "averaged_over_frames": f"1..{N - 1}", "budgets": res}), flush=True)


# ----------------------------------------------------------------------------
# the frame front end: q, k, v = rope(X W_Q), rope(X W_K), X W_V
# ----------------------------------------------------------------------------

def run_rope(args):
    """Time statekv_rope at the workload's shape: the frame's queries and keys
    (T x (Hq + Hkv) rows of d bf16) rotated in place at their positions, one
    call for q and one for k per frame, as a caller that leaves RoPE to the
    library does.  Algorithmic bytes: every element read and written once."""
    import torch

    import framegen
    import streaming_long_video_amd as skv

    spec = framegen.workload(args.workload)
    T, Hq, Hkv, d = spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    dev = torch.device("cuda", 0)
    layer = skv.Layer(Hq, Hkv, d, T, spec.state_budget, detailed_capacity=T,
                      rope_theta=spec.rope_theta)
    g = torch.Generator(device="cpu").manual_seed(spec.seed)
    q = torch.randn((T, Hq, d), generator=g).to(dev, torch.bfloat16)
    k = torch.randn((T, Hkv, d), generator=g).to(dev, torch.bfloat16)
    for i in range(args.warmup + 8):
        layer.rope(q, i * T)
        layer.rope(k, i * T)
    torch.cuda.synchronize()
    # the launches of 16 frames recorded once as a HIP graph and replayed, so
    # that the host-side cost of the Python calls (several us each) does not
    # set the rate
    per_graph = 16
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(per_graph):
            layer.rope(q, i * T)
            layer.rope(k, i * T)
    replays = max(1, (args.steps + per_graph - 1) // per_graph)
    graph.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(replays):
        graph.replay()
    ev[1].record()
    torch.cuda.synchronize()
    frames = replays * per_graph
    us = ev[0].elapsed_time(ev[1]) * 1e3 / frames
    # the same calls from Python, for comparison (host-bound)
    t0 = time.perf_counter()
    for i in range(args.steps):
        layer.rope(q, i * T)
        layer.rope(k, i * T)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) * 1e6 / args.steps
    del graph
    layer.close()
    nbytes = 2 * T * (Hq + Hkv) * d * 2
    print(json.dumps({
        "mode": "rope", "workload": args.workload, "tokens": T, "heads": Hq + Hkv,
        "head_dim": d, "calls_per_frame": 2, "frames": frames,
        "us_per_frame": us, "eager_us_per_frame": eager_us, "algorithmic_bytes": nbytes,
        "achieved_gbs": nbytes / (us * 1e-6) / 1e9,
        "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "timing": "HIP events around replays of a HIP graph of 16 frames' launches",
    }), flush=True)


def run_frontend(args):
    """Time statekv_qkv_rope at the workload's shape (hidden = Hq * d).  The
    calls cycle through --frontend-layers distinct weight copies (together
    larger than the 256 MB last-level cache), as the layers of a model would,
    so that every call reads its weights from HBM."""
    import torch

    import framegen
    import streaming_long_video_amd as skv

    spec = framegen.workload(args.workload)
    T, Hq, Hkv, d = spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    hid = framegen.hidden_width(spec)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(
        torch.bfloat16)
    w0 = up(framegen.projection_weights(spec))
    ws = [w0] + [w0.clone() for _ in range(args.frontend_layers - 1)]
    xs = [up(framegen.hidden_states(spec, n)) for n in range(8)]
    outs = (torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev),
            torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=dev),
            torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=dev))
    L = len(ws)
    need = skv.qkv_rope_workspace_bytes(T, hid, Hq, Hkv, d)
    work = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None
    for i in range(args.warmup + L):
        skv.qkv_rope(xs[i % 8], ws[i % L], Hq, Hkv, d, i * T, spec.rope_theta, out=outs,
                     workspace=work)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    t0 = time.perf_counter()
    for i in range(args.steps):
        skv.qkv_rope(xs[i % 8], ws[i % L], Hq, Hkv, d, i * T, spec.rope_theta, out=outs,
                     workspace=work)
    host_us = (time.perf_counter() - t0) * 1e6 / args.steps
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / args.steps
    rows = (Hq + 2 * Hkv) * d
    nbytes = rows * hid * 2 + T * hid * 2 + T * rows * 2
    flops = 2.0 * T * hid * rows
    print(json.dumps({
        "mode": "frontend", "workload": args.workload, "tokens": T, "hidden": hid,
        "out_features": rows, "weight_copies": L, "calls": args.steps,
        "us_per_call": us, "host_us_per_call": host_us, "workspace_bytes": need,
        "algorithmic_bytes": nbytes,
        "achieved_gbs": nbytes / (us * 1e-6) / 1e9,
        "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "gflop": flops / 1e9, "tflops": flops / (us * 1e-6) / 1e12,
        "frac_of_mfma_peak": flops / (us * 1e-6) / 1e12 / PEAK_MFMA_TFLOPS,
        "timing": "HIP events around the calls on the launch stream",
    }), flush=True)


# ----------------------------------------------------------------------------
# 28 layers of the 2B shape, layer-major per frame
# ----------------------------------------------------------------------------

def run_depth28(args):
    import torch

    import framegen
    import streaming_long_video_amd as skv

    spec = framegen.workload("internvl3_2b_28layers")
    T, Hq, Hkv, d, Bs = (spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                         spec.state_budget)
    N, L = spec.n_frames, spec.n_layers
    dev = torch.device("cuda", 0)
    layers, frames = [], []
    for l in range(L):
        s = spec.for_layer(l)
        qs, ks, vs = framegen.stacked_frames(s, 0, N, workers=gen_workers(args))
        up = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        frames.append((up(qs), up(ks), up(vs)))
        layers.append(skv.Layer(Hq, Hkv, d, T, Bs, detailed_capacity=N * T,
                                num_splits=args.splits, flags=layout_flags(args)))
    out = torch.empty((T, Hq, d), dtype=torch.float32, device=dev)
    # untimed warm-up through the first evictions on a scratch layer (the
    # first launch of each kernel loads its code object)
    warm_frames = Bs // T + 2
    warm = skv.Layer(Hq, Hkv, d, T, Bs, detailed_capacity=warm_frames * T,
                     num_splits=args.splits, flags=layout_flags(args))
    for n in range(warm_frames):
        warm.prefill(frames[0][0][n], frames[0][1][n], frames[0][2][n], out=out)
    torch.cuda.synchronize()
    warm.close()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(N + 1)]
    ev[0].record()
    for n in range(N):
        for l in range(L):
            q, k, v = frames[l]
            layers[l].prefill(q[n], k[n], v[n], out=out)
        ev[n + 1].record()
    torch.cuda.synchronize()
    per = [ev[n].elapsed_time(ev[n + 1]) for n in range(N)]
    pick = {f"frame_{n + 1}": per[n] for n in (0, 8, 64, N - 1)}
    print(json.dumps({"mode": "depth28", "workload": "internvl3_2b_28layers",
                      "splits": args.splits or "auto", "state_layout": args.state_layout,
                      "ms_per_frame_all_layers": pick,
                      "ms_mean_steady": float(np.mean(per[Bs // T + 1:])),
                      "ms_first_frame": per[0]}), flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=496,
                    help="timed frames (all at the full state)")
    ap.add_argument("--warmup", type=int, default=0,
                    help="untimed frames after the state-fill frames (ceil(B/T), never timed)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--mode", choices=["headline", "crossover", "depth28", "decode", "mass",
                                       "frontend", "rope"],
                    default="headline")
    ap.add_argument("--decode-queries", type=int, nargs="+", default=[1, 4],
                    help="text tokens per decoding call (decode mode)")
    ap.add_argument("--events", choices=["none", "dominant", "all"], default="none",
                    help="kernels timed with HIP events during the timed region (each timed "
                         "launch costs a few microseconds of dispatch serialisation)")
    ap.add_argument("--breakdown-steps", type=int, default=32,
                    help="frames after the timed region with every kernel timed")
    ap.add_argument("--dist-steps", type=int, default=64,
                    help="frames after those with one event per frame (median, p5, p95)")
    ap.add_argument("--gen-workers", type=int, default=0,
                    help="processes generating the synthetic frames (0: up to 16; 1 under "
                         "a profiler)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run a plain device copy of this size before the timed region "
                         "(reference kernel for rocprofv3 byte counters)")
    ap.add_argument("--splits", type=int, default=0, help="attention key splits (0 = auto)")
    ap.add_argument("--state-layout", choices=["rows", "positions", "inplace", "inplace-positions"],
                    default="inplace",
                    help="C as its own K/V rows rewritten on update (rows), as positions into "
                         "D (positions), updated in place (inplace), or both")
    ap.add_argument("--mass-frames", type=int, default=64,
                    help="frames of the App. A diagnostics run (--mode mass)")
    ap.add_argument("--frontend-layers", type=int, default=12,
                    help="distinct weight copies the front-end timing cycles through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        _fail_multi_gpu(max(args.gpus, int(os.environ.get("WORLD_SIZE", "1"))))
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")
    {"headline": run_headline, "crossover": run_crossover, "depth28": run_depth28,
     "decode": run_decode, "mass": run_mass, "frontend": run_frontend,
     "rope": run_rope}[args.mode](args)


if __name__ == "__main__":
    main()
