"""Benchmark of the StateKV per-layer video-prefill step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one frame through one layer: attention over [C_{n-1} ; frame]
with importance scores, top-B select, the state update C_n and the append to
D (every row of the hot path).  By default C is updated in place (kept rows
stay, kept frame tokens fill the freed rows; --state-layout rows rewrites C_n
in position order with a separate gather launch).  Default workload: the InternVL3-8B-like layer
(Hq=28, Hkv=4, d=128, T=256, B=4096), W=16 warm-up frames (they fill the
state: 16*256 = B) and K=496 timed frames, i.e. the pages' 512-frame stream.
All frames are generated on the host (seeded, synthetic) and staged in HBM
before the timed region.

Prints ONE JSON line: frames/s per layer over the K timed frames (no
per-launch instrumentation inside them), a roofline entry for the dominant
kernel and the per-kernel breakdown (launch durations from HIP events that the
dispatch itself timestamps on the launch stream, over the 32 frames right
after the timed region, state still full), and the float64 CPU oracle timed
on a bounded sample of the same stream.

Other measurements (not the headline line):
    --mode crossover   StateKV vs quadratic full attention, 1B shape,
                       B in {1024, 2048, 4096}, N in {32, ..., 512}
    --mode depth28     28 independent 2B-shaped layers, layer-major per
                       frame, per-frame latency at frames 1, 9, 65, 256
    --mode decode      decoding attention over the detailed state after the
                       512-frame 8B stream (1 and 4 text tokens): time per
                       call and HBM bandwidth of the decode kernel
    --mode mass        App. A diagnostics (top-b historical mass, recency
                       mass, candidate-pool recall) of a layer that keeps
                       every token, averaged over --mass-frames frames
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


def gen_workers(args) -> int:
    """Processes that generate the synthetic frames (forked from this one).
    Under a profiler that set up the GPU before the program started, forked
    workers inherit its state and its signal handlers, and their shutdown can
    hang: profiled runs pass --gen-workers 1."""
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


def select_bytes(Hkv, Hq, d, T, B, c, plan, in_place) -> float:
    """The select launch's bytes that must cross HBM once (state moves excluded:
    at most Hkv*T rows, data-dependent).

    Read the row tiles' score partials and write the scores; write the
    selection (kept indices, or in place the move lists); when the output pass
    ran in several key splits, read their O partials and write O; in place,
    also the D append (read the frame's K and V rows, write them to D)."""
    pool = c + T
    scores = Hkv * plan["row_tiles"] * pool * 4 + Hkv * pool * 4
    sel = Hkv * (2 * T + 1 if in_place else min(B, pool)) * 4
    S = plan["out_splits"]
    osum = (S + 1) * T * Hq * d * 4 if S > 1 else 0
    append = Hkv * T * 2 * (2 * d * 2) if in_place else 0
    return float(scores + sel + osum + append)


# ----------------------------------------------------------------------------
# CPU baseline: the float64 oracle on host cores
# ----------------------------------------------------------------------------

def cpu_baseline(spec, qs, ks, vs, warm: int, budget_s: float):
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
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    return {
        "value": done / dt,
        "unit": "frames/s per layer",
        "cores": int(max(blas) if blas else 1),
        "host_cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle, frames {warm}..{warm + done - 1} of the same "
                   f"stream after it ran frames 0..{warm - 1} untimed; {dt:.1f} s"),
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

def run_headline(args):
    import torch

    import framegen
    import streaming_long_video_amd as skv

    spec = framegen.workload(args.workload)
    if spec.n_layers != 1:
        raise SystemExit("the headline mode runs single-layer workloads")
    W, K = args.warmup, args.steps
    KB = args.breakdown_steps  # extra frames after the timed region, every kernel timed
    N = W + K + KB
    T, Hq, Hkv, d, Bs = (spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                         spec.state_budget)
    t_gen = time.perf_counter()
    qs, ks, vs = framegen.stacked_frames(spec, 0, N, workers=gen_workers(args))
    t_gen = time.perf_counter() - t_gen

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    q_all, k_all, v_all = up(qs), up(ks), up(vs)
    flags = {"rows": 0, "positions": skv.STATEKV_FLAG_C_IN_D,
             "inplace": skv.STATEKV_FLAG_SLOT_STABLE,
             "inplace-positions": skv.STATEKV_FLAG_SLOT_STABLE | skv.STATEKV_FLAG_C_IN_D,
             }[args.state_layout]
    layer = skv.Layer(Hq, Hkv, d, T, Bs, detailed_capacity=N * T, num_splits=args.splits,
                      flags=flags)
    out = torch.empty((T, Hq, d), dtype=torch.float32, device=dev)
    for n in range(W):
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

    all_mask = (1 << len(skv.STATEKV_KERNELS)) - 1
    mask = {"none": 0, "dominant": 1 << skv.STATEKV_KERNELS.index(DOMINANT),
            "all": all_mask}[args.events]
    skv.statekv_profile_start(layer.handle, mask, K * len(skv.STATEKV_KERNELS))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        layer.prefill(q_all[W + i], k_all[W + i], v_all[W + i], out=out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = skv.statekv_profile_stop(layer.handle)

    # per-kernel breakdown on the frames after the timed region (events around
    # every launch cost a little time, so they stay out of the timed frames)
    kernels_us = {k: (ms / cnt * 1e3 if cnt else None) for k, (ms, cnt) in prof.items()}
    if KB > 0:
        skv.statekv_profile_start(layer.handle, all_mask, KB * len(skv.STATEKV_KERNELS))
        for i in range(KB):
            n = W + K + i
            layer.prefill(q_all[n], k_all[n], v_all[n], out=out)
        torch.cuda.synchronize()
        bd = skv.statekv_profile_stop(layer.handle)
        breakdown_us = {k: ms / cnt * 1e3 for k, (ms, cnt) in bd.items() if cnt}
    else:
        breakdown_us = {k: v for k, v in kernels_us.items() if v}

    cs = [min(Bs, n * T) for n in range(W, W + K)]
    dominant = DOMINANT
    flops = float(np.mean([attn_out_flops(Hq, d, T, c) for c in cs]))
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
                   "frames": N, "detailed_capacity": N * T},
    }
    # the dominant kernel's launch duration: HIP events timestamped by the
    # dispatch on the launch stream -- from the timed region when it was
    # instrumented, else from the breakdown frames that follow it
    att = kernels_us.get("attn_out") or breakdown_us.get("attn_out")
    att_src = ("timed region" if kernels_us.get("attn_out") else
               f"frames {W + K}..{W + K + KB - 1}, right after the timed region")
    if att:
        achieved = flops / (att * 1e-6) / 1e12
        result["roofline"] = {
            "kernel": "attn_out (attention pass 2: QK^T recompute, P, PV, column sums)",
            "bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / PEAK_MFMA_TFLOPS,
            "traffic": measured_traffic("attn_out"),
            "flops_per_launch": flops, "avg_launch_us": att,
            "avg_launch_us_from": "HIP events on the launch stream, " + att_src,
        }
    if breakdown_us.get("attn_stats") and breakdown_us.get("attn_out"):
        useful = float(np.mean([useful_attention_flops(Hq, d, T, c) for c in cs]))
        t_att = (breakdown_us["attn_stats"] + breakdown_us["attn_out"]) * 1e-6
        result["attention"] = {
            "useful_tflops": useful / t_att / 1e12,
            "useful_frac_of_peak": useful / t_att / 1e12 / PEAK_MFMA_TFLOPS,
            "executed_frac_of_peak": 1.5 * useful / t_att / 1e12 / PEAK_MFMA_TFLOPS,
        }
    if breakdown_us.get("gather"):
        gb = float(np.mean([gather_bytes(Hkv, d, T, Bs, c, rows=args.state_layout == "rows")
                            for c in cs]))
        tg = breakdown_us["gather"]
        result["gather_append"] = {
            "bytes_per_launch": gb, "avg_launch_us": tg,
            "achieved_gbs": gb / (tg * 1e-6) / 1e9,
            "frac_of_hbm_peak": gb / (tg * 1e-6) / 1e9 / PEAK_HBM_GBS,
        }
    if breakdown_us.get("select"):
        in_place = args.state_layout.startswith("inplace")
        sb = float(np.mean([select_bytes(Hkv, Hq, d, T, Bs, c, layer.launch_plan(c + T), in_place)
                            for c in cs]))
        ts = breakdown_us["select"]
        result["select_launch"] = {
            "bytes_per_launch": sb, "avg_launch_us": ts,
            "achieved_gbs": sb / (ts * 1e-6) / 1e9,
            "frac_of_hbm_peak": sb / (ts * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "includes": "score sums, selection, O split sum" + (", D append" if in_place else ""),
        }
    result["kernels_us"] = {k: v for k, v in breakdown_us.items()}
    result["kernels_us_frames"] = f"{W + K}..{W + K + KB - 1}" if KB > 0 else "timed frames"
    result["dominant_kernel"] = dominant
    result["event_mode"] = args.events
    result["input_generation_s"] = t_gen
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, qs, ks, vs, W, args.cpu_seconds)
    print(json.dumps(result), flush=True)


# ----------------------------------------------------------------------------
# crossover sweep: StateKV vs quadratic full attention at the 1B shape
# ----------------------------------------------------------------------------

def run_crossover(args):
    import torch

    import framegen
    import streaming_long_video_amd as skv

    spec = framegen.workload("crossover_1b")
    T, Hq, Hkv, d = spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    Ns = [32, 64, 128, 256, 512]
    Nmax = max(Ns)
    qs, ks, vs = framegen.stacked_frames(spec, 0, Nmax, workers=gen_workers(args))
    dev = torch.device("cuda", 0)

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    q_all, k_all, v_all = up(qs), up(ks), up(vs)
    out = torch.empty((T, Hq, d), dtype=torch.float32, device=dev)
    rows = []
    # StateKV: per-frame time of every frame (events around each call)
    for B in (1024, 2048, 4096):
        layer = skv.Layer(Hq, Hkv, d, T, B, detailed_capacity=Nmax * T)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(Nmax + 1)]
        ev[0].record()
        for n in range(Nmax):
            layer.prefill(q_all[n], k_all[n], v_all[n], out=out)
            ev[n + 1].record()
        torch.cuda.synchronize()
        per = np.array([ev[n].elapsed_time(ev[n + 1]) for n in range(Nmax)])
        for N in Ns:
            steady = per[min(B // T + 1, N - 1):N]
            rows.append({"method": "statekv", "B": B, "N": N,
                         "ms_per_frame_steady": float(np.mean(steady)),
                         "ms_last_frame": float(per[N - 1]),
                         "ms_cumulative": float(per[:N].sum()),
                         "gflop_last_frame": useful_attention_flops(Hq, d, T, min(B, (N - 1) * T))
                         / 1e9,
                         "gflop_cumulative": sum(useful_attention_flops(Hq, d, T, min(B, n * T))
                                                 for n in range(N)) / 1e9})
        layer.close()
    # quadratic full attention: frame n attends over all n*T earlier tokens
    layer = skv.Layer(Hq, Hkv, d, T, 1024, detailed_capacity=Nmax * T)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(Nmax + 1)]
    ev[0].record()
    for n in range(Nmax):
        layer.full_attention(q_all[n], k_all[n], v_all[n], out=out)
        ev[n + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[n].elapsed_time(ev[n + 1]) for n in range(Nmax)])
    for N in Ns:
        rows.append({"method": "full_attention", "N": N,
                     "ms_last_frame": float(per[N - 1]),
                     "ms_cumulative": float(per[:N].sum()),
                     "gflop_last_frame": useful_attention_flops(Hq, d, T, (N - 1) * T) / 1e9,
                     "gflop_cumulative": sum(useful_attention_flops(Hq, d, T, n * T)
                                             for n in range(N)) / 1e9})
    print(json.dumps({"mode": "crossover", "workload": "crossover_1b", "rows": rows}), flush=True)


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
        layers.append(skv.Layer(Hq, Hkv, d, T, Bs, detailed_capacity=N * T))
    out = torch.empty((T, Hq, d), dtype=torch.float32, device=dev)
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
                      "ms_per_frame_all_layers": pick,
                      "ms_mean_steady": float(np.mean(per[Bs // T + 1:])),
                      "ms_first_frame": per[0]}), flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=496)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--mode", choices=["headline", "crossover", "depth28", "decode", "mass"],
                    default="headline")
    ap.add_argument("--decode-queries", type=int, nargs="+", default=[1, 4],
                    help="text tokens per decoding call (decode mode)")
    ap.add_argument("--events", choices=["none", "dominant", "all"], default="none",
                    help="kernels timed with HIP events during the timed region (each timed "
                         "launch costs a few microseconds of dispatch serialisation)")
    ap.add_argument("--breakdown-steps", type=int, default=32,
                    help="frames after the timed region with every kernel timed")
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        _fail_multi_gpu(max(args.gpus, int(os.environ.get("WORLD_SIZE", "1"))))
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")
    {"headline": run_headline, "crossover": run_crossover, "depth28": run_depth28,
     "decode": run_decode, "mass": run_mass}[args.mode](args)


if __name__ == "__main__":
    main()
