"""Summaries of rocprofv3 output for the StateKV kernels.

    python -m streaming_long_video_amd.profiling trace DIR [--last N]
        DIR holds the CSV output of
        `rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run -- <program>`;
        prints a markdown table: per kernel, the dispatch count, the mean
        duration over all dispatches and over the last N dispatches of that
        kernel (steady state), and the min / max.

    python -m streaming_long_video_amd.profiling traffic --fetch DIR --write DIR
            --copy-mib M [--last N] [--out FILE]
        DIRs hold the CSV output of one `rocprofv3 --pmc FETCH_SIZE` run and one
        `rocprofv3 --pmc WRITE_SIZE` run of `bench.py --copy-probe-mib M`.  The
        probe (an elementwise negation reading and writing M MiB) calibrates
        the counters: bytes = counter_KiB * 1024 * (M MiB / probe counter).
        Prints per-kernel calibrated bytes per launch (mean over the last N
        dispatches) and, with --out, writes them as JSON together with a hash of
        the kernel sources they were taken on.

Only reads files; runs nothing on the GPU.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

# kernel id -> pattern of its rocprofv3 name (d = 128 instantiations)
KERNELS = {
    "attn_stats": r"attn_kernel<128, 1(, false)?>",
    "attn_out": r"attn_kernel<128, 2(, false)?>",
    "select": r"select_sum_kernel",
    "gather": r"gather_append_kernel<128>",
    "full_attn": r"attn_kernel<128, 3(, false)?>",
    "full_combine": r"full_combine_kernel<128>",
    "decode": r"decode_kernel<128>",
    "decode_merge": r"decode_merge_kernel<128>",
    "qkv_rope": r"qkv_rope_kernel<128>",
}
PROBE = r"neg"  # torch's negation kernel: the copy probe

SOURCES = (
    # the host plan and launch code choose split counts and grids, which
    # decide part of the measured traffic
    "csrc/plan.h",
    "csrc/plan.cpp",
    "csrc/skv_internal.h",
    "csrc/statekv_api.hip",
    "csrc/kernels/attention.hip",
    "csrc/kernels/select.hip",
    "csrc/kernels/gather.hip",
    "csrc/kernels/decode.hip",
    "csrc/kernels/rope.hip",
)


def source_hash() -> str:
    """Hash of the kernel and launch-plan sources: counters taken on other
    sources are stale."""
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(here, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one(pattern: str, root: str) -> str:
    hits = sorted(glob.glob(os.path.join(root, "**", pattern), recursive=True))
    if not hits:
        raise SystemExit(f"no {pattern} under {root}")
    return hits[-1]


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0]


def kernel_durations(root: str):
    """{kernel name: [durations in ns, dispatch order]} from a kernel trace."""
    path = _one("*kernel_trace.csv", root)
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out = collections.defaultdict(list)
    for r in rows:
        out[_short(r["Kernel_Name"])].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def trace_table(root: str, last: int) -> str:
    durs = kernel_durations(root)
    lines = ["| kernel | dispatches | mean us (all) | mean us (last %d) | min us | max us |" % last,
             "|---|---:|---:|---:|---:|---:|"]
    total = {k: sum(v) for k, v in durs.items()}
    for k in sorted(durs, key=lambda k: -total[k]):
        v = durs[k]
        tail = v[-last:]
        lines.append(f"| `{k}` | {len(v)} | {sum(v) / len(v) / 1e3:.2f} | "
                     f"{sum(tail) / len(tail) / 1e3:.2f} | {min(v) / 1e3:.2f} | {max(v) / 1e3:.2f} |")
    return "\n".join(lines)


def counter_per_dispatch(root: str, counter: str):
    """{kernel name: [value per dispatch, dispatch order]} for one counter."""
    path = _one("*counter_collection.csv", root)
    per = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        per[d] += float(r["Counter_Value"])
        names[d] = _short(r["Kernel_Name"])
    out = collections.defaultdict(list)
    for d in sorted(per):
        out[names[d]].append(per[d])
    return out


def _match(values: dict, pattern: str):
    hits = [k for k in values if re.search(pattern, k)]
    if len(hits) != 1:
        return None
    return values[hits[0]]


def traffic(fetch_root: str, write_root: str, copy_mib: int, last: int):
    fetch = counter_per_dispatch(fetch_root, "FETCH_SIZE")
    write = counter_per_dispatch(write_root, "WRITE_SIZE")
    probe_bytes = copy_mib * float(1 << 20)
    pf, pw = _match(fetch, PROBE), _match(write, PROBE)
    if not pf or not pw:
        raise SystemExit("copy probe kernel not found in the counter output")
    # median of the probe dispatches (the first can include cold misses)
    pf_kib = sorted(pf)[len(pf) // 2]
    pw_kib = sorted(pw)[len(pw) // 2]
    f_fetch = probe_bytes / (pf_kib * 1024.0)
    f_write = probe_bytes / (pw_kib * 1024.0)
    result = {"probe": {"bytes": probe_bytes, "fetch_kib": pf_kib, "write_kib": pw_kib,
                        "fetch_factor": f_fetch, "write_factor": f_write},
              "source_hash": source_hash(), "kernels": {}}
    for kid, pat in KERNELS.items():
        fv, wv = _match(fetch, pat), _match(write, pat)
        if not fv or not wv:
            continue
        fk = sum(fv[-last:]) / len(fv[-last:])
        wk = sum(wv[-last:]) / len(wv[-last:])
        result["kernels"][kid] = {
            "fetch_kib": fk, "write_kib": wk,
            "fetch_bytes": fk * 1024.0 * f_fetch, "write_bytes": wk * 1024.0 * f_write,
            "bytes_per_launch": fk * 1024.0 * f_fetch + wk * 1024.0 * f_write,
            "dispatches_averaged": len(fv[-last:]),
        }
    return result


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--last", type=int, default=400)
    c = sub.add_parser("traffic")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-mib", type=int, required=True)
    c.add_argument("--last", type=int, default=400)
    c.add_argument("--out")
    args = ap.parse_args(argv)
    if args.cmd == "trace":
        print(trace_table(args.dir, args.last))
        return
    res = traffic(args.fetch, args.write, args.copy_mib, args.last)
    text = json.dumps(res, indent=1)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")
    print(text)


if __name__ == "__main__":
    sys.exit(main())
