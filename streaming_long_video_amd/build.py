"""Build libstatekv.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python streaming_long_video_amd/build.py [--verbose]

(run as a file: importing the package loads the library, which this builds)

Each source is compiled to an object in ``_build/`` next to this file, then
linked into ``streaming_long_video_amd/libstatekv.so``.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libstatekv.so")

SOURCES = [
    os.path.join(CSRC, "plan.cpp"),
    os.path.join(CSRC, "statekv_api.hip"),
    os.path.join(CSRC, "frontend_api.hip"),
    os.path.join(CSRC, "kernels", "attention.hip"),
    os.path.join(CSRC, "kernels", "select.hip"),
    os.path.join(CSRC, "kernels", "gather.hip"),
    os.path.join(CSRC, "kernels", "decode.hip"),
    os.path.join(CSRC, "kernels", "rope.hip"),
    os.path.join(CSRC, "kernels", "diagnostics.hip"),
    os.path.join(CSRC, "kernels", "frontend.hip"),
]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


# per-source flags: the attention kernels take finite inputs, so the row
# maxima need no NaN-quieting of their operands
EXTRA = {
    os.path.join(CSRC, "kernels", "attention.hip"): ["-fno-honor-nans"],
}


def _obj(src: str) -> str:
    rel = os.path.relpath(src, CSRC).replace(os.sep, "_")
    return os.path.join(BUILD, rel + ".o")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        line for line in (r.stdout + r.stderr).splitlines()
        if "packed-fp32-ops" not in line)  # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link libstatekv.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cmds = []
    for src in SOURCES:
        lang = [] if src.endswith(".cpp") else ["-x", "hip"]
        cmds.append([HIPCC, *COMMON, *EXTRA.get(src, []), *lang, "-c", src, "-o", _obj(src)])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
          *[_obj(s) for s in SOURCES]], verbose)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(verbose=args.verbose)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
