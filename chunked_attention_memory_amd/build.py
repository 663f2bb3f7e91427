"""Build libgecko.so (the C-ABI HIP library) in-tree for gfx950.

Usage: python -m chunked_attention_memory_amd.build [--jobs N] [--verbose]

Each source under csrc/ is compiled to an object with hipcc, in parallel, then
linked into chunked_attention_memory_amd/_lib/libgecko.so. Always rebuilds.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libgecko.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep the compiler from emitting packed fp32 (v_pk_*_f32) instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l)
    if out.strip() and (verbose or r.returncode):
        print(out, flush=True)
    if r.returncode:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}")


def build(jobs: int | None = None, verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]
    flags = common_flags()

    def compile_one(pair):
        src, obj = pair
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([cc, *flags, *lang, "-c", src, "-o", obj], verbose)

    with ThreadPoolExecutor(max_workers=jobs or min(8, os.cpu_count() or 4)) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = os.path.join(OUT_DIR, LIB_NAME + ".tmp")
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    final = os.path.join(OUT_DIR, LIB_NAME)
    os.replace(tmp, final)
    return final


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(args.jobs, args.verbose)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
