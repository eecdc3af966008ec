"""Build libkvq.so (HIP, gfx950) in-tree with hipcc.

    python -m sub_byte_quantized_amd.build [--jobs N]

Each source is compiled to an object in parallel, then linked into
sub_byte_quantized_amd/libkvq.so.  The benchmark's read-ceiling kernel is
linked on its own into libkvq_bench.so.  Always rebuilds.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvq.so")
SOURCES = ["kvq_host.cpp", "kvq_write.hip", "kvq_decode.hip", "kvq_prefill.hip", "kvq_gather.hip"]
BENCH_LIB = os.path.join(PKG, "libkvq_bench.so")
BENCH_SOURCES = ["bench_stream_read.hip"]
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def common_flags():
    return ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
            "-fhip-fp32-correctly-rounded-divide-sqrt",
            # packed fp32 VALU ops are kept out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def compile_one(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *lang, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int = 4, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES + BENCH_SOURCES))
    link(objs[:len(SOURCES)], LIB)
    link(objs[len(SOURCES):], BENCH_LIB)
    if verbose:
        print(f"built {LIB} and {BENCH_LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    a = ap.parse_args(argv)
    build(a.jobs)


if __name__ == "__main__":
    sys.exit(main())
