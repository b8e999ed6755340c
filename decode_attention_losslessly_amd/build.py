"""Builds the HIP libraries for gfx950, in-tree next to this file.

hipcc compiles each source of csrc/ (device code for gfx950 only) and links them into
libkvz.so, the shared library exporting the C ABI of include/kvz.h, and libkvz_bench.so, the
measurement kernels of include/kvz_bench.h.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
OUT = os.path.join(HERE, "libkvz.so")
SOURCES = ["kvz_api.hip", "compress.hip", "decompress.hip", "attn_mha.hip", "attn_gqa.hip", "attn_dense.hip",
           "merge.hip", "attn_zf.hip", "pool.hip"]
BENCH_OUT = os.path.join(HERE, "libkvz_bench.so")
BENCH_SOURCES = ["read_ceiling.hip"]
ARCH = os.environ.get("KVZ_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
         "-I", CSRC, "-I", os.path.join(ROOT, "include")]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise and verbose:
        print("\n".join(noise), flush=True)
    return obj


def _link(objs, out: str, verbose: bool) -> None:
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], OUT, verbose)
    _link([objs[s] for s in BENCH_SOURCES], BENCH_OUT, verbose)
    return OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
