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


# Host code only (the C-ABI validation and launch code) under AddressSanitizer and
# UndefinedBehaviorSanitizer, every report fatal: each flag applies to the host pass alone.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, verbose: bool, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, src + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
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


def _link(objs, out: str, verbose: bool, extra=()) -> None:
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", out + ".tmp"]
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


def build_sanitized(out: str, verbose: bool = False) -> str:
    """libkvz with its host code under ASan and UBSan, at `out` (for the CPU test of the C-ABI host
    code; a process that loads it must preload sanitizer_runtime())."""
    build_dir = os.path.join(os.path.dirname(out), "_build_sanitized")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, SANITIZE), SOURCES))
    _link(objs, out, verbose, ["-shared-libasan", "-fsanitize=address,undefined"])
    return out


def sanitizer_runtime() -> str:
    """hipcc's (clang's) AddressSanitizer runtime, to preload into a process that loads a
    sanitized libkvz."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True,
                       check=True)
    return r.stdout.strip()


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
