"""Builds tests/c/abi_decode, the decode loop that drives libkvz through its C ABI alone (gcc,
against the HIP runtime's C API). It links the built libkvz.so and, for its reference values,
the C oracle (test infrastructure), so it is built after both."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_decode.c")
OUT = os.path.join(HERE, "abi_decode")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    pkg, orc = os.path.join(ROOT, "decode_attention_losslessly_amd"), os.path.join(ROOT, "oracle")
    # gcc is not hipcc, so the HIP runtime header needs to be told which runtime it declares
    # (the AMD one; this is the only platform the library is built for)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), SRC, "-L", pkg, "-lkvz", "-L", orc, "-lkvz_oracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../decode_attention_losslessly_amd:$ORIGIN/../../oracle:" + os.path.join(ROCM, "lib"),
           "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
