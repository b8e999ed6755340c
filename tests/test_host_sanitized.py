"""The C-ABI host code of libkvz (argument validation, split and workspace sizing, launch set-up)
built with AddressSanitizer and UndefinedBehaviorSanitizer on the host pass (every report fatal),
and the library's CPU tests run against that build in a child process that preloads the
sanitizer runtime; extreme shapes go through the host size functions as well. No device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

EXTREMES = r'''
import ctypes, sys
sys.path.insert(0, sys.argv[1])
from decode_attention_losslessly_amd import kvz
L = kvz.lib()
assert kvz.LIB_PATH == sys.argv[2], kvz.LIB_PATH
big = (1 << 31) - 1
assert L.kvz_workspace_bytes(big, big, big, 64, 16, big, -4096) == 0     # does not fit in size_t
assert L.kvz_workspace_bytes(-1, 32, 32, 128, 16, 1, 0) == 0 and L.kvz_num_splits(-1, 32, 32, 128, 16, 1, 0) == 0
assert L.kvz_unit_bytes(1 << 16, 1 << 14) == 0 and L.kvz_unit_bytes(1024, 64) > 0   # P * D at most 65536
for B, Hq, Hkv, D, P, mp, pps in [(big, 64, 64, 128, 16, big, 0), (1, big, 1, 128, 16, 1, 0),
                                  (big, big, big, 64, 16, big, -4096), (65536, 64, 8, 128, 16, 1 << 20, 0),
                                  (1, 32, 32, 128, 1 << 30, 1, 0), (-1, 32, 32, 128, 16, 1, 0),
                                  (32, 32, 32, 128, 16, -5, 0), (32, 32, 32, 128, 16, 513, -(1 << 31))]:
    L.kvz_workspace_bytes(B, Hq, Hkv, D, P, mp, pps)
    L.kvz_num_splits(B, Hq, Hkv, D, P, mp, pps)
for P, D in [(big, 64), (16, big), (0, 0), (-16, 128), (1 << 16, 1 << 14)]:
    L.kvz_unit_bytes(P, D); L.kvz_meta_bytes(P, D); L.kvz_payload_bytes(P, D); L.kvz_inline_capacity(P, D)
    L.kvz_unit_bytes_for(1, P, D)
print("extremes ok")
'''


def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from decode_attention_losslessly_amd import build
    lib = build.build_sanitized(str(tmp_path / "libkvz_hostsan.so"))
    env = dict(os.environ, KVZ_LIB=lib, LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", EXTREMES, ROOT, lib], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "extremes ok" in r.stdout, (r.stdout + r.stderr)[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0 and "passed" in r.stdout, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
