"""The C oracle's pins run again with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (every report fatal), in a child process that preloads the sanitizer
runtime: an out-of-bounds access, a use after free or undefined behaviour anywhere in the oracle
code those tests reach fails this test. CPU only."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build(out=str(tmp_path / "libkvz_oracle_asan.so"), sanitize=True)
    env = dict(os.environ, KVZ_ORACLE_LIB=lib, LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_codec.py", "tests/test_oracle_attention.py", "tests/test_oracle_zipfusion.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
