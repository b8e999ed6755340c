"""The C ABI driven from C alone: tests/c/abi_decode (built by __graft_entry__.build()) allocates
with hipMalloc, compresses pages, runs decode steps that append and attend across page fills, the
uncompressed baseline, the allocation-free call and every decode route, for a multi-head and a
grouped-query shape, and checks them against the fp64 oracle and the source bits."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "abi_decode")

pytestmark = pytest.mark.gpu


def test_decode_loop_through_the_c_abi():
    assert os.path.exists(EXE), "tests/c/abi_decode is built by __graft_entry__.build()"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(": ok") == 2, r.stdout
