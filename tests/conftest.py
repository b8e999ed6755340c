import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload")


def pytest_terminal_summary(terminalreporter):
    kvz_testlib = sys.modules.get("kvz_testlib")
    if kvz_testlib is not None and kvz_testlib.CONDITIONED:
        terminalreporter.write_line(f"attention rows that passed only under their first-order score-rounding bound: "
                                    f"{len(kvz_testlib.CONDITIONED)}")


_FULL = {}


@pytest.fixture(scope="session")
def full_workloads():
    """Full-size workload `cfg`, built once: (workload, K pages, V pages, device cache, seq_lens).
    Only the most recent one is kept, so host and device memory hold one full cache at a time."""
    def get(cfg):
        if cfg not in _FULL:
            import gc

            import torch

            from kvz_testlib import build_cache
            from synth import make_workload
            _FULL.clear()
            gc.collect()
            torch.cuda.empty_cache()
            w = make_workload(cfg)
            print(f"\n[full workload {cfg}: {w.name}, generating {w.num_pages} pages]", flush=True)
            kp, vp = w.pages(0), w.pages(1)
            cache, lens = build_cache(w, kp, vp)
            _FULL[cfg] = (w, kp, vp, cache, lens)
        return _FULL[cfg]
    yield get
    _FULL.clear()
