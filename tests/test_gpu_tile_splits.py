"""Splits that start and end inside units. With pages of several 16-token tiles and too few of
them to fill the GPU page by page, the multi-head kernel over the compressed cache counts its
splits in tiles: a split that starts inside a unit takes its first tile's escape cursors from the
escapes of the unit's earlier tiles, and the merge counts the same splits. Parity against the
fp64 oracle for inline units (few escapes) and pool units (escape-heavy magnitudes: every split
then runs the pool-capable loop from a cut unit), both group geometries, head dims 64 and 128,
grouped queries at head dim 64 (one wave per query head), and lengths that end inside pages;
the split kernel records that it counted tiles, and a fixed split size (whole pages) gives the
same attention within fp32 rounding of the summation order."""
import numpy as np
import pytest
import torch

import decode_attention_losslessly_amd as kvz
from synth import make_workload

from kvz_testlib import DEV, build_cache, check_rows, dev, host16, oracle_rows

pytestmark = pytest.mark.gpu

CASES = [
    # (config, overrides)
    (1, dict()),                                                       # 1 page of 256 tokens, 2 heads
    (1, dict(B=2, lens=[700, 300], Hq=3, Hkv=3)),                      # cut pages and 188/44-row tails
    (3, dict(B=2, lens=[1000, 333], Hq=4, Hkv=4, P=64)),               # outlier channels, P = 64
    (4, dict(B=2, lens=[900, 1500], Hq=2, Hkv=2, P=128)),              # Student-t keys: some pool units
    (5, dict(B=1, L=1100, Hq=2, Hkv=2, P=256)),                        # escape-heavy: pool loop from a cut unit
    (5, dict(B=2, lens=[500, 129], Hq=4, Hkv=4, P=64, D=64)),
    (1, dict(B=1, L=1030, Hq=8, Hkv=2, P=256)),                        # grouped queries at head dim 64
    (3, dict(B=1, L=2000, Hq=2, Hkv=2, P=512, D=64)),                  # 32 tiles a page
]


def _attend(w, cache, lens, q, pps=0):
    ws = torch.empty(kvz.workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages, pps), dtype=torch.uint8,
                     device=DEV)
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, dev(w.page_table), lens, w.sm_scale, out, out32, workspace=ws,
                         pages_per_split=pps)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    return host16(out), out32.cpu().numpy(), kvz.chosen_split(ws, w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages, pps)


@pytest.mark.parametrize("fmt", [kvz.FORMAT_ESCAPE, kvz.FORMAT_CHANNEL])
@pytest.mark.parametrize("cfg,kw", CASES)
def test_splits_inside_units_match_oracle(cfg, kw, fmt):
    w = make_workload(cfg, n_append=0, **kw)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp, fmt=fmt)
    q = w.q()
    o16, o32, (c, tpp) = _attend(w, cache, lens, q)
    assert tpp == w.P // 16 and c > 0, (c, tpp)
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    what = f"cfg{cfg} {kw} fmt{fmt} tiles of {c}"
    check_rows(o16.reshape(-1, w.D), o32.reshape(-1, w.D), ref, what)
    # whole pages per split (a fixed split size): the same attention up to the summation order
    p16, p32, (cp, tp) = _attend(w, cache, lens, q, pps=1)
    assert (cp, tp) == (1, 1)
    check_rows(p16.reshape(-1, w.D), p32.reshape(-1, w.D), ref, what + " (whole pages)")
    nrm = np.abs(p32).max(axis=-1, keepdims=True)
    assert np.all(np.abs(o32 - p32) <= 1e-5 * np.maximum(nrm, 1e-30)), what
