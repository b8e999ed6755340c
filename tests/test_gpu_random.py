"""Seeded random shapes through the compressed and the uncompressed attention paths, against the
fp64 oracle within the stated tolerance: page sizes of one to four tiles, head dims 64 and 128,
query groups from 1 to 16 heads, uneven lengths with empty requests and partial pages, the
value distributions of all five workloads (the escape-stress one included, for the pool paths)
and every kind of split choice (chosen on the device, fixed, and the ranked schedule forced).
Each case also rebuilds its units bit for bit through every decode route of the kernels, and runs
again over the same pages in ZipFusion's block format (multi-head or grouped-query kernel) and
with channel groups (same schedule, every decode route).
Each case is drawn from its own seed, so a failure names a reproducible case. A second set draws
larger batches, longer requests and pages of up to 512 tokens."""
import numpy as np
import pytest
import torch

import decode_attention_losslessly_amd as kvz
from kvz_testlib import DEV, build_cache, check_rows, dev, full_page_ids, host16, oracle_rows
from synth import make_workload

pytestmark = pytest.mark.gpu

N_CASES = 24


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    P = int(rng.choice([16, 32, 48, 64]))
    D = int(rng.choice([64, 128]))
    grp = 1 if D == 64 else int(rng.choice([1, 2, 4, 7, 8, 16]))
    Hkv = int(rng.integers(1, 5))
    B = int(rng.integers(1, 7))
    lens = rng.integers(0, 6 * P + 1, size=B)
    if B > 2:
        lens[rng.integers(0, B)] = 0
    cfg = int(rng.integers(1, 6))
    pps = int(rng.choice([0, 1, 2, -1, -3]))
    return dict(cfg=cfg, B=B, lens=lens, Hq=Hkv * grp, Hkv=Hkv, D=D, P=P), pps


def _large_case(seed):
    """larger batches (up to 39 requests), longer requests (up to 40 pages), pages of up to 256
    tokens (512 at head dim 64), two requests ending on a page boundary, query groups of up to 32
    heads (and grouped queries at head dim 64)"""
    rng = np.random.default_rng(90000 + seed)
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 16, 32, 64, 128, 256] + ([512] if D == 64 else [])))
    grp = int(rng.choice([1, 2, 4])) if D == 64 else int(rng.choice([1, 2, 4, 7, 8, 16, 24, 32]))
    Hkv = int(rng.integers(1, 5))
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, int(rng.choice([3, 10, 40])) * P + 1, size=B)
    for _ in range(2):
        k = rng.integers(0, B)
        lens[k] = (lens[k] // P) * P
    cfg = int(rng.integers(1, 7))
    pps = int(rng.choice([0, 0, 0, 1, 4, 9, -1, -4]))
    return dict(cfg=cfg, B=B, lens=lens, Hq=Hkv * grp, Hkv=Hkv, D=D, P=P), pps


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shapes_match_oracle(seed):
    _check_case(seed, *_case(seed))


@pytest.mark.parametrize("seed", range(16))
def test_random_large_shapes_match_oracle(seed):
    _check_case(seed, *_large_case(seed))


def _check_case(seed, kw, pps):
    cfg = kw.pop("cfg")
    what = f"seed {seed}: cfg{cfg} B={kw['B']} {kw['Hq']}/{kw['Hkv']} D={kw['D']} P={kw['P']} pps={pps}"
    print(what, flush=True)
    w = make_workload(cfg, n_append=0, **kw)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp)
    q = w.q()
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, dev(w.page_table), lens, w.sm_scale, out, out32, pages_per_split=pps)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0, what
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, what + " compressed")
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvz.decode_attention_dense(dev(q), dev(kp), dev(vp), dev(w.page_table), dev(w.seq_lens), w.sm_scale, out, out32,
                               status=status, pages_per_split=pps)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, what
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, what + " dense")
    # the kernels' own decode of every full page, on every route of this head dim
    ids = full_page_ids(w)
    if len(ids):
        for lane_map in ([0, 1, 2, 3] if w.D == 128 else [0, 2]):
            kd = torch.zeros((len(ids), w.Hkv, w.P, w.D), dtype=torch.int16, device=DEV)
            vd = torch.zeros_like(kd)
            kvz.decompress_pages(cache, dev(ids), kd, vd, lane_map=lane_map)
            torch.cuda.synchronize()
            assert np.array_equal(host16(kd), kp[ids]) and np.array_equal(host16(vd), vp[ids]), f"{what} lane map {lane_map}"
    # the same pages in ZipFusion's block format
    zc, zl = build_cache(w, kp, vp, fmt=kvz.FORMAT_ZIPFUSION)
    assert int(zc.status.item()) == 0, what
    kvz.decode_attention(dev(q), zc, dev(w.page_table), zl, w.sm_scale, out, out32,
                         pages_per_split=max(pps, 0))
    torch.cuda.synchronize()
    assert int(zc.status.item()) == 0, what
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, what + " zipfusion")
    if len(ids):
        for lane_map in ([0, 1] if w.D == 128 else [0]):
            kd = torch.zeros((len(ids), w.Hkv, w.P, w.D), dtype=torch.int16, device=DEV)
            vd = torch.zeros_like(kd)
            kvz.decompress_pages(zc, dev(ids), kd, vd, lane_map=lane_map)
            torch.cuda.synchronize()
            assert np.array_equal(host16(kd), kp[ids]) and np.array_equal(host16(vd), vp[ids]), \
                f"{what} zipfusion lane map {lane_map}"
    # the same pages with channel groups, the same schedule
    cc, cl = build_cache(w, kp, vp, fmt=kvz.FORMAT_CHANNEL)
    assert int(cc.status.item()) == 0, what
    kvz.decode_attention(dev(q), cc, dev(w.page_table), cl, w.sm_scale, out, out32, pages_per_split=pps)
    torch.cuda.synchronize()
    assert int(cc.status.item()) == 0, what
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, what + " channel")
    if len(ids):
        for lane_map in ([0, 1, 2, 3] if w.D == 128 else [0, 2]):
            kd = torch.zeros((len(ids), w.Hkv, w.P, w.D), dtype=torch.int16, device=DEV)
            vd = torch.zeros_like(kd)
            kvz.decompress_pages(cc, dev(ids), kd, vd, lane_map=lane_map)
            torch.cuda.synchronize()
            assert np.array_equal(host16(kd), kp[ids]) and np.array_equal(host16(vd), vp[ids]), \
                f"{what} channel lane map {lane_map}"
