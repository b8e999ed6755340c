"""Attention parity on shapes the five workloads do not reach: pages of several 16-token tiles
(including a count that is not a power of two), query groups of 2 and 16 heads (16 = two MFMA
row chunks), head_dim 64, and ragged lengths around page boundaries. Compressed and dense paths
against the fp64 oracle within the stated tolerance. Blocks of the format's largest size (65,536
values: 512-token pages at head dim 128, 1,024-token pages at 64) are also compressed byte-exact,
appended into and rebuilt bit for bit."""
import numpy as np
import pytest
import torch

import decode_attention_losslessly_amd as kvz
from kvz_testlib import (DEV, build_cache, check_rows, decode_units, dev, full_page_ids, host16, lane_maps,
                         oracle_rows, unit_equal)
from oracle import c_oracle
from synth import make_workload

pytestmark = pytest.mark.gpu

SHAPES = [  # (P, D, Hq, Hkv)
    (32, 128, 8, 2),
    (48, 128, 6, 3),
    (64, 128, 32, 2),
    (256, 128, 4, 1),
    (32, 128, 4, 4),
    (16, 64, 4, 4),
    (64, 64, 8, 8),
    (16, 64, 8, 2),     # grouped queries at head dim 64: one wave per query head
    (48, 64, 6, 1),
]


@pytest.mark.parametrize("P,D,Hq,Hkv", SHAPES)
def test_shapes_match_oracle(P, D, Hq, Hkv):
    lens = [1, P - 1, P, P + 1, 5 * P + 3, 2 * P]
    for cfg in (1, 5):   # smooth per-channel scales, and the escape-stress distribution (pool path)
        w = make_workload(cfg, B=len(lens), lens=lens, Hq=Hq, Hkv=Hkv, D=D, P=P, n_append=0)
        kp, vp = w.pages(0), w.pages(1)
        cache, seq = build_cache(w, kp, vp)
        q = w.q()
        rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
        ref = oracle_rows(w, kp, vp, q, rows)
        for pps in (0, 1, 3, -2):   # -2: the multi-head kernel's ranked schedule
            out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
            out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
            kvz.decode_attention(dev(q), cache, dev(w.page_table), seq, w.sm_scale, out, out32, pages_per_split=pps)
            torch.cuda.synchronize()
            assert int(cache.status.item()) == 0
            check_rows(host16(out).reshape(-1, D), out32.cpu().numpy().reshape(-1, D), ref,
                       f"cfg{cfg} P{P} D{D} {Hq}/{Hkv} pps{pps} compressed")
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        kvz.decode_attention_dense(dev(q), dev(kp), dev(vp), dev(w.page_table), dev(w.seq_lens), w.sm_scale, out,
                                   out32, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        check_rows(host16(out).reshape(-1, D), out32.cpu().numpy().reshape(-1, D), ref,
                   f"cfg{cfg} P{P} D{D} {Hq}/{Hkv} dense")


@pytest.mark.parametrize("P,D,Hq,Hkv", [(512, 128, 2, 2), (512, 128, 8, 2), (1024, 64, 2, 2)])
@pytest.mark.parametrize("cfg", [1, 5])
def test_largest_blocks(P, D, Hq, Hkv, cfg):
    """P * D = 65536, where a storage position takes all 16 bits of an inline escape entry and
    compression stages 128 KB of V per wave. The last token is appended through kvz_append_token,
    which fills request 1's second page and compresses it. Units byte-exact against the oracle
    (escape-stress data puts them in the pool), every decode route bit-exact, attention within
    tolerance under every split choice."""
    lens = [P - 1, 2 * P, 2 * P + 5]
    w = make_workload(cfg, B=len(lens), lens=lens, Hq=Hq, Hkv=Hkv, D=D, P=P, n_append=1)
    kp, vp = w.pages(0), w.pages(1)
    ids = full_page_ids(w)
    assert len(ids) == 4
    cache, seq = build_cache(w, kp, vp, esc_capacity=len(ids) * Hkv * 2 * P * D)   # room for every value
    assert int(cache.status.item()) == 0
    units = cache.units.cpu().numpy()
    pool = host16(cache.esc_pool)
    ref_units, ref_pool, _ = c_oracle.encode_pages(kp[ids], vp[ids])
    for i, pid in enumerate(ids):
        for h in range(Hkv):
            assert unit_equal(units[pid, h], pool, ref_units[i, h], ref_pool, P, D), (int(pid), h)
    for lane_map in lane_maps(D):
        kd, vd = decode_units(cache, ids, Hkv, P, D, lane_map)
        assert np.array_equal(kd, kp[ids]) and np.array_equal(vd, vp[ids]), lane_map
    q = w.q()
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    for pps in (0, 1, -2):
        out = torch.zeros((w.B, w.Hq, D), dtype=torch.int16, device=DEV)
        out32 = torch.full((w.B, w.Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        kvz.decode_attention(dev(q), cache, dev(w.page_table), seq, w.sm_scale, out, out32, pages_per_split=pps)
        torch.cuda.synchronize()
        assert int(cache.status.item()) == 0
        check_rows(host16(out).reshape(-1, D), out32.cpu().numpy().reshape(-1, D), ref,
                   f"cfg{cfg} P{P} D{D} {Hq}/{Hkv} pps{pps}")


@pytest.mark.parametrize("kw", [
    dict(B=12, lens=[26, 32, 5, 53, 0, 1, 24, 13, 50, 53, 42, 55], Hq=16, Hkv=8, P=32),
    dict(B=3, lens=[37, 0, 48], Hq=40, Hkv=5, P=16),
])
def test_wide_dynamic_range_batch(kw):
    """Escape-stress batches with rows of test_tolerance.py: the first has the row whose small
    elements need the fp32 budget in the BF16 bound (16 query heads over 8 KV heads, 32-token
    pages, requests with a tail only, with one full page, and empty); the second a near-tie row,
    (0, 29), that only its first-order score-rounding bound admits (40 query heads over 5). Every
    row within the bounds, compressed under the device's split choice, one page per split and
    two, and dense."""
    kw = dict(kw)
    w = make_workload(5, n_append=0, lens=np.array(kw.pop("lens")), D=128, **kw)
    kp, vp = w.pages(0), w.pages(1)
    cache, seq = build_cache(w, kp, vp)
    q = w.q()
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.zeros((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
    for pps in (0, 1, 2):
        kvz.decode_attention(dev(q), cache, dev(w.page_table), seq, w.sm_scale, out, out32, pages_per_split=pps)
        torch.cuda.synchronize()
        assert int(cache.status.item()) == 0
        check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, f"compressed pps{pps}")
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvz.decode_attention_dense(dev(q), dev(kp), dev(vp), dev(w.page_table), dev(w.seq_lens), w.sm_scale, out, out32,
                               status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, "dense")


@pytest.mark.parametrize("Hq,Hkv,P,D", [(24, 1, 32, 128), (32, 1, 16, 128), (64, 2, 16, 128), (32, 4, 32, 64),
                                        (16, 1, 16, 64)])
def test_large_query_groups(Hq, Hkv, P, D):
    """Query groups beyond 16 heads at head dim 128 (3, 4 and 8 chunks of 8 query heads per KV
    head; the last two multi-query shapes) and grouped queries at head dim 64 (a wave per query
    head): both cache formats and the uncompressed baseline against the oracle, smooth and
    escape-stress data, under the device's split choice and one page per split."""
    lens = [1, P - 1, 3 * P + 5, 7 * P]
    for cfg in (1, 5):
        w = make_workload(cfg, B=len(lens), lens=lens, Hq=Hq, Hkv=Hkv, D=D, P=P, n_append=0)
        kp, vp = w.pages(0), w.pages(1)
        q = w.q()
        rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
        ref = oracle_rows(w, kp, vp, q, rows)
        out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
        out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
        for fmt in (kvz.FORMAT_ESCAPE, kvz.FORMAT_ZIPFUSION):
            cache, seq = build_cache(w, kp, vp, fmt=fmt)
            for pps in (0, 1):
                kvz.decode_attention(dev(q), cache, dev(w.page_table), seq, w.sm_scale, out, out32,
                                     pages_per_split=pps)
                torch.cuda.synchronize()
                assert int(cache.status.item()) == 0
                check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref,
                           f"cfg{cfg} {Hq}/{Hkv} P{P} format {fmt} pps{pps}")
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        kvz.decode_attention_dense(dev(q), dev(kp), dev(vp), dev(w.page_table), dev(w.seq_lens), w.sm_scale, out,
                                   out32, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, f"cfg{cfg} {Hq}/{Hkv} dense")
