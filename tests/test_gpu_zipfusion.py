"""GPU parity of the second cache format, ZipFusion's block format (include/kvz.h,
KVZ_FORMAT_ZIPFUSION; oracle/zipfusion.py): compression byte-exact against the oracle (raw
blocks compared at the pool offset the library chose), the attention kernels' in-register
rebuild bit-exact in both K lane layouts (multi-head and grouped-query), attention of the
multi-head and grouped-query kernels against the fp64 oracle within the stated tolerance
(reduced workloads, and sampled rows of the full grouped-query workloads), and append with
compress-on-fill. Workloads cover mostly compressed blocks (smooth values) and all-raw blocks
(the escape-stress distribution)."""
import numpy as np
import pytest
import torch

import decode_attention_losslessly_amd as kvz
from kvz_testlib import DEV, build_cache, check_rows, dev, full_page_ids, host16, oracle_rows
from oracle import zipfusion as zf
from synth import make_workload

pytestmark = pytest.mark.gpu
ZF = kvz.FORMAT_ZIPFUSION

SMALL = {
    1: dict(),
    2: dict(L=100),
    3: dict(B=3, L=97),
    4: dict(B=5, lens=[1, 16, 33, 150, 47]),     # grouped queries, 28 over 4 KV heads
    5: dict(B=2, L=70),
    6: dict(B=2, L=70, Hq=8, Hkv=8),
    7: dict(cfg=6, B=3, lens=[70, 161, 16]),        # grouped queries, 32 over 8 KV heads
    8: dict(cfg=5, B=2, L=70, Hq=8, Hkv=2),         # grouped queries, every block raw
}


def _workload(key):
    a = dict(SMALL[key])
    return make_workload(a.pop("cfg", key), **a)


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_compress_matches_oracle(cfg):
    w = _workload(cfg)
    kp, vp = w.pages(0), w.pages(1)
    cache, _ = build_cache(w, kp, vp, fmt=ZF)
    assert int(cache.status.item()) == 0
    units = cache.units.cpu().numpy()
    pool = host16(cache.esc_pool)
    ids = full_page_ids(w, w.seq_lens - w.n_append)
    n_raw = 0
    for pid in ids:
        for h in range(w.Hkv):
            got = units[pid, h].tobytes()
            off = zf.unit_raw_offset(got, w.P, w.D)
            want, raw = zf.encode_unit(kp[pid, h], vp[pid, h], pool_offset=off)
            assert got == want, f"unit ({pid}, {h}) differs"
            if raw.size:
                assert np.array_equal(pool[off:off + raw.size], raw)
                n_raw += raw.size // zf.BLOCK
    assert int(cache.esc_cursor.item()) == n_raw * zf.BLOCK


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_in_kernel_rebuild_is_bit_exact(cfg):
    w = _workload(cfg)
    kp, vp = w.pages(0), w.pages(1)
    cache, _ = build_cache(w, kp, vp, fmt=ZF)
    ids = full_page_ids(w, w.seq_lens - w.n_append)
    for lane_map in ([0, 1] if w.D == 128 else [0]):
        kd = torch.empty((len(ids), w.Hkv, w.P, w.D), dtype=torch.int16, device=DEV)
        vd = torch.empty_like(kd)
        kvz.decompress_pages(cache, dev(ids), kd, vd, lane_map=lane_map)
        torch.cuda.synchronize()
        assert np.array_equal(host16(kd), kp[ids]) and np.array_equal(host16(vd), vp[ids]), lane_map


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_attention_matches_oracle(cfg):
    w = _workload(cfg)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp, fmt=ZF)
    q = w.q()
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    for pps in (0, 1):
        out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
        out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
        kvz.decode_attention(dev(q), cache, dev(w.page_table), lens, w.sm_scale, out, out32, pages_per_split=pps)
        torch.cuda.synchronize()
        assert int(cache.status.item()) == 0
        check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, f"zf cfg{cfg} pps{pps}")


@pytest.mark.parametrize("P,D,Hq", [(16, 128, 4), (48, 128, 4), (64, 64, 4), (16, 128, 16), (48, 128, 8)])
def test_mixed_units_and_page_fills(P, D, Hq):
    # half the requests smooth (compressed blocks), half escape-stress (raw blocks); appends cross
    # page fills; 4 KV heads under 4 query heads (multi-head kernel) or 8 and 16 (grouped-query)
    n_steps = P + 3
    lens = np.array([3 * P - 2, P + 5, 2 * P, 4 * P + 7])
    smooth = make_workload(1, B=4, lens=lens + n_steps, Hq=Hq, Hkv=4, D=D, P=P, n_append=0)
    stress = make_workload(5, B=4, lens=lens + n_steps, Hq=Hq, Hkv=4, D=D, P=P, n_append=0)
    kp, vp = smooth.pages(0), smooth.pages(1)
    ks, vs = stress.pages(0), stress.pages(1)
    odd = np.zeros(smooth.num_pages, bool)
    for r in (1, 3):
        odd[smooth.page_table[r][smooth.page_table[r] >= 0]] = True
    kp[odd], vp[odd] = ks[odd], vs[odd]
    w = smooth
    L0 = (w.seq_lens - n_steps).astype(np.int32)
    ids = full_page_ids(w, L0)
    cache = kvz.Cache.allocate(P, w.Hkv, D, w.num_pages, w.B, w.num_pages * w.Hkv * 2 * P * D, device=DEV, fmt=ZF)
    kvz.compress_pages(cache, dev(kp[ids]), dev(vp[ids]), dev(ids))
    tk = np.zeros((w.B, w.Hkv, P, D), np.uint16)
    tv = np.zeros_like(tk)
    for r in range(w.B):
        if L0[r] % P:
            tk[r], tv[r] = kp[w.page_table[r, L0[r] // P]], vp[w.page_table[r, L0[r] // P]]
    cache.k_tail.copy_(dev(tk))
    cache.v_tail.copy_(dev(tv))
    lens_d, table = dev(L0), dev(w.page_table)
    tok = lambda pages, r, t: pages[w.page_table[r, t // P]][:, t % P, :]
    for i in range(n_steps):
        kn = np.stack([tok(kp, r, int(L0[r]) + i) for r in range(w.B)])
        vn = np.stack([tok(vp, r, int(L0[r]) + i) for r in range(w.B)])
        kvz.append_token(cache, dev(kn), dev(vn), table, lens_d)
    torch.cuda.synchronize()
    assert np.array_equal(lens_d.cpu().numpy(), w.seq_lens) and int(cache.status.item()) == 0
    full = full_page_ids(w)
    kd = torch.empty((len(full), w.Hkv, P, D), dtype=torch.int16, device=DEV)
    vd = torch.empty_like(kd)
    kvz.decompress_pages(cache, dev(full), kd, vd, lane_map=1 if Hq > w.Hkv else 0)
    torch.cuda.synchronize()
    assert np.array_equal(host16(kd), kp[full]) and np.array_equal(host16(vd), vp[full])
    q = w.q()
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    out = torch.zeros((w.B, w.Hq, D), dtype=torch.int16, device=DEV)
    out32 = torch.zeros((w.B, w.Hq, D), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, table, lens_d, w.sm_scale, out, out32)
    torch.cuda.synchronize()
    check_rows(host16(out).reshape(-1, D), out32.cpu().numpy().reshape(-1, D), ref, f"zf mixed P{P} D{D}")


@pytest.mark.parametrize("cfg", [4, 6])
def test_grouped_queries_full_size_sampled(cfg):
    """The grouped-query workloads at full size in this format (the pages' benchmark shape,
    32 query over 8 KV heads at 64 x 8192, and 28 over 4 at 64 requests of 1K-8K tokens):
    sampled units rebuilt bit for bit in the grouped-query K layout, sampled rows against the
    fp64 oracle."""
    w = make_workload(cfg)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp, fmt=ZF)
    assert int(cache.status.item()) == 0
    rng = np.random.default_rng(cfg)
    ids = full_page_ids(w)
    sample = ids[rng.choice(len(ids), size=64, replace=False)]
    kd = torch.empty((len(sample), w.Hkv, w.P, w.D), dtype=torch.int16, device=DEV)
    vd = torch.empty_like(kd)
    kvz.decompress_pages(cache, dev(sample), kd, vd, lane_map=1)
    torch.cuda.synchronize()
    assert np.array_equal(host16(kd), kp[sample]) and np.array_equal(host16(vd), vp[sample])
    q = w.q()
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, dev(w.page_table), lens, w.sm_scale, out, out32)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0 and np.isfinite(out32.cpu().numpy()).all()
    rows = sorted(set(zip(rng.integers(0, w.B, 24).tolist(), rng.integers(0, w.Hq, 24).tolist())))
    ref = oracle_rows(w, kp, vp, q, rows)
    idx = tuple(np.array(rows).T)
    check_rows(host16(out)[idx], out32.cpu().numpy()[idx], ref, f"zf full cfg{cfg}")
