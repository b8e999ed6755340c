"""GPU parity of the third cache format, channel groups (include/kvz.h, KVZ_FORMAT_CHANNEL; the
oracle's codec with geometry "channel"): compression byte-exact against the oracle (escape lists
compared wherever the pool holds them), the kernels' in-register rebuild bit-exact in every lane
layout and route (inline lists, per-unit pool patch, pool-capable loops), attention of the
multi-head and grouped-query kernels against the fp64 oracle within the stated tolerance on both
schedules, and appends with compress-on-fill. Workloads cover smooth values, x20 outlier
channels, the escape-stress distribution (pool units) and head dims 64 and 128."""
import numpy as np
import pytest
import torch

import decode_attention_losslessly_amd as kvz
from kvz_testlib import (DEV, build_cache, check_rows, decode_units, dev, full_page_ids, host16, lane_maps,
                         oracle_rows, unit_equal)
from oracle import codec
from synth import make_workload

pytestmark = pytest.mark.gpu
CHF = kvz.FORMAT_CHANNEL

SMALL = {
    1: dict(),                                       # head dim 64, one 256-token page
    2: dict(L=100),                                  # x20 outlier channels in K
    3: dict(B=3, L=97),
    4: dict(B=5, lens=[1, 16, 33, 150, 47]),         # grouped queries, 28 over 4 KV heads
    5: dict(B=2, L=70),                              # escape stress: units in the pool
    6: dict(B=2, L=70, Hq=8, Hkv=8),
    7: dict(cfg=6, B=3, lens=[70, 161, 16]),         # grouped queries, 32 over 8 KV heads
    8: dict(cfg=5, B=2, L=70, Hq=8, Hkv=2),          # grouped queries over pool units
    9: dict(cfg=6, B=2, L=100, Hq=16, Hkv=4, D=64),  # grouped queries at head dim 64
}


def _workload(key):
    a = dict(SMALL[key])
    return make_workload(a.pop("cfg", key), **a)


def _compare_units(w, cache, kp, vp, ids):
    units = cache.units.cpu().numpy()
    pool = host16(cache.esc_pool)
    bad = []
    for pid in ids:
        for h in range(w.Hkv):
            ref, ref_pool = codec.encode_unit(kp[pid, h], vp[pid, h], geometry=codec.CHANNEL)
            if not unit_equal(units[pid, h], pool, ref, ref_pool, w.P, w.D):
                bad.append((int(pid), h))
    assert not bad, f"{len(bad)} units differ, first {bad[:4]}"


@pytest.mark.parametrize("key", sorted(SMALL))
def test_compress_matches_oracle(key):
    w = _workload(key)
    kp, vp = w.pages(0), w.pages(1)
    cache, _ = build_cache(w, kp, vp, fmt=CHF)
    assert int(cache.status.item()) == 0
    _compare_units(w, cache, kp, vp, full_page_ids(w))


@pytest.mark.parametrize("key", sorted(SMALL))
def test_in_kernel_rebuild_is_bit_exact(key):
    w = _workload(key)
    kp, vp = w.pages(0), w.pages(1)
    cache, _ = build_cache(w, kp, vp, fmt=CHF)
    ids = full_page_ids(w)
    for lane_map in lane_maps(w.D):
        kd, vd = decode_units(cache, ids, w.Hkv, w.P, w.D, lane_map)
        assert np.array_equal(kd, kp[ids]) and np.array_equal(vd, vp[ids]), lane_map


@pytest.mark.parametrize("P,D", [(16, 128), (32, 128), (16, 64), (256, 64)])
def test_all_bit_patterns(P, D):
    """Every BF16 pattern through compression and every rebuild route: in order (consecutive
    patterns share exponents: inline units) and permuted (escapes everywhere: pool units)."""
    rng = np.random.default_rng(P * D)
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    n = max(4, 65536 // (P * D))
    need = n * 2 * 2 * P * D
    vals = np.concatenate([allp, allp] + [rng.permutation(allp) for _ in range(need // 65536)])[:need]
    x = vals.reshape(n, 2, 2, P, D)
    kp, vp = np.ascontiguousarray(x[:, 0]), np.ascontiguousarray(x[:, 1])
    ids = np.arange(n, dtype=np.int32)[::-1].copy()
    cache = kvz.Cache.allocate(P, 2, D, n, 1, esc_capacity=4 * n * 2 * P * D, device=DEV, fmt=CHF)
    kvz.compress_pages(cache, dev(kp[ids]), dev(vp[ids]), dev(ids))
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    units, pool = cache.units.cpu().numpy(), host16(cache.esc_pool)
    for i, pid in enumerate(ids):
        for h in range(2):
            ref, ref_pool = codec.encode_unit(kp[ids][i, h], vp[ids][i, h], geometry=codec.CHANNEL)
            assert unit_equal(units[pid, h], pool, ref, ref_pool, P, D), (int(pid), h)
    order = np.arange(n, dtype=np.int32)
    for lane_map in lane_maps(D):
        kd, vd = decode_units(cache, order, 2, P, D, lane_map)
        assert np.array_equal(kd, kp[ids][::-1]) and np.array_equal(vd, vp[ids][::-1]), lane_map


@pytest.mark.parametrize("key", sorted(SMALL))
def test_attention_matches_oracle(key):
    w = _workload(key)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp, fmt=CHF)
    q = w.q()
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    # split schedule with its own size, single-page splits, the ranked schedule (forced)
    for pps in (0, 1, -2):
        out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
        out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
        kvz.decode_attention(dev(q), cache, dev(w.page_table), lens, w.sm_scale, out, out32, pages_per_split=pps)
        torch.cuda.synchronize()
        assert int(cache.status.item()) == 0
        check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref,
                   f"channel {key} pps{pps}")


@pytest.mark.parametrize("P,D,Hq", [(16, 128, 4), (32, 128, 4), (16, 64, 4), (16, 128, 16)])
def test_mixed_units_and_page_fills(P, D, Hq):
    """Requests with smooth pages next to escape-stress ones (inline and pool units in one
    split: the pipelined loop, the per-unit pool path and the pool-capable loop all run), then
    appends across page fills; units byte-exact against the oracle, rebuild bit-exact,
    attention against the fp64 oracle."""
    n_steps = P + 3
    lens = np.array([3 * P - 2, P + 5, 2 * P, 4 * P + 7])
    smooth = make_workload(2, B=4, lens=lens + n_steps, Hq=Hq, Hkv=4, D=D, P=P, n_append=0)
    stress = make_workload(5, B=4, lens=lens + n_steps, Hq=Hq, Hkv=4, D=D, P=P, n_append=0)
    kp, vp = smooth.pages(0), smooth.pages(1)
    ks, vs = stress.pages(0), stress.pages(1)
    rng = np.random.default_rng(P + D + Hq)
    odd = rng.random(smooth.num_pages) < 0.5
    kp[odd], vp[odd] = ks[odd], vs[odd]
    w = smooth
    L0 = (w.seq_lens - n_steps).astype(np.int32)
    ids = full_page_ids(w, L0)
    cache = kvz.Cache.allocate(P, w.Hkv, D, w.num_pages, w.B, w.num_pages * w.Hkv * 2 * P * D, device=DEV, fmt=CHF)
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
    _compare_units(w, cache, kp, vp, full)
    for lane_map in lane_maps(D):
        kd, vd = decode_units(cache, full, w.Hkv, P, D, lane_map)
        assert np.array_equal(kd, kp[full]) and np.array_equal(vd, vp[full]), lane_map
    q = w.q()
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    for pps in (0, 1):
        out = torch.zeros((w.B, w.Hq, D), dtype=torch.int16, device=DEV)
        out32 = torch.zeros((w.B, w.Hq, D), dtype=torch.float32, device=DEV)
        kvz.decode_attention(dev(q), cache, table, lens_d, w.sm_scale, out, out32, pages_per_split=pps)
        torch.cuda.synchronize()
        check_rows(host16(out).reshape(-1, D), out32.cpu().numpy().reshape(-1, D), ref,
                   f"channel mixed P{P} D{D} Hq{Hq} pps{pps}")


@pytest.mark.parametrize("cfg", [3, 5, 6])
def test_full_size_sampled(cfg):
    """Configs 3 (8K x 32 heads), 5 (escape stress, 32K) and 6 (the pages' grouped-query shape)
    at full size in this format: sampled units byte-exact and rebuilt bit for bit, sampled rows
    against the fp64 oracle."""
    w = make_workload(cfg)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp, fmt=CHF)
    assert int(cache.status.item()) == 0
    rng = np.random.default_rng(cfg)
    ids = full_page_ids(w, w.seq_lens - w.n_append)
    sample = ids[rng.choice(len(ids), size=32, replace=False)]
    _compare_units(w, cache, kp, vp, sample)
    kd, vd = decode_units(cache, sample, w.Hkv, w.P, w.D, 1 if w.Hq > w.Hkv else 0)
    assert np.array_equal(kd, kp[sample]) and np.array_equal(vd, vp[sample])
    q = w.q()
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, dev(w.page_table), lens, w.sm_scale, out, out32)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0 and np.isfinite(out32.cpu().numpy()).all()
    rows = sorted(set(zip(rng.integers(0, w.B, 16).tolist(), rng.integers(0, w.Hq, 16).tolist())))
    ref = oracle_rows(w, kp, vp, q, rows)
    idx = tuple(np.array(rows).T)
    check_rows(host16(out)[idx], out32.cpu().numpy()[idx], ref, f"channel full cfg{cfg}")
