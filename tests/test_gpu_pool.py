"""kvz_compact_pool: the pool data of the units still in use moves to a new, smaller pool and the
units point at it; attention of the live requests is bit-identical before and after, with the old
pool overwritten so that any read of it would show. All three cache formats (escape lists with
token or channel groups; ZipFusion raw blocks), on escape-heavy data. An undersized new pool drops the data of the units that do not
fit (status bit set) and nothing reads past a pool. A pool filled exactly to its capacity, ending
inside a 16-byte chunk, escape-heavy units under grouped-query attention, and splits that start on
inline units and go on into pool units (both pool routes in one wave) still give attention within
tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

import decode_attention_losslessly_amd as kvz
from kvz_testlib import DEV, build_cache, check_rows, dev, full_page_ids, host16, oracle_rows
from synth import make_workload

pytestmark = pytest.mark.gpu


def _attend(w, cache, lens, q):
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.zeros((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
    kvz.decode_attention(q, cache, dev(w.page_table), lens, w.sm_scale, out, out32)
    torch.cuda.synchronize()
    return out.clone(), out32.clone()


def _pool_use(cache, w, ids, fmt):
    """pool elements the units `ids` own, read from their headers"""
    u = cache.units.cpu().numpy()
    P, D = w.P, w.D
    total = 0
    for pid in ids:
        for h in range(w.Hkv):
            b = u[pid, h]
            if fmt == kvz.FORMAT_ZIPFUSION:
                nb = 2 * (P // 16) * (D // 32)
                total += 512 * int((b[:nb] == 0xFF).sum())
            else:
                hdr = 2 * P * (D // 64)
                off = int(b[hdr + 8:hdr + 16].view(np.uint64)[0])
                if off != (1 << 64) - 1:
                    total += int(b[hdr:hdr + 8].view(np.uint32).sum())
    return total


@pytest.mark.parametrize("fmt", [kvz.FORMAT_ESCAPE, kvz.FORMAT_ZIPFUSION, kvz.FORMAT_CHANNEL])
def test_compaction_keeps_live_results(fmt):
    w = make_workload(5, B=4, lens=[70, 45, 100, 33], Hq=4, Hkv=4, D=128)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp, fmt=fmt)
    q = dev(w.q())
    o16, o32 = _attend(w, cache, lens, q)
    live_rows = [0, 2]
    lens_live = lens.clone()
    lens_live[[1, 3]] = 0
    live = np.array([w.page_table[r, i] for r in live_rows for i in range(int(w.seq_lens[r]) // w.P)], np.int32)
    need = _pool_use(cache, w, live, fmt)
    used_before = int(cache.esc_cursor.item())
    assert 0 < need < used_before
    old_pool = cache.esc_pool
    kvz.compact_pool(cache, dev(live), new_capacity=need)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    assert int(cache.esc_cursor.item()) == need and cache.esc_capacity == need
    old_pool.fill_(0x7F7F)      # nothing may read the old pool any more
    n16, n32 = _attend(w, cache, lens_live, q)
    for r in live_rows:
        assert torch.equal(n16[r], o16[r]) and torch.equal(n32[r], o32[r])
    assert not n16[[1, 3]].any()


@pytest.mark.parametrize("fmt", [kvz.FORMAT_ESCAPE, kvz.FORMAT_ZIPFUSION, kvz.FORMAT_CHANNEL])
def test_undersized_pool_drops_and_stays_in_bounds(fmt):
    w = make_workload(5, B=2, L=64, Hq=4, Hkv=4, D=128)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp, fmt=fmt)
    ids = full_page_ids(w)
    kvz.compact_pool(cache, dev(ids), new_capacity=1000)
    torch.cuda.synchronize()
    assert int(cache.status.item()) & kvz.kvz.STATUS_ESC_POOL_FULL
    assert int(cache.esc_cursor.item()) > 1000          # the cursor counts every request
    _attend(w, cache, lens, dev(w.q()))   # outputs unspecified (status says so); the run must stay in bounds


@pytest.mark.parametrize("D,P", [(128, 16), (64, 32)])
@pytest.mark.parametrize("pps", [0, 64])
def test_pool_filled_to_capacity_matches_oracle(D, P, pps):
    """The pool holds exactly what the cache needs and ends inside a 16-byte chunk, so the escape
    windows of the last units reach its end and are read element by element up to the capacity.
    pages_per_split 64 gives each row one split; 0 lets the device choose (shorter splits). Every
    split starts with an escape-heavy unit, so either way its wave walks it in the pool-capable
    loop from the first step."""
    w = make_workload(5, n_append=0, B=2, L=12 * P, Hq=4, Hkv=4, D=D, P=P)
    kp, vp = w.pages(0), w.pages(1)
    probe, _ = build_cache(w, kp, vp)
    need = int(probe.esc_cursor.item())
    del probe
    assert need % 8 != 0, need
    cache, lens = build_cache(w, kp, vp, esc_capacity=need)
    assert int(cache.status.item()) == 0 and int(cache.esc_cursor.item()) == need
    q = w.q()
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, dev(w.page_table), lens, w.sm_scale, out, out32, pages_per_split=pps)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    check_rows(host16(out).reshape(-1, D), out32.cpu().numpy().reshape(-1, D), ref,
               f"D={D} P={P} pps={pps}, pool of {need} elements")


@pytest.mark.parametrize("P", [16, 32])
@pytest.mark.parametrize("pps", [0, 64])
def test_grouped_query_pool_loop_matches_oracle(P, pps):
    """Escape-heavy units under grouped-query attention (8 query heads over 2 KV heads): the
    first unit has a quarter or more of its values escaped, so a wave moves to the pool-capable
    loop at once; with 32-token pages a unit spans two tiles, whose escape windows start at the
    block cursors. One split per row (64) or the device's choice (0)."""
    w = make_workload(5, n_append=0, B=3, lens=np.array([10 * P + 5, 7 * P, 12 * P + 9]), Hq=8, Hkv=2, D=128, P=P)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp)
    q = w.q()
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, dev(w.page_table), lens, w.sm_scale, out, out32, pages_per_split=pps)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, f"P={P} pps={pps}")


def _mixed_pages(w, light_pages):
    """K and V pages of escape-stress workload w, except that the logical pages light_pages[r]
    of request r hold light data (per-channel log-normal values, whose few escapes stay in the
    unit's inline list)."""
    kp, vp = w.pages(0), w.pages(1)
    light = make_workload(3, n_append=0, B=w.B, lens=w.seq_lens, Hq=w.Hq, Hkv=w.Hkv, D=w.D, P=w.P)
    for r in range(w.B):
        for i in light_pages[r]:
            pid = int(w.page_table[r, i])
            kp[pid], vp[pid] = light.page(pid, 0), light.page(pid, 1)
    return kp, vp


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2)])
@pytest.mark.parametrize("P", [16, 32])
@pytest.mark.parametrize("pps", [0, 64])
@pytest.mark.parametrize("spare", [0, 3])
def test_splits_from_inline_into_pool_units(Hq, Hkv, P, pps, spare):
    """Requests whose first pages are light (inline escapes) and whose later pages are escape-heavy
    (pool lists). With `spare` times the workload's unit slots in the cache, its pool holds less
    than a quarter of a unit's values per slot, so the splits start in the pipelined loop: it
    computes the light pages and skips the first heavy ones until most tiles seen went to the
    pool; the wave then walks the rest of its split in the pool-capable loop (which also meets
    light pages here: request 1 has some between heavy ones) and, after it, adds the skipped heavy
    pages through the per-unit path (a split that starts on a heavy page goes to the pool-capable
    loop at once). Without spare slots the cache counts as escape-heavy and every split starts in
    the pool-capable loop. Multi-head and grouped-query kernels; one split per row (64) or the
    device's choice (0)."""
    lens = np.array([24 * P + 5, 20 * P, 30 * P + 11])
    w = make_workload(5, n_append=0, B=3, lens=lens, Hq=Hq, Hkv=Hkv, D=128, P=P)
    light = [range(0, 3), list(range(0, 4)) + [9, 10, 15], range(0, 8)]
    kp, vp = _mixed_pages(w, light)
    cache, lt = build_cache(w, kp, vp, num_pages=w.num_pages * (1 + spare))
    heavy_cache = int(cache.esc_cursor.item()) >= cache.num_pages * Hkv * P * 128 // 2
    assert heavy_cache == (spare == 0)
    units = cache.units.cpu().numpy()
    hdr = 2 * P * 2
    inline = [[bool((units[w.page_table[r, i], :, hdr + 8:hdr + 16].view(np.uint64) == (1 << 64) - 1).all())
               for i in range(int(lens[r]) // P)] for r in range(w.B)]
    for r in range(w.B):
        assert [i for i, x in enumerate(inline[r]) if x] == list(light[r]), r
    q = w.q()
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, dev(w.page_table), lt, w.sm_scale, out, out32, pages_per_split=pps)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref,
               f"Hq={Hq} Hkv={Hkv} P={P} pps={pps}")
