"""GPU codec parity: kvz_compress_pages is byte-exact against the CPU oracle and the attention
kernels' in-register decode (kvz_decompress_pages) gives back every input bit pattern, through
every decode route the attention kernels take:
  lane maps 0 / 1   multi-head / grouped-query lane layout, escapes patched as the main loops and
                    the per-unit path after them do (inline list walk; pool list staged whole);
  lane maps 2 / 3   the same layouts through the pool-capable loops' route (a pool unit's escape
                    windows staged with its payload, every offset word patched from them)."""
import numpy as np
import pytest
import torch

import decode_attention_losslessly_amd as kvz
from oracle import c_oracle, codec
from synth import make_workload

from kvz_testlib import DEV, build_cache, decode_units, dev, full_page_ids, host16, lane_maps, unit_equal

pytestmark = pytest.mark.gpu

SMALL = {
    1: dict(),
    2: dict(L=100),
    3: dict(B=3, L=97),
    4: dict(B=5, lens=[1, 16, 33, 150, 47]),
    5: dict(B=2, L=70),
    6: dict(B=2, L=70),
}


def _compare_units(w, cache, kp, vp, ids):
    units = cache.units.cpu().numpy()
    pool = cache.esc_pool.cpu().numpy().view(np.uint16)
    ref_units, ref_pool, _ = c_oracle.encode_pages(kp[ids], vp[ids])
    bad = []
    for i, pid in enumerate(ids):
        for h in range(w.Hkv):
            if not unit_equal(units[pid, h], pool, ref_units[i, h], ref_pool, w.P, w.D):
                bad.append((int(pid), h))
    assert not bad, f"{len(bad)} units differ, first {bad[:4]}"


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_compress_matches_oracle(cfg):
    w = make_workload(cfg, **SMALL[cfg])
    kp, vp = w.pages(0), w.pages(1)
    cache, _ = build_cache(w, kp, vp)
    assert int(cache.status.item()) == 0
    ids = full_page_ids(w, w.seq_lens - w.n_append)
    _compare_units(w, cache, kp, vp, ids)


def _pattern_pages(P, D, n, seed):
    """n pages x (K, V) x H=2 heads of P x D values, page by page: all 65,536 patterns in order,
    twice (consecutive patterns share their exponent, so these units have no escapes and stay
    inline), then seeded permutations of them (escapes everywhere: pool units)."""
    rng = np.random.default_rng(seed)
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    need = n * 2 * 2 * P * D
    vals = np.concatenate([allp, allp] + [rng.permutation(allp) for _ in range(need // 65536)])[:need]
    x = vals.reshape(n, 2, 2, P, D)
    return np.ascontiguousarray(x[:, 0]), np.ascontiguousarray(x[:, 1])


@pytest.mark.parametrize("P,D", [(16, 128), (32, 128), (16, 64), (256, 64)])
def test_compress_all_bit_patterns(P, D):
    n = max(4, 65536 // (P * D))
    kp, vp = _pattern_pages(P, D, n, P + D)
    ids = np.arange(n, dtype=np.int32)[::-1].copy()
    cache = kvz.Cache.allocate(P, 2, D, n, 1, esc_capacity=4 * n * 2 * P * D, device=DEV)
    kvz.compress_pages(cache, dev(kp[ids]), dev(vp[ids]), dev(ids))
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    units = cache.units.cpu().numpy()
    pool = cache.esc_pool.cpu().numpy().view(np.uint16)
    ref_units, ref_pool, _ = c_oracle.encode_pages(kp[ids], vp[ids])
    for i, pid in enumerate(ids):
        for h in range(2):
            assert unit_equal(units[pid, h], pool, ref_units[i, h], ref_pool, P, D), (pid, h)
    heads = [codec.unit_header(units[pid, h], P, D) for pid in ids for h in range(2)]
    assert any(off == codec.INLINE for _, _, off in heads) and any(off != codec.INLINE for _, _, off in heads)
    # the in-kernel decode gives every pattern back, on every route
    for lane_map in lane_maps(D):
        kd, vd = decode_units(cache, ids, 2, P, D, lane_map)
        assert np.array_equal(kd, kp[ids]), lane_map
        assert np.array_equal(vd, vp[ids]), lane_map


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_in_kernel_decode_is_bit_exact(cfg):
    w = make_workload(cfg, **SMALL[cfg])
    kp, vp = w.pages(0), w.pages(1)
    cache, _ = build_cache(w, kp, vp)
    ids = full_page_ids(w, w.seq_lens - w.n_append)
    for lane_map in lane_maps(w.D):
        kd, vd = decode_units(cache, ids, w.Hkv, w.P, w.D, lane_map)
        assert np.array_equal(kd, kp[ids]), lane_map
        assert np.array_equal(vd, vp[ids]), lane_map


@pytest.mark.parametrize("P,D", [(16, 128), (32, 128), (16, 64)])
def test_decode_from_a_pool_filled_to_capacity(P, D):
    """Escape-heavy units (every one keeps its escapes in the pool) in a pool sized to exactly
    what they need, ending inside a 16-byte chunk: the windows of the last units reach the pool's
    end and are read element by element up to it. Every route gives every value back."""
    for L in range(12 * P, 20 * P, P):
        w = make_workload(5, n_append=0, B=2, L=L, Hq=2, Hkv=2, D=D, P=P)
        kp, vp = w.pages(0), w.pages(1)
        probe, _ = build_cache(w, kp, vp)
        need = int(probe.esc_cursor.item())
        del probe
        if need % 8:
            break
    assert need % 8, need
    cache, _ = build_cache(w, kp, vp, esc_capacity=need)
    assert int(cache.status.item()) == 0 and int(cache.esc_cursor.item()) == need
    ids = full_page_ids(w)
    units = cache.units.cpu().numpy()
    heads = [codec.unit_header(units[pid, h], P, D) for pid in ids for h in range(w.Hkv)]
    assert all(off != codec.INLINE for _, _, off in heads)
    assert max(off + kc + vc for kc, vc, off in heads) == need     # some unit's list ends at the pool's end
    for lane_map in lane_maps(D):
        kd, vd = decode_units(cache, ids, w.Hkv, P, D, lane_map)
        assert np.array_equal(kd, kp[ids]), lane_map
        assert np.array_equal(vd, vp[ids]), lane_map


def test_escape_pool_overflow_sets_status_and_stays_in_bounds():
    w = make_workload(5, B=1, L=64, Hq=2, Hkv=2)
    kp, vp = w.pages(0), w.pages(1)
    ids = np.arange(w.num_pages, dtype=np.int32)
    cache = kvz.Cache.allocate(w.P, w.Hkv, w.D, w.num_pages, 1, esc_capacity=3000, device=DEV)
    guard = cache.esc_pool.clone()
    kvz.compress_pages(cache, dev(kp), dev(vp), dev(ids))
    torch.cuda.synchronize()
    assert int(cache.status.item()) & kvz.kvz.STATUS_ESC_POOL_FULL
    assert int(cache.esc_cursor.item()) > 3000        # cursor counts the refused request too
    units = cache.units.cpu().numpy()
    for pid in ids:
        for h in range(w.Hkv):
            kc, vc, off = codec.unit_header(units[pid, h], w.P, w.D)
            assert off == codec.INLINE or off + kc + vc <= 3000
    assert guard.numel() == cache.esc_pool.numel()


def test_bad_page_id_sets_status():
    w = make_workload(2, L=32, Hq=2, Hkv=2)
    kp, vp = w.pages(0), w.pages(1)
    cache = kvz.Cache.allocate(w.P, w.Hkv, w.D, 2, 1, esc_capacity=1 << 12, device=DEV)
    ids = np.array([0, 7], np.int32)
    kvz.compress_pages(cache, dev(kp[:2]), dev(vp[:2]), dev(ids))
    torch.cuda.synchronize()
    assert int(cache.status.item()) & kvz.kvz.STATUS_BAD_PAGE_ID


@pytest.mark.parametrize("cfg", [2, 3, 4, 5, 6])
def test_compress_full_size_sampled(cfg, full_workloads):
    """Full shapes: sampled units byte-exact against the oracle and rebuilt bit for bit by every
    decode route of the kernel that serves the workload (multi-head or grouped-query)."""
    w, kp, vp, cache, _ = full_workloads(cfg)
    ids = full_page_ids(w, w.seq_lens - w.n_append)
    rng = np.random.default_rng(cfg)
    sample = ids[rng.choice(len(ids), size=min(96, len(ids)), replace=False)]
    _compare_units(w, cache, kp, vp, sample)
    for lane_map in ([1, 3] if w.Hq > w.Hkv else [0, 2]):
        kd, vd = decode_units(cache, sample, w.Hkv, w.P, w.D, lane_map)
        assert np.array_equal(kd, kp[sample]) and np.array_equal(vd, vp[sample]), lane_map
