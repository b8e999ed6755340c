"""GPU append parity: kvz_append_token writes the new row into the uncompressed tail and, when the
tail fills, compresses it into the unit the page table names (ZipFusion summary, §III.D "KV Cache
Management and Scheduling": partially filled pages stay uncompressed; a full page is compressed).
The units it writes are byte-exact against the oracle and attention afterwards matches it. Seeded
random cases run appends across page fills in all three cache formats, then a pool compaction that
keeps a random half of the requests."""
import numpy as np
import pytest
import torch

import decode_attention_losslessly_amd as kvz
from oracle import c_oracle, codec
from synth import make_workload

from kvz_testlib import (DEV, check_rows, decode_units, dev, full_page_ids, host16, lane_maps, oracle_rows, tails,
                         unit_equal)
from oracle import zipfusion as zf

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("prepared", [False, True])
@pytest.mark.parametrize("cfg,H,Hq", [(3, 4, 4), (4, 2, 14), (5, 2, 2)])
def test_append_across_page_fill(cfg, H, Hq, prepared):
    """prepared: the steps go through one prepare_append_token call, the new rows copied into the
    buffers it was prepared with."""
    n_app = 19
    L0 = np.array([14, 15, 31, 0, 40], np.int32)
    w = make_workload(cfg, B=5, lens=L0 + n_app, Hq=Hq, Hkv=H, n_append=0)
    kp, vp = w.pages(0), w.pages(1)
    ids0 = full_page_ids(w, L0)
    cache = kvz.Cache.allocate(w.P, w.Hkv, w.D, w.num_pages, w.B, esc_capacity=1 << 22, device=DEV)
    if len(ids0):
        kvz.compress_pages(cache, dev(kp[ids0]), dev(vp[ids0]), dev(ids0))
    tk, tv = tails(w, kp, vp, L0)
    cache.k_tail.copy_(dev(tk))
    cache.v_tail.copy_(dev(tv))
    lens = dev(L0)
    table = dev(w.page_table)
    kbuf = torch.zeros((w.B, w.Hkv, w.D), dtype=torch.int16, device=DEV)
    vbuf = torch.zeros_like(kbuf)
    app = kvz.prepare_append_token(cache, kbuf, vbuf, table, lens) if prepared else None
    for j in range(n_app):
        kn = np.stack([w.token(r, int(L0[r]) + j, 0) for r in range(w.B)])
        vn = np.stack([w.token(r, int(L0[r]) + j, 1) for r in range(w.B)])
        if prepared:
            kbuf.copy_(dev(kn))
            vbuf.copy_(dev(vn))
            app()
        else:
            kvz.append_token(cache, dev(kn), dev(vn), table, lens)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    assert np.array_equal(lens.cpu().numpy(), L0 + n_app)
    # every full page (old and newly filled) matches the oracle's encoding of the raw page
    ids = full_page_ids(w)
    units = cache.units.cpu().numpy()
    pool = cache.esc_pool.cpu().numpy().view(np.uint16)
    ref_units, ref_pool, _ = c_oracle.encode_pages(kp[ids], vp[ids])
    for i, pid in enumerate(ids):
        for h in range(w.Hkv):
            assert unit_equal(units[pid, h], pool, ref_units[i, h], ref_pool, w.P, w.D), (pid, h)
    # tails hold the rows of the partial page
    tk2, tv2 = tails(w, kp, vp)
    Lf = L0 + n_app
    gk, gv = host16(cache.k_tail), host16(cache.v_tail)
    for r in range(w.B):
        rows = int(Lf[r]) % w.P
        assert np.array_equal(gk[r, :, :rows], tk2[r, :, :rows])
        assert np.array_equal(gv[r, :, :rows], tv2[r, :, :rows])
    # attention over the appended cache
    q = w.q()
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.zeros((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, table, lens, w.sm_scale, out, out32)
    torch.cuda.synchronize()
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, "after append")


def test_append_past_page_table_sets_status():
    w = make_workload(2, B=1, L=32, Hq=2, Hkv=2)
    cache = kvz.Cache.allocate(w.P, w.Hkv, w.D, w.num_pages, 1, esc_capacity=1 << 12, device=DEV)
    lens = dev(np.array([32], np.int32))                     # 2 pages of 16: the table is full
    kn = dev(np.zeros((1, 2, w.D), np.uint16))
    kvz.append_token(cache, kn, kn, dev(w.page_table), lens)
    torch.cuda.synchronize()
    assert int(cache.status.item()) & kvz.kvz.STATUS_SEQ_TOO_LONG
    assert int(lens.item()) == 32


def _append_case(seed):
    rng = np.random.default_rng(70000 + seed)
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 48, 64, 128]))
    grp = 1 if D == 64 else int(rng.choice([1, 2, 4, 7, 8]))
    Hkv = int(rng.integers(1, 5))
    B = int(rng.integers(1, 9))
    fmt = int(rng.integers(0, 2))
    n = int(rng.integers(1, 2 * P + 4))
    L0 = rng.integers(0, 4 * P, size=B).astype(np.int32)
    return int(rng.integers(1, 7)), D, P, Hkv * grp, Hkv, B, fmt, n, L0


@pytest.mark.parametrize("seed", range(16))
def test_random_append_and_compaction(seed):
    """Random shapes and the first two formats: n appends from lengths L0 (crossing page fills),
    every full page byte-exact against the oracle and rebuilt bit for bit on every decode route,
    attention within tolerance; then the pool is compacted to a random half of the requests and
    their attention is bit-identical."""
    _random_append_case(seed)


@pytest.mark.parametrize("seed", range(16, 24))
def test_random_append_and_compaction_channel_groups(seed):
    """The same random cases with the channel-group format."""
    _random_append_case(seed, kvz.FORMAT_CHANNEL)


def _random_append_case(seed, force_fmt=None):
    cfg, D, P, Hq, Hkv, B, fmt, n, L0 = _append_case(seed)
    fmt = fmt if force_fmt is None else force_fmt
    what = f"seed {seed}: cfg{cfg} D={D} P={P} {Hq}/{Hkv} B={B} fmt={fmt} n={n} L0={L0.tolist()}"
    print(what, flush=True)
    w = make_workload(cfg, n_append=0, B=B, lens=L0 + n, Hq=Hq, Hkv=Hkv, D=D, P=P)
    kp, vp = w.pages(0), w.pages(1)
    ids0 = full_page_ids(w, L0)
    cap = w.num_pages * Hkv * 2 * P * D
    cache = kvz.Cache.allocate(P, Hkv, D, w.num_pages, B, cap, device=DEV, fmt=fmt)
    if len(ids0):
        kvz.compress_pages(cache, dev(kp[ids0]), dev(vp[ids0]), dev(ids0))
    tk, tv = tails(w, kp, vp, L0)
    cache.k_tail.copy_(dev(tk))
    cache.v_tail.copy_(dev(tv))
    lens, table = dev(L0), dev(w.page_table)
    for j in range(n):
        kn = np.stack([w.token(r, int(L0[r]) + j, 0) for r in range(B)])
        vn = np.stack([w.token(r, int(L0[r]) + j, 1) for r in range(B)])
        kvz.append_token(cache, dev(kn), dev(vn), table, lens)
    torch.cuda.synchronize()
    assert np.array_equal(lens.cpu().numpy(), w.seq_lens) and int(cache.status.item()) == 0, what
    ids = full_page_ids(w)
    units, pool = cache.units.cpu().numpy(), host16(cache.esc_pool)
    if len(ids):
        if fmt == kvz.FORMAT_ESCAPE:
            ref_units, ref_pool, _ = c_oracle.encode_pages(kp[ids], vp[ids])
            for i, pid in enumerate(ids):
                for h in range(Hkv):
                    assert unit_equal(units[pid, h], pool, ref_units[i, h], ref_pool, P, D), (what, pid, h)
        elif fmt == kvz.FORMAT_CHANNEL:
            for pid in ids:
                for h in range(Hkv):
                    ref, ref_pool = codec.encode_unit(kp[pid, h], vp[pid, h], geometry=codec.CHANNEL)
                    assert unit_equal(units[pid, h], pool, ref, ref_pool, P, D), (what, pid, h)
        else:
            for pid in ids:
                for h in range(Hkv):
                    got = units[pid, h].tobytes()
                    off = zf.unit_raw_offset(got, P, D)
                    want, raw = zf.encode_unit(kp[pid, h], vp[pid, h], pool_offset=off)
                    assert got == want, (what, pid, h)
                    assert not raw.size or np.array_equal(pool[off:off + raw.size], raw), (what, pid, h)
        for lm in (lane_maps(D) if fmt != kvz.FORMAT_ZIPFUSION else ([0, 1] if D == 128 else [0])):
            kd, vd = decode_units(cache, ids, Hkv, P, D, lm)
            assert np.array_equal(kd, kp[ids]) and np.array_equal(vd, vp[ids]), (what, lm)
    q = w.q()
    rows = [(r, h) for r in range(B) for h in range(Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    out = torch.zeros((B, Hq, D), dtype=torch.int16, device=DEV)
    out32 = torch.zeros((B, Hq, D), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, table, lens, w.sm_scale, out, out32)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0, what
    check_rows(host16(out).reshape(-1, D), out32.cpu().numpy().reshape(-1, D), ref, what)
    live = [r for r in range(B) if np.random.default_rng(seed).random(B)[r] < 0.5]
    live_ids = np.array([w.page_table[r, i] for r in live for i in range(int(w.seq_lens[r]) // P)], np.int32)
    o16, o32 = out.clone(), out32.clone()
    kvz.compact_pool(cache, dev(live_ids), new_capacity=cap)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0, what
    lens_live = lens.clone()
    dead = [r for r in range(B) if r not in live]
    if dead:
        lens_live[dead] = 0
    out.zero_()
    out32.zero_()
    kvz.decode_attention(dev(q), cache, table, lens_live, w.sm_scale, out, out32)
    torch.cuda.synchronize()
    for r in live:
        assert torch.equal(out[r], o16[r]) and torch.equal(out32[r], o32[r]), (what, "after compaction", r)
