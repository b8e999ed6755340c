"""GPU attention parity: the compressed kernels (kvz_decode_attention) and the dense baseline
(kvz_decode_attention_dense) against the fp64 CPU oracle, within the stated tolerance:
|out_bf16 - o| <= max(2e-2, 2^-7 |o|) per element and max_d |out_f32 - o| <= 1e-4 max_d |o| per row."""
import math

import numpy as np
import pytest
import torch

import decode_attention_losslessly_amd as kvz
from oracle import attention as oa
from synth import f32_to_bf16_bits, make_workload

from kvz_testlib import DEV, build_cache, check_rows, dev, host16, oracle_rows

pytestmark = pytest.mark.gpu

SMALL = {
    1: dict(),
    2: dict(L=333),
    3: dict(B=3, L=161),
    4: dict(B=6, lens=[1, 15, 16, 17, 300, 1024]),
    5: dict(B=2, L=517),
    6: dict(B=3, L=161),
}


def _run(w, cache, lens, q, dense_pages=None, pages_per_split=0):
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    if dense_pages is None:
        kvz.decode_attention(dev(q), cache, dev(w.page_table), lens, w.sm_scale, out, out32,
                             pages_per_split=pages_per_split)
    else:
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        kvz.decode_attention_dense(dev(q), dense_pages[0], dense_pages[1], dev(w.page_table), lens, w.sm_scale, out,
                                   out32, status=status, pages_per_split=pages_per_split)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
    torch.cuda.synchronize()
    return host16(out), out32.cpu().numpy()


def _all_rows(w):
    return [(r, h) for r in range(w.B) for h in range(w.Hq)]


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_compressed_matches_oracle(cfg):
    w = make_workload(cfg, **SMALL[cfg])
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp)
    q = w.q()
    o16, o32 = _run(w, cache, lens, q)
    assert int(cache.status.item()) == 0
    rows = _all_rows(w)
    ref = oracle_rows(w, kp, vp, q, rows)
    check_rows(o16.reshape(-1, w.D), o32.reshape(-1, w.D), ref, f"cfg{cfg} compressed")


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_dense_matches_oracle(cfg):
    w = make_workload(cfg, **SMALL[cfg])
    kp, vp = w.pages(0), w.pages(1)
    q = w.q()
    o16, o32 = _run(w, None, dev(w.seq_lens), q, dense_pages=(dev(kp), dev(vp)))
    rows = _all_rows(w)
    ref = oracle_rows(w, kp, vp, q, rows)
    check_rows(o16.reshape(-1, w.D), o32.reshape(-1, w.D), ref, f"cfg{cfg} dense")


@pytest.mark.parametrize("cfg", [2, 4])
def test_split_count_does_not_change_the_result_and_runs_repeat(cfg):
    w = make_workload(cfg, **SMALL[cfg])
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp)
    q = w.q()
    base16, base32 = _run(w, cache, lens, q)
    for pps in [1, 3, 64, 100000]:
        o16, o32 = _run(w, cache, lens, q, pages_per_split=pps)
        nrm = np.abs(base32).max(axis=-1, keepdims=True)
        assert np.all(np.abs(o32 - base32) <= 1e-5 * nrm), pps     # fp32 reduction order only
    again16, again32 = _run(w, cache, lens, q)
    assert np.array_equal(again32.view(np.uint32), base32.view(np.uint32))    # repeatable bit for bit
    assert np.array_equal(again16, base16)


def _run_table(w, cache, lens, q, table, fmt_pps=0):
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, dev(table), lens, w.sm_scale, out, out32, pages_per_split=fmt_pps)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    return host16(out), out32.cpu().numpy()


@pytest.mark.parametrize("cfg,fmt", [(2, kvz.FORMAT_ESCAPE), (4, kvz.FORMAT_ESCAPE), (5, kvz.FORMAT_ESCAPE),
                                     (6, kvz.FORMAT_ESCAPE), (4, kvz.FORMAT_ZIPFUSION)])
def test_unit_placement_and_token_order(cfg, fmt):
    """Moving every unit to another slot (the page table follows it; pool offsets inside the units
    stay valid) gives the same result bit for bit: the kernels depend on a page's slot only for its
    address. Shuffling the order of each request's full pages in the page table permutes its
    tokens, which attention does not see: the result moves by fp32 rounding order only."""
    w = make_workload(cfg, **SMALL[cfg])
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp, fmt=fmt)
    q = w.q()
    base16, base32 = _run_table(w, cache, lens, q, w.page_table)
    rng = np.random.default_rng(11)
    perm = rng.permutation(w.num_pages).astype(np.int32)          # slot pid moves to perm[pid]
    moved = cache.units[torch.from_numpy(np.argsort(perm)).to(DEV)].clone()
    cache.units.copy_(moved)
    ok = (w.page_table >= 0) & (w.page_table < w.num_pages)
    table = np.where(ok, perm[np.clip(w.page_table, 0, w.num_pages - 1)], w.page_table).astype(np.int32)
    m16, m32 = _run_table(w, cache, lens, q, table)
    assert np.array_equal(m32.view(np.uint32), base32.view(np.uint32)) and np.array_equal(m16, base16)
    shuffled = table.copy()
    L = lens.cpu().numpy()
    for r in range(w.B):
        nfull = int(L[r]) // w.P
        shuffled[r, :nfull] = table[r, rng.permutation(nfull)]
    ref = oracle_rows(w, kp, vp, q, _all_rows(w))      # over the tokens in their original order
    for pps in (0, 1):
        s16, s32 = _run_table(w, cache, lens, q, shuffled, pps)
        nrm = np.abs(base32).max(axis=-1, keepdims=True)
        assert np.all(np.abs(s32 - base32) <= 1e-5 * nrm), pps
        check_rows(s16.reshape(-1, w.D), s32.reshape(-1, w.D), ref, f"cfg {cfg} fmt {fmt} shuffled pages, pps {pps}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_ranked_schedule_matches_oracle(cfg):
    """The multi-head kernel's ranked schedule (pages_per_split = -R forces it: every row is cut
    into 2R chunks, each a share of its request's own pages, the last R shrinking) gives the
    oracle's attention and the default schedule's fp32 result up to reduction order; the kernel
    records -2R where the merge reads it. The escape-stress workload takes the pool paths inside
    the chunks. The uncompressed baseline under the same schedule matches the oracle too."""
    w = make_workload(cfg, **SMALL[cfg])
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp)
    q = w.q()
    base16, base32 = _run(w, cache, lens, q)
    rows = _all_rows(w)
    ref = oracle_rows(w, kp, vp, q, rows)
    nrm = np.abs(base32).max(axis=-1, keepdims=True)
    for pps in [-1, -2, -5]:
        o16, o32 = _run(w, cache, lens, q, pages_per_split=pps)
        assert int(cache.status.item()) == 0
        check_rows(o16.reshape(-1, w.D), o32.reshape(-1, w.D), ref, f"cfg{cfg} ranked {pps}")
        assert np.all(np.abs(o32 - base32) <= 1e-5 * nrm), pps
        ws = torch.empty(kvz.workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages, pps), dtype=torch.uint8,
                         device=DEV)
        kvz.decode_attention_splits(dev(q), cache, dev(w.page_table), lens, w.sm_scale, ws, pages_per_split=pps)
        assert kvz.chosen_pages_per_split(ws, w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages, pps) == 2 * pps
        # the uncompressed baseline under the same schedule
        d16, d32 = _run(w, None, dev(w.seq_lens), q, dense_pages=(dev(kp), dev(vp)), pages_per_split=pps)
        check_rows(d16.reshape(-1, w.D), d32.reshape(-1, w.D), ref, f"cfg{cfg} dense ranked {pps}")


@pytest.mark.parametrize("lens,ranked", [([6000] * 8, True), ([4000, 10000, 5000, 9000, 4500, 8000, 6000, 7000], False)])
def test_schedule_choice(lens, ranked):
    """Without pages_per_split the multi-head kernel takes the ranked schedule for even lengths
    whose big chunks would be long (8 x 32 rows: R = 16, 300 of 375 pages in them), and the
    split schedule when the longest request exceeds 5/4 of the mean, where chunks proportional
    to each length would make the longest requests' chunks the longest waves. Sampled rows
    against the oracle either way."""
    w = make_workload(3, B=8, lens=lens, Hq=32, Hkv=32, n_append=0)
    kp, vp = w.pages(0), w.pages(1)
    cache, lt = build_cache(w, kp, vp)
    q = w.q()
    ws = torch.empty(kvz.workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages), dtype=torch.uint8, device=DEV)
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.zeros((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
    kvz.decode_attention_splits(dev(q), cache, dev(w.page_table), lt, w.sm_scale, ws)
    kvz.merge_splits(ws, lt, w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages, out, out32)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    assert (kvz.chosen_pages_per_split(ws, w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages) < 0) == ranked
    rows = _sampled_rows(w, 16, 7)
    ref = oracle_rows(w, kp, vp, q, rows)
    idx = tuple(np.array(rows).T)
    check_rows(host16(out)[idx], out32.cpu().numpy()[idx], ref, f"schedule ranked={ranked}")


def test_dense_and_compressed_agree():
    w = make_workload(3, **SMALL[3])
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp)
    q = w.q()
    c16, c32 = _run(w, cache, lens, q)
    d16, d32 = _run(w, None, dev(w.seq_lens), q, dense_pages=(dev(kp), dev(vp)))
    nrm = np.abs(d32).max(axis=-1, keepdims=True)
    assert np.all(np.abs(c32 - d32) <= 2e-5 * nrm + 1e-30)


def _synthetic_cache(B, H, Hq, D, P, L, K, V, q):
    """Cache and dense pages from explicit token arrays K, V [B][L][H][D] (BF16 bits)."""
    npg = (L + P - 1) // P
    table = np.arange(B * npg, dtype=np.int32).reshape(B, npg)
    kp = np.zeros((B * npg, H, P, D), np.uint16)
    vp = np.zeros_like(kp)
    for r in range(B):
        for t in range(L):
            kp[table[r, t // P], :, t % P] = K[r, t]
            vp[table[r, t // P], :, t % P] = V[r, t]

    class W:
        pass
    w = W()
    w.B, w.Hq, w.Hkv, w.D, w.P, w.page_table = B, Hq, H, D, P, table
    w.seq_lens = np.full(B, L, np.int32)
    w.n_append, w.num_pages, w.sm_scale, w.k_dist = 0, B * npg, 1 / math.sqrt(D), "x"
    w.appended = None
    cache, lens = build_cache(w, kp, vp)
    return w, cache, lens, kp, vp


@pytest.mark.parametrize("Hq,H", [(4, 4), (8, 2)])
def test_closed_forms(Hq, H):
    rng = np.random.default_rng(7)
    B, D, P = 3, 128, 16
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32))
    # 1) a single token returns that token's V exactly
    K = f32_to_bf16_bits(rng.standard_normal((B, 1, H, D)).astype(np.float32) * 4)
    V = f32_to_bf16_bits(rng.standard_normal((B, 1, H, D)).astype(np.float32))
    w, cache, lens, kp, vp = _synthetic_cache(B, H, Hq, D, P, 1, K, V, q)
    o16, o32 = _run(w, cache, lens, q)
    want = np.repeat(V[:, 0], Hq // H, axis=1)
    assert np.array_equal(o16, want)
    assert np.array_equal(o32, oa.bf16_to_f64(want).astype(np.float32))
    # 2) V constant along the tokens returns that constant exactly (in BF16)
    L = 77
    K = f32_to_bf16_bits(rng.standard_normal((B, L, H, D)).astype(np.float32) * 3)
    row = f32_to_bf16_bits(rng.standard_normal((B, 1, H, D)).astype(np.float32))
    V = np.repeat(row, L, axis=1)
    w, cache, lens, kp, vp = _synthetic_cache(B, H, Hq, D, P, L, K, V, q)
    o16, o32 = _run(w, cache, lens, q)
    assert np.array_equal(o16, np.repeat(row[:, 0], Hq // H, axis=1))
    # 3) q = 0 gives uniform weights: the mean of V
    V = f32_to_bf16_bits(rng.standard_normal((B, L, H, D)).astype(np.float32))
    w, cache, lens, kp, vp = _synthetic_cache(B, H, Hq, D, P, L, K, V, q)
    qz = np.zeros_like(q)
    o16, o32 = _run(w, cache, lens, qz)
    mean = np.repeat(oa.bf16_to_f64(V).mean(axis=1), Hq // H, axis=1)
    assert np.all(np.abs(o32 - mean) <= 1e-5 * np.abs(mean).max(axis=-1, keepdims=True))


def test_empty_and_short_requests():
    w = make_workload(2, B=4, lens=[0, 1, 15, 16], Hq=4, Hkv=4)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp)
    q = w.q()
    o16, o32 = _run(w, cache, lens, q)
    assert not o16[0].any() and not o32[0].any()
    rows = [(r, h) for r in range(1, 4) for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    check_rows(o16[1:].reshape(-1, w.D), o32[1:].reshape(-1, w.D), ref, "short")
    d16, d32 = _run(w, None, dev(w.seq_lens), q, dense_pages=(dev(kp), dev(vp)))
    assert not d16[0].any()


@pytest.mark.parametrize("B,Hq,Hkv", [(70, 4, 4), (70, 8, 2), (300, 4, 4), (300, 8, 2), (300, 32, 32)])
def test_many_ragged_requests(B, Hq, Hkv):
    """The split kernels number their work from the sequence lengths (a prefix over the requests,
    64 at a time, held in registers up to 256 requests and re-read beyond; directly, one split
    per item, when the items alone fill the resident waves, as 300 x 32 heads do): a batch of
    uneven lengths with empty requests among them still gives every (request, head) row exactly
    its attention, and empty requests zeros."""
    rng = np.random.default_rng(B + Hq)
    lens = rng.integers(0, 200, size=B)
    lens[rng.choice(B, size=B // 7, replace=False)] = 0
    w = make_workload(4, B=B, lens=lens, Hq=Hq, Hkv=Hkv, D=128, n_append=0)
    kp, vp = w.pages(0), w.pages(1)
    cache, lt = build_cache(w, kp, vp)
    q = w.q()
    o16, o32 = _run(w, cache, lt, q)
    assert int(cache.status.item()) == 0
    empty = np.flatnonzero(w.seq_lens == 0)
    assert not o16[empty].any() and not o32[empty].any()
    rows = [(r, h) for r in np.flatnonzero(w.seq_lens > 0).tolist() for h in range(w.Hq)]
    ref = oracle_rows(w, kp, vp, q, rows)
    idx = np.array([r * w.Hq + h for r, h in rows])
    check_rows(o16.reshape(-1, w.D)[idx], o32.reshape(-1, w.D)[idx], ref, f"B={B}")
    d16, d32 = _run(w, None, dev(w.seq_lens), q, dense_pages=(dev(kp), dev(vp)))
    check_rows(d16.reshape(-1, w.D)[idx], d32.reshape(-1, w.D)[idx], ref, f"dense B={B}")
    # the ranked schedule (multi-head kernel; the grouped-query one keeps its splits) over the
    # same uneven batch
    r16, r32 = _run(w, cache, lt, q, pages_per_split=-3)
    assert not r16[empty].any() and not r32[empty].any()
    check_rows(r16.reshape(-1, w.D)[idx], r32.reshape(-1, w.D)[idx], ref, f"pps -3 B={B}")


def test_bad_page_id_sets_status():
    w = make_workload(2, B=1, L=64, Hq=2, Hkv=2)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp)
    table = w.page_table.copy()
    table[0, 1] = 10 ** 6
    out = torch.zeros((1, 2, w.D), dtype=torch.int16, device=DEV)
    kvz.decode_attention(dev(w.q()), cache, dev(table), lens, w.sm_scale, out)
    torch.cuda.synchronize()
    assert int(cache.status.item()) & kvz.kvz.STATUS_BAD_PAGE_ID


def _sampled_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    rs = rng.integers(0, w.B, size=n)
    hs = rng.integers(0, w.Hq, size=n)
    return sorted(set(zip(rs.tolist(), hs.tolist())))


@pytest.mark.parametrize("cfg", [2, 3, 4, 5, 6])
def test_full_size_sampled_rows(cfg, full_workloads):
    """Full shapes, the launch configuration the benchmark times, sampled (request, head) rows."""
    w, kp, vp, cache, lens = full_workloads(cfg)
    q = w.q()
    o16, o32 = _run(w, cache, lens, q)
    assert int(cache.status.item()) == 0
    rows = _sampled_rows(w, 24, cfg)
    ref = oracle_rows(w, kp, vp, q, rows)
    idx = tuple(np.array(rows).T)
    check_rows(o16[idx], o32[idx], ref, f"cfg{cfg} full compressed")
    assert np.isfinite(o32).all()
    if cfg in (3, 5):   # these launches take the multi-head kernel's ranked schedule
        ws = torch.empty(kvz.workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages), dtype=torch.uint8, device=DEV)
        kvz.decode_attention_splits(dev(q), cache, dev(w.page_table), lens, w.sm_scale, ws)
        assert kvz.chosen_pages_per_split(ws, w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages) < 0
    d16, d32 = _run(w, None, dev(w.seq_lens), q, dense_pages=(dev(kp), dev(vp)))
    check_rows(d16[idx], d32[idx], ref, f"cfg{cfg} full dense")


def test_two_phase_calls_equal_the_one_call():
    w = make_workload(4, **SMALL[4])
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp)
    q = dev(w.q())
    o16, o32 = _run(w, cache, lens, w.q())
    ws = torch.empty(kvz.workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages), dtype=torch.uint8, device=DEV)
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.zeros((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
    kvz.decode_attention_splits(q, cache, dev(w.page_table), lens, w.sm_scale, ws)
    kvz.merge_splits(ws, lens, w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages, out, out32)
    torch.cuda.synchronize()
    assert np.array_equal(host16(out), o16) and np.array_equal(out32.cpu().numpy(), o32)


@pytest.mark.parametrize("cfg,fmt", [(2, kvz.FORMAT_ESCAPE), (4, kvz.FORMAT_ESCAPE), (4, kvz.FORMAT_ZIPFUSION)])
def test_prepared_calls_equal_the_one_call(cfg, fmt):
    """A prepared call (buffers checked and marshalled once) gives the one-call result bit for bit,
    and keeps doing so while appends change the lengths in device memory between its calls (it
    reads them at every call), for the compressed path in both formats and the uncompressed
    baseline."""
    kw = dict(SMALL[cfg], **({"lens": [1, 15, 16, 17, 300, 1000]} if cfg == 4 else {}))   # room to append
    w = make_workload(cfg, n_append=0, **kw)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp, fmt=fmt)
    q, table = dev(w.q()), dev(w.page_table)
    kd, vd = dev(kp), dev(vp)
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.zeros((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
    dense_lens = dev(w.seq_lens.astype(np.int32))
    step = kvz.prepare_decode_attention(q, cache, table, lens, w.sm_scale, out, out32)
    dstep = kvz.prepare_decode_attention_dense(q, kd, vd, table, dense_lens, w.sm_scale, out, out32)
    rng = np.random.default_rng(5)
    for it in range(3):
        ref16 = torch.zeros_like(out)
        ref32 = torch.zeros_like(out32)
        kvz.decode_attention(q, cache, table, lens, w.sm_scale, ref16, ref32)
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, ref16) and torch.equal(out32, ref32), it
        kvz.decode_attention_dense(q, kd, vd, table, dense_lens, w.sm_scale, ref16, ref32)
        dstep()
        torch.cuda.synchronize()
        assert torch.equal(out, ref16) and torch.equal(out32, ref32), it
        # one more token per request (its tail row only: the lengths stay within the pages laid out)
        assert ((w.max_pages * w.P - lens.cpu().numpy()) > 0).all()
        kn = torch.from_numpy(rng.integers(0, 1 << 14, size=(w.B, w.Hkv, w.D)).astype(np.int16)).to(DEV)
        kvz.append_token(cache, kn, kn, table, lens)
        torch.cuda.synchronize()
        assert int(cache.status.item()) == 0


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2)])
def test_sequence_longer_than_the_page_table(Hq, Hkv):
    """A length beyond max_pages_per_seq * P sets KVZ_STATUS_SEQ_TOO_LONG and is clamped to the
    pages the table holds: the result is attention over those tokens. Compressed and dense."""
    w = make_workload(2, B=2, lens=[100, 60], Hq=Hq, Hkv=Hkv, n_append=0)
    kp, vp = w.pages(0), w.pages(1)
    cache, _ = build_cache(w, kp, vp)
    table = np.ascontiguousarray(w.page_table[:, :5])          # 5 pages = 80 tokens per request
    lens = dev(w.seq_lens)
    q = w.q()
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.zeros((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, dev(table), lens, w.sm_scale, out, out32)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == kvz.kvz.STATUS_SEQ_TOO_LONG
    assert np.array_equal(lens.cpu().numpy(), w.seq_lens)        # the lengths are not written
    rows = _all_rows(w)
    from oracle import c_oracle
    ref = c_oracle.dense_attention_rows(q, kp, vp, table, np.array([80, 60], np.int32), w.sm_scale, rows)
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, "clamped")
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvz.decode_attention_dense(dev(q), dev(kp), dev(vp), dev(table), lens, w.sm_scale, out, out32, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == kvz.kvz.STATUS_SEQ_TOO_LONG
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, "dense clamped")


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2)])
@pytest.mark.parametrize("fmt", [kvz.FORMAT_ESCAPE, kvz.FORMAT_ZIPFUSION])
def test_cache_of_tails_only(Hq, Hkv, fmt):
    """A cache allocated with no unit slots (no unit array) serves requests shorter than a page:
    attention over their tail rows, appends that do not fill a page, status clear."""
    P, D = 16, 128
    w = make_workload(3, B=3, lens=[5, 0, 13], Hq=Hq, Hkv=Hkv, n_append=0)
    kp, vp = w.pages(0), w.pages(1)
    cache = kvz.Cache.allocate(P, Hkv, D, 0, w.B, esc_capacity=0, device=DEV, fmt=fmt)
    assert cache.units.numel() == 0
    lens = w.seq_lens.copy()
    rows_k = np.zeros((w.B, Hkv, P, D), np.uint16)
    rows_v = np.zeros_like(rows_k)
    for r, L in enumerate(lens):
        rows_k[r], rows_v[r] = kp[w.page_table[r, 0]], vp[w.page_table[r, 0]]
    cache.k_tail.copy_(dev(rows_k))
    cache.v_tail.copy_(dev(rows_v))
    lens_d = dev((lens - 1).clip(0).astype(np.int32))
    table = dev(np.zeros((w.B, 1), np.int32))
    nxt_k = np.stack([rows_k[r][:, max(int(L) - 1, 0)] for r, L in enumerate(lens)])
    nxt_v = np.stack([rows_v[r][:, max(int(L) - 1, 0)] for r, L in enumerate(lens)])
    kvz.append_token(cache, dev(nxt_k), dev(nxt_v), table, lens_d)      # row L-1 of each request again
    torch.cuda.synchronize()
    assert np.array_equal(lens_d.cpu().numpy(), lens.clip(1)) and int(cache.status.item()) == 0
    lens_d = dev(lens.astype(np.int32))
    q = w.q()
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, table, lens_d, w.sm_scale, out, out32)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == 0
    from oracle import c_oracle
    tail_table = np.arange(w.B, dtype=np.int32).reshape(w.B, 1)
    ref = c_oracle.dense_attention_rows(q, rows_k, rows_v, tail_table, lens, w.sm_scale, _all_rows(w))
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, f"tails only, format {fmt}")


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2)])
@pytest.mark.parametrize("pps", [0, 1])
def test_cache_without_unit_slots(Hq, Hkv, pps):
    """num_pages = 0: every full page is a bad id (KVZ_STATUS_BAD_PAGE_ID) and is skipped; each
    split the merge counts still leaves an empty partial, so the result is attention over the
    tail rows alone (one split per page with pages_per_split 1)."""
    P, D = 16, 128
    w = make_workload(2, B=2, lens=[3 * P + 5, 7], Hq=Hq, Hkv=Hkv, n_append=0)
    kp, vp = w.pages(0), w.pages(1)
    cache = kvz.Cache.allocate(P, Hkv, D, 1, w.B, esc_capacity=16, device=DEV)
    cache.num_pages = 0
    rows_k = np.zeros((w.B, Hkv, P, D), np.uint16)
    rows_v = np.zeros_like(rows_k)
    for r, L in enumerate(w.seq_lens):
        pid = w.page_table[r, L // P]
        rows_k[r], rows_v[r] = kp[pid], vp[pid]
    cache.k_tail.copy_(dev(rows_k))
    cache.v_tail.copy_(dev(rows_v))
    q = w.q()
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32 = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    kvz.decode_attention(dev(q), cache, dev(w.page_table), dev(w.seq_lens), w.sm_scale, out, out32,
                         pages_per_split=pps)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == kvz.kvz.STATUS_BAD_PAGE_ID
    from oracle import c_oracle
    tail_table = np.arange(w.B, dtype=np.int32).reshape(w.B, 1)
    ref = c_oracle.dense_attention_rows(q, rows_k, rows_v, tail_table, w.seq_lens % P, w.sm_scale, _all_rows(w))
    check_rows(host16(out).reshape(-1, w.D), out32.cpu().numpy().reshape(-1, w.D), ref, f"tail only, pps {pps}")
