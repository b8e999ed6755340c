#!/usr/bin/env python3
"""Decode attention over a losslessly compressed BF16 KV cache on one MI355X.

Workload (default): 32 requests x 32 heads (one KV head per query head), head_dim 128, 8192
cached tokens per request plus one appended token (8193), 16-token pages with a shuffled page
table; K and V ~ N(0, 1) times a per-channel log-uniform scale in [0.1, 10]. Synthetic data.

One step = the decode-attention hot path over that batch: the split kernel (compressed blocks
rebuilt in registers, split-K partials) and the merge kernel, which is what the pages time for
attention (ZipFusion summary, §IV.B: attention, fused reconstruction and split merge). Prefill,
the initial compression and the append are set-up (excluded there too, §IV.A) and are reported
as separate fields.

Order: set-up; whole steps for --settle-seconds of wall time while the clocks ramp up (set-up);
--warmup untimed steps; exactly --steps timed steps (the headline `value` and `ms_per_step`);
the split kernel's mean launch duration over --steps launches back to back (`roofline`); the
same for the uncompressed baseline; --rounds rounds of alternated compressed and dense loops
(`interleaved`); cache-flushed launches; the streaming-read ceiling (`read_ceiling`); the CPU
oracle on this host (`cpu_baseline`), whose fp64 outputs check the timed call (`parity`: a
failure exits with status 1; for the other cache formats, fp64 rows from the raw pages); appends.

Prints one JSON line. `python bench.py --gpus N` with N > 1 exits with a message: the library
runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0


def source_digest(kernel_source: str = "attn_mha.hip") -> str:
    """Digest of one attention kernel's sources: its translation unit and the headers it
    includes (the counters in profiles/ stay valid while these are unchanged)."""
    csrc = os.path.join(ROOT, "decode_attention_losslessly_amd", "csrc")
    h = hashlib.sha256()
    seen, todo = set(), [kernel_source]
    while todo:
        f = todo.pop()
        if f in seen or not os.path.exists(os.path.join(csrc, f)):
            continue
        seen.add(f)
        text = open(os.path.join(csrc, f), "rb").read()
        todo += [ln.split(b'"')[1].decode() for ln in text.splitlines() if ln.startswith(b'#include "')]
    for f in sorted(seen):
        h.update(f.encode() + open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the first ~30 launches after set-up run up to 20 % slower while the clocks settle
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=3, help="workload number (3 = the headline workload)")
    ap.add_argument("--format", choices=["escape", "zipfusion", "channel"], default="escape",
                    help="cache format: exponent offsets with escapes (the library's), ZipFusion's blocks, or "
                         "the first with channel groups (4 dims over a tile's 16 tokens per base)")
    ap.add_argument("--pages-per-split", type=int, default=0,
                    help="pages per split-K work item (0: the library's choice)")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch size")
    ap.add_argument("--context", type=int, default=None, help="override the workload's context length")
    ap.add_argument("--q-heads", type=int, default=None, help="override the workload's query heads")
    ap.add_argument("--kv-heads", type=int, default=None, help="override the workload's KV heads")
    ap.add_argument("--head-dim", type=int, default=None, help="override the workload's head dim (64 or 128)")
    ap.add_argument("--page-size", type=int, default=None, help="override the workload's page size (a multiple of 16)")
    ap.add_argument("--no-dense", action="store_true", help="skip the uncompressed baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-requests", type=int, default=32, help="requests in the CPU baseline sample")
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="wall seconds of whole steps run before the warm-up, while the clocks ramp up (set-up)")
    ap.add_argument("--rounds", type=int, default=3,
                    help="rounds of alternated compressed / dense whole-step loops of --steps steps each")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling kernel")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra launches timed after a 1 GiB cache flush each (reported as attn_us.cold_median)")
    ap.add_argument("--graph-layers", type=int, default=0, metavar="N",
                    help="also time N layers of attention (N copies of the cache) launched eagerly and "
                         "replayed as one HIP graph")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 5 times (calibrates HBM byte counters) and exit")
    return ap.parse_args()


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path", file=sys.stderr, flush=True)
        return 2

    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    if args.copy_probe:
        a = torch.ones(args.copy_probe << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": a.numel(), "launches": 5}), flush=True)
        return 0

    import decode_attention_losslessly_amd as kvz
    from synth import make_workload

    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if a.dtype == np.uint16 else a.dtype)).to(dev)

    w = make_workload(args.config, B=args.batch, L=args.context, Hq=args.q_heads, Hkv=args.kv_heads, D=args.head_dim,
                      P=args.page_size)
    if any(a is not None for a in (args.batch, args.context, args.q_heads, args.kv_heads, args.head_dim,
                                   args.page_size)):
        w.name = f"{w.name}@b{w.B}_ctx{int(w.seq_lens.max())}_h{w.Hq}x{w.Hkv}_d{w.D}_p{w.P}"
    B, Hq, H, D, P = w.B, w.Hq, w.Hkv, w.D, w.P
    t0 = time.perf_counter()
    kp, vp = w.pages(0), w.pages(1)
    log(f"workload {w.name}: {w.num_pages} pages generated in {time.perf_counter() - t0:.1f}s")

    # ---- set-up: dense pages on the device, compression of the full pages, tails, append
    L = w.seq_lens.astype(np.int64)
    L0 = (w.seq_lens - w.n_append).astype(np.int32)
    kd, vd = t16(kp), t16(vp)
    ids = np.array([w.page_table[r, i] for r in range(B) for i in range(int(L0[r]) // P)], np.int32)
    n_units = len(ids) * H
    fmt = {"escape": kvz.FORMAT_ESCAPE, "zipfusion": kvz.FORMAT_ZIPFUSION, "channel": kvz.FORMAT_CHANNEL}[args.format]
    if fmt != kvz.FORMAT_ESCAPE:
        w.name = f"{w.name}+{args.format}"
    if fmt == kvz.FORMAT_ZIPFUSION:
        pool_cap = (n_units + B * H) * 2 * P * D          # room for every block raw
    else:
        frac = 0.6 if w.k_dist == "log_uniform" else 0.02
        pool_cap = int(n_units * 2 * P * D * frac) + (1 << 20)
    cache = kvz.Cache.allocate(P, H, D, w.num_pages, B, pool_cap, device=dev, fmt=fmt)
    ids_d = t16(ids)
    torch.cuda.synchronize()
    kd_sel, vd_sel = kd[ids_d.long()], vd[ids_d.long()]
    torch.cuda.synchronize()
    # one unit first, so that the timed call does not carry the kernel's first-launch cost (the
    # timed call compresses that unit again, into the same slot)
    kvz.compress_pages(cache, kd_sel[:1].contiguous(), vd_sel[:1].contiguous(), ids_d[:1].contiguous())
    torch.cuda.synchronize()
    ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ce0.record()
    kvz.compress_pages(cache, kd_sel, vd_sel, ids_d)
    ce1.record()
    torch.cuda.synchronize()
    compress_s = ce0.elapsed_time(ce1) * 1e-3
    del kd_sel, vd_sel
    tk = np.zeros((B, H, P, D), np.uint16)
    tv = np.zeros_like(tk)
    for r in range(B):
        if L0[r] % P:
            tk[r], tv[r] = kp[w.page_table[r, L0[r] // P]], vp[w.page_table[r, L0[r] // P]]
    cache.k_tail.copy_(t16(tk))
    cache.v_tail.copy_(t16(tv))
    lens = t16(L0)
    table = t16(w.page_table)
    if w.n_append:
        kvz.append_token(cache, t16(w.appended(0)), t16(w.appended(1)), table, lens)   # advances the lengths
        torch.cuda.synchronize()
    assert np.array_equal(lens.cpu().numpy(), w.seq_lens), "append did not advance the lengths"
    status = int(cache.status.item())
    assert status == 0, f"cache status {status}"
    q = t16(w.q())
    log(f"compressed {n_units} units in {compress_s * 1e3:.1f} ms")

    # ---- algorithmic bytes of one split-kernel launch
    U = kvz.unit_bytes(P, D, fmt)
    full = (w.seq_lens // P).astype(np.int64)
    live = np.array([w.page_table[r, i] for r in range(B) for i in range(int(full[r]))], np.int64)
    if fmt == kvz.FORMAT_ZIPFUSION:
        # pool elements read = raw blocks of the live units (512 values each)
        nb = 2 * (P // 16) * (D // 32)
        metas = cache.units[:, :, :nb][torch.from_numpy(live).to(dev)]
        n_raw = int((metas == 0xFF).sum().item())
        pool_esc = n_raw * 512
        raw_frac = n_raw / max(1, metas.numel())
    else:
        G = D // 64
        hdr = 2 * P * G
        heads = cache.units[:, :, hdr:hdr + 16][torch.from_numpy(live).to(dev)].contiguous()
        cnt = heads[:, :, :8].view(torch.int32).to(torch.int64).sum(-1)
        off = heads[:, :, 8:16].view(torch.int64).squeeze(-1)
        pool_esc = int(torch.where(off != -1, cnt, torch.zeros_like(cnt)).sum().item())
        raw_frac = None
    S = kvz.num_splits(B, Hq, H, D, P, w.max_pages, args.pages_per_split)   # split slots per row
    units_bytes = int(full.sum()) * H * U
    tail_bytes = int((w.seq_lens % P).sum()) * H * D * 2 * 2
    dense_kv_bytes = int(L.sum()) * H * D * 2 * 2

    def partial_bytes(C, pages):
        # (m, l, acc) written per (request, query head, split): at C pages per split, or -C
        # chunks per row when the kernel used the ranked schedule (C < 0)
        if C < 0:
            return len(pages) * Hq * (-C) * (D + 2) * 4, -C
        splits = np.where(pages > 0, (pages + C - 1) // C, 1)
        return int(splits.sum()) * Hq * (D + 2) * 4, int(splits.max())

    pps = args.pages_per_split
    ws = torch.empty(kvz.workspace_bytes(B, Hq, H, D, P, w.max_pages, pps), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.int16, device=dev)

    def pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed_steps(split_fn, merge_fn, steps):
        """`steps` whole steps (split kernel then merge) launched back to back, bracketed by a
        device synchronisation on both sides: wall seconds, and GPU microseconds per step from
        one event pair on the launch stream."""
        g0, g1 = pair()
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        g0.record()
        for _ in range(steps):
            split_fn()
            merge_fn()
        g1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - s0, g0.elapsed_time(g1) * 1e3 / steps

    def launch_stats(split_fn, merge_fn, steps):
        """(1) `steps` split launches back to back under one event pair: the split kernel's mean
        launch duration; (2) an event pair around each split and each merge launch, for their
        spread (each pair adds a few microseconds of its own, which (1) does not carry)."""
        a0, a1 = pair()
        a0.record()
        for _ in range(steps):
            split_fn()
        a1.record()
        torch.cuda.synchronize()
        split_mean_us = a0.elapsed_time(a1) * 1e3 / steps
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1, e2 in ev:
            e0.record()
            split_fn()
            e1.record()
            merge_fn()
            e2.record()
        torch.cuda.synchronize()
        attn = np.array([a.elapsed_time(b) for a, b, _ in ev]) * 1e3
        merge = np.array([b.elapsed_time(c) for _, b, c in ev]) * 1e3
        return split_mean_us, attn, merge

    def settle(split_fn, merge_fn, seconds):
        """Keeps the device busy with whole steps for `seconds` of wall time: the clocks ramp up
        over the first tens of milliseconds of work after an idle set-up, and steps timed before
        they settle run up to 20% slower. Part of the set-up, like the compression; returns the
        steps it ran."""
        n, s0 = 0, time.perf_counter()
        while time.perf_counter() - s0 < seconds:
            for _ in range(10):
                split_fn()
                merge_fn()
            torch.cuda.synchronize()
            n += 10
        return n

    # the two paths as prepared calls (arguments checked and marshalled once), so that a short step
    # is not paced by Python: the split kernel and the merge, on the current stream
    c_step = kvz.prepare_decode_attention(q, cache, table, lens, w.sm_scale, out, workspace=ws, pages_per_split=pps)
    d_step = kvz.prepare_decode_attention_dense(q, kd, vd, table, lens, w.sm_scale, out, workspace=ws,
                                                pages_per_split=pps)
    c_split, c_merge = c_step.splits, c_step.merge
    d_split, d_merge = d_step.splits, d_step.merge
    settle_steps = settle(c_split, c_merge, args.settle_seconds)
    # the headline: W warm-up steps, then exactly K timed steps of the compressed path
    for _ in range(args.warmup):
        c_split()
        c_merge()
    wall, step_gpu_us = timed_steps(c_split, c_merge, args.steps)
    ms_per_step = wall / args.steps * 1e3
    # the split size the kernel chose for this batch (in pages, or in 16-token tiles when it
    # counted tiles), and the bytes that follow from it: page-table entries, q and the partials
    C_used, tpp_used = kvz.chosen_split(ws, B, Hq, H, D, P, w.max_pages, pps)
    part_bytes, splits_used = partial_bytes(C_used, full * tpp_used)
    small_bytes = int(full.sum()) * H * 4 + B * Hq * D * 2 + part_bytes
    comp_bytes = units_bytes + 2 * pool_esc + tail_bytes + small_bytes
    split_mean_us, attn_us, merge_us = launch_stats(c_split, c_merge, args.steps)
    assert int(cache.status.item()) == 0

    # the output of the timed call, with its fp32 copy, for the parity check against the oracle
    out_bf16 = out.clone()
    out32 = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    kvz.decode_attention(q, cache, table, lens, w.sm_scale, out, out32, workspace=ws, pages_per_split=pps)
    torch.cuda.synchronize()
    same_bits = bool(torch.equal(out, out_bf16))

    dense = None
    if not args.no_dense:
        for _ in range(args.warmup):
            d_split()
            d_merge()
        dwall, dstep_gpu = timed_steps(d_split, d_merge, args.steps)
        dC = kvz.chosen_pages_per_split(ws, B, Hq, H, D, P, w.max_pages, pps)
        dpages = (L + P - 1) // P
        dense_bytes = dense_kv_bytes + int(dpages.sum()) * H * 4 + B * Hq * D * 2 + partial_bytes(dC, dpages)[0]
        dsplit_mean, dattn, dmerge = launch_stats(d_split, d_merge, args.steps)
        dense = dict(ms_per_step=dwall / args.steps * 1e3, step_gpu_us=round(dstep_gpu, 2),
                     attn_us=float(np.median(dattn)), attn_us_mean=dsplit_mean, merge_us=float(np.median(dmerge)),
                     bytes=dense_bytes, gbps=dense_bytes / (dsplit_mean * 1e-6) / 1e9,
                     pct_peak=100 * dense_bytes / (dsplit_mean * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                     tokens_per_s=B / (dwall / args.steps))

    # compressed and dense whole-step loops alternated, K steps each, after all of the above:
    # neither path's figure can carry a clock ramp or another transient alone
    inter = None
    if dense is not None and args.rounds > 0:
        cw, dw = [], []
        for _ in range(args.rounds):
            cw.append(timed_steps(c_split, c_merge, args.steps)[0] / args.steps * 1e3)
            dw.append(timed_steps(d_split, d_merge, args.steps)[0] / args.steps * 1e3)
        inter = {"rounds": args.rounds, "ms_per_step_median": round(float(np.median(cw)), 4),
                 "dense_ms_per_step_median": round(float(np.median(dw)), 4),
                 "speedup_vs_dense_median": round(float(np.median(np.array(dw) / np.array(cw))), 4)}

    # same kernel with the caches flushed before every launch (the pages clear L2, §IV.B)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(args.cold_steps):
        flush.zero_()
        e0, e1 = pair()
        e0.record()
        c_split()
        e1.record()
        c_merge()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    cold = np.array(cold) if cold else np.array([np.nan])
    del flush

    ceiling = None
    if fmt != kvz.FORMAT_ZIPFUSION and not args.no_ceiling:   # the channel format's units read alike
        ceiling = read_ceiling(kvz, cache, table, lens, full, H, U, args.steps, dev, pair)

    layers = layer_loop(kvz, cache, q, table, lens, w, ws, pps, args.graph_layers, dev) if args.graph_layers > 0 else None

    attn_mean = split_mean_us   # mean launch duration of the split kernel, back to back
    achieved = comp_bytes / (attn_mean * 1e-6) / 1e9
    traffic = None
    mha = Hq == H or D != 128   # grouped queries at head dim 64 run on the multi-head kernels
    ksrc = "attn_zf.hip" if fmt == kvz.FORMAT_ZIPFUSION else ("attn_mha.hip" if mha else "attn_gqa.hip")
    tfile = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if os.path.exists(tfile):
        t = json.load(open(tfile))
        if t.get("source_digest") == source_digest(ksrc):
            traffic = t.get("bytes_per_launch")
    if fmt == kvz.FORMAT_ZIPFUSION:
        kname = f"attn_zf_kernel<{D}>" if mha else "attn_zf_gqa_kernel"
    else:
        ch = "true" if fmt == kvz.FORMAT_CHANNEL else "false"
        kname = f"attn_mha_kernel<{D}, {ch}>" if mha else f"attn_gqa_kernel<{ch}>"
    roofline = dict(kernel=kname, bound="hbm",
                    achieved=round(achieved, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBPS, 4), traffic=traffic,
                    algorithmic_bytes_per_launch=comp_bytes, attn_us_mean=round(attn_mean, 2))
    if ceiling is not None:
        ceiling["pct_of_read_ceiling"] = round(100 * achieved / ceiling["gbps"], 2)

    cpu = parity = None
    if not args.no_cpu and fmt == kvz.FORMAT_ESCAPE:   # the CPU oracle baseline decodes the library's format
        cpu, ref_rows, ref = cpu_baseline(w, kp, vp, min(args.cpu_requests, B), units_bytes, pool_esc, tail_bytes, log)
        parity = parity_check(out_bf16.cpu().numpy().view(np.uint16), out32.cpu().numpy(), ref_rows, ref, same_bits,
                              score_bound_of(w, kp, vp, ref_rows))
        log(f"parity: {parity}")
    elif not args.no_cpu:
        # the other formats: no CPU baseline of their own (the oracle's timed decode is the first
        # format's), but the timed call is still checked against fp64 rows from the raw pages
        from oracle import c_oracle
        ref_rows = [(r, h) for r in range(min(args.cpu_requests, B)) for h in range(Hq)]
        ref = c_oracle.dense_attention_rows(w.q(), kp, vp, w.page_table, w.seq_lens, w.sm_scale, ref_rows)
        parity = parity_check(out_bf16.cpu().numpy().view(np.uint16), out32.cpu().numpy(), ref_rows, ref, same_bits,
                              score_bound_of(w, kp, vp, ref_rows))
        log(f"parity: {parity}")

    # Appends in steady state, after everything else (they overwrite the tails): up to one page
    # of tokens, each call timed alone; a call in which some request's tail fills compresses
    # that page, so those calls are reported apart.
    append_us = append_fill_us = None
    lens2 = lens.clone()
    lh = lens2.cpu().numpy().astype(np.int64)
    kz = torch.zeros((B, H, D), dtype=torch.int16, device=dev)
    nofill, fill = [], []
    for _ in range(P):
        if np.any(lh + 1 > w.max_pages * P):
            break
        fills = bool(np.any(lh % P == P - 1))
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        kvz.append_token(cache, kz, kz, table, lens2)
        a1.record()
        torch.cuda.synchronize()
        (fill if fills else nofill).append(a0.elapsed_time(a1) * 1e3)
        lh += 1
    if nofill:
        append_us = float(np.median(nofill))
    if fill:
        append_fill_us = float(np.median(fill))
    # the same number of calls back to back through a prepared call, as a decode loop issues them
    # (every request's tail fills once among P calls, so the mean includes that request's page
    # compression)
    append_steady_us = None
    n_app = 0
    lens2.copy_(lens)   # from the same lengths again (the tails and units hold zeros by now)
    lh = lens2.cpu().numpy().astype(np.int64)
    for _ in range(P):
        if np.any(lh + 1 > w.max_pages * P):
            break
        lh += 1
        n_app += 1
    if n_app:
        app = kvz.prepare_append_token(cache, kz, kz, table, lens2)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(n_app):
            app()
        a1.record()
        torch.cuda.synchronize()
        append_steady_us = a0.elapsed_time(a1) * 1e3 / n_app

    res = {
        "metric": "decode-attn tokens/s + compressed HBM GB/s (% peak), 8K ctx batch 32",
        "value": round(B / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": H, "head_dim": D,
                   "context": int(w.seq_lens.max()), "page_size": P, "splits": splits_used,
                   "schedule": "ranked" if C_used < 0 else "split",
                   "pages_per_split": C_used if C_used > 0 and tpp_used == 1 else None,
                   "tiles_per_split": C_used if C_used > 0 and tpp_used > 1 else None,
                   "parallelism": "none (1 GPU)"},
        "compressed_gbps": round(achieved, 1),
        "pct_peak_hbm": round(100 * achieved / PEAK_HBM_GBPS, 2),
        "uncompressed_equiv_gbps": round(dense_kv_bytes / (attn_mean * 1e-6) / 1e9, 1),
        "step_gpu_us": round(step_gpu_us, 2),
        "settle_steps": settle_steps,
        "interleaved": inter,
        "read_ceiling": ceiling,
        "parity": parity,
        "attn_us": {"mean": round(attn_mean, 2), "median": round(float(np.median(attn_us)), 2),
                    "p10": round(float(np.percentile(attn_us, 10)), 2),
                    "p90": round(float(np.percentile(attn_us, 90)), 2), "cold_median": round(float(np.median(cold)), 2) if args.cold_steps else None},
        "merge_us": round(float(np.median(merge_us)), 2),
        "compressed_bytes": comp_bytes,
        "dense_kv_bytes": dense_kv_bytes,
        "compression_ratio": round((units_bytes + 2 * pool_esc + tail_bytes) / dense_kv_bytes, 4),
        "format": args.format,
        "pool_escapes": pool_esc,
        "raw_block_fraction": raw_frac,
        "dense": dense,
        "speedup_vs_dense": round(dense["ms_per_step"] / ms_per_step, 4) if dense else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "layers": layers,
        "append_us": round(append_us, 1) if append_us is not None else None,
        "append_fill_us": round(append_fill_us, 1) if append_fill_us is not None else None,
        "append_steady_us": round(append_steady_us, 2) if append_steady_us is not None else None,
        "compress_gbps_dense_input": round(len(ids) * H * P * D * 4 / compress_s / 1e9, 1),
        "gpu": f"{torch.cuda.get_device_name(0)} ({torch.cuda.get_device_properties(0).gcnArchName})",
        "software": {"torch": torch.__version__, "hip": torch.version.hip},
        "source_digest": source_digest(ksrc),
    }
    print(json.dumps(res), flush=True)
    if parity is not None and not parity["ok"]:
        log("parity check against the oracle FAILED")
        return 1
    return 0


def read_ceiling(kvz, cache, table, lens, full, H, U, steps, dev, pair):
    """The streaming-read ceiling (kvzb_read_units): the same unit bytes and page-table entries,
    read in the attention kernels' pattern, with 1, 2, 4, 8 and 16 waves per SIMD of the device
    (the kernel keeps up to 8 resident); the best rate is the ceiling."""
    import numpy as np
    import torch

    from decode_attention_losslessly_amd import kvz_bench
    if U > 16384 or U % 16:
        return None   # the read kernel holds a whole unit in registers: at most 16 KB
    B = int(lens.numel())
    rows = B * H
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes = int(full.sum()) * H * (U + 4)
    best = None
    for waves_per_simd in (1, 2, 4, 8, 16):
        chunks = max(1, round(waves_per_simd * 4 * cus / rows))
        sink = torch.empty(rows * chunks * 64, dtype=torch.int32, device=dev)
        fn = lambda: kvz_bench.read_units(cache, table, lens, chunks, sink)
        for _ in range(5):
            fn()
        e0, e1 = pair()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        gbps = nbytes / (us * 1e-6) / 1e9
        if best is None or gbps > best["gbps"]:
            best = {"gbps": round(gbps, 1), "us": round(us, 2), "chunks_per_row": chunks,
                    "waves": rows * chunks, "bytes": nbytes}
    best["pct_peak"] = round(100 * best["gbps"] / PEAK_HBM_GBPS, 2)
    return best


def parity_check(out16, out32, rows, ref, same_bits, bound_of=None):
    """The timed call's output against this run's oracle rows (the CPU baseline's): BF16 within
    max(2e-2, 2^-7 |o|) + 1e-4 max_d |o| per element (the row's fp32 budget: a rounded fp32
    result is no closer to o than the fp32 result), fp32 within 1e-4 max_d |o| per row. A row
    that misses them may pass within those bounds plus its first-order score-rounding bound
    (bound_of(i); rows whose top logits nearly tie at a large scale): counted apart."""
    import numpy as np
    idx = tuple(np.array(rows).T)
    got16 = (out16[idx].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got32 = out32[idx].astype(np.float64)
    err16 = np.abs(got16 - ref)
    nrm = np.abs(ref).max(axis=-1)
    tol16 = np.maximum(2e-2, 2.0 ** -7 * np.abs(ref)) + 1e-4 * nrm[:, None]
    e32 = np.abs(got32 - ref).max(axis=-1)
    miss = (err16 > tol16).any(axis=-1) | (e32 > 1e-4 * nrm)
    n_bound = 0
    if bound_of is not None:
        for i in np.flatnonzero(miss):
            e = bound_of(int(i))
            if (err16[i] <= tol16[i] + e).all() and e32[i] <= 1e-4 * nrm[i] + e:
                miss[i] = False
                n_bound += 1
    ok16 = bool(not ((err16 > tol16) & miss[:, None]).any())
    ok32 = bool(not (miss & (e32 > 1e-4 * nrm)).any())
    rel = e32 / np.where(nrm > 0, nrm, 1.0)
    return {"rows": len(rows), "max_bf16_abs_err": float(err16.max()), "max_f32_normwise_err": float(rel.max()),
            "rows_within_first_order_bound": n_bound, "bf16_ok": ok16, "f32_ok": ok32,
            "timed_output_reproduced": same_bits, "ok": ok16 and ok32 and same_bits}


def score_bound_of(w, kp, vp, rows):
    """bound_of(i) for parity_check: the oracle's first-order score-rounding bound of row i."""
    from oracle import attention as oa
    q, grp = w.q(), w.Hq // w.Hkv

    def bound_of(i):
        r, h = rows[i]
        K, V = oa.gather_dense(kp, vp, w.page_table[r], int(w.seq_lens[r]), w.P)
        return oa.score_rounding_bound(q[r, h], K[:, h // grp], V[:, h // grp], w.sm_scale)
    return bound_of


def layer_loop(kvz, cache, q, table, lens, w, ws, pps, nl, dev, reps=20):
    """One decode step of an nl-layer model's attention: nl calls of decode_attention (split
    kernel + merge), one per layer, each on its own copy of the cache (separate memory, as the
    layers of a model hold). Timed launched one call after another from Python (prepared calls:
    one C call per launch), then captured once as a HIP graph and replayed; the replayed outputs
    must equal the eager ones bit for bit. Launch overhead is what a decode step at batch 1 pays
    per layer."""
    import torch

    caches = [cache] + [kvz.Cache(cache.P, cache.H, cache.D, cache.num_pages, cache.max_batch, cache.units.clone(),
                                  cache.esc_pool.clone(), cache.esc_cursor.clone(), cache.k_tail.clone(),
                                  cache.v_tail.clone(), cache.status.clone(), cache.fmt) for _ in range(nl - 1)]
    B, Hq, D = q.shape
    outs = torch.empty((nl, B, Hq, D), dtype=torch.int16, device=dev)

    def step():
        for i, c in enumerate(caches):
            kvz.decode_attention(q, c, table, lens, w.sm_scale, outs[i], workspace=ws, pages_per_split=pps)

    prepared = [kvz.prepare_decode_attention(q, c, table, lens, w.sm_scale, outs[i], workspace=ws, pages_per_split=pps)
                for i, c in enumerate(caches)]

    def eager_step():   # the same calls, each launched as one prepared C call
        for p in prepared:
            p()

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps / nl

    eager_us = timed(eager_step)
    ref = outs.clone()
    outs.zero_()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph_us = timed(graph.replay)
    assert torch.equal(outs, ref), "graph replay differs from the eager layers"
    assert all(int(c.status.item()) == 0 for c in caches)
    del graph, caches, prepared
    return {"layers": nl, "eager_us_per_layer": round(eager_us, 2), "graph_us_per_layer": round(graph_us, 2),
            "graph_tokens_per_s": round(B / (graph_us * 1e-6), 1)}


def _host_cpu() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, kp, vp, n_req, units_bytes, pool_esc, tail_bytes, log):
    """The C oracle (scalar decode of the compressed units + fp64 attention, OpenMP over rows) on
    the rows of the first n_req requests, timed, and scaled to the whole batch. Returns the
    baseline record, the rows and their fp64 outputs (this run's parity reference)."""
    import numpy as np

    from oracle import c_oracle
    L = w.seq_lens
    full = L // w.P
    reqs = list(range(n_req))
    ids = np.array([w.page_table[r, i] for r in reqs for i in range(int(full[r]))], np.int32)
    t0 = time.perf_counter()
    units_s, pool_s, _ = c_oracle.encode_pages(kp[ids], vp[ids])
    enc_s = time.perf_counter() - t0
    # units indexed by physical id as the oracle expects
    units = np.zeros((w.num_pages, w.Hkv, units_s.shape[2]), np.uint8)
    units[ids] = units_s
    tk = np.zeros((w.B, w.Hkv, w.P, w.D), np.uint16)
    tv = np.zeros_like(tk)
    for r in reqs:
        if L[r] % w.P:
            tk[r], tv[r] = kp[w.page_table[r, L[r] // w.P]], vp[w.page_table[r, L[r] // w.P]]
    rows = [(r, h) for r in reqs for h in range(w.Hq)]
    q = w.q()
    t0 = time.perf_counter()
    ref = c_oracle.decode_attention_rows(q, units, pool_s, w.page_table, L, tk, tv, w.Hkv, w.P, w.sm_scale, rows)
    dt = time.perf_counter() - t0
    threads = c_oracle.num_threads()
    scale = (w.B * w.Hq) / len(rows)
    step_s = dt * scale
    # what the whole batch's call processes: its compressed bytes (units, pool escapes, tail
    # rows) and its context tokens
    comp = units_bytes + 2 * pool_esc + tail_bytes
    log(f"cpu oracle: {len(rows)} rows in {dt:.2f}s on {threads} threads (encode set-up {enc_s:.1f}s)")
    # the same oracle on one core, over the first request's rows
    one = rows[:w.Hq]
    c_oracle.set_num_threads(1)
    t0 = time.perf_counter()
    c_oracle.decode_attention_rows(q, units, pool_s, w.page_table, L, tk, tv, w.Hkv, w.P, w.sm_scale, one)
    dt1 = time.perf_counter() - t0
    c_oracle.set_num_threads(threads)
    step1_s = dt1 * (w.B * w.Hq) / len(one)
    log(f"cpu oracle on 1 core: {len(one)} rows in {dt1:.2f}s")
    rec = {"value": round(w.B / step_s, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{len(rows)} of {w.B * w.Hq} (request, head) rows: scalar decode of their compressed "
                     f"pages + fp64 attention, {dt:.2f}s wall, scaled to the full batch",
           "cpu_seconds": round(dt * threads, 2),
           "kv_tokens_per_s": round(float(L.sum()) / step_s, 1),
           "compressed_gbps": round(comp / step_s / 1e9, 4),
           "one_core": {"value": round(w.B / step1_s, 3), "unit": "tokens/s",
                        "kv_tokens_per_s": round(float(L.sum()) / step1_s, 1),
                        "compressed_gbps": round(comp / step1_s / 1e9, 4),
                        "sample": f"{len(one)} rows of request 0, {dt1:.2f}s, scaled to the full batch"},
           "host_cpu": _host_cpu()}
    return rec, rows, ref

if __name__ == "__main__":
    sys.exit(main())
