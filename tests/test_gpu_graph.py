"""One decode step (append a token to every request, then attention and merge) captured once in
a HIP graph and replayed step after step: every replay gives exactly what the same step gives
run eagerly, including steps whose append fills a page and compresses it; likewise a step over
several layers, each appending to its own cache before its attention. The library launches only
stream work (no allocation, no synchronisation, no memset) and reads sequence lengths from device
memory, so a single captured step serves every later step of a decode loop."""
import numpy as np
import pytest
import torch

import decode_attention_losslessly_amd as kvz
from kvz_testlib import DEV, check_rows, dev, escape_capacity, full_page_ids, host16, oracle_rows, tails
from synth import make_workload

pytestmark = pytest.mark.gpu

N_STEPS = 24


def copy_cache(c: kvz.Cache) -> kvz.Cache:
    return kvz.Cache(c.P, c.H, c.D, c.num_pages, c.max_batch, c.units.clone(), c.esc_pool.clone(),
                     c.esc_cursor.clone(), c.k_tail.clone(), c.v_tail.clone(), c.status.clone(), c.fmt)


def decode_loop_inputs(cfg, Hq, Hkv, lens, n_steps):
    """A cache N tokens short of workload `cfg` at the final lengths lens + n_steps, and the
    tokens the steps append: (w, kp, vp, cache, L0, new_k[step], new_v[step])."""
    w = make_workload(cfg, B=len(lens), lens=np.array(lens) + n_steps, Hq=Hq, Hkv=Hkv, D=128, n_append=0)
    kp, vp = w.pages(0), w.pages(1)
    L0 = (w.seq_lens - n_steps).astype(np.int32)
    ids = full_page_ids(w, L0)
    cache = kvz.Cache.allocate(w.P, w.Hkv, w.D, w.num_pages, w.B, escape_capacity(w, len(w.page_table.ravel()) * w.Hkv),
                               device=DEV)
    kvz.compress_pages(cache, dev(kp[ids]), dev(vp[ids]), dev(ids))
    tk, tv = tails(w, kp, vp, L0)
    cache.k_tail.copy_(dev(tk))
    cache.v_tail.copy_(dev(tv))
    new_k = [dev(np.stack([w.token(r, int(L0[r]) + i, 0) for r in range(w.B)])) for i in range(n_steps)]
    new_v = [dev(np.stack([w.token(r, int(L0[r]) + i, 1) for r in range(w.B)])) for i in range(n_steps)]
    return w, kp, vp, cache, L0, new_k, new_v


# pps -2: the multi-head kernel's ranked schedule (chosen on the device, like the split size)
@pytest.mark.parametrize("cfg,Hq,Hkv,lens,pps", [(3, 4, 4, [100, 37, 250], 0), (3, 4, 4, [100, 37, 250], -2),
                                                 (4, 8, 2, [60, 17, 200], 0)])
def test_replayed_decode_steps_match_eager(cfg, Hq, Hkv, lens, pps):
    # the workload holds the final lengths; the cache starts N_STEPS tokens shorter
    w, kp, vp, cache, L0, new_k, new_v = decode_loop_inputs(cfg, Hq, Hkv, lens, N_STEPS)
    table, q = dev(w.page_table), dev(w.q())
    ws = torch.empty(kvz.workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages, pps), dtype=torch.uint8,
                     device=DEV)
    torch.cuda.synchronize()

    # eager
    ce, le = copy_cache(cache), dev(L0)
    eager = []
    for i in range(N_STEPS):
        out = torch.empty((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
        out32 = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
        kvz.append_token(ce, new_k[i], new_v[i], table, le)
        kvz.decode_attention(q, ce, table, le, w.sm_scale, out, out32, workspace=ws, pages_per_split=pps)
        eager.append((out, out32))
    torch.cuda.synchronize()

    # one captured step, replayed with the next token copied into its static inputs each time
    cg, lg = copy_cache(cache), dev(L0)
    k_in, v_in = torch.empty_like(new_k[0]), torch.empty_like(new_v[0])
    out_g = torch.empty((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out32_g = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
    ws_g = torch.empty_like(ws)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            kvz.append_token(cg, k_in, v_in, table, lg)
            kvz.decode_attention(q, cg, table, lg, w.sm_scale, out_g, out32_g, workspace=ws_g, pages_per_split=pps)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(lg.cpu().numpy(), L0), "capturing must not run the step"
    for i in range(N_STEPS):
        k_in.copy_(new_k[i])
        v_in.copy_(new_v[i])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager[i][0]), f"bf16 output differs at step {i}"
        assert torch.equal(out32_g, eager[i][1]), f"fp32 output differs at step {i}"
    assert np.array_equal(lg.cpu().numpy(), w.seq_lens) and np.array_equal(le.cpu().numpy(), w.seq_lens)
    assert int(cg.status.item()) == 0 and int(ce.status.item()) == 0
    # and the last step is the attention of the full workload
    rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
    o = oracle_rows(w, kp, vp, w.q(), rows)
    check_rows(host16(out_g).reshape(-1, w.D), out32_g.cpu().numpy().reshape(-1, w.D), o, "graph replay")


@pytest.mark.parametrize("cfgs,Hq,Hkv", [((2, 3, 5), 4, 4), ((4, 3, 5), 8, 2)])
def test_layers_in_one_graph(cfgs, Hq, Hkv):
    """A decode step over several layers, each with its own cache, page table and queries (here
    the workloads of different configurations at one shape, so the layers differ in their
    escapes and pool use), captured as one graph. Every replay, with other eager work in between,
    equals the eager layers bit for bit, and the layers match the oracle."""
    from kvz_testlib import build_cache
    lens = [100, 37, 250]
    layers = []
    for c in cfgs:
        w = make_workload(c, B=len(lens), lens=np.array(lens), Hq=Hq, Hkv=Hkv, D=128, n_append=0)
        kp, vp = w.pages(0), w.pages(1)
        cache, lt = build_cache(w, kp, vp)
        layers.append((w, kp, vp, cache, lt, dev(w.page_table), dev(w.q())))
    w0 = layers[0][0]
    ws = torch.empty(kvz.workspace_bytes(w0.B, Hq, Hkv, 128, w0.P, w0.max_pages), dtype=torch.uint8, device=DEV)
    nl = len(layers)
    out = torch.empty((nl, w0.B, Hq, 128), dtype=torch.int16, device=DEV)
    out32 = torch.empty((nl, w0.B, Hq, 128), dtype=torch.float32, device=DEV)

    def step(o, o32):
        for i, (w, _, _, cache, lt, table, q) in enumerate(layers):
            kvz.decode_attention(q, cache, table, lt, w.sm_scale, o[i], o32[i], workspace=ws)

    eo, eo32 = torch.empty_like(out), torch.empty_like(out32)
    step(eo, eo32)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(out, out32)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    scratch_o, scratch_o32 = torch.empty_like(out), torch.empty_like(out32)
    for rep in range(3):
        out.zero_()
        out32.zero_()
        graph.replay()
        step(scratch_o, scratch_o32)     # eager work between replays, on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(out, eo) and torch.equal(out32, eo32), f"replay {rep} differs from the eager layers"
    for i, (w, kp, vp, cache, _, _, _) in enumerate(layers):
        assert int(cache.status.item()) == 0
        rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
        o = oracle_rows(w, kp, vp, w.q(), rows)
        check_rows(host16(eo[i]).reshape(-1, w.D), eo32[i].cpu().numpy().reshape(-1, w.D), o, f"layer {i} (config {cfgs[i]})")


@pytest.mark.parametrize("cfgs,Hq,Hkv", [((2, 3, 5), 4, 4), ((4, 3, 5), 8, 2)])
def test_layers_with_append_in_one_graph(cfgs, Hq, Hkv):
    """The real decode step: every layer appends the new token to its own cache (its own tails
    and lengths) and then attends, all layers captured as one graph, which is replayed step after
    step across page fills (with eager work between replays). Every replay equals the same step
    run eagerly on copies of the caches, bit for bit, and the last step of every layer matches
    the oracle."""
    n_steps = 20
    lens = [100, 37, 250]      # 100 + 12 and 250 + 6 fill a 16-token page during the loop
    layers = [decode_loop_inputs(c, Hq, Hkv, lens, n_steps) for c in cfgs]
    w0 = layers[0][0]
    ws = torch.empty(kvz.workspace_bytes(w0.B, Hq, Hkv, 128, w0.P, w0.max_pages), dtype=torch.uint8, device=DEV)
    tables = [dev(L[0].page_table) for L in layers]
    qs = [dev(L[0].q()) for L in layers]
    nl = len(layers)

    def make_state():
        return [copy_cache(L[3]) for L in layers], [dev(L[4]) for L in layers]

    def step(caches, lts, ks, vs, o, o32):
        for i, (w, *_rest) in enumerate(layers):
            kvz.append_token(caches[i], ks[i], vs[i], tables[i], lts[i])
            kvz.decode_attention(qs[i], caches[i], tables[i], lts[i], w.sm_scale, o[i], o32[i], workspace=ws)

    shape = (nl, w0.B, Hq, 128)
    ce, le = make_state()
    eager = []
    for t in range(n_steps):
        eo, eo32 = torch.empty(shape, dtype=torch.int16, device=DEV), torch.empty(shape, dtype=torch.float32, device=DEV)
        step(ce, le, [L[5][t] for L in layers], [L[6][t] for L in layers], eo, eo32)
        eager.append((eo, eo32))
    torch.cuda.synchronize()

    cg, lg = make_state()
    k_in = [torch.empty_like(L[5][0]) for L in layers]
    v_in = [torch.empty_like(L[6][0]) for L in layers]
    out, out32 = torch.empty(shape, dtype=torch.int16, device=DEV), torch.empty(shape, dtype=torch.float32, device=DEV)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(cg, lg, k_in, v_in, out, out32)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert all(np.array_equal(l.cpu().numpy(), L[4]) for l, L in zip(lg, layers)), "capturing must not run the step"
    scratch = torch.empty_like(out32)
    for t in range(n_steps):
        for i, L in enumerate(layers):
            k_in[i].copy_(L[5][t])
            v_in[i].copy_(L[6][t])
        graph.replay()
        scratch.copy_(out32).mul_(2.0)      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager[t][0]) and torch.equal(out32, eager[t][1]), f"step {t} differs from eager"
    for i, (w, kp, vp, *_rest) in enumerate(layers):
        assert np.array_equal(lg[i].cpu().numpy(), w.seq_lens)
        assert int(cg[i].status.item()) == 0 and int(ce[i].status.item()) == 0
        rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
        o = oracle_rows(w, kp, vp, w.q(), rows)
        check_rows(host16(out[i]).reshape(-1, w.D), out32[i].cpu().numpy().reshape(-1, w.D), o,
                   f"layer {i} (config {cfgs[i]}) after {n_steps} steps")
