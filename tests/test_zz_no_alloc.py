"""kvz_decode_attention_noalloc: the allocation-free variant of kvz_decode_attention, whose split
partials live in the library's own per-GPU scratch array. Called through the C ABI, it gives the
same bits as kvz_decode_attention with a caller workspace (same kernels, same schedule) on two
calls in a row, the second smaller than the first, allocates no device memory, and refuses a call
that needs more scratch than the array holds, enqueueing nothing."""
import numpy as np
import pytest
import torch

import decode_attention_losslessly_amd as kvz
from kvz_testlib import DEV, build_cache, check_rows, dev, host16, oracle_rows
from synth import make_workload

pytestmark = pytest.mark.gpu


def _both(w, cache, lens, q, pps=0):
    """(noalloc out, out32), (workspace out, out32) for the same call."""
    shape = (w.B, w.Hq, w.D)
    a16, a32 = torch.zeros(shape, dtype=torch.int16, device=DEV), torch.full(shape, float("nan"), device=DEV)
    b16, b32 = torch.zeros_like(a16), torch.full(shape, float("nan"), device=DEV)
    table = dev(w.page_table)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats(DEV).get("allocation.all.allocated", 0)
    kvz.decode_attention_noalloc(q, cache, table, lens, w.sm_scale, a16, a32, pages_per_split=pps)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats(DEV).get("allocation.all.allocated", 0) == before, "the call allocated"
    kvz.decode_attention(q, cache, table, lens, w.sm_scale, b16, b32, pages_per_split=pps)
    torch.cuda.synchronize()
    return (a16, a32), (b16, b32)


@pytest.mark.parametrize("first,second", [
    (dict(cfg=3, B=3, L=161, Hq=8, Hkv=8), dict(cfg=2, B=2, L=70, Hq=4, Hkv=4)),
    (dict(cfg=4, B=5, lens=[1, 16, 33, 150, 47], Hq=28, Hkv=4), dict(cfg=6, B=2, L=40, Hq=8, Hkv=2)),
    (dict(cfg=5, B=2, L=300, Hq=4, Hkv=4), dict(cfg=5, B=1, L=33, Hq=4, Hkv=4)),
])
def test_noalloc_equals_workspace_call_twice(first, second):
    for args in (first, second):
        a = dict(args)
        w = make_workload(a.pop("cfg"), D=128, n_append=0, **a)
        kp, vp = w.pages(0), w.pages(1)
        cache, lens = build_cache(w, kp, vp)
        q = dev(w.q())
        (a16, a32), (b16, b32) = _both(w, cache, lens, q)
        assert int(cache.status.item()) == 0
        assert torch.equal(a16, b16), w.name
        assert torch.equal(a32.view(torch.int32), b32.view(torch.int32)), w.name
        rows = [(r, h) for r in range(w.B) for h in range(w.Hq)]
        ref = oracle_rows(w, kp, vp, w.q(), rows)
        check_rows(host16(a16).reshape(-1, w.D), a32.cpu().numpy().reshape(-1, w.D), ref, f"noalloc {w.name}")


def test_noalloc_ranked_and_fixed_splits():
    w = make_workload(3, B=3, L=400, Hq=4, Hkv=4, n_append=0)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp)
    q = dev(w.q())
    for pps in (-2, 3, 0):
        (a16, a32), (b16, b32) = _both(w, cache, lens, q, pps)
        assert torch.equal(a16, b16) and torch.equal(a32.view(torch.int32), b32.view(torch.int32)), pps


def test_noalloc_refuses_more_than_its_scratch():
    w = make_workload(3, B=8, L=16 * 1024, Hq=32, Hkv=32, n_append=0)
    assert kvz.workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.P, w.max_pages, 1) > kvz.kvz.NOALLOC_SCRATCH_BYTES
    cache = kvz.Cache.allocate(w.P, w.Hkv, w.D, 1, w.B, esc_capacity=16, device=DEV)
    q = torch.zeros((w.B, w.Hq, w.D), dtype=torch.int16, device=DEV)
    out = torch.full((w.B, w.Hq, w.D), 7, dtype=torch.int16, device=DEV)
    with pytest.raises(kvz.KvzError) as e:
        kvz.decode_attention_noalloc(q, cache, dev(w.page_table), dev(w.seq_lens), w.sm_scale, out, pages_per_split=1)
    assert e.value.code == kvz.kvz.KVZ_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7).all()) and int(cache.status.item()) == 0      # nothing was enqueued


def test_noalloc_under_graph_capture():
    """The caller this entry point is for: a decode step captured in a HIP graph. One eager call
    first (the library takes the array's device address there), then the captured call replayed
    three times with eager work between the replays; every replay equals the workspace call."""
    w = make_workload(3, B=3, L=161, Hq=8, Hkv=8, n_append=0)
    kp, vp = w.pages(0), w.pages(1)
    cache, lens = build_cache(w, kp, vp)
    q, table = dev(w.q()), dev(w.page_table)
    shape = (w.B, w.Hq, w.D)
    want16, want32 = torch.zeros(shape, dtype=torch.int16, device=DEV), torch.zeros(shape, device=DEV)
    kvz.decode_attention(q, cache, table, lens, w.sm_scale, want16, want32)
    out16, out32 = torch.zeros_like(want16), torch.zeros_like(want32)
    kvz.decode_attention_noalloc(q, cache, table, lens, w.sm_scale, out16, out32)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            kvz.decode_attention_noalloc(q, cache, table, lens, w.sm_scale, out16, out32)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    other16, other32 = torch.zeros_like(want16), torch.zeros_like(want32)
    for rep in range(3):
        out16.zero_()
        out32.zero_()
        graph.replay()
        kvz.decode_attention_noalloc(q, cache, table, lens, w.sm_scale, other16, other32)   # eager, same array
        torch.cuda.synchronize()
        assert torch.equal(out16, want16) and torch.equal(out32.view(torch.int32), want32.view(torch.int32)), rep
        assert torch.equal(other16, want16), rep
