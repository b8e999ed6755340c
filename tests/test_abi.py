"""The C ABI library loads, exports every entry point include/kvz.h declares, and its host-side
size and argument checks agree with the format and with the oracle. No device work is done."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (one HIP runtime for torch and libkvz)

import decode_attention_losslessly_amd as kvz
from decode_attention_losslessly_amd import kvz as binding
from oracle import codec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvz.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvz_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 10
    L = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(binding.EXPORTS) == set(names)


def test_bench_library_exports_every_declared_symbol():
    from decode_attention_losslessly_amd import kvz_bench
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "kvz_bench.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(kvzb_[a-z_0-9]+)\s*\(", text)))
    assert names and set(kvz_bench.EXPORTS) == set(names)
    L = ctypes.CDLL(kvz_bench.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    # argument checks come before any device work
    assert kvz_bench.lib().kvzb_read_units(None, 1, 6272, None, 1, None, 1, 1, 16, 1, None, None) == \
        binding.KVZ_ERR_INVALID_ARG


# the calls the hot path's boundary is built from: sizes, compress, append, attention over the
# compressed cache and over the uncompressed baseline, the test decode, error strings
BOUNDARY = ("kvz_payload_bytes", "kvz_meta_bytes", "kvz_workspace_bytes", "kvz_compress_pages", "kvz_append_token",
            "kvz_decode_attention", "kvz_decode_attention_dense", "kvz_decompress_pages", "kvz_strerror")


def test_boundary_calls_are_declared_and_exported():
    names = set(_declared())
    L = ctypes.CDLL(binding.LIB_PATH)
    for n in BOUNDARY:
        assert n in names, n
        assert hasattr(L, n), n


@pytest.mark.parametrize("P,D", [(16, 64), (16, 128), (32, 128), (256, 64), (16, 256)])
def test_sizes_agree_with_format(P, D):
    assert kvz.payload_bytes(P, D) == 3 * P * D // 2          # 12 bits per value
    assert kvz.unit_bytes(P, D) == kvz.meta_bytes(P, D) + 2 * kvz.payload_bytes(P, D)
    assert kvz.unit_bytes(P, D) == codec.unit_bytes(P, D)
    assert kvz.meta_bytes(P, D) == codec.meta_bytes(P, D)
    assert kvz.inline_capacity(P, D) == codec.inline_capacity(P, D)
    # channel groups change which values share a base, not the sizes
    assert kvz.unit_bytes(P, D, kvz.FORMAT_CHANNEL) == kvz.unit_bytes(P, D)


def test_unsupported_shapes_have_zero_size():
    assert kvz.unit_bytes(15, 128) == 0
    assert kvz.unit_bytes(16, 96) == 0
    assert kvz.payload_bytes(16, 96) == 0 and kvz.payload_bytes(8, 128) == 0


def test_split_geometry():
    # the workspace holds (D + 2) floats per (request, query head, split slot), then the
    # 16-byte slot where the split kernel records the split size it chose
    for args in [(32, 32, 32, 128, 16, 513), (1, 32, 32, 128, 16, 256), (64, 28, 4, 128, 16, 512),
                 (4, 32, 32, 128, 16, 2048), (1, 2, 2, 64, 256, 1)]:
        S = kvz.num_splits(*args)
        B, Hq, _, D, _, mp = args
        assert S >= 1
        assert kvz.workspace_bytes(*args) == B * Hq * S * (D + 2) * 4 + 16
        assert kvz.num_splits(*args, pages_per_split=mp) == 1
        assert kvz.num_splits(*args, pages_per_split=1) == mp
    # batch-1 context: enough splits to spread one request over the chip
    assert kvz.num_splits(1, 32, 32, 128, 16, 256) >= 32


def test_tile_split_slots():
    # Pages of several 16-token tiles that give fewer than 2,048 (item, page) waves at the table's
    # full width: the multi-head kernel counts its splits in tiles, each at least the fewest tiles
    # that keep the splits at full width to 2,048 waves, and the workspace holds those slots.
    # Grouped queries at head dim 128, fixed split sizes and batches with pages enough keep
    # whole pages.
    assert kvz.num_splits(1, 2, 2, 64, 256, 1) == 16            # 32 tiles: 1-tile splits
    assert kvz.num_splits(1, 32, 32, 128, 256, 16) == 64        # 8,192 tiles: 4-tile splits, 256 / 4
    assert kvz.num_splits(1, 32, 32, 128, 128, 32) == 64        # 1,024 pages of 8 tiles: 4-tile splits
    assert kvz.num_splits(1, 32, 32, 128, 64, 64) == 64         # 2,048 pages: one page a split
    assert kvz.num_splits(1, 32, 8, 128, 256, 16) == 16         # grouped queries: whole pages
    assert kvz.num_splits(1, 2, 2, 64, 256, 1, pages_per_split=1) == 1
    assert kvz.workspace_bytes(1, 2, 2, 64, 256, 1) == 2 * 16 * (64 + 2) * 4 + 16


def test_ranked_slots_reserved_only_when_usable():
    # Multi-head calls reserve slots for the ranked schedule's chunks (two per big rank, R big
    # ranks from about 4096 waves over the batch's items) only when requests of the table's full
    # width could give big chunks (80% of a row over R) of at least half the ranked minimum of
    # 5 pages; otherwise the workspace, and the grid, hold the split schedule's slots only.
    def split_only(B, Hq, mp):   # the split schedule's slots: C >= ceil(mp / (2 * 4096 / items))
        cap = (2 * 4096 + B * Hq - 1) // (B * Hq)
        c = max(4, (mp + cap - 1) // cap)
        return (mp + c - 1) // c
    # batch 1 x 4K: R = 128, 204.8 pages of big chunks < 320: split slots only
    assert kvz.num_splits(1, 32, 32, 128, 16, 256) == split_only(1, 32, 256) == 64
    # batch 1 x 16K: R = 128, 819.2 >= 320: 2 R = 256 chunk slots
    assert kvz.num_splits(1, 32, 32, 128, 16, 1024) == 256
    # 32 x 8K: R = 4, 8 chunk slots; the split schedule needs 8 as well
    assert kvz.num_splits(32, 32, 32, 128, 16, 513) == 8
    # 4 x 32K: R = 32, 64 chunk slots
    assert kvz.num_splits(4, 32, 32, 128, 16, 2048) == 64
    # grouped-query calls and fixed split sizes never reserve them
    assert kvz.num_splits(1, 32, 8, 128, 16, 1024) == split_only(1, 8, 1024)
    assert kvz.num_splits(1, 32, 32, 128, 16, 1024, pages_per_split=4) == 256
    # a negative split size forces -pps big ranks: 2 chunks each
    assert kvz.num_splits(1, 32, 32, 128, 16, 256, pages_per_split=-3) == max(6, split_only(1, 32, 256))


def test_invalid_arguments_enqueue_nothing():
    L = binding.lib()
    assert L.kvz_compress_pages(None, None, None, None, 0, None) == binding.KVZ_ERR_INVALID_ARG
    assert L.kvz_decode_attention(None, None, None, 0, None, 0, 1, 1.0, 0, None, None, None, 0, None) == \
        binding.KVZ_ERR_INVALID_ARG
    # shape checks happen before any pointer is used
    rc = L.kvz_decode_attention_dense(None, None, None, 0, 4, 96, 16, None, 0, None, 1, 4, 1.0, 0, None, None, None,
                                      0, None, None)
    assert rc == binding.KVZ_ERR_UNSUPPORTED
    rc = L.kvz_decode_attention_dense(None, None, None, 0, 4, 128, 16, None, 0, None, 1, 6, 1.0, 0, None, None, None,
                                      0, None, None)
    assert rc == binding.KVZ_ERR_UNSUPPORTED       # 6 query heads on 4 KV heads
    rc = L.kvz_decode_attention_dense(None, None, None, 0, 1, 128, 16, None, 0, None, 1, 32, 1.0, 0, None, None,
                                      None, 0, None, None)
    assert rc == binding.KVZ_ERR_INVALID_ARG       # a group of 32 is served; the null pointers are not
    rc = L.kvz_decode_attention_dense(None, None, None, 0, 2, 64, 16, None, 0, None, 1, 8, 1.0, 0, None, None, None,
                                      0, None, None)
    assert rc == binding.KVZ_ERR_INVALID_ARG       # grouped queries at head dim 64 are served too
    assert L.kvz_compact_pool(None, None, 0, None, 0, None, None) == binding.KVZ_ERR_INVALID_ARG
    assert kvz.kvz.strerror(binding.KVZ_ERR_WORKSPACE) == "workspace too small"
    # a page table whose width times P overflows a 32-bit length
    wide = (1 << 31) // 16
    rc = L.kvz_decode_attention_dense(None, None, None, 0, 4, 128, 16, None, wide, None, 1, 4, 1.0, 0, None, None,
                                      None, 0, None, None)
    assert rc == binding.KVZ_ERR_UNSUPPORTED
    fake = 256
    cs = binding._CacheStruct(16, 4, 128, 1, 8, 0, fake, fake, 16, fake, fake, fake, fake)
    assert L.kvz_append_token(ctypes.byref(cs), fake, fake, fake, wide, fake, 1, None) == binding.KVZ_ERR_UNSUPPORTED
    assert L.kvz_decode_attention(fake, ctypes.byref(cs), fake, wide, fake, 1, 4, 0.1, 0, fake, None, fake, 1 << 40,
                                  None) == binding.KVZ_ERR_UNSUPPORTED
    # compression stages a unit on chip: up to the format's largest block (P * D = 65536) for the
    # first format at head dim 64 or 128, half of it otherwise (n = 0: checked, nothing enqueued)
    for fmt, P, D, want in ((0, 512, 128, binding.KVZ_OK), (0, 1024, 64, binding.KVZ_OK),
                            (1, 512, 128, binding.KVZ_ERR_UNSUPPORTED), (1, 256, 128, binding.KVZ_OK),
                            (2, 512, 128, binding.KVZ_ERR_UNSUPPORTED), (2, 256, 128, binding.KVZ_OK),
                            (3, 16, 128, binding.KVZ_ERR_INVALID_ARG),
                            (0, 256, 192, binding.KVZ_ERR_UNSUPPORTED), (0, 128, 192, binding.KVZ_OK)):
        c = binding._CacheStruct(P, 4, D, 1, 8, fmt, fake, fake, 16, fake, fake, fake, fake)
        assert L.kvz_compress_pages(ctypes.byref(c), fake, fake, fake, 0, None) == want, (fmt, P, D)
        assert L.kvz_append_token(ctypes.byref(c), fake, fake, fake, 4, fake, 0, None) == want, (fmt, P, D)
    # a cache without unit slots needs no unit array; with slots it does
    for npages, units, want in ((0, None, binding.KVZ_OK), (1, None, binding.KVZ_ERR_INVALID_ARG)):
        c = binding._CacheStruct(16, 4, 128, npages, 8, 0, units, fake, 16, fake, fake, fake, fake)
        assert L.kvz_compress_pages(ctypes.byref(c), fake, fake, fake, 0, None) == want, npages
    # a workspace that does not fit in size_t: zero size, and the call refuses it
    big = (1 << 31) - 1
    assert kvz.workspace_bytes(big, 1024, 1024, 128, 16, 1 << 20, 1) == 0
    huge = binding._CacheStruct(16, 1024, 128, 1, big, 0, fake, fake, 16, fake, fake, fake, fake)
    rc = L.kvz_decode_attention_splits(fake, ctypes.byref(huge), fake, 1 << 20, fake, big, 1024, 0.1, 1, fake,
                                       (1 << 64) - 1, None)
    assert rc == binding.KVZ_ERR_INVALID_ARG


def test_binding_checks_buffers_before_calling_the_library():
    """Wrong types, too-small buffers and mixed devices raise in the binding; nothing reaches the
    library (these calls never get past their checks, so they run without a GPU)."""
    cache = kvz.Cache.allocate(16, 4, 128, 8, 2, 64, device="cpu")
    q = torch.zeros((2, 8, 128), dtype=torch.int16)
    table = torch.zeros((2, 4), dtype=torch.int32)
    lens = torch.zeros(2, dtype=torch.int32)
    out = torch.zeros((2, 8, 128), dtype=torch.int16)
    bad = [dict(q=q.float()), dict(page_table=table.long()), dict(seq_lens=lens[:1]), dict(out=out[:1]),
           dict(out_f32=torch.zeros((2, 8, 128), dtype=torch.float16)), dict(page_table=table[:1]),
           dict(q=q[:, :, :64].transpose(0, 1))]
    for b in bad:
        args = dict(q=q, page_table=table, seq_lens=lens, out=out, out_f32=None)
        args.update(b)
        with pytest.raises(ValueError):
            kvz.decode_attention(args["q"], cache, args["page_table"], args["seq_lens"], 0.1, args["out"],
                                 args["out_f32"])
    # a query of another head dim than the cache's: the library would read q and write out with
    # the cache's head dim, past the end of both
    q64, out64 = torch.zeros((2, 8, 64), dtype=torch.int16), torch.zeros((2, 8, 64), dtype=torch.int16)
    with pytest.raises(ValueError):
        kvz.decode_attention(q64, cache, table, lens, 0.1, out64)
    with pytest.raises(ValueError):
        kvz.prepare_decode_attention(q64, cache, table, lens, 0.1, out64)
    with pytest.raises(ValueError):
        kvz.decode_attention_splits(q64, cache, table, lens, 0.1, torch.zeros(1 << 20, dtype=torch.uint8))
    kp = torch.zeros((8, 4, 16, 128), dtype=torch.int16)
    with pytest.raises(ValueError):
        kvz.decode_attention_dense(q64, kp, kp, table, lens, 0.1, out64)
    with pytest.raises(ValueError):
        kvz.decode_attention_splits(q, cache, table, lens, 0.1, None)        # the two-phase calls take a workspace
    with pytest.raises(ValueError):
        kvz.merge_splits(None, lens, 2, 8, 4, 128, 16, 4, out)
    with pytest.raises(ValueError):
        kvz.append_token(cache, torch.zeros((2, 4, 64), dtype=torch.int16), torch.zeros((2, 4, 128), dtype=torch.int16),
                         table, lens)
    with pytest.raises(ValueError):
        kvz.compress_pages(cache, torch.zeros((1, 4, 16, 128), dtype=torch.int16),
                           torch.zeros((1, 4, 16, 128), dtype=torch.int16), torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError):
        kvz.decompress_pages(cache, torch.zeros(2, dtype=torch.int32), torch.zeros((1, 4, 16, 128), dtype=torch.int16),
                             torch.zeros((2, 4, 16, 128), dtype=torch.int16))


def test_noalloc_checks_come_before_any_device_work():
    L = binding.lib()
    assert L.kvz_decode_attention_noalloc(None, None, None, 0, None, 0, 1, 1.0, 0, None, None, None) == \
        binding.KVZ_ERR_INVALID_ARG
    # a well-formed description (the pointers are never dereferenced on the host) whose call would
    # need more than the library's scratch array: refused with KVZ_ERR_SCRATCH, nothing enqueued
    fake = 256
    cs = binding._CacheStruct(16, 32, 128, 1, 8, 0, fake, fake, 16, fake, fake, fake, fake)
    need = kvz.workspace_bytes(8, 32, 32, 128, 16, 1024, 1)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    rc = L.kvz_decode_attention_noalloc(fake, ctypes.byref(cs), fake, 1024, fake, 8, 32, 0.1, 1, fake, None, None)
    assert rc == binding.KVZ_ERR_SCRATCH
    assert "scratch" in kvz.kvz.strerror(binding.KVZ_ERR_SCRATCH)
    # unsupported shapes are refused first
    rc = L.kvz_decode_attention_noalloc(fake, ctypes.byref(cs), fake, 1024, fake, 8, 33, 0.1, 0, fake, None, None)
    assert rc == binding.KVZ_ERR_UNSUPPORTED


def test_cache_struct_layout_matches_header():
    # field order and sizes of kvz_cache: 6 int32, then pointers/int64 (8 bytes each)
    s = binding._CacheStruct
    assert ctypes.sizeof(s) == 6 * 4 + 7 * 8
    assert s.units.offset == 24 and s.status.offset == 24 + 6 * 8


def test_package_has_no_cpu_fallback():
    src = open(os.path.join(ROOT, "decode_attention_losslessly_amd", "kvz.py")).read()
    assert "oracle" not in src
    for f in os.listdir(os.path.join(ROOT, "decode_attention_losslessly_amd")):
        if f.endswith(".py"):
            assert "import oracle" not in open(os.path.join(ROOT, "decode_attention_losslessly_amd", f)).read()
