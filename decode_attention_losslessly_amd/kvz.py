"""Python binding of libkvz (include/kvz.h): argument marshalling only.

Every step of the path runs in the HIP library; this module turns torch tensors into device
pointers and the current HIP stream into the `stream` argument. PyTorch is used for device
memory and streams only. There is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVZ_LIB names another build of the same sources (the host-sanitized one of the tests)
LIB_PATH = os.environ.get("KVZ_LIB") or os.path.join(_HERE, "libkvz.so")

KVZ_OK, KVZ_ERR_INVALID_ARG, KVZ_ERR_UNSUPPORTED, KVZ_ERR_WORKSPACE, KVZ_ERR_HIP, KVZ_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 32 << 20   # KVZ_NOALLOC_SCRATCH_BYTES
STATUS_ESC_POOL_FULL, STATUS_BAD_PAGE_ID, STATUS_SEQ_TOO_LONG = 1, 2, 4
FORMAT_ESCAPE, FORMAT_ZIPFUSION, FORMAT_CHANNEL = 0, 1, 2

EXPORTS = ("kvz_payload_bytes", "kvz_unit_bytes", "kvz_meta_bytes", "kvz_inline_capacity", "kvz_workspace_bytes",
           "kvz_num_splits", "kvz_compress_pages", "kvz_append_token", "kvz_decode_attention", "kvz_decode_attention_dense",
           "kvz_decompress_pages", "kvz_strerror", "kvz_decode_attention_splits",
           "kvz_decode_attention_dense_splits", "kvz_merge_splits", "kvz_unit_bytes_for", "kvz_compact_pool",
           "kvz_decode_attention_noalloc")


class KvzError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


class _CacheStruct(ctypes.Structure):
    _fields_ = [("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_batch", ctypes.c_int32), ("format", ctypes.c_int32),
                ("units", ctypes.c_void_p), ("esc_pool", ctypes.c_void_p), ("esc_capacity", ctypes.c_int64),
                ("esc_cursor", ctypes.c_void_p), ("k_tail", ctypes.c_void_p), ("v_tail", ctypes.c_void_p),
                ("status", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkvz.so (torch is imported first so that one HIP runtime serves both)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python __graft_entry__.py build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, sz, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p
        cp = ctypes.POINTER(_CacheStruct)
        sig = {
            "kvz_payload_bytes": (sz, [i32, i32]),
            "kvz_unit_bytes": (sz, [i32, i32]),
            "kvz_unit_bytes_for": (sz, [i32, i32, i32]),
            "kvz_compact_pool": (ctypes.c_int, [cp, vp, i32, vp, i64, vp, vp]),
            "kvz_meta_bytes": (sz, [i32, i32]),
            "kvz_inline_capacity": (i32, [i32, i32]),
            "kvz_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32, i32]),
            "kvz_num_splits": (i32, [i32, i32, i32, i32, i32, i32, i32]),
            "kvz_compress_pages": (ctypes.c_int, [cp, vp, vp, vp, i32, vp]),
            "kvz_append_token": (ctypes.c_int, [cp, vp, vp, vp, i32, vp, i32, vp]),
            "kvz_decode_attention": (ctypes.c_int, [vp, cp, vp, i32, vp, i32, i32, f32, i32, vp, vp, vp, sz, vp]),
            "kvz_decode_attention_noalloc": (ctypes.c_int, [vp, cp, vp, i32, vp, i32, i32, f32, i32, vp, vp, vp]),
            "kvz_decode_attention_dense": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, i32, vp, i32, vp, i32, i32,
                                                          f32, i32, vp, vp, vp, sz, vp, vp]),
            "kvz_decompress_pages": (ctypes.c_int, [cp, vp, i32, i32, vp, vp, vp]),
            "kvz_decode_attention_splits": (ctypes.c_int, [vp, cp, vp, i32, vp, i32, i32, f32, i32, vp, sz, vp]),
            "kvz_decode_attention_dense_splits": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, i32, vp, i32, vp, i32,
                                                                 i32, f32, i32, vp, sz, vp, vp]),
            "kvz_merge_splits": (ctypes.c_int, [vp, sz, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp]),
            "kvz_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().kvz_strerror(code).decode()


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libkvz must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_HALF = (torch.int16, torch.bfloat16)   # BF16 values, as bits or as bfloat16


def _arg(t: torch.Tensor | None, name: str, dtypes, numel: int, device) -> None:
    """Checks a device buffer the library reads or writes: its type, that it holds at least `numel`
    elements (the library touches exactly that many) and that it is on the call's device, so that
    a wrong argument raises here instead of being read or written past its end."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, the call needs {numel}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _on(t: torch.Tensor | None, name: str, device, required: bool = False) -> None:
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _table(page_table: torch.Tensor, B: int, device) -> int:
    """max_pages of a [B, max_pages] int32 page table"""
    if page_table.dim() != 2 or page_table.shape[0] < B:
        raise ValueError(f"page_table: shape {tuple(page_table.shape)}, expected [>= {B}, max_pages]")
    _arg(page_table, "page_table", (torch.int32,), 0, device)
    return int(page_table.shape[1])


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _scratch(nbytes: int, device, stream) -> torch.Tensor:
    """A workspace for one call on `stream`: allocated from the caching allocator on that stream,
    so that its memory is not handed out again before the call's kernels are done with it."""
    if stream is None:
        return torch.empty(max(nbytes, 4), dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(max(nbytes, 4), dtype=torch.uint8, device=device)


def _check(rc: int, what: str):
    if rc != KVZ_OK:
        raise KvzError(rc, what)


# ---------------------------------------------------------------- sizes
def unit_bytes(P: int, D: int, fmt: int = FORMAT_ESCAPE) -> int:
    return int(lib().kvz_unit_bytes_for(fmt, P, D))


def payload_bytes(P: int, D: int) -> int:
    return int(lib().kvz_payload_bytes(P, D))


def meta_bytes(P: int, D: int) -> int:
    return int(lib().kvz_meta_bytes(P, D))


def inline_capacity(P: int, D: int) -> int:
    return int(lib().kvz_inline_capacity(P, D))


def workspace_bytes(B, Hq, Hkv, D, P, max_pages, pages_per_split=0) -> int:
    return int(lib().kvz_workspace_bytes(B, Hq, Hkv, D, P, max_pages, pages_per_split))


def num_splits(B, Hq, Hkv, D, P, max_pages, pages_per_split=0) -> int:
    return int(lib().kvz_num_splits(B, Hq, Hkv, D, P, max_pages, pages_per_split))


def chosen_split(workspace: torch.Tensor, B, Hq, Hkv, D, P, max_pages, pages_per_split=0) -> tuple[int, int]:
    """What the last split kernel run on `workspace` recorded in the slot after the partials:
    (plan pages per split, or minus its chunks per (request, query head) when it used the ranked
    schedule; plan pages per page of the table, P // 16 when it counted its splits in 16-token
    tiles, else 1). Synchronises with the device."""
    S = num_splits(B, Hq, Hkv, D, P, max_pages, pages_per_split)
    off = B * Hq * S * (D + 2) * 4
    c, tpp = workspace[off:off + 8].view(torch.int32).tolist()
    return int(c), int(tpp)


def chosen_pages_per_split(workspace: torch.Tensor, B, Hq, Hkv, D, P, max_pages, pages_per_split=0) -> int:
    """The first element of chosen_split: plan pages per split (pages, or 16-token tiles when the
    kernel counted tiles), or minus the chunks per row under the ranked schedule."""
    return chosen_split(workspace, B, Hq, Hkv, D, P, max_pages, pages_per_split)[0]


# ---------------------------------------------------------------- cache
@dataclass
class Cache:
    """Device buffers of a compressed cache (owned by torch), described to libkvz per call."""
    P: int
    H: int
    D: int
    num_pages: int
    max_batch: int
    units: torch.Tensor        # uint8 [num_pages, H, unit_bytes]
    esc_pool: torch.Tensor     # int16 [esc_capacity]
    esc_cursor: torch.Tensor   # int64 [1]
    k_tail: torch.Tensor       # int16 [max_batch, H, P, D]
    v_tail: torch.Tensor
    status: torch.Tensor       # int32 [1]
    fmt: int = FORMAT_ESCAPE   # FORMAT_ESCAPE, FORMAT_ZIPFUSION (esc_pool then holds raw blocks) or FORMAT_CHANNEL

    @classmethod
    def allocate(cls, P: int, H: int, D: int, num_pages: int, max_batch: int, esc_capacity: int,
                 device="cuda", fmt: int = FORMAT_ESCAPE) -> "Cache":
        U = unit_bytes(P, D, fmt)
        if U == 0:
            raise KvzError(KVZ_ERR_UNSUPPORTED, "Cache.allocate")
        z = dict(device=device)
        return cls(P, H, D, num_pages, max_batch,
                   units=torch.zeros((num_pages, H, U), dtype=torch.uint8, **z),
                   esc_pool=torch.zeros(max(1, esc_capacity), dtype=torch.int16, **z),
                   esc_cursor=torch.zeros(1, dtype=torch.int64, **z),
                   k_tail=torch.zeros((max_batch, H, P, D), dtype=torch.int16, **z),
                   v_tail=torch.zeros((max_batch, H, P, D), dtype=torch.int16, **z),
                   status=torch.zeros(1, dtype=torch.int32, **z), fmt=fmt)

    @property
    def esc_capacity(self) -> int:
        return int(self.esc_pool.numel())

    def struct(self) -> _CacheStruct:
        return _CacheStruct(self.P, self.H, self.D, self.num_pages, self.max_batch, self.fmt, self.units.data_ptr(),
                            self.esc_pool.data_ptr(), self.esc_capacity, self.esc_cursor.data_ptr(),
                            self.k_tail.data_ptr(), self.v_tail.data_ptr(), self.status.data_ptr())


# ---------------------------------------------------------------- entry points
def _io(q, page_table, seq_lens, out, out_f32, device, D_kv: int) -> int:
    """Checks an attention call's query, table, lengths and outputs against the head dim D_kv of
    the keys and values (the library reads q and writes the outputs with that head dim); returns
    max_pages."""
    if q.dim() != 3:
        raise ValueError(f"q: shape {tuple(q.shape)}, expected [B, H_q, D]")
    B, Hq, D = q.shape
    if D != D_kv:
        raise ValueError(f"q: head dim {D}, the keys and values have {D_kv}")
    _arg(q, "q", _HALF, 0, device)
    max_pages = _table(page_table, B, device)
    _arg(seq_lens, "seq_lens", (torch.int32,), B, device)
    if out is not None:
        _arg(out, "out", _HALF, B * Hq * D, device)
    if out_f32 is not None:
        _arg(out_f32, "out_f32", (torch.float32,), B * Hq * D, device)
    return max_pages


def _dense_pages(k_pages, v_pages, status, device) -> None:
    if k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError(f"k_pages, v_pages: shapes {tuple(k_pages.shape)}, {tuple(v_pages.shape)}, "
                         "expected two equal [num_pages, H, P, D]")
    _arg(k_pages, "k_pages", _HALF, 0, device)
    _arg(v_pages, "v_pages", _HALF, 0, device)
    if status is not None:
        _arg(status, "status", (torch.int32,), 1, device)


def compress_pages(cache: Cache, k_src: torch.Tensor, v_src: torch.Tensor, dst_page_ids: torch.Tensor,
                   stream=None) -> None:
    """k_src, v_src: int16 [n, H, P, D]; dst_page_ids: int32 [n]."""
    n = int(dst_page_ids.numel())
    dev, blk = cache.units.device, n * cache.H * cache.P * cache.D
    _arg(k_src, "k_src", _HALF, blk, dev)
    _arg(v_src, "v_src", _HALF, blk, dev)
    _arg(dst_page_ids, "dst_page_ids", (torch.int32,), n, dev)
    cs = cache.struct()
    _check(lib().kvz_compress_pages(ctypes.byref(cs), _ptr(k_src), _ptr(v_src), _ptr(dst_page_ids), n,
                                    _stream(stream)), "kvz_compress_pages")


def append_token(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, page_table: torch.Tensor,
                 seq_lens: torch.Tensor, stream=None) -> None:
    """k_new, v_new: int16 [B, H, D]; page_table int32 [B, max_pages]; seq_lens int32 [B] (updated)."""
    dev = cache.units.device
    B = int(page_table.shape[0])
    max_pages = _table(page_table, B, dev)
    _arg(k_new, "k_new", _HALF, B * cache.H * cache.D, dev)
    _arg(v_new, "v_new", _HALF, B * cache.H * cache.D, dev)
    _arg(seq_lens, "seq_lens", (torch.int32,), B, dev)
    cs = cache.struct()
    _check(lib().kvz_append_token(ctypes.byref(cs), _ptr(k_new), _ptr(v_new), _ptr(page_table), max_pages,
                                  _ptr(seq_lens), B, _stream(stream)), "kvz_append_token")


def decode_attention(q: torch.Tensor, cache: Cache, page_table: torch.Tensor, seq_lens: torch.Tensor,
                     sm_scale: float, out: torch.Tensor, out_f32: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, pages_per_split: int = 0, stream=None) -> None:
    """q, out: int16 [B, Hq, D] (BF16 bits); out_f32 optional float32 [B, Hq, D]."""
    B, Hq, D = q.shape
    max_pages = _io(q, page_table, seq_lens, out, out_f32, cache.units.device, cache.D)
    _on(workspace, "workspace", cache.units.device)
    if workspace is None:
        workspace = _scratch(workspace_bytes(B, Hq, cache.H, D, cache.P, max_pages, pages_per_split), q.device, stream)
    cs = cache.struct()
    _check(lib().kvz_decode_attention(_ptr(q), ctypes.byref(cs), _ptr(page_table), max_pages, _ptr(seq_lens), B, Hq,
                                      float(sm_scale), pages_per_split, _ptr(out), _ptr(out_f32), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)),
           "kvz_decode_attention")


def decode_attention_noalloc(q: torch.Tensor, cache: Cache, page_table: torch.Tensor, seq_lens: torch.Tensor,
                             sm_scale: float, out: torch.Tensor, out_f32: torch.Tensor | None = None,
                             pages_per_split: int = 0, stream=None) -> None:
    """decode_attention with its workspace in the library's own per-GPU scratch array: nothing is
    allocated, here or in the library (for callers that cannot allocate device memory)."""
    B, Hq, D = q.shape
    max_pages = _io(q, page_table, seq_lens, out, out_f32, cache.units.device, cache.D)
    cs = cache.struct()
    _check(lib().kvz_decode_attention_noalloc(_ptr(q), ctypes.byref(cs), _ptr(page_table), max_pages,
                                              _ptr(seq_lens), B, Hq, float(sm_scale), pages_per_split, _ptr(out),
                                              _ptr(out_f32), _stream(stream)), "kvz_decode_attention_noalloc")


def decode_attention_dense(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, page_table: torch.Tensor,
                           seq_lens: torch.Tensor, sm_scale: float, out: torch.Tensor,
                           out_f32: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                           status: torch.Tensor | None = None, pages_per_split: int = 0, stream=None) -> None:
    """k_pages, v_pages: int16 [num_pages, H, P, D]; other arguments as decode_attention."""
    B, Hq, D = q.shape
    num_pages, H, P, _ = k_pages.shape
    max_pages = _io(q, page_table, seq_lens, out, out_f32, q.device, k_pages.shape[-1])
    _dense_pages(k_pages, v_pages, status, q.device)
    _on(workspace, "workspace", q.device)
    if workspace is None:
        workspace = _scratch(workspace_bytes(B, Hq, H, D, P, max_pages, pages_per_split), q.device, stream)
    _check(lib().kvz_decode_attention_dense(_ptr(q), _ptr(k_pages), _ptr(v_pages), num_pages, H, D, P,
                                            _ptr(page_table), max_pages, _ptr(seq_lens), B, Hq, float(sm_scale),
                                            pages_per_split, _ptr(out), _ptr(out_f32), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _ptr(status),
                                            _stream(stream)), "kvz_decode_attention_dense")


def decode_attention_splits(q: torch.Tensor, cache: Cache, page_table: torch.Tensor, seq_lens: torch.Tensor,
                            sm_scale: float, workspace: torch.Tensor, pages_per_split: int = 0, stream=None) -> None:
    """First phase of decode_attention: the split kernel, partials into `workspace`."""
    B, Hq, D = q.shape
    max_pages = _io(q, page_table, seq_lens, None, None, cache.units.device, cache.D)
    _on(workspace, "workspace", cache.units.device, required=True)
    cs = cache.struct()
    _check(lib().kvz_decode_attention_splits(_ptr(q), ctypes.byref(cs), _ptr(page_table), max_pages,
                                             _ptr(seq_lens), B, Hq, float(sm_scale), pages_per_split,
                                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                                             _stream(stream)), "kvz_decode_attention_splits")


def decode_attention_dense_splits(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                                  page_table: torch.Tensor, seq_lens: torch.Tensor, sm_scale: float,
                                  workspace: torch.Tensor, status: torch.Tensor | None = None,
                                  pages_per_split: int = 0, stream=None) -> None:
    B, Hq, D = q.shape
    num_pages, H, P, _ = k_pages.shape
    max_pages = _io(q, page_table, seq_lens, None, None, q.device, k_pages.shape[-1])
    _dense_pages(k_pages, v_pages, status, q.device)
    _on(workspace, "workspace", q.device, required=True)
    _check(lib().kvz_decode_attention_dense_splits(_ptr(q), _ptr(k_pages), _ptr(v_pages), num_pages, H, D, P,
                                                   _ptr(page_table), max_pages, _ptr(seq_lens), B, Hq,
                                                   float(sm_scale), pages_per_split, _ptr(workspace),
                                                   workspace.numel() * workspace.element_size(), _ptr(status),
                                                   _stream(stream)), "kvz_decode_attention_dense_splits")


def merge_splits(workspace: torch.Tensor, seq_lens: torch.Tensor, B: int, Hq: int, H: int, D: int, P: int,
                 max_pages: int, out: torch.Tensor, out_f32: torch.Tensor | None = None, dense: bool = False,
                 pages_per_split: int = 0, stream=None) -> None:
    """Second phase: merges the partials left by one of the split kernels."""
    _on(workspace, "workspace", seq_lens.device, required=True)
    dev = workspace.device
    _arg(seq_lens, "seq_lens", (torch.int32,), B, dev)
    _arg(out, "out", _HALF, B * Hq * D, dev)
    if out_f32 is not None:
        _arg(out_f32, "out_f32", (torch.float32,), B * Hq * D, dev)
    _check(lib().kvz_merge_splits(_ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(seq_lens), B,
                                  Hq, H, D, P, max_pages, pages_per_split, 1 if dense else 0, _ptr(out),
                                  _ptr(out_f32), _stream(stream)), "kvz_merge_splits")


def compact_pool(cache: Cache, page_ids: torch.Tensor, new_capacity: int, stream=None) -> None:
    """Moves the pool data of the units page_ids (int32 [n], all heads) into a new pool of
    new_capacity u16 elements and installs it in `cache` (the old pool is then released). The new
    buffers are allocated and cleared on the call's stream, and the old pool is kept from reuse
    until the work enqueued there so far is done."""
    _arg(page_ids, "page_ids", (torch.int32,), int(page_ids.numel()), cache.units.device)
    s = torch.cuda.current_stream() if stream is None else stream
    with torch.cuda.stream(s):
        new_pool = torch.zeros(max(1, new_capacity), dtype=torch.int16, device=cache.esc_pool.device)
        new_cursor = torch.zeros(1, dtype=torch.int64, device=cache.esc_pool.device)
    cs = cache.struct()
    _check(lib().kvz_compact_pool(ctypes.byref(cs), _ptr(page_ids), int(page_ids.numel()), _ptr(new_pool),
                                  new_pool.numel(), _ptr(new_cursor), _stream(s)), "kvz_compact_pool")
    cache.esc_pool.record_stream(s)
    cache.esc_pool, cache.esc_cursor = new_pool, new_cursor


def decompress_pages(cache: Cache, page_ids: torch.Tensor, k_dst: torch.Tensor, v_dst: torch.Tensor,
                     lane_map: int = 0, stream=None) -> None:
    """Test entry point: the attention kernels' in-register decode written out as BF16 bits."""
    n, dev = int(page_ids.numel()), cache.units.device
    _arg(page_ids, "page_ids", (torch.int32,), n, dev)
    _arg(k_dst, "k_dst", _HALF, n * cache.H * cache.P * cache.D, dev)
    _arg(v_dst, "v_dst", _HALF, n * cache.H * cache.P * cache.D, dev)
    cs = cache.struct()
    _check(lib().kvz_decompress_pages(ctypes.byref(cs), _ptr(page_ids), int(page_ids.numel()), lane_map,
                                      _ptr(k_dst), _ptr(v_dst), _stream(stream)), "kvz_decompress_pages")


# ---------------------------------------------------------------- prepared calls
class PreparedAttention:
    """One decode-attention call, its buffers checked and its arguments marshalled once, for a loop
    that repeats it (the same buffers every step, their contents changing on the device: a decode
    loop reads its lengths and page table from memory each call). `splits()` enqueues the split
    kernel, `merge()` the merge, a call both, on the stream given at preparation (default: the
    current stream then). It keeps its buffers alive and holds their addresses: prepare again after
    anything replaces a buffer (kvz_compact_pool installs a new pool)."""

    def __init__(self, split_fn, split_args, merge_args, keep, what):
        self._split = split_fn
        self._split_args = split_args
        self._merge = lib().kvz_merge_splits
        self._merge_args = merge_args
        self._keep = keep          # the tensors and the cache description the addresses point into
        self._what = what

    def splits(self) -> None:
        rc = self._split(*self._split_args)
        if rc:
            raise KvzError(rc, self._what)

    def merge(self) -> None:
        rc = self._merge(*self._merge_args)
        if rc:
            raise KvzError(rc, "kvz_merge_splits")

    def __call__(self) -> None:
        self.splits()
        self.merge()


class PreparedAppend:
    """One append_token call, its buffers checked and its arguments marshalled once, for a decode
    loop that appends the new token's K and V from the same buffers every step (the lengths
    advance on the device). A call enqueues kvz_append_token on the stream given at preparation.
    It keeps its buffers alive and holds their addresses: prepare again after anything replaces a
    buffer (kvz_compact_pool installs a new pool)."""

    def __init__(self, args, keep):
        self._fn = lib().kvz_append_token
        self._args = args
        self._keep = keep

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc:
            raise KvzError(rc, "kvz_append_token")


def prepare_append_token(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, page_table: torch.Tensor,
                         seq_lens: torch.Tensor, stream=None) -> PreparedAppend:
    """append_token as a PreparedAppend (arguments as append_token)."""
    dev = cache.units.device
    B = int(page_table.shape[0])
    max_pages = _table(page_table, B, dev)
    _arg(k_new, "k_new", _HALF, B * cache.H * cache.D, dev)
    _arg(v_new, "v_new", _HALF, B * cache.H * cache.D, dev)
    _arg(seq_lens, "seq_lens", (torch.int32,), B, dev)
    s = torch.cuda.current_stream() if stream is None else stream
    cs = cache.struct()
    args = (ctypes.byref(cs), _ptr(k_new), _ptr(v_new), _ptr(page_table), max_pages, _ptr(seq_lens), B, _stream(s))
    return PreparedAppend(args, (cache, cs, k_new, v_new, page_table, seq_lens, s))


def _merge_args(workspace, seq_lens, B, Hq, H, D, P, max_pages, pps, dense, out, out_f32, s):
    return (_ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(seq_lens), B, Hq, H, D, P, max_pages,
            pps, 1 if dense else 0, _ptr(out), _ptr(out_f32), s)


def prepare_decode_attention(q: torch.Tensor, cache: Cache, page_table: torch.Tensor, seq_lens: torch.Tensor,
                             sm_scale: float, out: torch.Tensor, out_f32: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None, pages_per_split: int = 0,
                             stream=None) -> PreparedAttention:
    """decode_attention as a PreparedAttention (arguments as decode_attention)."""
    B, Hq, D = q.shape
    dev = cache.units.device
    max_pages = _io(q, page_table, seq_lens, out, out_f32, dev, cache.D)
    _on(workspace, "workspace", dev)
    s = torch.cuda.current_stream() if stream is None else stream
    if workspace is None:
        workspace = _scratch(workspace_bytes(B, Hq, cache.H, D, cache.P, max_pages, pages_per_split), q.device, s)
    cs = cache.struct()
    st = _stream(s)
    split = (_ptr(q), ctypes.byref(cs), _ptr(page_table), max_pages, _ptr(seq_lens), B, Hq, float(sm_scale),
             pages_per_split, _ptr(workspace), workspace.numel() * workspace.element_size(), st)
    merge = _merge_args(workspace, seq_lens, B, Hq, cache.H, D, cache.P, max_pages, pages_per_split, False, out,
                        out_f32, st)
    keep = (q, cache, cs, page_table, seq_lens, out, out_f32, workspace, s)
    return PreparedAttention(lib().kvz_decode_attention_splits, split, merge, keep, "kvz_decode_attention_splits")


def prepare_decode_attention_dense(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                                   page_table: torch.Tensor, seq_lens: torch.Tensor, sm_scale: float,
                                   out: torch.Tensor, out_f32: torch.Tensor | None = None,
                                   workspace: torch.Tensor | None = None, status: torch.Tensor | None = None,
                                   pages_per_split: int = 0, stream=None) -> PreparedAttention:
    """decode_attention_dense as a PreparedAttention (arguments as decode_attention_dense)."""
    B, Hq, D = q.shape
    num_pages, H, P, _ = k_pages.shape
    max_pages = _io(q, page_table, seq_lens, out, out_f32, q.device, k_pages.shape[-1])
    _dense_pages(k_pages, v_pages, status, q.device)
    _on(workspace, "workspace", q.device)
    s = torch.cuda.current_stream() if stream is None else stream
    if workspace is None:
        workspace = _scratch(workspace_bytes(B, Hq, H, D, P, max_pages, pages_per_split), q.device, s)
    st = _stream(s)
    split = (_ptr(q), _ptr(k_pages), _ptr(v_pages), num_pages, H, D, P, _ptr(page_table), max_pages, _ptr(seq_lens),
             B, Hq, float(sm_scale), pages_per_split, _ptr(workspace), workspace.numel() * workspace.element_size(),
             _ptr(status), st)
    merge = _merge_args(workspace, seq_lens, B, Hq, H, D, P, max_pages, pages_per_split, True, out, out_f32, st)
    keep = (q, k_pages, v_pages, page_table, seq_lens, out, out_f32, workspace, status, s)
    return PreparedAttention(lib().kvz_decode_attention_dense_splits, split, merge, keep,
                             "kvz_decode_attention_dense_splits")
