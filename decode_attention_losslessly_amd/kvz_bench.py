"""Python binding of libkvz_bench (include/kvz_bench.h): argument marshalling only. The
measurement kernels there are the references the decode-attention kernels are compared with."""
from __future__ import annotations

import ctypes
import os

import torch

from .kvz import Cache, KvzError, _ptr, _stream

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvz_bench.so")
EXPORTS = ("kvzb_read_units",)

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python __graft_entry__.py build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, sz, vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
        L.kvzb_read_units.restype = ctypes.c_int
        L.kvzb_read_units.argtypes = [vp, i32, sz, vp, i32, vp, i32, i32, i32, i32, vp, vp]
        _lib = L
    return _lib


def read_units(cache: Cache, page_table: torch.Tensor, seq_lens: torch.Tensor, chunks_per_row: int,
               sink: torch.Tensor, stream=None) -> None:
    """Streams the unit bytes an attention call over `cache` reads (kvzb_read_units).
    sink: int32 [B * H * chunks_per_row * 64]."""
    B, max_pages = page_table.shape
    rc = lib().kvzb_read_units(_ptr(cache.units), cache.num_pages, cache.units.shape[2], _ptr(page_table), max_pages,
                               _ptr(seq_lens), B, cache.H, cache.P, chunks_per_row, _ptr(sink), _stream(stream))
    if rc != 0:
        raise KvzError(rc, "kvzb_read_units")
