"""ctypes front end of the C oracle (oracle/c/kvz_oracle.c). Test infrastructure only."""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        # KVZ_ORACLE_LIB names another build of the same source (the sanitized one of the tests)
        path = os.environ.get("KVZ_ORACLE_LIB") or os.path.join(_HERE, "libkvz_oracle.so")
        if not os.path.exists(path):
            from . import build
            build.build()
        L = ctypes.CDLL(path)
        i32, i64, u64, dbl, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        L.kvzo_meta_bytes.restype = ctypes.c_size_t
        L.kvzo_meta_bytes.argtypes = [i32, i32]
        L.kvzo_unit_bytes.restype = ctypes.c_size_t
        L.kvzo_unit_bytes.argtypes = [i32, i32]
        L.kvzo_inline_capacity.restype = i32
        L.kvzo_inline_capacity.argtypes = [i32, i32]
        L.kvzo_group_base.restype = i32
        L.kvzo_group_base.argtypes = [vp]
        L.kvzo_encode_unit.restype = i64
        L.kvzo_encode_unit.argtypes = [vp, vp, i32, i32, u64, vp, vp]
        L.kvzo_encode_pages.restype = i64
        L.kvzo_encode_pages.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp, i64, i64]
        L.kvzo_decode_unit.restype = None
        L.kvzo_decode_unit.argtypes = [vp, vp, i32, i32, vp, vp]
        L.kvzo_decode_pages.restype = None
        L.kvzo_decode_pages.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp, vp]
        L.kvzo_decode_attention_rows.restype = None
        L.kvzo_decode_attention_rows.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32,
                                                 dbl, vp, i32, vp]
        L.kvzo_dense_attention_rows.restype = None
        L.kvzo_dense_attention_rows.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, dbl, vp,
                                                i32, vp]
        L.kvzo_num_threads.restype = i32
        L.kvzo_num_threads.argtypes = []
        _LIB = L
    return _LIB


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


def unit_bytes(P: int, D: int) -> int:
    return int(lib().kvzo_unit_bytes(P, D))


def meta_bytes(P: int, D: int) -> int:
    return int(lib().kvzo_meta_bytes(P, D))


def inline_capacity(P: int, D: int) -> int:
    return int(lib().kvzo_inline_capacity(P, D))


def group_base(exps) -> int:
    e = np.ascontiguousarray(exps, np.int32)
    assert e.shape == (64,)
    return int(lib().kvzo_group_base(_p(e)))


def encode_unit(K: np.ndarray, V: np.ndarray, pool_offset: int = 0):
    P, D = K.shape
    K = np.ascontiguousarray(K, np.uint16)
    V = np.ascontiguousarray(V, np.uint16)
    unit = np.zeros(unit_bytes(P, D), np.uint8)
    esc = np.zeros(2 * P * D, np.uint16)
    n = lib().kvzo_encode_unit(_p(K), _p(V), P, D, pool_offset, _p(unit), _p(esc))
    return unit, esc[:n].copy()


def encode_pages(K: np.ndarray, V: np.ndarray, pool_capacity: int | None = None):
    """K/V [n][H][P][D] -> (units [n][H][U], pool u16, pool length)."""
    n, H, P, D = K.shape
    K = np.ascontiguousarray(K, np.uint16)
    V = np.ascontiguousarray(V, np.uint16)
    units = np.zeros((n, H, unit_bytes(P, D)), np.uint8)
    cap = 2 * n * H * P * D if pool_capacity is None else pool_capacity
    pool = np.zeros(max(cap, 1), np.uint16)
    end = lib().kvzo_encode_pages(_p(K), _p(V), n, H, P, D, _p(units), _p(pool), 0, cap)
    if end < 0:
        raise RuntimeError("escape pool capacity exceeded")
    return units, pool[:max(end, 1)].copy(), int(end)


def decode_unit(unit: np.ndarray, pool: np.ndarray | None, P: int, D: int):
    unit = np.ascontiguousarray(unit, np.uint8)
    pool = np.zeros(1, np.uint16) if pool is None or len(pool) == 0 else np.ascontiguousarray(pool, np.uint16)
    K = np.zeros((P, D), np.uint16)
    V = np.zeros((P, D), np.uint16)
    lib().kvzo_decode_unit(_p(unit), _p(pool), P, D, _p(K), _p(V))
    return K, V


def decode_pages(units: np.ndarray, pool: np.ndarray, page_ids, P: int, D: int):
    """units [num_pages][H][U] -> K, V [len(page_ids)][H][P][D]."""
    units = np.ascontiguousarray(units, np.uint8)
    H = units.shape[1]
    ids = np.ascontiguousarray(page_ids, np.int32)
    pool = np.ascontiguousarray(pool if pool is not None and len(pool) else np.zeros(1, np.uint16), np.uint16)
    K = np.zeros((len(ids), H, P, D), np.uint16)
    V = np.zeros((len(ids), H, P, D), np.uint16)
    lib().kvzo_decode_pages(_p(units), _p(pool), _p(ids), len(ids), H, P, D, _p(K), _p(V))
    return K, V


def decode_attention_rows(q, units, pool, page_table, seq_lens, tail_k, tail_v, Hkv, P, sm_scale, rows):
    """fp64 outputs [len(rows)][D] for (request, query head) pairs, from compressed units."""
    q = np.ascontiguousarray(q, np.uint16)
    B, Hq, D = q.shape
    units = np.ascontiguousarray(units, np.uint8)
    pool = np.ascontiguousarray(pool if pool is not None and len(pool) else np.zeros(1, np.uint16), np.uint16)
    pt = np.ascontiguousarray(page_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    tk = np.ascontiguousarray(tail_k, np.uint16)
    tv = np.ascontiguousarray(tail_v, np.uint16)
    rw = np.ascontiguousarray(np.asarray(rows, np.int32).reshape(-1, 2))
    out = np.zeros((rw.shape[0], D), np.float64)
    lib().kvzo_decode_attention_rows(_p(q), _p(units), _p(pool), _p(pt), pt.shape[1], _p(sl), _p(tk), _p(tv),
                                     Hq, Hkv, D, P, float(sm_scale), _p(rw), rw.shape[0], _p(out))
    return out


def dense_attention_rows(q, k_pages, v_pages, page_table, seq_lens, sm_scale, rows):
    """fp64 outputs [len(rows)][D] for (request, query head) pairs, from dense pages."""
    q = np.ascontiguousarray(q, np.uint16)
    B, Hq, D = q.shape
    kp = np.ascontiguousarray(k_pages, np.uint16)
    vp = np.ascontiguousarray(v_pages, np.uint16)
    _, Hkv, P, _ = kp.shape
    pt = np.ascontiguousarray(page_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    rw = np.ascontiguousarray(np.asarray(rows, np.int32).reshape(-1, 2))
    out = np.zeros((rw.shape[0], D), np.float64)
    lib().kvzo_dense_attention_rows(_p(q), _p(kp), _p(vp), _p(pt), pt.shape[1], _p(sl), Hq, Hkv, D, P,
                                    float(sm_scale), _p(rw), rw.shape[0], _p(out))
    return out


def num_threads() -> int:
    return int(lib().kvzo_num_threads())


def set_num_threads(n: int) -> None:
    lib().kvzo_set_num_threads(int(n))
