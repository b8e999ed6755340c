"""CPU oracle of single-token decode attention, in float64.

TEST INFRASTRUCTURE ONLY (see oracle/codec.py).

What is computed (ZipFusion summary, §II.A "KV Cache and BF16": decoding compares the current
query with the stored keys, then combines the stored values; §III.C: attention over the
compressed cache is ordinary attention over the exactly rebuilt values):

    s_t = sm_scale * sum_d q_d k_{t,d}
    o   = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s)

for each request r and query head h, over the L_r tokens of the request; the KV head of
query head h is h // (H_q / H_kv) (grouped-query attention: consecutive query heads share
one KV head). Tokens are the full pages listed in the page table, in logical order, then
the rows of the request's uncompressed tail (the ZipFusion summary, §III.D: partially
filled pages stay uncompressed). The online-softmax rescaling a kernel uses is the same
quantity as this plain softmax (FlashSVD review, "FlashAttention-2 and the Cached-Decode
Kernel").

score_rounding_bound gives the tests an allowance for rows that no fp32 evaluation resolves to
the stated tolerances (top logits nearly tied at a large scale); parity of such a row is
unpinned beyond that bound.
"""
from __future__ import annotations

import numpy as np

from . import codec


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """q [D], K [L][D], V [L][D] (BF16 bits) -> o [D] float64. L = 0 gives zeros."""
    if K.shape[0] == 0:
        return np.zeros(q.shape[-1], np.float64)
    qf, Kf, Vf = bf16_to_f64(q), bf16_to_f64(K), bf16_to_f64(V)
    s = sm_scale * (Kf @ qf)
    w = np.exp(s - s.max())
    return (w @ Vf) / w.sum()


def score_rounding_bound(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> float:
    """q [D], K [L][D], V [L][D] (BF16 bits) -> a first-order bound on max_d |o~ - o| for any
    evaluation o~ whose scores carry the rounding of a D-term sum in fp32:

        D * 2^-24 * sm_scale * sum_t p_t * (sum_d |q_d k_{t,d}|) * max_d |v_{t,d} - o_d|

    The products of two BF16 values are exact in fp32; an fp32 sum of D terms in any order is
    within (D - 1) 2^-24 sum |terms| of the exact sum, and do/ds_t = p_t (v_t - o). The pages
    give no tolerance; this is the allowance for rows whose top logits nearly tie at a large
    scale (escape-stress values reach 2^20, logits 1e5 and more), where any fp32 evaluation
    moves the output by far more than the stated bounds. Such rows are not pinned beyond it."""
    if K.shape[0] == 0:
        return 0.0
    qf, Kf, Vf = bf16_to_f64(q), bf16_to_f64(K), bf16_to_f64(V)
    s = sm_scale * (Kf @ qf)
    p = np.exp(s - s.max())
    p /= p.sum()
    o = p @ Vf
    S = sm_scale * np.abs(Kf * qf).sum(axis=1)
    return float(qf.shape[0] * 2.0 ** -24 * (p * S * np.abs(Vf - o).max(axis=1)).sum())


def attend_heads(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """q [Hq][D], K/V [L][Hkv][D] -> o [Hq][D] float64."""
    Hq, Hkv = q.shape[0], K.shape[1]
    grp = Hq // Hkv
    return np.stack([attend(q[h], K[:, h // grp], V[:, h // grp], sm_scale) for h in range(Hq)])


def gather_compressed(units: np.ndarray, pool: np.ndarray, page_ids, tail_k: np.ndarray,
                      tail_v: np.ndarray, L: int, P: int, D: int):
    """Tokens of one request from compressed units and its tail -> K, V [L][Hkv][D].

    units: uint8 [num_pages][Hkv][unit_bytes]; tail_*: uint16 [Hkv][P][D].
    """
    Hkv = units.shape[1]
    full = L // P
    K = np.empty((L, Hkv, D), np.uint16)
    V = np.empty((L, Hkv, D), np.uint16)
    for i in range(full):
        pid = int(page_ids[i])
        for h in range(Hkv):
            k, v = codec.decode_unit(units[pid, h], pool, P, D)
            K[i * P:(i + 1) * P, h] = k
            V[i * P:(i + 1) * P, h] = v
    rest = L - full * P
    K[full * P:] = np.transpose(tail_k[:, :rest], (1, 0, 2))
    V[full * P:] = np.transpose(tail_v[:, :rest], (1, 0, 2))
    return K, V


def gather_dense(k_pages: np.ndarray, v_pages: np.ndarray, page_ids, L: int, P: int):
    """Tokens of one request from dense pages [num_pages][Hkv][P][D] -> K, V [L][Hkv][D]."""
    n = (L + P - 1) // P
    K = np.concatenate([k_pages[int(page_ids[i])].transpose(1, 0, 2) for i in range(n)])[:L] \
        if n else np.zeros((0,) + k_pages.shape[1:2] + k_pages.shape[3:], np.uint16)
    V = np.concatenate([v_pages[int(page_ids[i])].transpose(1, 0, 2) for i in range(n)])[:L] \
        if n else np.zeros((0,) + v_pages.shape[1:2] + v_pages.shape[3:], np.uint16)
    return K, V


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 straight to BF16 (nearest, ties to even), no intermediate float32."""
    x = np.asarray(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    flat, o = x.reshape(-1), out.reshape(-1)
    for i, v in enumerate(flat):
        o[i] = _round_one(float(v))
    return out


def _round_one(v: float) -> int:
    sign = 0x8000 if (v < 0 or (v == 0 and np.signbit(v))) else 0
    a = abs(v)
    if a == 0:
        return sign
    if np.isnan(a):
        return 0x7FC0
    m, e = np.frexp(a)                       # a = m * 2**e, 0.5 <= m < 1
    if e - 1 >= -126:                        # normal BF16: 8 significant bits
        r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    else:                                    # subnormal BF16: multiples of 2**-133
        r = np.ldexp(np.rint(np.ldexp(a, 133)), -133)
    if r >= 2.0 ** 128:
        return sign | 0x7F80
    bits = int(np.array([r], np.float32).view(np.uint32)[0]) >> 16
    return sign | bits
