"""Pins of the fp64 attention oracle to closed forms, a library routine and brute force.

* One token -> that token's V; constant V -> that constant; q = 0 -> mean of V (softmax closed forms).
* torch.nn.functional.scaled_dot_product_attention in float64 on the CPU (a library routine).
* A pure-Python loop with math.exp on tiny inputs.
* GQA head mapping, paging and the tail boundary; Python vs C oracle.
* Rounding of float64 to BF16 against hand values and torch's float32 -> bfloat16 cast.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import c_oracle, codec
from synth import f32_to_bf16_bits, make_workload


def _bf(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def test_single_token_returns_its_value():
    rng = np.random.default_rng(0)
    q = _bf(rng.standard_normal(64))
    K = _bf(rng.standard_normal((1, 64)) * 5)
    V = _bf(rng.standard_normal((1, 64)))
    o = oa.attend(q, K, V, 0.125)
    assert np.array_equal(o, oa.bf16_to_f64(V[0]))
    assert np.array_equal(oa.f64_to_bf16_bits(o), V[0])


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(1)
    q = _bf(rng.standard_normal(128))
    K = _bf(rng.standard_normal((37, 128)) * 3)
    row = _bf(rng.standard_normal(128))
    V = np.tile(row, (37, 1))
    o = oa.attend(q, K, V, 1 / math.sqrt(128))
    assert np.allclose(o, oa.bf16_to_f64(row), rtol=1e-14, atol=0)
    assert np.array_equal(oa.f64_to_bf16_bits(o), row)


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    K = _bf(rng.standard_normal((50, 64)) * 10)
    V = _bf(rng.standard_normal((50, 64)))
    o = oa.attend(np.zeros(64, np.uint16), K, V, 0.125)
    assert np.allclose(o, oa.bf16_to_f64(V).mean(axis=0), rtol=1e-13, atol=1e-15)


def test_empty_context_gives_zero():
    o = oa.attend(np.zeros(64, np.uint16), np.zeros((0, 64), np.uint16), np.zeros((0, 64), np.uint16), 1.0)
    assert not o.any()


@pytest.mark.parametrize("L", [1, 2, 3, 7, 16, 17, 40])
def test_matches_torch_sdpa_fp64(L):
    rng = np.random.default_rng(L)
    q = _bf(rng.standard_normal(64))
    K = _bf(rng.standard_normal((L, 64)) * 2)
    V = _bf(rng.standard_normal((L, 64)))
    o = oa.attend(q, K, V, 0.125)
    tq = torch.from_numpy(oa.bf16_to_f64(q)).view(1, 1, 1, 64)
    tk = torch.from_numpy(oa.bf16_to_f64(K)).view(1, 1, L, 64)
    tv = torch.from_numpy(oa.bf16_to_f64(V)).view(1, 1, L, 64)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.125).view(64).numpy()
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-14)


def test_matches_python_loop():
    rng = np.random.default_rng(9)
    q = _bf(rng.standard_normal(64))
    K = _bf(rng.standard_normal((9, 64)))
    V = _bf(rng.standard_normal((9, 64)))
    qf, Kf, Vf = oa.bf16_to_f64(q), oa.bf16_to_f64(K), oa.bf16_to_f64(V)
    s = [0.3 * sum(qf[d] * Kf[t][d] for d in range(64)) for t in range(9)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    ref = [sum(w[t] * Vf[t][d] for t in range(9)) / sum(w) for d in range(64)]
    assert np.allclose(oa.attend(q, K, V, 0.3), ref, rtol=1e-13, atol=1e-15)


def test_gqa_head_mapping():
    # 6 query heads on 2 KV heads: heads 0-2 read KV head 0, heads 3-5 read KV head 1.
    rng = np.random.default_rng(4)
    q = _bf(rng.standard_normal((6, 64)))
    K = _bf(rng.standard_normal((5, 2, 64)))
    V = np.empty((5, 2, 64), np.uint16)
    V[:, 0] = _bf(np.full(64, 1.0))
    V[:, 1] = _bf(np.full(64, -3.0))
    o = oa.attend_heads(q, K, V, 0.125)
    assert np.all(o[:3] == 1.0) and np.all(o[3:] == -3.0)


def test_paging_and_tail_match_flat_attention():
    w = make_workload(4, B=3, lens=[5, 16, 45], Hq=4, Hkv=2, D=64)
    kp, vp = w.pages(0), w.pages(1)
    units, pool, _ = c_oracle.encode_pages(kp, vp)
    q = w.q()
    for r in range(w.B):
        L = int(w.seq_lens[r])
        K, V = oa.gather_dense(kp, vp, w.page_table[r], L, w.P)
        full = L // w.P
        tail_pid = w.page_table[r, full] if L % w.P else None
        tk = kp[tail_pid] if tail_pid is not None else np.zeros((w.Hkv, w.P, w.D), np.uint16)
        tv = vp[tail_pid] if tail_pid is not None else np.zeros((w.Hkv, w.P, w.D), np.uint16)
        K2, V2 = oa.gather_compressed(units, pool, w.page_table[r], tk, tv, L, w.P, w.D)
        assert np.array_equal(K, K2) and np.array_equal(V, V2)
        flat_k = np.stack([w.token(r, t, 0) for t in range(L)])
        assert np.array_equal(K, flat_k)
        o = oa.attend_heads(q[r], K, V, w.sm_scale)
        rows = [(r, h) for h in range(w.Hq)]
        co = c_oracle.decode_attention_rows(q, units, pool, w.page_table, w.seq_lens,
                                            _tails(w, kp, 0), _tails(w, vp, 1), w.Hkv, w.P, w.sm_scale, rows)
        assert np.allclose(co, o, rtol=1e-12, atol=1e-14)
        do = c_oracle.dense_attention_rows(q, kp, vp, w.page_table, w.seq_lens, w.sm_scale, rows)
        assert np.allclose(do, o, rtol=1e-12, atol=1e-14)


def _tails(w, pages, tensor):
    t = np.zeros((w.B, w.Hkv, w.P, w.D), np.uint16)
    for r in range(w.B):
        L = int(w.seq_lens[r])
        if L % w.P:
            t[r] = pages[w.page_table[r, L // w.P]]
    return t


def test_f64_to_bf16_rounding():
    # 1 + 2^-8 is halfway between 1.0 (0x3F80) and 1 + 2^-7 (0x3F81): ties to even -> 0x3F80;
    # 1 + 3*2^-8 is halfway between 0x3F81 and 0x3F82 -> 0x3F82; just above the tie rounds up.
    assert oa.f64_to_bf16_bits(np.array([1 + 2 ** -8]))[0] == 0x3F80
    assert oa.f64_to_bf16_bits(np.array([1 + 3 * 2 ** -8]))[0] == 0x3F82
    assert oa.f64_to_bf16_bits(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 0x3F81
    assert oa.f64_to_bf16_bits(np.array([-2.0]))[0] == 0xC000
    assert oa.f64_to_bf16_bits(np.array([-0.0]))[0] == 0x8000
    assert oa.f64_to_bf16_bits(np.array([2.0 ** -133]))[0] == 0x0001
    assert oa.f64_to_bf16_bits(np.array([3.5e38]))[0] == 0x7F80
    # float32-representable inputs: agrees with torch's nearest-even cast
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(oa.f64_to_bf16_bits(x.astype(np.float64)), ref)
