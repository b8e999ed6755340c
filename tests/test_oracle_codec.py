"""Pins of the CPU codec oracle to facts that do not come from the oracle itself.

* BF16 field split and known encodings (tests/golden/bf16_fields.txt; ZipFusion summary §II.A).
* Losslessness over all 65,536 BF16 patterns (§II.A, §III.B: every bit pattern preserved).
* The base rule, checked by brute force over all 256 candidate exponents.
* Hand-derived encodings of small groups and blocks (closed forms of the definition).
* Payload size against the 768-of-1024-byte figure (tests/golden/block_size.txt; §III.B).
* The Python and C oracles, written separately, agree byte for byte.
"""
import os

import numpy as np
import pytest

from oracle import c_oracle, codec
from synth import make_workload

GOLD = os.path.join(os.path.dirname(__file__), "golden")
ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _golden_rows(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


def test_bf16_fields_golden():
    for hx, s, e, m, val in _golden_rows("bf16_fields.txt"):
        x = np.uint16(int(hx, 16))
        assert int(codec.exponent(x)) == int(e)
        assert int(codec.sm_byte(x)) == (int(s) << 7) | int(m)
        f = np.array([int(hx, 16) << 16], np.uint32).view(np.float32)[0]
        if val == "nan":
            assert np.isnan(f)
        else:
            assert f == np.float32(float(val)), hx


def test_exponent_matches_frexp_for_normals():
    f = (ALL.astype(np.uint32) << 16).view(np.float32)
    e = codec.exponent(ALL)
    normal = (e > 0) & (e < 255)
    _, fe = np.frexp(f[normal].astype(np.float64))
    assert np.array_equal(e[normal], fe + 126)          # |x| in [2^(e-127), 2^(e-126))
    sign = (codec.sm_byte(ALL) >> 7).astype(bool)
    assert np.array_equal(sign[~np.isnan(f)], np.signbit(f[~np.isnan(f)]))


def _groups_exhaustive(seed):
    """All 65,536 patterns as 64-value groups: in order, permuted, and with random partners."""
    rng = np.random.default_rng(seed)
    out = [ALL.reshape(1024, 64)]
    for _ in range(3):
        out.append(rng.permutation(ALL).reshape(1024, 64))
    part = rng.integers(0, 65536, size=(65536, 64), dtype=np.uint32).astype(np.uint16)
    part[:, 0] = ALL
    out.append(part[rng.choice(65536, 4096, replace=False)])
    return np.concatenate(out)


def test_group_round_trip_exhaustive():
    g = _groups_exhaustive(0)
    for x in g[::7]:
        b, off, sm, esc = codec.encode_group(x)
        assert np.array_equal(codec.decode_group(b, off, sm, esc), x)


def _brute_cov(e, c):
    return int(((e - c >= 0) & (e - c <= 14)).sum())


def test_base_is_optimal_brute_force():
    rng = np.random.default_rng(1)
    groups = [codec.exponent(x).astype(np.int32) for x in _groups_exhaustive(2)[::41]]
    for _ in range(300):   # narrow spans: many ties and near ties
        lo = int(rng.integers(0, 230))
        groups.append(rng.integers(lo, lo + int(rng.integers(1, 26)), size=64).astype(np.int32))
    bases = codec.choose_bases(np.stack(groups))
    for e, b in zip(groups, bases):
        covs = np.array([_brute_cov(e, c) for c in range(256)])
        best = covs.max()
        assert _brute_cov(e, b) == best
        assert b in e
        assert b == min(c for c in np.unique(e) if covs[c] == best)     # smallest on ties
        assert int((codec.offsets(e, b) == 15).sum()) == 64 - best
        assert c_oracle.group_base(e) == b


def test_narrow_span_has_min_base_and_no_escape():
    rng = np.random.default_rng(3)
    for _ in range(500):
        lo = int(rng.integers(0, 242))
        e = rng.integers(lo, lo + int(rng.integers(1, 16)), size=64).astype(np.int32)
        b = int(codec.choose_bases(e[None])[0])
        assert b == e.min()
        assert not (codec.offsets(e, b) == 15).any()


def test_hand_derived_group():
    # 61 values of 1.0 (0x3F80, exponent 127), one each of 2.0 (0x4000, exponent 128), -0.5 (0xBF00, exp 126),
    # and 2^14 = 16384.0 (0x4680, exponent 141) -> window [126, 140] covers 63 values, [127, 141]
    # covers 63 too (1.0 x61, 2.0, 2^14); both tie at 63, so the base is 126 and
    # 2^14 (offset 15 from 126) escapes. sm bytes: 1.0 -> 0x00, 2.0 -> 0x00, -0.5 -> 0x80,
    # 2^14 -> 0x00. Offsets: 1.0 -> 1, 2.0 -> 2, -0.5 -> 0.
    x = np.full(64, 0x3F80, np.uint16)
    x[10], x[20], x[30] = 0x4000, 0xBF00, 0x4680
    b, off, sm, esc = codec.encode_group(x)
    assert b == 126
    want = np.ones(64, np.uint8)
    want[10], want[20], want[30] = 2, 0, 15
    assert np.array_equal(off, want)
    assert sm[20] == 0x80 and sm.sum() == 0x80
    assert list(esc) == [0x4680]
    # dropping -0.5: window [127, 141] now covers all 64 and the base moves to 127
    x[20] = 0x3F80
    b, off, _, esc = codec.encode_group(x)
    assert b == 127 and len(esc) == 0 and off[30] == 14


def test_hand_derived_offset_word_layout():
    # storage offsets 0..7 -> even positions in the low half-word, odd in the high half-word
    off = np.array([1, 2, 3, 4, 5, 6, 7, 8], np.uint8)
    w = int(codec.pack_offsets(off)[0])
    assert w == (1 | 3 << 4 | 5 << 8 | 7 << 12 | 2 << 16 | 4 << 20 | 6 << 24 | 8 << 28)
    assert np.array_equal(codec.unpack_offsets(np.array([w], np.uint32)), off)


def test_hand_derived_block_layout():
    # A K block and a V block of one tile: value (tok, d) = exponent 100 + (tok % 15), mantissa
    # d % 128, sign tok % 2. Every group spans exponents 100..114 only within one token row, so
    # each row's base is that row's exponent and no value escapes; offsets are all 0.
    P, D = 16, 64
    X = np.zeros((P, D), np.uint16)
    for tok in range(P):
        for d in range(D):
            X[tok, d] = ((tok % 2) << 15) | ((100 + tok % 15) << 7) | (d % 128)
    kb, kp, ke = codec.encode_block(X, codec.K_KIND)
    vb, vp, ve = codec.encode_block(X, codec.V_KIND)
    assert len(ke) == 0 and len(ve) == 0
    # bases: [group][tok] -> one group per row here
    assert list(kb) == [100 + tok % 15 for tok in range(P)]
    assert list(vb) == list(kb)
    # K sm bytes token-major: byte tok*D + d = sign<<7 | d
    assert kp[5 * D + 7] == (1 << 7) | 7
    # V sm bytes dim-major: byte d*16 + tok
    assert vp[7 * 16 + 5] == (1 << 7) | 7
    assert vp[7 * 16 + 4] == 7
    # offsets all zero
    assert not kp[P * D:].any() and not vp[P * D:].any()
    assert len(kp) == P * D * 3 // 2


def test_escape_order_is_storage_order():
    # a V tile where (tok 3, d 1) and (tok 1, d 2) escape: dim-major order puts d=1 first;
    # token-major K order puts tok 1 first.
    P, D = 16, 64
    X = np.full((P, D), 0x3F80, np.uint16)
    X[3, 1] = 0x7F00
    X[1, 2] = 0x7E80
    _, _, ke = codec.encode_block(X, codec.K_KIND)
    _, _, ve = codec.encode_block(X, codec.V_KIND)
    assert list(ke) == [0x7E80, 0x7F00]
    assert list(ve) == [0x7F00, 0x7E80]


def test_inline_positions_repeat_the_offset_codes():
    # the position recorded with each inline escape is where its offset code 15 sits
    w = make_workload(3, B=1, L=64, Hq=4, Hkv=4)
    K, V = w.pages(0), w.pages(1)
    seen = 0
    for p in range(K.shape[0]):
        for h in range(w.Hkv):
            unit, pool = codec.encode_unit(K[p, h], V[p, h])
            pos = codec.inline_positions(unit, w.P, w.D)
            assert pos is not None
            for kind, X, ps in ((codec.K_KIND, K[p, h], pos[0]), (codec.V_KIND, V[p, h], pos[1])):
                order = codec.storage_order(w.P, w.D, kind)
                off = codec.offsets(codec.exponent(X).reshape(w.P, -1, 64),
                                    codec.choose_bases(codec.exponent(X).reshape(w.P, -1, 64))).reshape(-1)
                assert list(ps) == list(np.nonzero(off[order] == 15)[0])
                seen += len(ps)
    assert seen > 0


def test_sizes():
    assert codec.block_bytes(16, 128) == 3072
    # meta = bases (2*P*D/64 bytes) + 16-byte header + 4-byte inline entries, rounded to 128
    assert codec.meta_bytes(16, 128) == 128 and codec.inline_capacity(16, 128) == 12
    assert codec.unit_bytes(16, 128) == 128 + 6144
    assert codec.meta_bytes(256, 64) == 640 and codec.inline_capacity(256, 64) == 28
    for P, D in [(16, 64), (16, 128), (32, 256), (256, 64)]:
        assert c_oracle.unit_bytes(P, D) == codec.unit_bytes(P, D)
        assert c_oracle.inline_capacity(P, D) == codec.inline_capacity(P, D)


def test_payload_size_golden():
    for P, D, n, comp, dense in _golden_rows("block_size.txt"):
        P, D, n = int(P), int(D), int(n)
        assert codec.block_bytes(P, D) * n // (P * D) == int(comp)
        assert 2 * n == int(dense)


@pytest.mark.parametrize("P,D", [(16, 64), (16, 128), (32, 128), (256, 64)])
def test_unit_round_trip_all_patterns(P, D):
    rng = np.random.default_rng(P * 1000 + D)
    vals = np.concatenate([ALL, rng.permutation(ALL)])
    n = P * D
    for s in range(0, len(vals) - 2 * n + 1, 2 * n):
        K = vals[s:s + n].reshape(P, D)
        V = vals[s + n:s + 2 * n].reshape(P, D)
        unit, pool = codec.encode_unit(K, V, pool_offset=0)
        k2, v2 = codec.decode_unit(unit, pool, P, D)
        assert np.array_equal(k2, K) and np.array_equal(v2, V)
        cu, cp = c_oracle.encode_unit(K, V, 0)
        assert np.array_equal(cu, unit) and np.array_equal(cp, pool)
        k3, v3 = c_oracle.decode_unit(unit, pool, P, D)
        assert np.array_equal(k3, K) and np.array_equal(v3, V)


def test_every_pattern_round_trips_in_c_oracle():
    P, D = 16, 128
    blocks = _groups_exhaustive(5).reshape(-1, P, D)
    n = blocks.shape[0] // 2
    K, V = blocks[:n][:, None], blocks[n:2 * n][:, None]
    units, pool, _ = c_oracle.encode_pages(np.ascontiguousarray(K), np.ascontiguousarray(V))
    k2, v2 = c_oracle.decode_pages(units, pool, np.arange(n), P, D)
    assert np.array_equal(k2, K) and np.array_equal(v2, V)
    seen = np.zeros(65536, bool)
    seen[K.reshape(-1)] = True
    seen[V.reshape(-1)] = True
    assert seen.all()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6])
def test_python_and_c_oracles_agree_on_configs(cfg):
    w = make_workload(cfg)
    ids = np.arange(min(6, w.num_pages))
    K, V = w.pages(0, ids), w.pages(1, ids)
    units, pool, end = c_oracle.encode_pages(K, V)
    off = 0
    for i in range(len(ids)):
        for h in range(0, w.Hkv, max(1, w.Hkv // 3)):
            u, p = codec.encode_unit(K[i, h], V[i, h], pool_offset=off)
            kc, vc, o = codec.unit_header(units[i, h], w.P, w.D)
            if o != codec.INLINE:
                u, p = codec.encode_unit(K[i, h], V[i, h], pool_offset=o)
                assert np.array_equal(pool[o:o + kc + vc], p)
            assert np.array_equal(u, units[i, h])
            k, v = codec.decode_unit(units[i, h], pool, w.P, w.D)
            assert np.array_equal(k, K[i, h]) and np.array_equal(v, V[i, h])
