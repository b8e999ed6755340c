"""Pins of the CPU codec oracle's channel groups (format 2: a group is the 16 tokens of one tile
over 4 adjacent dims) to facts that do not come from the oracle itself.

* Losslessness over all 65,536 BF16 patterns (ZipFusion summary, §II.A "KV Cache and BF16" and
  §III.B "Lossless KV Cache Format": every bit pattern comes back).
* Which values share a base, and where that base is stored: a hand-built block whose only
  exponent outliers fill exactly one channel group.
* The bases and escape counts against a brute force that walks every value's group by its
  definition, with the base rule evaluated over all 256 candidate exponents.
* Only the bases differ from the token groups: payload sign/mantissa bytes and sizes agree.
"""
import numpy as np
import pytest

from oracle import codec

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)
CH = codec.CHANNEL


@pytest.mark.parametrize("D", [64, 128])
def test_all_bit_patterns_round_trip(D):
    rng = np.random.default_rng(D)
    for vals in (ALL, rng.permutation(ALL)):
        blocks = vals.reshape(-1, 2, 16, D)          # (K, V) pairs of 16-token pages
        for K, V in blocks[::7]:
            unit, pool = codec.encode_unit(K, V, geometry=CH)
            k, v = codec.decode_unit(unit, pool if len(pool) else None, 16, D, geometry=CH)
            assert np.array_equal(k, K) and np.array_equal(v, V)
        # every pattern, through blocks of one page each
        flat = vals.reshape(-1, 16, D)
        for X in flat:
            for kind in (codec.K_KIND, codec.V_KIND):
                b, p, e = codec.encode_block(X, kind, geometry=CH)
                assert np.array_equal(codec.decode_block(b, p, e, 16, D, kind, geometry=CH), X)


@pytest.mark.parametrize("P,D,t,j", [(16, 128, 0, 5), (32, 128, 1, 31), (32, 64, 1, 0), (48, 64, 2, 15)])
def test_one_channel_group_of_outliers(P, D, t, j):
    """Values of exponent 127 except tokens [16t, 16t + 16) x dims [4j, 4j + 4), exponent 60: in
    channel groups those 64 values are one group of their own (base 60, stored at byte
    t * D/4 + j), nothing escapes; in token groups each of the 16 rows holds 4 outliers among
    64, which escape."""
    X = np.full((P, D), 0x3F80, np.uint16)          # 1.0: exponent 127
    X[16 * t:16 * t + 16, 4 * j:4 * j + 4] = (60 << 7) | 0x15
    bases, _, esc = codec.encode_block(X, codec.K_KIND, geometry=CH)
    want = np.full(P * D // 64, 127)
    want[t * (D // 4) + j] = 60
    assert np.array_equal(bases, want) and len(esc) == 0
    _, _, esc_tok = codec.encode_block(X, codec.K_KIND)
    assert len(esc_tok) == 64


def _brute_bases(X):
    """Base of every channel group, by its definition: for tile t and dims group j, the exponent
    c (over all 256) that the most group values satisfy 0 <= e - c <= 14, among those present in
    the group, smallest on ties."""
    P, D = X.shape
    e = (X.astype(np.int64) >> 7) & 0xFF
    out = []
    for t in range(P // 16):
        for j in range(D // 4):
            vals = [int(e[tok, d]) for tok in range(16 * t, 16 * t + 16) for d in range(4 * j, 4 * j + 4)]
            best, arg = -1, None
            for c in range(256):
                if c not in vals:
                    continue
                n = sum(1 for x in vals if 0 <= x - c <= 14)
                if n > best:
                    best, arg = n, c
            out.append(arg)
    return np.array(out)


@pytest.mark.parametrize("kind", [codec.K_KIND, codec.V_KIND])
def test_bases_and_escapes_by_brute_force(kind):
    rng = np.random.default_rng(7 + kind)
    P, D = 32, 64
    # exponents spread over ~40 binades so that groups escape and ties occur
    e = rng.integers(100, 140, size=(P, D))
    X = ((rng.integers(0, 2, size=(P, D)) << 15) | (e << 7) | rng.integers(0, 128, size=(P, D))).astype(np.uint16)
    bases, payload, esc = codec.encode_block(X, kind, geometry=CH)
    bb = _brute_bases(X)
    assert np.array_equal(bases, bb)
    # escapes: values outside [base, base + 14] of their own group
    vb = np.array([[bb[(tok // 16) * (D // 4) + d // 4] for d in range(D)] for tok in range(P)])
    ee = (X.astype(np.int64) >> 7) & 0xFF
    n_esc = int(((ee < vb) | (ee > vb + 14)).sum())
    assert len(esc) == n_esc > 0


def test_only_the_bases_differ_from_token_groups():
    rng = np.random.default_rng(3)
    K = rng.integers(0, 65536, size=(32, 128), dtype=np.uint32).astype(np.uint16)
    V = rng.integers(0, 65536, size=(32, 128), dtype=np.uint32).astype(np.uint16)
    ut, _ = codec.encode_unit(K, V)
    uc, _ = codec.encode_unit(K, V, geometry=CH)
    assert len(ut) == len(uc) == codec.unit_bytes(32, 128)
    mb, per_tile = codec.meta_bytes(32, 128), 16 * 128
    for blk in range(2):                          # K then V block: tiles of sm bytes, then offsets
        for t in range(2):
            a = mb + blk * codec.block_bytes(32, 128) + t * (per_tile * 3 // 2)
            assert np.array_equal(ut[a:a + per_tile], uc[a:a + per_tile])
