"""Pins of the ZipFusion block-format oracle (oracle/zipfusion.py) to what the pages fix and to
the mathematics, independent of the oracle's own code:

* the 768-of-1024-byte size of an eligible 512-value block (tests/golden/block_size.txt; ZipFusion
  summary §III.B);
* the eligibility rule at its boundary, for an even and an odd smallest exponent (§III.B);
* exhaustive round trip: every BF16 pattern whose exponent lies in a window [b, b + 15], b even,
  for every such window (zeros, subnormals, Inf and NaN payloads included);
* the rebuilt high byte equals sign << 7 | (b/2 + k) and b/2 + k never exceeds 127, so one 32-bit
  add of four such bytes cannot carry between them (§III.C);
* raw blocks (exponent span above 15) round-trip through the pool;
* a hand-derived unit: meta bytes, slot order, V blocks dim-major.
"""
import os

import numpy as np
import pytest

from oracle import zipfusion as zf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(sign, exp, mant):
    return np.uint16((sign << 15) | (exp << 7) | mant)


def test_block_size_golden():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "block_size.txt")) if ln.strip() and ln[0] != "#"]
    P, D, n, comp, dense = map(int, rows[0])
    assert n == zf.BLOCK and zf.blocks_per_tile(D) * zf.BLOCK == 16 * D
    rng = np.random.default_rng(0)
    x = np.array([_bf16(int(s), 120 + int(e), int(m)) for s, e, m in
                  zip(rng.integers(0, 2, n), rng.integers(0, 16, n), rng.integers(0, 128, n))], np.uint16)
    meta, data = zf.encode_block(x)
    assert meta != zf.RAW and len(data) == comp
    assert x.nbytes == dense


@pytest.mark.parametrize("lo", [100, 101])
def test_eligibility_boundary(lo):
    b = lo & ~1
    base = np.array([_bf16(0, lo, 5)] * zf.BLOCK, np.uint16)
    inside, outside = base.copy(), base.copy()
    inside[7] = _bf16(1, b + 15, 3)        # top of the window [b, b + 15]
    outside[7] = _bf16(1, b + 16, 3)
    assert zf.eligible(inside) and zf.encode_block(inside)[0] == b // 2
    assert not zf.eligible(outside) and zf.encode_block(outside) == (zf.RAW, None)


def test_every_pattern_in_every_window_round_trips():
    for b in range(0, 241, 2):
        pats = np.array([_bf16(s, e, m) for e in range(b, b + 16) for s in (0, 1) for m in range(128)], np.uint16)
        assert pats.size == 4096
        rng = np.random.default_rng(b)
        for order in (pats, rng.permutation(pats)):
            for j in range(0, pats.size, zf.BLOCK):
                blk = order[j:j + zf.BLOCK]
                meta, data = zf.encode_block(blk)
                assert meta != zf.RAW
                out = zf.decode_block(meta, data)
                assert np.array_equal(out, blk)


def test_high_byte_formula_and_no_carry():
    rng = np.random.default_rng(1)
    for _ in range(200):
        b = int(rng.integers(0, 121)) * 2
        e = rng.integers(b, b + 16, zf.BLOCK)
        x = ((rng.integers(0, 2, zf.BLOCK) << 15) | (e << 7) | rng.integers(0, 128, zf.BLOCK)).astype(np.uint16)
        meta, data = zf.encode_block(x)
        buf = np.frombuffer(data, np.uint8)
        low, packed = buf[:512], buf[512:]
        codes = np.empty(512, np.int64)
        codes[0::2], codes[1::2] = packed & 15, packed >> 4
        k = codes & 7
        assert np.all(meta + k <= 127)                       # the 7-bit field never reaches the sign bit
        high = ((codes >> 3) << 7) | (meta + k)
        assert np.array_equal((high << 8) | low, x.astype(np.int64))
        assert np.array_equal(low, x & 0xFF)                 # the low byte is kept as is


def test_raw_blocks_round_trip_through_the_pool():
    rng = np.random.default_rng(2)
    P, D = 32, 64
    K = rng.integers(0, 1 << 16, (P, D)).astype(np.uint16)   # exponent span far above 15
    V = np.full((P, D), _bf16(0, 127, 1), np.uint16)         # one exponent: compressed
    unit, pool = zf.encode_unit(K, V, pool_offset=40)
    nb = 2 * (P // 16) * zf.blocks_per_tile(D)
    assert zf.raw_blocks(unit, P, D) == nb // 2 and pool.size == zf.BLOCK * nb // 2
    full_pool = np.concatenate([np.zeros(40, np.uint16), pool])
    K2, V2 = zf.decode_unit(unit, full_pool, P, D)
    assert np.array_equal(K2, K) and np.array_equal(V2, V)
    unit2, pool2 = zf.encode_unit(V, V)
    assert zf.unit_raw_offset(unit2, P, D) == zf.NO_RAW and pool2.size == 0


def test_hand_derived_unit_layout():
    P, D = 16, 64                                            # one tile, 2 K blocks + 2 V blocks
    K = np.zeros((P, D), np.uint16)
    V = np.zeros((P, D), np.uint16)
    K[:8, :] = _bf16(0, 130, 0)                              # K block 0 = tokens 0..7 (token-major)
    K[8:, :] = _bf16(1, 140, 9)                              # K block 1 = tokens 8..15
    V[:, :32] = _bf16(0, 121, 2)                             # V block 0 = dims 0..31 (dim-major)
    V[:, 32:] = _bf16(0, 125, 4)
    unit, pool = zf.encode_unit(K, V)
    assert zf.meta_bytes(P, D) == 128 and len(unit) == 128 + 4 * 768 == zf.unit_bytes(P, D)
    assert list(unit[:4]) == [65, 70, 60, 62]                # b/2 of each block, K then V
    assert unit[8:16] == b"\xff" * 8                         # no raw block
    slot = lambda j: np.frombuffer(unit[128 + 768 * j:128 + 768 * (j + 1)], np.uint8)
    assert np.all(slot(1)[:512] == 9) and np.all(slot(1)[512:] == 0x88)   # sign 1, k 0 in both nibbles
    assert np.all(slot(2)[:512] == 0x82)                     # exponent 121: low bit 1, mantissa 2
    assert np.all(slot(3)[512:] == 0x00)                     # 125 // 2 - 124 // 2 = 0
