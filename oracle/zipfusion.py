"""CPU oracle of ZipFusion's own KV block format, the second codec of this repository.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may import this package; the library under decode_attention_losslessly_amd/ never does.
It shares no code, constants or helpers with the HIP path.

What the pages fix (ZipFusion: Fusing Lossless KV Decompression with Attention, the
paperlayer.ai summary, §III.B "Lossless KV Cache Format" and §III.C "Attention over the
Compressed KV Cache"):
  * a block is compressed only when every exponent in it lies in [b, b + 15], b being the
    smallest exponent of the block rounded down to an even number; other blocks stay raw;
  * a compressed value keeps its low byte (lowest exponent bit and the 7 fraction bits) and a
    4-bit code made of its sign and 3 exponent-offset bits; two codes share a byte, so a value
    costs 12 bits and a 512-value block 768 instead of 1024 bytes;
  * the low bytes come first, contiguous, then the packed codes;
  * the rebuild is exact (integer fields only).

Readings of this repository (the pages leave them open):
  * a block is 512 consecutive storage positions of a 16-token tile, in the same storage order
    as the main format: K token-major (tok*D + d), V dim-major (d*16 + tok); a tile holds D/32
    blocks;
  * code = sign << 3 | k with k = e//2 - b//2 (0..7); the lowest exponent bit travels in the
    low byte; the even position of a code byte is its low nibble;
  * per block one metadata byte: b//2 when compressed, 0xFF when raw;
  * a raw block is its 512 BF16 values in storage order, kept outside the unit (a pool).

Unit layout (one page of one head, K blocks then V blocks, tile by tile):
  meta   [K block bytes: T*G2] [V block bytes: T*G2] zero pad to 8 bytes, u64 raw-pool offset
         (u16 elements; all ones when the unit has no raw block), zero pad to 128 bytes;
         T = P/16 tiles, G2 = D/32 blocks per tile
  slots  2*T*G2 slots of 768 bytes in the same block order; a raw block's slot is zero and its
         values are in the pool at offset + 512 * (its rank among the unit's raw blocks).
"""
from __future__ import annotations

import numpy as np

BLOCK = 512             # values per block
COMPRESSED_BYTES = 768  # 512 low bytes + 256 code bytes
RAW = 0xFF
NO_RAW = (1 << 64) - 1


def exponent(x):
    """8-bit exponent field of BF16 bit patterns (§II.A)."""
    return (np.asarray(x, dtype=np.uint32) >> 7) & 0xFF


def block_base(x) -> int:
    """The block's minimum exponent rounded down to an even number (§III.B)."""
    return int(exponent(x).min()) & ~1


def eligible(x) -> bool:
    """Every exponent within [b, b + 15] (§III.B)."""
    e = exponent(x)
    return int(e.max()) - block_base(x) <= 15


def encode_block(x) -> tuple[int, bytes | None]:
    """One block of 512 BF16 patterns (storage order) -> (meta byte, 768 bytes or None if raw)."""
    x = np.asarray(x, dtype=np.uint16)
    assert x.shape == (BLOCK,)
    if not eligible(x):
        return RAW, None
    b = block_base(x)
    e = exponent(x)
    sign = (x.astype(np.uint32) >> 15) & 1
    k = (e >> 1) - (b >> 1)
    assert np.all((k >= 0) & (k <= 7))
    code = ((sign << 3) | k).astype(np.uint8)
    low = (x & 0xFF).astype(np.uint8)                 # lowest exponent bit + 7 fraction bits
    packed = (code[0::2] | (code[1::2] << 4)).astype(np.uint8)
    return b >> 1, low.tobytes() + packed.tobytes()


def decode_block(meta: int, data: bytes) -> np.ndarray:
    """Inverse of encode_block for a compressed block: bits = sign<<15 | (b/2 + k)<<8 | low byte."""
    assert meta != RAW and len(data) == COMPRESSED_BYTES
    buf = np.frombuffer(data, dtype=np.uint8)
    low = buf[:BLOCK].astype(np.uint16)
    packed = buf[BLOCK:]
    code = np.empty(BLOCK, dtype=np.uint16)
    code[0::2] = packed & 0xF
    code[1::2] = packed >> 4
    sign = (code >> 3) & 1
    high = (sign << 7) | (meta + (code & 7))
    return ((high << 8) | low).astype(np.uint16)


# ---------------------------------------------------------------- unit
def blocks_per_tile(D: int) -> int:
    return 16 * D // BLOCK


def meta_bytes(P: int, D: int) -> int:
    nb = 2 * (P // 16) * blocks_per_tile(D)
    return (((nb + 7) // 8 * 8 + 8) + 127) // 128 * 128


def unit_bytes(P: int, D: int) -> int:
    return meta_bytes(P, D) + 2 * (P // 16) * blocks_per_tile(D) * COMPRESSED_BYTES


def _storage(X: np.ndarray, kind: str) -> np.ndarray:
    """[P][D] token-major values -> storage order, tile by tile."""
    P, D = X.shape
    out = []
    for t in range(P // 16):
        tile = X[16 * t:16 * t + 16]
        out.append(tile.reshape(-1) if kind == "K" else tile.T.reshape(-1))
    return np.concatenate(out)


def _from_storage(s: np.ndarray, P: int, D: int, kind: str) -> np.ndarray:
    X = np.empty((P, D), dtype=np.uint16)
    n = 16 * D
    for t in range(P // 16):
        chunk = s[t * n:(t + 1) * n]
        X[16 * t:16 * t + 16] = chunk.reshape(16, D) if kind == "K" else chunk.reshape(D, 16).T
    return X


def encode_unit(K, V, pool_offset: int = 0) -> tuple[bytes, np.ndarray]:
    """K, V: uint16 [P][D] token-major. Returns (unit bytes, raw-pool values of this unit).
    pool_offset is where the caller places the unit's raw values (used only if there are any)."""
    K = np.asarray(K, dtype=np.uint16)
    V = np.asarray(V, dtype=np.uint16)
    P, D = K.shape
    metas, slots, raw = [], [], []
    for X, kind in ((K, "K"), (V, "V")):
        s = _storage(X, kind)
        for j in range(len(s) // BLOCK):
            m, data = encode_block(s[j * BLOCK:(j + 1) * BLOCK])
            metas.append(m)
            if data is None:
                raw.append(s[j * BLOCK:(j + 1) * BLOCK])
                slots.append(bytes(COMPRESSED_BYTES))
            else:
                slots.append(data)
    nb = len(metas)
    meta = bytearray(meta_bytes(P, D))
    meta[:nb] = bytes(metas)
    off = (nb + 7) // 8 * 8
    meta[off:off + 8] = int(pool_offset if raw else NO_RAW).to_bytes(8, "little")
    pool = np.concatenate(raw).astype(np.uint16) if raw else np.zeros(0, dtype=np.uint16)
    return bytes(meta) + b"".join(slots), pool


def unit_raw_offset(unit: bytes, P: int, D: int) -> int:
    nb = 2 * (P // 16) * blocks_per_tile(D)
    off = (nb + 7) // 8 * 8
    return int.from_bytes(unit[off:off + 8], "little")


def decode_unit(unit: bytes, pool: np.ndarray, P: int, D: int) -> tuple[np.ndarray, np.ndarray]:
    """Unit bytes (+ the raw pool it points into) -> K, V uint16 [P][D]."""
    nb = 2 * (P // 16) * blocks_per_tile(D)
    mb = meta_bytes(P, D)
    base = unit_raw_offset(unit, P, D)
    rank = 0
    vals = []
    for j in range(nb):
        m = unit[j]
        if m == RAW:
            vals.append(np.asarray(pool[base + BLOCK * rank: base + BLOCK * (rank + 1)], dtype=np.uint16))
            rank += 1
        else:
            vals.append(decode_block(m, unit[mb + j * COMPRESSED_BYTES: mb + (j + 1) * COMPRESSED_BYTES]))
    s = np.concatenate(vals)
    half = len(s) // 2
    return _from_storage(s[:half], P, D, "K"), _from_storage(s[half:], P, D, "V")


def raw_blocks(unit: bytes, P: int, D: int) -> int:
    nb = 2 * (P // 16) * blocks_per_tile(D)
    return sum(1 for j in range(nb) if unit[j] == RAW)
