"""CPU oracle of the lossless BF16 KV-cache format.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may import this package; the library under decode_attention_losslessly_amd/ never does.
It shares no code, constants or helpers with the HIP path.

What the pages fix (ZipFusion: Fusing Lossless KV Decompression with Attention, the
paperlayer.ai summary):
  * §II.A "KV Cache and BF16": a BF16 value is 1 sign, 8 exponent and 7 fraction bits, and a
    lossless format preserves every value's bit pattern.
  * §III.B "Lossless KV Cache Format": values keep their sign and fraction information, the
    exponent is coded as an offset from a per-block base, and the original bits come back
    exactly with no floating-point rounding.
  * §III.C "Attention over the Compressed KV Cache": the values are rebuilt with plain
    integer bit operations.
The layout itself is this repository's (the pages' own 12-bit layout is prior art):

  group      the 64 values of one token row of one head, dims [64g, 64g + 64)
  sm byte    (sign << 7) | mantissa, stored for every value, escaped or not
  base b     of a group: among the group's own exponents, the one that maximises
             cov(c) = #{j : 0 <= e_j - c <= 14}; ties go to the smallest exponent
  offset     e - b when 0 <= e - b <= 14, else 15 = escape; an escaped value's 16 raw bits
             go to the block's escape list
  tile       16 consecutive tokens of a page (P is a multiple of 16)
  storage    K: position tok*D + d inside a tile (token-major)
  order      V: position d*16 + tok inside a tile (dim-major)
  block      the P x D values of one page, one head, one of K / V: for each tile, its
             16*D sm bytes in storage order, then 2*D little-endian u32 offset words;
             word w holds positions 8w..8w+7 with position 8w+2k in bits 4k..4k+3 and
             position 8w+2k+1 in bits 16+4k..16+4k+3
  escapes    a block's escaped values in storage order (tiles in order)
  unit       one (page, KV head): meta region, then the K block, then the V block
  meta       [0, P*G)          K bases, byte t*16G + g*16 + tok for tile t
             [P*G, 2P*G)       V bases, same order
             [2PG, 2PG+4)      u32 number of K escapes
             [2PG+4, 2PG+8)    u32 number of V escapes
             [2PG+8, 2PG+16)   u64 escape-pool offset in u16 elements, or all ones when the
                               escapes are inline
             [2PG+16, MR)      when all escapes fit, one little-endian u32 entry per escape,
                               K's then V's in list order: value | (storage position << 16),
                               the position (within its block) repeating what the offset
                               codes already say; unused bytes zero
             MR = round_up(2PG + 16, 128)

Second geometry, the channel groups (format 2; group shape: §III.B fixes a block's exponent
range, not the shape of the values that share a base): a group is the 16 tokens of one tile
over 4 adjacent dims [4j, 4j + 4), still 64 values, so every size above is unchanged; the base
of tile t's group j is byte t*16G + j of the block's base table (16G = D/4 groups per tile).
Everything else (sm bytes, offsets, storage order, escapes, meta) is the same.
"""
from __future__ import annotations

import numpy as np

GROUP = 64
TILE = 16
CHANNEL_DIMS = 4           # dims of a channel group (over the TILE tokens of a tile)
TOKEN, CHANNEL = "token", "channel"
ESCAPE = 15
MAX_OFFSET = 14
INLINE = 0xFFFF_FFFF_FFFF_FFFF
K_KIND, V_KIND = 0, 1


# ---------------------------------------------------------------- BF16 fields (§II.A)
def exponent(x: np.ndarray) -> np.ndarray:
    return ((np.asarray(x, np.uint16) >> 7) & 0xFF).astype(np.int32)


def sm_byte(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.uint16)
    return (((x >> 8) & 0x80) | (x & 0x7F)).astype(np.uint8)


def rebuild(sm: np.ndarray, e: np.ndarray) -> np.ndarray:
    """BF16 bits from an sm byte and an 8-bit exponent: sign, exponent, mantissa."""
    sm = np.asarray(sm, np.uint16)
    e = np.asarray(e, np.uint16)
    return (((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)).astype(np.uint16)


# ---------------------------------------------------------------- group codec
def coverage(exps: np.ndarray) -> np.ndarray:
    """cov[..., i] = number of j with 0 <= e_j - e_i <= 14, for a [..., 64] exponent array."""
    d = exps[..., None, :] - exps[..., :, None]          # d[..., i, j] = e_j - e_i
    return ((d >= 0) & (d <= MAX_OFFSET)).sum(axis=-1)


def choose_bases(exps: np.ndarray) -> np.ndarray:
    """Base per group: the group exponent of largest coverage, smallest on ties."""
    exps = np.asarray(exps, np.int32)
    flat = exps.reshape(-1, GROUP)
    out = np.empty(flat.shape[0], np.int32)
    step = 4096
    for s in range(0, flat.shape[0], step):
        e = flat[s:s + step]
        cov = coverage(e)
        best = cov.max(axis=-1, keepdims=True)
        cand = np.where(cov == best, e, 256)              # exponents reaching the best coverage
        out[s:s + step] = cand.min(axis=-1)
    return out.reshape(exps.shape[:-1])


def offsets(exps: np.ndarray, bases: np.ndarray) -> np.ndarray:
    d = np.asarray(exps, np.int32) - np.asarray(bases, np.int32)[..., None]
    return np.where((d >= 0) & (d <= MAX_OFFSET), d, ESCAPE).astype(np.uint8)


def encode_group(x: np.ndarray):
    """One group of 64 BF16 values -> (base, offsets[64], sm[64], escaped values in order)."""
    x = np.asarray(x, np.uint16)
    assert x.shape == (GROUP,)
    e = exponent(x)
    b = int(choose_bases(e[None])[0])
    off = offsets(e, np.int32(b))
    return b, off, sm_byte(x), x[off == ESCAPE].copy()


def decode_group(base: int, off: np.ndarray, sm: np.ndarray, escapes: np.ndarray) -> np.ndarray:
    off = np.asarray(off, np.int32)
    out = rebuild(sm, (base + np.minimum(off, MAX_OFFSET)) & 0xFF)
    esc = off == ESCAPE
    assert int(esc.sum()) == len(escapes)
    out[esc] = np.asarray(escapes, np.uint16)
    return out


# ---------------------------------------------------------------- storage order
def storage_order(P: int, D: int, kind: int) -> np.ndarray:
    """Flat [P*D] token-major index of each storage position of a block, in storage order."""
    idx = np.arange(P * D).reshape(P, D)
    parts = []
    for t in range(P // TILE):
        tile = idx[t * TILE:(t + 1) * TILE]
        parts.append(tile.reshape(-1) if kind == K_KIND else tile.T.reshape(-1))
    return np.concatenate(parts)


def pack_offsets(off: np.ndarray) -> np.ndarray:
    """Offsets of consecutive storage positions -> little-endian u32 words (8 per word)."""
    o = np.asarray(off, np.uint32).reshape(-1, 8)
    w = np.zeros(o.shape[0], np.uint32)
    for k in range(4):
        w |= o[:, 2 * k] << np.uint32(4 * k)
        w |= o[:, 2 * k + 1] << np.uint32(16 + 4 * k)
    return w


def unpack_offsets(words: np.ndarray) -> np.ndarray:
    w = np.asarray(words, np.uint32)
    o = np.zeros((w.shape[0], 8), np.uint8)
    for k in range(4):
        o[:, 2 * k] = (w >> np.uint32(4 * k)) & 0xF
        o[:, 2 * k + 1] = (w >> np.uint32(16 + 4 * k)) & 0xF
    return o.reshape(-1)


def block_bytes(P: int, D: int) -> int:
    return (P * D) + (P * D) // 2


def meta_bytes(P: int, D: int) -> int:
    used = 2 * P * (D // GROUP) + 16
    return (used + 127) // 128 * 128


def inline_capacity(P: int, D: int) -> int:
    """Escapes a unit can hold inline: 4-byte (value, position) entries after the header."""
    return (meta_bytes(P, D) - 2 * P * (D // GROUP) - 16) // 4


def unit_bytes(P: int, D: int) -> int:
    return meta_bytes(P, D) + 2 * block_bytes(P, D)


def group_values(A: np.ndarray, geometry: str = TOKEN) -> np.ndarray:
    """Block array [P][D] -> its groups [n_groups][64], in base-table order."""
    P, D = A.shape
    if geometry == TOKEN:        # token t's dims [64g, 64g + 64); table order t*16G + g*16 + tok
        g = A.reshape(P // TILE, TILE, D // GROUP, GROUP).transpose(0, 2, 1, 3)
    else:                        # tile t's tokens over dims [4j, 4j + 4); table order t*16G + j
        g = A.reshape(P // TILE, TILE, D // CHANNEL_DIMS, CHANNEL_DIMS).transpose(0, 2, 1, 3)
    return g.reshape(-1, GROUP)


def value_bases(bases: np.ndarray, P: int, D: int, geometry: str = TOKEN) -> np.ndarray:
    """Base table [P*G] (table order) -> the base of every value, [P][D]."""
    b = np.asarray(bases, np.int32)
    tok, dim = np.meshgrid(np.arange(P), np.arange(D), indexing="ij")
    if geometry == TOKEN:
        idx = (tok // TILE) * TILE * (D // GROUP) + (dim // GROUP) * TILE + tok % TILE
    else:
        idx = (tok // TILE) * (D // CHANNEL_DIMS) + dim // CHANNEL_DIMS
    return b[idx]


def encode_block(X: np.ndarray, kind: int, with_positions: bool = False, geometry: str = TOKEN):
    """Block [P][D] BF16 bits -> (base bytes [P*G], block payload bytes, escapes u16
    [, storage positions of the escapes])."""
    X = np.asarray(X, np.uint16)
    P, D = X.shape
    bases = choose_bases(group_values(exponent(X), geometry))          # table order
    e = exponent(X)
    d = e - value_bases(bases, P, D, geometry)
    off = np.where((d >= 0) & (d <= MAX_OFFSET), d, ESCAPE).astype(np.uint8)
    sm = sm_byte(X)
    order = storage_order(P, D, kind)
    sm_s, off_s, x_s = sm.reshape(-1)[order], off.reshape(-1)[order], X.reshape(-1)[order]
    payload, per_tile = [], TILE * D
    for t in range(P // TILE):
        sl = slice(t * per_tile, (t + 1) * per_tile)
        payload.append(sm_s[sl])
        payload.append(pack_offsets(off_s[sl]).astype('<u4').view(np.uint8))
    esc = off_s == ESCAPE
    out = (bases.astype(np.uint8), np.concatenate(payload), x_s[esc].copy())
    if with_positions:
        out = out + (np.nonzero(esc)[0].astype(np.uint32),)
    return out


def decode_block(bases: np.ndarray, payload: np.ndarray, escapes: np.ndarray, P: int, D: int,
                 kind: int, geometry: str = TOKEN) -> np.ndarray:
    per_tile = TILE * D
    sm_s, off_s = [], []
    for t in range(P // TILE):
        chunk = payload[t * (per_tile + per_tile // 2):(t + 1) * (per_tile + per_tile // 2)]
        sm_s.append(chunk[:per_tile])
        off_s.append(unpack_offsets(chunk[per_tile:].view('<u4')))
    sm_s, off_s = np.concatenate(sm_s), np.concatenate(off_s)
    order = storage_order(P, D, kind)
    b_s = value_bases(bases, P, D, geometry).reshape(-1)[order]
    x_s = rebuild(sm_s, (b_s + np.minimum(off_s, MAX_OFFSET)) & 0xFF)
    esc = off_s == ESCAPE
    assert int(esc.sum()) == len(escapes)
    x_s[esc] = escapes
    X = np.empty(P * D, np.uint16)
    X[order] = x_s
    return X.reshape(P, D)


def encode_unit(K: np.ndarray, V: np.ndarray, pool_offset: int | None = None, geometry: str = TOKEN):
    """One (page, head) unit from its K and V blocks [P][D], with token or channel groups.

    Returns (unit bytes uint8[unit_bytes], escapes that go to the pool: u16, K's then V's).
    When the escapes do not fit inline they go to the pool at `pool_offset` (0 when None).
    """
    P, D = K.shape
    G = D // GROUP
    kb, kp, ke, kpos = encode_block(K, K_KIND, with_positions=True, geometry=geometry)
    vb, vp, ve, vpos = encode_block(V, V_KIND, with_positions=True, geometry=geometry)
    meta = np.zeros(meta_bytes(P, D), np.uint8)
    meta[:P * G] = kb
    meta[P * G:2 * P * G] = vb
    h = 2 * P * G
    meta[h:h + 8] = np.array([len(ke), len(ve)], '<u4').view(np.uint8)
    esc = np.concatenate([ke, ve]).astype(np.uint16)
    if len(esc) <= inline_capacity(P, D):
        meta[h + 8:h + 16] = np.array([INLINE], '<u8').view(np.uint8)
        pos = np.concatenate([kpos, vpos]).astype(np.uint32)
        entries = esc.astype(np.uint32) | (pos << np.uint32(16))
        meta[h + 16:h + 16 + 4 * len(esc)] = entries.astype('<u4').view(np.uint8)
        pool = np.zeros(0, np.uint16)
    else:
        meta[h + 8:h + 16] = np.array([pool_offset or 0], '<u8').view(np.uint8)
        pool = esc
    return np.concatenate([meta, kp, vp]), pool


def unit_header(unit: np.ndarray, P: int, D: int):
    """(K escape count, V escape count, pool offset or INLINE)."""
    h = 2 * P * (D // GROUP)
    kc, vc = np.asarray(unit[h:h + 8]).view('<u4')
    off = int(np.asarray(unit[h + 8:h + 16]).view('<u8')[0])
    return int(kc), int(vc), off


def unit_escapes(unit: np.ndarray, pool: np.ndarray | None, P: int, D: int):
    kc, vc, off = unit_header(unit, P, D)
    if off == INLINE:
        h = 2 * P * (D // GROUP) + 16
        entries = np.asarray(unit[h:h + 4 * (kc + vc)]).view('<u4')
        esc = (entries & 0xFFFF).astype(np.uint16)
    else:
        esc = np.asarray(pool[off:off + kc + vc], np.uint16)
    return esc[:kc], esc[kc:]


def inline_positions(unit: np.ndarray, P: int, D: int):
    """Storage positions recorded with inline escapes (K's, V's), or None for a pool list."""
    kc, vc, off = unit_header(unit, P, D)
    if off != INLINE:
        return None
    h = 2 * P * (D // GROUP) + 16
    pos = (np.asarray(unit[h:h + 4 * (kc + vc)]).view('<u4') >> 16).astype(np.int64)
    return pos[:kc], pos[kc:]


def decode_unit(unit: np.ndarray, pool: np.ndarray | None, P: int, D: int, geometry: str = TOKEN):
    """Unit bytes (+ escape pool) -> (K [P][D], V [P][D]) BF16 bits."""
    unit = np.asarray(unit, np.uint8)
    G = D // GROUP
    mb, bb = meta_bytes(P, D), block_bytes(P, D)
    ke, ve = unit_escapes(unit, pool, P, D)
    K = decode_block(unit[:P * G], unit[mb:mb + bb], ke, P, D, K_KIND, geometry)
    V = decode_block(unit[P * G:2 * P * G], unit[mb + bb:mb + 2 * bb], ve, P, D, V_KIND, geometry)
    return K, V
