// Lane layouts of the attention kernels: which storage positions each lane of a wave loads
// and rebuilds, for one 16-token tile of one unit. A K tile is cut into pieces of 16 storage
// positions (16 dims of one token); lane l holds the pieces k_piece(l, i), i < D/64:
//
//   K, multi-head layout      pieces l + 64*i: with D = 128, token l/8 and token 8 + l/8, dims
//                             16*(l%8) .. +16 of both; with D = 64, token l/4, dims 16*(l%4)..
//                             Every load instruction of the wave reads 64 consecutive pieces,
//                             i.e. whole cache lines.
//   K, grouped-query layout   (D = 128) the MFMA operand layout: lane l -> token l%16, dims
//                             32*(l/16) .. +32, i.e. pieces 2c and 2c + 1 of chunk
//                             c = 4*(l%16) + l/16.
//   V                         lane l -> dims l + 64*s (s < D/64), all 16 tokens: storage
//                             positions [16*d, 16*d + 16), segment s in lane order.
//
// Loading is split from decoding so that kernels can issue the next tile's loads before they
// decode the current one.
#pragma once

#include "kvz_device.hpp"

namespace kvz {

// ---------------------------------------------------------------- streaming loads
// The compressed units are read once per attention call and are far larger than the caches,
// so their loads carry the non-temporal hint: they then do not displace the page table, q
// and the partials in L2 and the Infinity Cache.
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 stream16(const void* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 stream8(const void* p) {
  const nt_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t stream4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint32_t stream1(const uint8_t* p) { return __builtin_nontemporal_load(p); }

// Loads of one unit go through a buffer resource whose base is the unit (wave-uniform, so it
// sits in SGPRs) and whose extent is the unit's size. The lane's part of an offset is the same
// for every tile and every unit, so it is computed once; the tile's part is a scalar offset.
// No vector instruction is then spent on addresses, and a read past the unit returns zeros.
// A stage that a pipeline issues only to keep its wait counts fixed (past its last step) is
// given an extent of 0: its loads return zeros without touching memory.
typedef __amdgpu_buffer_rsrc_t UnitRsrc;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer: no swizzle, 32-bit data format field
constexpr int kNonTemporal = 2;          // cache-policy operand: non-temporal
__device__ __forceinline__ UnitRsrc unit_rsrc(const uint8_t* unit, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(unit), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 uload16(UnitRsrc r, uint32_t voff, uint32_t soff) {
  const nt_u32x4 v = __builtin_bit_cast(nt_u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kNonTemporal));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 uload8(UnitRsrc r, uint32_t voff, uint32_t soff) {
  const nt_u32x2 v = __builtin_bit_cast(nt_u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kNonTemporal));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t uload4(UnitRsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, kNonTemporal);
}
__device__ __forceinline__ uint32_t uload1(UnitRsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, kNonTemporal);
}
// the same without the non-temporal hint, for bytes other waves read at about the same time
__device__ __forceinline__ uint4 cload16(UnitRsrc r, uint32_t voff, uint32_t soff) {
  const nt_u32x4 v = __builtin_bit_cast(nt_u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 cload8(UnitRsrc r, uint32_t voff, uint32_t soff) {
  const nt_u32x2 v = __builtin_bit_cast(nt_u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
  return make_uint2(v.x, v.y);
}

// ---------------------------------------------------------------- K
// Channel groups (CH, format 2): a base covers 4 adjacent dims over the tile's 16 tokens, so the
// 16 dims of a piece take 4 bases, one dword of the tile's base table (byte dim/4): base[i] then
// holds that dword for piece i. In the multi-head layout a lane's pieces share their dims, and
// so their dword.
template <int D>
struct KRaw {
  static constexpr int VK = 2 * (D / kGroup) * 8;   // values per lane: D / 4
  static constexpr int NP = VK / 16;                 // pieces per lane
  static constexpr int NW = VK / 8;                  // offset words per lane
  uint32_t sm[VK / 4];
  uint32_t nib[NW];
  uint32_t base[NP];   // base of each piece's group (the grouped-query pieces share one)
};

// storage piece (16 positions) held as piece i by this lane
template <int D, bool GQA>
__device__ __forceinline__ int k_piece(int lane, int i) {
  if constexpr (GQA) return 2 * (4 * (lane & 15) + (lane >> 4)) + i;
  else return lane + 64 * i;
}

// token and first dim of a storage piece
template <int D>
__device__ __forceinline__ int piece_token(int piece) { return (16 * piece) / D; }
template <int D>
__device__ __forceinline__ int piece_dim(int piece) { return (16 * piece) % D; }

// BASES: the pieces' bases are loaded with the payload (the pipelined loops, whose meta window
// arrives in the same round trip); without, the caller takes them from the tile's meta window
// (k_bases_from_meta), which the pool-capable loops load a step ahead: a second read of those
// bytes a step later could miss the caches and fetch the line again.
template <int D, bool GQA, bool BASES = true, bool CH = false>
__device__ __forceinline__ void load_k(const uint8_t* unit, int P, int tile, int lane, KRaw<D>& r, bool live = true) {
  constexpr int NP = KRaw<D>::NP;
  const UnitRsrc u = unit_rsrc(unit, live ? unit_bytes(P, D) : 0u);
  const uint32_t tb = kblock_offset(P, D) + tile * tile_bytes(D);   // scalar parts
  const uint32_t bases = kbase_offset(D, tile);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int pc = k_piece<D, GQA>(lane, i);
    const uint4 a = uload16(u, 16 * pc, tb);
    r.sm[4 * i] = a.x; r.sm[4 * i + 1] = a.y; r.sm[4 * i + 2] = a.z; r.sm[4 * i + 3] = a.w;
    if constexpr (!GQA) {
      const uint2 n = uload8(u, 16 * D + 8 * pc, tb);
      r.nib[2 * i] = n.x; r.nib[2 * i + 1] = n.y;
      if constexpr (BASES && !CH) r.base[i] = uload1(u, (piece_dim<D>(pc) / kGroup) * kTile + piece_token<D>(pc), bases);
    }
  }
  if constexpr (!GQA && BASES && CH) {   // the pieces' dims are the same: one dword for all
    const uint32_t b = uload4(u, piece_dim<D>(k_piece<D, GQA>(lane, 0)) / 4, bases);
#pragma unroll
    for (int i = 0; i < NP; ++i) r.base[i] = b;
  }
  if constexpr (GQA) {   // the two pieces are adjacent: one 16-byte offset load, one base
    const int pc = k_piece<D, GQA>(lane, 0);
    const uint4 n = uload16(u, 16 * D + 8 * pc, tb);
    r.nib[0] = n.x; r.nib[1] = n.y; r.nib[2] = n.z; r.nib[3] = n.w;
    if constexpr (BASES && CH) {   // 32 dims: two dwords of the base table
      const uint2 b = uload8(u, piece_dim<D>(pc) / 4, bases);
      r.base[0] = b.x;
      r.base[1] = b.y;
    } else if constexpr (BASES) {
      r.base[0] = r.base[1] = uload1(u, (piece_dim<D>(pc) / kGroup) * kTile + piece_token<D>(pc), bases);
    }
  }
}

// ---------------------------------------------------------------- meta window
// One dword per lane of the tile's metadata, loaded with the payload:
//   lanes [0, 4G)         K bases of the tile (16*G bytes)
//   lanes [4G, 8G)        V bases of the tile
//   lanes [8G, 8G + 32)   header (4 dwords) then the inline escapes
// (the other lanes read the region's first dword; they are not used).
__device__ __forceinline__ uint32_t load_meta(const uint8_t* unit, int P, int D, int tile, int lane, bool live = true) {
  const int G = D / kGroup;
  // the K and V base tables both advance by kTile*G bytes per tile (the scalar offset); the
  // header lanes take it back out
  const uint32_t toff = kbase_offset(D, tile);
  // lanes past the meta region's end (inline entries beyond kvz_inline_capacity, never read)
  // read its start instead, so that the window stays on the region's cache lines
  uint32_t off;
  if (lane < 4 * G) off = kbase_offset(D, 0) + 4 * lane;
  else if (lane < 8 * G) off = vbase_offset(P, D, 0) + 4 * (lane - 4 * G);
  else if (lane < 8 * G + 32 && hdr_offset(P, D) + 4 * (lane - 8 * G) < meta_bytes(P, D))
    off = hdr_offset(P, D) + 4 * (lane - 8 * G) - toff;
  else off = -toff;
  return uload4(unit_rsrc(unit, live ? unit_bytes(P, D) : 0u), off, toff);
}
template <int D>
__device__ __forceinline__ int hdr_lane() { return 8 * (D / kGroup); }

// Base of the group of storage piece pc of a K tile, from the tile's meta window (lanes [0, 4G)
// hold the tile's K base bytes, g * 16 + tok): one cross-lane read instead of a byte load.
template <int D>
__device__ __forceinline__ uint32_t k_piece_base(uint32_t meta, int pc) {
  const int idx = (piece_dim<D>(pc) / kGroup) * kTile + piece_token<D>(pc);
  return ((uint32_t)__shfl((int)meta, idx >> 2) >> (8 * (idx & 3))) & 0xFFu;
}

// the bases of a K tile loaded without them (load_k<D, GQA, false>); with channel groups, a
// piece's dword of the base table is window lane piece_dim / 16
template <int D, bool GQA, bool CH = false>
__device__ __forceinline__ void k_bases_from_meta(KRaw<D>& r, uint32_t meta, int lane) {
  if constexpr (CH) {
#pragma unroll
    for (int i = 0; i < KRaw<D>::NP; ++i)
      r.base[i] = (uint32_t)__shfl((int)meta, piece_dim<D>(k_piece<D, GQA>(lane, i)) / 16);
  } else if constexpr (GQA) {   // the lane's two pieces are one token's adjacent dims: one group
    r.base[0] = r.base[1] = k_piece_base<D>(meta, k_piece<D, GQA>(lane, 0));
  } else {
#pragma unroll
    for (int i = 0; i < KRaw<D>::NP; ++i) r.base[i] = k_piece_base<D>(meta, k_piece<D, GQA>(lane, i));
  }
}

// base byte k of a dword as the term b << 7 | b << 23 of a pair whose two values share it
template <int k>
__device__ __forceinline__ uint32_t byte_base_term(uint32_t w) {
  return ((w >> (8 * k)) & 0xFFu) * 0x00800080u;
}

template <int D, bool CH = false>
__device__ __forceinline__ void decode_k(const KRaw<D>& r, uint32_t (&pairs)[KRaw<D>::VK / 2]) {
#pragma unroll
  for (int i = 0; i < KRaw<D>::NP; ++i) {
    if constexpr (CH) {   // dims 4k .. 4k+3 of the piece (pairs 2k, 2k+1) share base byte k
      const uint32_t w = r.base[i];
      const uint32_t b0 = byte_base_term<0>(w), b1 = byte_base_term<1>(w);
      const uint32_t b2 = byte_base_term<2>(w), b3 = byte_base_term<3>(w);
      decode8(r.sm[4 * i], r.sm[4 * i + 1], r.nib[2 * i], b0, b0, b1, b1, &pairs[8 * i]);
      decode8(r.sm[4 * i + 2], r.sm[4 * i + 3], r.nib[2 * i + 1], b2, b2, b3, b3, &pairs[8 * i + 4]);
    } else {
      const uint32_t bb = opaque(r.base[i] * 0x00800080u);   // once per piece, not folded into each pair
      decode8(r.sm[4 * i], r.sm[4 * i + 1], r.nib[2 * i], bb, bb, bb, bb, &pairs[8 * i]);
      decode8(r.sm[4 * i + 2], r.sm[4 * i + 3], r.nib[2 * i + 1], bb, bb, bb, bb, &pairs[8 * i + 4]);
    }
  }
}

// ---------------------------------------------------------------- V
struct VSeg {
  uint4 sm;      // sm bytes of tokens 0..15 of one dim
  uint2 nib;     // offset words of those 16 values
};

template <int D>
struct VRaw {
  static constexpr int NS = D / kGroup;
  VSeg seg[NS];
};

template <int D>
__device__ __forceinline__ void load_v(const uint8_t* unit, int P, int tile, int lane, VRaw<D>& r, bool live = true) {
  const UnitRsrc u = unit_rsrc(unit, live ? unit_bytes(P, D) : 0u);
  const uint32_t tb = vblock_offset(P, D) + tile * tile_bytes(D);
#pragma unroll
  for (int s = 0; s < VRaw<D>::NS; ++s) {
    const int d = lane + 64 * s;
    r.seg[s].sm = uload16(u, 16 * d, tb);
    r.seg[s].nib = uload8(u, 16 * D + 8 * d, tb);
  }
}

// Base terms of the 8 token pairs of group g in tile `tile` (wave-uniform, in SGPRs). Every
// lane of the meta window spreads its 4 base bytes into two pair terms with one v_perm each
// (bytes b0, b1 -> b0 << 7 | b1 << 23, likewise b2, b3); the terms of group g are then read
// from lanes 4G + 4g .. 4G + 4g + 3.
struct VBases {
  uint32_t bb[8];
};

// With channel groups (CH) every token of the lane's dim d = lane + 64 g shares one base, byte
// d/4 of the tile's V base table: window lane 4G + d/16.
template <int D, bool CH = false>
__device__ __forceinline__ VBases v_bases(uint32_t meta, int g) {
  constexpr int G = D / kGroup;
  if constexpr (CH) {
    const int d = lane_id() + 64 * g;
    const uint32_t w = (uint32_t)__shfl((int)meta, 4 * G + d / 16);
    const uint32_t t = ((w >> (8 * ((d >> 2) & 3))) & 0xFFu) * 0x00800080u;
    VBases r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.bb[i] = t;
    return r;
  }
  const uint32_t lo = __builtin_amdgcn_perm(0u, meta, 0x0C010C00u) << 7;
  const uint32_t hi = __builtin_amdgcn_perm(0u, meta, 0x0C030C02u) << 7;
  VBases r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.bb[2 * i] = readlane(lo, 4 * G + 4 * g + i);
    r.bb[2 * i + 1] = readlane(hi, 4 * G + 4 * g + i);
  }
  return r;
}

// rebuilds the 16 tokens of one dim into pairs[0..7] (token pairs 2k, 2k+1)
__device__ __forceinline__ void decode_v_seg(const VSeg& s, const VBases& b, uint32_t* pairs) {
  decode8(s.sm.x, s.sm.y, s.nib.x, b.bb[0], b.bb[1], b.bb[2], b.bb[3], &pairs[0]);
  decode8(s.sm.z, s.sm.w, s.nib.y, b.bb[4], b.bb[5], b.bb[6], b.bb[7], &pairs[4]);
}

// ---------------------------------------------------------------- unit header
struct UnitHeader {
  uint32_t kc, vc;          // escapes of the K and V blocks
  uint64_t off;             // pool offset or kInline
};

// A pool extent that does not fit the pool (a damaged or dropped header) is treated as no escapes,
// so that no pool read ever leaves the pool.
__device__ __forceinline__ void clamp_to_pool(UnitHeader& h, int64_t pool_cap) {
  if (h.off != kInline && h.off + (uint64_t)h.kc + h.vc > (uint64_t)pool_cap) h.kc = h.vc = 0;
}

template <int D>
__device__ __forceinline__ UnitHeader header_from_meta(uint32_t meta) {
  constexpr int hl = 8 * (D / kGroup);
  UnitHeader r;
  r.kc = readlane(meta, hl);
  r.vc = readlane(meta, hl + 1);
  r.off = ((uint64_t)readlane(meta, hl + 3) << 32) | readlane(meta, hl + 2);
  return r;
}

// ---------------------------------------------------------------- escape patching per tile
// A unit's escapes are either inline (K's entries then V's, each value | position << 16, in
// storage order, in the header area of the meta window) or in the pool (values only).
//   inline: the entries of this tile are walked with wave-uniform control; each names its lane,
//           register and half directly, so no lane has to search its offsets;
//   pool:   every lane finds its escape codes, a wave scan ranks them in storage order, the
//           tile's part of the list and a copy of the pairs go to `lds` (16*D u16 of values,
//           then 64 lanes x (D/4 or D/8) u32 of pairs) and each lane patches its own copy.
// `cursor` is the block-level index of the tile's first escape and is advanced past the tile.

// Escapes of a unit's K and V blocks in its tiles before `t0`: the block-level cursors of tile t0's
// first escapes (the count of offset codes 15 in storage order before it, which is also the index
// of its first inline entry). For a split that starts inside a unit: each tile's offset codes
// (8*D bytes after its 16*D sign-and-mantissa bytes) are read once, a batch of tiles' worth of
// loads issued before any is counted, and counted with a SWAR test of the four bits of every code.
// The other splits of the unit read the same bytes at about the same time, so these loads keep
// them in the caches (no non-temporal hint: 3-4% faster on batch-1 steps over 128- and 256-token
// pages).
template <int D>
__device__ __forceinline__ void escapes_before(const uint8_t* unit, int P, int t0, int lane, uint32_t& kcur,
                                               uint32_t& vcur) {
  static_assert(D == 64 || D == 128, "head dims 64 and 128");
  constexpr int NW = D / 32;             // offset-code dwords per lane and tile
  constexpr int kBatch = 32 / (2 * NW);  // tiles per batch of loads: 32 VGPRs of codes
  const UnitRsrc u = unit_rsrc(unit, unit_bytes(P, D));
  auto codes15 = [](uint32_t x) {   // codes of value 15 among the 8 of x
    x &= x >> 1;
    x &= x >> 2;
    return (uint32_t)__builtin_popcount(x & 0x11111111u);
  };
  uint32_t ck = 0, cv = 0;
  for (int tb = 0; tb < t0; tb += kBatch) {
    uint32_t kw[kBatch][NW], vw[kBatch][NW];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int t = min(tb + j, t0 - 1);   // past t0: a tile already read, not counted
      const uint32_t ko = kblock_offset(P, D) + t * tile_bytes(D) + 16 * D;
      const uint32_t vo = vblock_offset(P, D) + t * tile_bytes(D) + 16 * D;
      if constexpr (NW == 4) {
        const uint4 a = cload16(u, 16 * lane, ko), b = cload16(u, 16 * lane, vo);
        kw[j][0] = a.x; kw[j][1] = a.y; kw[j][2] = a.z; kw[j][3] = a.w;
        vw[j][0] = b.x; vw[j][1] = b.y; vw[j][2] = b.z; vw[j][3] = b.w;
      } else {
        const uint2 a = cload8(u, 8 * lane, ko), b = cload8(u, 8 * lane, vo);
        kw[j][0] = a.x; kw[j][1] = a.y;
        vw[j][0] = b.x; vw[j][1] = b.y;
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      uint32_t nk = 0, nv = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        nk += codes15(kw[j][i]);
        nv += codes15(vw[j][i]);
      }
      const bool in = tb + j < t0;
      ck += in ? nk : 0u;
      cv += in ? nv : 0u;
    }
  }
  kcur = readlane(wave_incl_scan(ck), 63);
  vcur = readlane(wave_incl_scan(cv), 63);
}

// Storage position p of a K tile -> (lane, register, half) through its piece (see k_piece).
template <int D, bool GQA>
__device__ __forceinline__ void k_position(uint32_t p, int& lane, int& reg, int& half) {
  const uint32_t pc = p / 16, j = p % 16;
  uint32_t l, i;
  if constexpr (GQA) {
    const uint32_t c = pc / 2;
    l = 16 * (c & 3) + (c >> 2);
    i = pc & 1;
  } else {
    l = pc % 64;
    i = pc / 64;
  }
  lane = (int)l;
  reg = (int)(8 * i + j / 2);
  half = (int)(j & 1);
}

// Pool lists (many escapes, values only) are patched through LDS with loops that keep few
// registers live, so that this rarely-hot path does not raise the register count of the main
// loop. `lds` holds, per wave, the tile's escape values (16*D u16) followed by a copy of the
// lane's pairs (64 lanes x N u32).
//   chunks(lane)  the storage chunks this lane holds, in storage order, each `span` positions
//                 long and read from `nib` words of 8 positions

// u16 elements of the per-wave LDS area the escape paths use: a tile's escape list (at most 16*D
// values, staged from a 16-byte aligned start: + 16 of slack), then 64 lanes x D/8 pairs
template <int D>
constexpr int esc_lds_elems() { return 32 * D + 16; }
template <int D>
constexpr int esc_pairs_at() { return 16 * D + 16; }

// Copies pool[first, first + n) into lds, the element `first` landing at lds[first % 8]: every
// lane loads its 16-byte chunks of the aligned range, kBatch chunks at a time with
// all loads of a batch issued before its LDS writes (two round trips for the longest list instead
// of one per element; a batch, not the whole range, so that the registers held stay few); a chunk
// that would cross the end of the pool is read element by element up to that end.
// Returns first % 8.
template <int D, int kBatch>
__device__ __forceinline__ uint32_t stage_list(const uint16_t* pool, int64_t pool_cap, uint64_t first, uint32_t n,
                                               uint16_t* lds, int lane) {
  constexpr int kChunks = (2 * D + 2 + 63) / 64;   // 16-byte chunks per lane for n <= 16*D
  const uint64_t a0 = first & ~7ull;
  const uint32_t mis = (uint32_t)(first - a0);
  const uint32_t nch = (mis + n + 7) / 8;
#pragma unroll
  for (int c0 = 0; c0 < kChunks; c0 += kBatch) {
    if ((uint32_t)(64 * c0) >= nch) break;
    uint4 v[kBatch];
#pragma unroll
    for (int c = 0; c < kBatch; ++c) {
      const uint32_t ch = (uint32_t)lane + 64u * (c0 + c);
      const uint64_t e0 = a0 + 8ull * ch;
      v[c] = make_uint4(0, 0, 0, 0);
      if (c0 + c < kChunks && ch < nch) {
        if (e0 + 8 <= (uint64_t)pool_cap) {
          v[c] = *reinterpret_cast<const uint4*>(pool + e0);
        } else {
          uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e0 + e < (uint64_t)pool_cap) w[e >> 1] |= (uint32_t)pool[e0 + e] << (16 * (e & 1));
          v[c] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kBatch; ++c) {
      const uint32_t ch = (uint32_t)lane + 64u * (c0 + c);
      if (c0 + c < kChunks && ch < nch) *reinterpret_cast<uint4*>(lds + 8 * ch) = v[c];
    }
  }
  return mis;
}

// Writes escape x of position j (within this lane's run of pairs) into the LDS copy.
__device__ __forceinline__ void lds_pair_half(uint32_t* mine, int j, uint32_t x) {
  reinterpret_cast<uint16_t*>(mine)[j] = (uint16_t)x;   // pair j/2, half j%2 (little-endian)
}

template <int D, bool GQA>
__device__ __forceinline__ void pool_patch_k(uint32_t (&pairs)[KRaw<D>::VK / 2], const KRaw<D>& raw,
                                             const UnitHeader& h, uint32_t& cursor, uint16_t* lds,
                                             const uint16_t* pool, int64_t pool_cap, int lane) {
  constexpr int N = KRaw<D>::VK / 2, NP = KRaw<D>::NP;
  // rank (in storage order) of each piece's first escape
  uint32_t cnt[NP], rank[NP], total = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) cnt[i] = popc_flags(escape_flags(raw.nib[2 * i])) + popc_flags(escape_flags(raw.nib[2 * i + 1]));
  if constexpr (GQA) {
    // pieces 2c, 2c + 1 are adjacent: scan whole chunks in chunk order (lane 16*(c%4) + c/4)
    const uint32_t cl = cnt[0] + cnt[1];
    const uint32_t c_ord = (uint32_t)__shfl((int)cl, 16 * (lane & 3) + (lane >> 2));
    const uint32_t inc = wave_incl_scan(c_ord);
    total = readlane(inc, 63);
    const uint32_t first = (uint32_t)__shfl((int)(inc - c_ord), 4 * (lane & 15) + (lane >> 4));
    rank[0] = first;
    rank[1] = first + cnt[0];
  } else {
    // piece i of every lane precedes piece i + 1 of any lane
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const uint32_t inc = wave_incl_scan(cnt[i]);
      rank[i] = total + inc - cnt[i];
      total += readlane(inc, 63);
    }
  }
  if (total == 0) return;
  const uint32_t cur = uniform(cursor);
  const uint32_t avail = h.kc > cur ? min(total, h.kc - cur) : 0u;
  const uint32_t mis = stage_list<D, GQA ? 2 : 3>(pool, pool_cap, h.off + cur, avail, lds, lane);
  uint32_t* mine = reinterpret_cast<uint32_t*>(lds + esc_pairs_at<D>()) + lane * N;
#pragma unroll
  for (int i = 0; i < N; i += 4) *reinterpret_cast<uint4*>(mine + i) = make_uint4(pairs[i], pairs[i + 1], pairs[i + 2], pairs[i + 3]);
  wave_lds_sync();
  for (int i = 0; i < NP; ++i) {
    uint32_t rk = rank[i];
    for (int w = 0; w < 2; ++w) {
      uint32_t f = flags_in_order(escape_flags(raw.nib[2 * i + w]));
      while (f) {                                  // positions of the word in list order
        const int pos = ordered_bit_to_pos(__builtin_ctz(f));
        f &= f - 1;
        if (rk < avail) lds_pair_half(mine, 16 * i + 8 * w + pos, lds[mis + rk]);
        ++rk;
      }
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(mine + i);
    pairs[i] = v.x; pairs[i + 1] = v.y; pairs[i + 2] = v.z; pairs[i + 3] = v.w;
  }
  wave_lds_sync();
  cursor = cur + total;
}

template <int D, int kBatch>
__device__ __forceinline__ void pool_patch_v(uint32_t (&pairs)[D / 8], const VRaw<D>& raw, const UnitHeader& h,
                                             uint32_t& cursor, uint16_t* lds, const uint16_t* pool, int64_t pool_cap,
                                             int lane) {
  constexpr int NS = D / 64, N = D / 8;
  uint32_t packed = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    packed |= (popc_flags(escape_flags(raw.seg[s].nib.x)) + popc_flags(escape_flags(raw.seg[s].nib.y))) << (16 * s);
  const uint32_t inc = wave_incl_scan(packed);
  const uint32_t tot = readlane(inc, 63);
  const uint32_t exc = inc - packed;
  const uint32_t t0 = tot & 0xFFFFu;
  const uint32_t total = t0 + (tot >> 16);
  if (total == 0) return;
  const uint32_t cur = uniform(cursor);
  const uint32_t avail = h.vc > cur ? min(total, h.vc - cur) : 0u;
  const uint32_t mis = stage_list<D, kBatch>(pool, pool_cap, h.off + h.kc + cur, avail, lds, lane);
  uint32_t* mine = reinterpret_cast<uint32_t*>(lds + esc_pairs_at<D>()) + lane * N;
#pragma unroll
  for (int i = 0; i < N; i += 4) *reinterpret_cast<uint4*>(mine + i) = make_uint4(pairs[i], pairs[i + 1], pairs[i + 2], pairs[i + 3]);
  wave_lds_sync();
  for (int s = 0; s < NS; ++s) {
    uint32_t rank = s == 0 ? (exc & 0xFFFFu) : t0 + (exc >> 16);
    for (int w = 0; w < 2; ++w) {
      uint32_t f = flags_in_order(escape_flags(w == 0 ? raw.seg[s].nib.x : raw.seg[s].nib.y));
      while (f) {                                  // positions of the word in list order
        const int pos = ordered_bit_to_pos(__builtin_ctz(f));
        f &= f - 1;
        if (rank < avail) lds_pair_half(mine, 16 * s + 8 * w + pos, lds[mis + rank]);
        ++rank;
      }
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(mine + i);
    pairs[i] = v.x; pairs[i + 1] = v.y; pairs[i + 2] = v.z; pairs[i + 3] = v.w;
  }
  wave_lds_sync();
  cursor = cur + total;
}

// Returns false, patching nothing, when the unit's list is in the pool and POOL is off: the
// caller then leaves the work item to the general kernel.
template <int D, bool GQA, bool POOL = true>
__device__ __forceinline__ bool patch_k_tile(uint32_t (&pairs)[KRaw<D>::VK / 2], const KRaw<D>& raw,
                                             uint32_t meta, const UnitHeader& h, int P, int tile,
                                             uint32_t& cursor, uint16_t* lds, const uint16_t* pool,
                                             int64_t pool_cap, int lane) {
  constexpr int N = KRaw<D>::VK / 2;
  // everything that names an escape is wave-uniform: keep it in SGPRs
  const uint32_t lo = uniform((uint32_t)tile * kTile * D), hi = lo + kTile * D;
  if (h.off == kInline) {
    const uint32_t end = uniform(min(h.kc, (uint32_t)inline_capacity(P, D)));
    uint32_t e = uniform(cursor);
    while (e < end) {
      const uint32_t ent = readlane(meta, hdr_lane<D>() + 4 + (int)e);
      const uint32_t p = ent >> 16;
      if (p >= hi) break;
      int l, reg, half;
      k_position<D, GQA>(p - lo, l, reg, half);
      patch_one<N>(pairs, reg, l, half, ent & 0xFFFFu);
      ++e;
    }
    cursor = e;
    return true;
  }
  if constexpr (!POOL) return false;
  pool_patch_k<D, GQA>(pairs, raw, h, cursor, lds, pool, pool_cap, lane);
  return true;
}

// V: segments s = 0 .. D/64-1 (dims lane + 64 s), storage order segment-major then lane;
// pairs[s * 8 + k] holds tokens 2k, 2k+1 of dim lane + 64 s.
// kBatch: 16-byte pool chunks per lane held in registers at a time while staging the list
template <int D, bool POOL = true, int kBatch = 3>
__device__ __forceinline__ bool patch_v_tile(uint32_t (&pairs)[D / 8], const VRaw<D>& raw, uint32_t meta,
                                             const UnitHeader& h, int P, int tile, uint32_t& cursor, uint16_t* lds,
                                             const uint16_t* pool, int64_t pool_cap, int lane) {
  const uint32_t lo = uniform((uint32_t)tile * kTile * D), hi = lo + kTile * D;
  if (h.off == kInline) {
    const uint32_t end = uniform(min(h.kc + h.vc, (uint32_t)inline_capacity(P, D)));
    uint32_t e = uniform(h.kc + cursor);
    while (e < end) {
      const uint32_t ent = readlane(meta, hdr_lane<D>() + 4 + (int)e);
      const uint32_t p = ent >> 16;
      if (p >= hi) break;
      const uint32_t q = p - lo, d = q >> 4, tok = q & 15;
      patch_one<D / 8>(pairs, (int)((d >> 6) * 8 + (tok >> 1)), (int)(d & 63), (int)(tok & 1), ent & 0xFFFFu);
      ++e;
    }
    cursor = e - h.kc;
    return true;
  }
  if constexpr (!POOL) return false;
  pool_patch_v<D, kBatch>(pairs, raw, h, cursor, lds, pool, pool_cap, lane);
  return true;
}

}  // namespace kvz
