// Lane layouts of the attention kernels: which storage positions each lane of a wave loads
// and rebuilds, for one 16-token tile of one unit.
//
//   K, multi-head layout      lane l -> token l/4, dims (l%4)*D/4 .. +D/4: storage positions
//                             [l*D/4, (l+1)*D/4) of the tile, in lane order.
//   K, grouped-query layout   (D = 128) lane l -> token l%16, dims 32*(l/16) .. +32: the MFMA
//                             operand layout; storage chunk 4*(l%16) + l/16.
//   V                         lane l -> dims l + 64*s (s < D/64), all 16 tokens: storage
//                             positions [16*d, 16*d + 16), segment s in lane order.
//
// Loading is split from decoding so that kernels can issue the next tile's loads before they
// decode the current one.
#pragma once

#include "kvz_device.hpp"

namespace kvz {

// ---------------------------------------------------------------- K
template <int D>
struct KRaw {
  static constexpr int VK = (D == 128) ? 32 : 16;   // values per lane
  static constexpr int NW = VK / 8;                 // offset words per lane
  uint32_t sm[VK / 4];
  uint32_t nib[NW];
  uint32_t base;
};

// chunk index (storage order, units of VK values) of this lane
template <int D, bool GQA>
__device__ __forceinline__ int k_chunk(int lane) {
  if constexpr (GQA) return 4 * (lane & 15) + (lane >> 4);
  else return lane;
}

template <int D, bool GQA>
__device__ __forceinline__ void load_k(const uint8_t* unit, int P, int tile, int lane, KRaw<D>& r) {
  constexpr int VK = KRaw<D>::VK;
  const int c = k_chunk<D, GQA>(lane);
  const int tok = c / (D / VK), dim0 = (c % (D / VK)) * VK;
  const uint8_t* tb = unit + kblock_offset(P, D) + tile * tile_bytes(D);
  const uint4* s = reinterpret_cast<const uint4*>(tb + c * VK);
  if constexpr (VK == 32) {
    uint4 a = s[0], b = s[1];
    r.sm[0] = a.x; r.sm[1] = a.y; r.sm[2] = a.z; r.sm[3] = a.w;
    r.sm[4] = b.x; r.sm[5] = b.y; r.sm[6] = b.z; r.sm[7] = b.w;
    uint4 n = *reinterpret_cast<const uint4*>(tb + 16 * D + c * (VK / 2));
    r.nib[0] = n.x; r.nib[1] = n.y; r.nib[2] = n.z; r.nib[3] = n.w;
  } else {
    uint4 a = s[0];
    r.sm[0] = a.x; r.sm[1] = a.y; r.sm[2] = a.z; r.sm[3] = a.w;
    uint2 n = *reinterpret_cast<const uint2*>(tb + 16 * D + c * (VK / 2));
    r.nib[0] = n.x; r.nib[1] = n.y;
  }
  r.base = unit[kbase_offset(D, tile) + (dim0 / kGroup) * kTile + tok];
}

template <int D>
__device__ __forceinline__ void decode_k(const KRaw<D>& r, uint32_t (&pairs)[KRaw<D>::VK / 2],
                                         uint32_t (&flags)[KRaw<D>::NW]) {
  const uint32_t bb = r.base * 0x00800080u;
#pragma unroll
  for (int w = 0; w < KRaw<D>::NW; ++w) {
    decode8(r.sm[2 * w], r.sm[2 * w + 1], r.nib[w], bb, bb, bb, bb, &pairs[4 * w]);
    flags[w] = escape_flags(r.nib[w]);
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
__device__ __forceinline__ void load_v(const uint8_t* unit, int P, int tile, int lane, VRaw<D>& r) {
  const uint8_t* tb = unit + vblock_offset(P, D) + tile * tile_bytes(D);
#pragma unroll
  for (int s = 0; s < VRaw<D>::NS; ++s) {
    const int d = lane + 64 * s;
    r.seg[s].sm = *reinterpret_cast<const uint4*>(tb + 16 * d);
    r.seg[s].nib = *reinterpret_cast<const uint2*>(tb + 16 * D + 8 * d);
  }
}

// Base terms of the 8 token pairs of group g in tile `tile` (wave-uniform, from SGPRs).
struct VBases {
  uint32_t bb[8];
};

__device__ __forceinline__ VBases v_bases(const uint8_t* unit, int P, int D, int tile, int g) {
  const uint8_t* b = unit + vbase_offset(P, D, tile) + g * kTile;
  uint4 w = sload4(b);
  VBases r;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t word = ws[k >> 1];
    const int sh = (k & 1) * 16;
    r.bb[k] = pair_base((word >> sh) & 0xFFu, (word >> (sh + 8)) & 0xFFu);
  }
  return r;
}

__device__ __forceinline__ void decode_v_seg(const VSeg& s, const VBases& b, uint32_t (&pairs)[8],
                                             uint32_t (&flags)[2]) {
  decode8(s.sm.x, s.sm.y, s.nib.x, b.bb[0], b.bb[1], b.bb[2], b.bb[3], &pairs[0]);
  decode8(s.sm.z, s.sm.w, s.nib.y, b.bb[4], b.bb[5], b.bb[6], b.bb[7], &pairs[4]);
  flags[0] = escape_flags(s.nib.x);
  flags[1] = escape_flags(s.nib.y);
}

// ---------------------------------------------------------------- unit header
struct UnitHeader {
  uint32_t kc, vc;          // escapes of the K and V blocks
  uint64_t off;             // pool offset or kInline
};

__device__ __forceinline__ UnitHeader load_header(const uint8_t* unit, int P, int D) {
  uint4 h = sload4(unit + hdr_offset(P, D));
  UnitHeader r;
  r.kc = h.x;
  r.vc = h.y;
  r.off = ((uint64_t)h.w << 32) | h.z;
  return r;
}

// ---------------------------------------------------------------- escape patching per tile
// Escapes of one tile of one block: count and patch. `rank` is the block-level rank of the
// tile's first escape and is advanced past the tile. Inline lists use the wave-uniform walk;
// pool lists are staged into `lds` (room for 16*D values) and patched per lane.

template <int D, bool GQA>
__device__ __forceinline__ void patch_k_tile(uint32_t (&pairs)[KRaw<D>::VK / 2],
                                             const uint32_t (&flags)[KRaw<D>::NW], const uint8_t* unit,
                                             int P, const UnitHeader& h, uint32_t& rank, uint16_t* lds,
                                             const uint16_t* pool, int lane) {
  constexpr int NW = KRaw<D>::NW;
  if (h.off == kInline) {
    rank += patch_inline<NW>(pairs, flags, GQA, unit + hdr_offset(P, D) + 16, rank, h.kc);
    return;
  }
  uint32_t c = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) c += popc_flags(flags[w]);
  // counts in storage order -> exclusive scan -> back to this lane
  const int src = GQA ? (16 * (lane & 3) + (lane >> 2)) : lane;      // lane holding chunk `lane`
  const uint32_t c_ord = GQA ? (uint32_t)__shfl((int)c, src) : c;
  const uint32_t inc = wave_incl_scan(c_ord);
  const uint32_t total = readlane(inc, 63);
  const uint32_t exc_ord = inc - c_ord;
  const uint32_t exc = GQA ? (uint32_t)__shfl((int)exc_ord, k_chunk<D, GQA>(lane)) : exc_ord;
  if (total == 0) return;
  // never read past this block's list, even if the offsets disagree with the header
  const uint32_t avail = h.kc > rank ? min(total, h.kc - rank) : 0u;
  const uint16_t* src_list = pool + h.off + rank;
  for (uint32_t i = lane; i < avail; i += 64) lds[i] = src_list[i];
  wave_lds_sync();
  patch_lds<NW>(pairs, flags, lds, exc, avail);
  wave_lds_sync();
  rank += total;
}

// V: segments s = 0 .. D/64-1 (dims lane + 64 s), storage order segment-major then lane.
template <int D>
__device__ __forceinline__ void patch_v_tile(uint32_t (&pairs)[D / 64][8], const uint32_t (&flags)[D / 64][2],
                                             const uint8_t* unit, int P, const UnitHeader& h, uint32_t& rank,
                                             uint16_t* lds, const uint16_t* pool, int lane) {
  constexpr int NS = D / 64;
  if (h.off == kInline) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      rank += patch_inline<2>(pairs[s], flags[s], false, unit + hdr_offset(P, D) + 16, h.kc + rank,
                              h.kc + h.vc);
    return;
  }
  uint32_t packed = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) packed |= (popc_flags(flags[s][0]) + popc_flags(flags[s][1])) << (16 * s);
  const uint32_t inc = wave_incl_scan(packed);
  const uint32_t tot = readlane(inc, 63);
  const uint32_t exc = inc - packed;
  const uint32_t t0 = tot & 0xFFFFu;
  const uint32_t total = t0 + (tot >> 16);
  if (total == 0) return;
  const uint32_t avail = h.vc > rank ? min(total, h.vc - rank) : 0u;
  const uint16_t* src_list = pool + h.off + h.kc + rank;
  for (uint32_t i = lane; i < avail; i += 64) lds[i] = src_list[i];
  wave_lds_sync();
  patch_lds<2>(pairs[0], flags[0], lds, exc & 0xFFFFu, avail);
  if constexpr (NS > 1) patch_lds<2>(pairs[1], flags[1], lds, t0 + (exc >> 16), avail);
  wave_lds_sync();
  rank += total;
}

}  // namespace kvz
