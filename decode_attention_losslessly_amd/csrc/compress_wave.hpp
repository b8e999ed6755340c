// Compression of one full page of one head into a unit by a single wave (§III.B "Lossless KV
// Cache Format": exponents coded as offsets from a per-group base, sign and fraction kept; §III.D:
// a page is compressed once it is full). The same unit bytes as the workgroup compressor in
// compress.hpp, for head dims 64 and 128, with no workgroup barrier anywhere:
//   1. the V block [P][D] is staged in the wave's LDS (its storage order transposes it); K is
//      read from memory where it is used (its storage order is the source order);
//   2. bases, eight groups at a time: the eight lanes of a group hold its 64 values as 16-byte
//      pieces and reduce their exponents' minimum and maximum; a group whose exponents span at
//      most 15 binades takes the minimum (nothing escapes, and the largest-coverage rule gives the
//      same base); the others take the histogram rule, one group at a time when there are one
//      or two of them, else all eight at once, each group in its own 256 LDS bins;
//   3. escapes are counted per block; the list goes inline when K + V escapes fit the meta
//      region, else to the pool at an atomically bumped cursor;
//   4. storage positions are encoded 8 per lane (one offset word, 8 sm bytes) in storage order,
//      a wave scan giving each escape its rank.
#pragma once

#include "compress.hpp"

namespace kvz {

// LDS of one wave: the V block (P D values), the bases in meta order (2 P G bytes, rounded up to
// 16), and 2 KB of histogram bins (256 one-byte bins for each of 8 groups, or 256 u32 bins for
// one group)
__host__ __device__ constexpr size_t compress_wave_lds(int P, int D) {
  return 2 * (size_t)P * D + ((size_t)2 * P * (D / kGroup) + 15) / 16 * 16 + 2048;
}

// exponent of the low / high BF16 value of a packed pair
__device__ __forceinline__ uint32_t exp_lo(uint32_t w) { return (w >> 7) & 0xFFu; }
__device__ __forceinline__ uint32_t exp_hi(uint32_t w) { return (w >> 23) & 0xFFu; }

// Bases of the eight groups held by the wave, eight lanes per group (lane 8j + i holds values
// 8i .. 8i+7 of group j as the packed pairs w[0..3]): the largest-coverage rule for each group,
// counted in its own 256 bins (`bins8`: 8 x 256 bytes; a group has 64 values, so every count
// and running sum fits in a byte, four bins to a dword). With C[k] = #{values with exponent
// <= k} (the running sum of the group's histogram), the count of exponent e's window [e, e+14]
// is C[min(e+14, 255)] - C[e-1]; the largest count wins, the smallest exponent on ties.
__device__ __forceinline__ uint32_t group_bases8(const uint32_t (&w)[4], uint8_t* bins8, int lane) {
  uint8_t* hb = bins8 + (lane >> 3) * 256;
  uint32_t* hw = reinterpret_cast<uint32_t*>(hb);
  uint4* hv = reinterpret_cast<uint4*>(hb) + (lane & 7) * 2;   // this lane's 32 bins
  hv[0] = make_uint4(0, 0, 0, 0);
  hv[1] = make_uint4(0, 0, 0, 0);
  wave_lds_sync();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t el = exp_lo(w[j]), eh = exp_hi(w[j]);
    atomicAdd(&hw[el >> 2], 1u << (8 * (el & 3)));
    atomicAdd(&hw[eh >> 2], 1u << (8 * (eh & 3)));
  }
  wave_lds_sync();
  // running sums: a dword times 0x01010101 holds its bytes' prefix sums (no byte carries past 64)
  const uint4 a = hv[0], b = hv[1];
  const uint32_t x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t tot = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) tot += (x[k] * 0x01010101u) >> 24;
  uint32_t inc = tot;
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
    const uint32_t o = (uint32_t)__shfl_up((int)inc, d, 8);
    if ((lane & 7) >= d) inc += o;
  }
  uint32_t run = inc - tot;   // the counts of the group's lower lanes' bins
  uint32_t y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    y[k] = x[k] * 0x01010101u + run * 0x01010101u;
    run = y[k] >> 24;
  }
  hv[0] = make_uint4(y[0], y[1], y[2], y[3]);
  hv[1] = make_uint4(y[4], y[5], y[6], y[7]);
  wave_lds_sync();
  uint32_t key = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t e = (j & 1) ? exp_hi(w[j >> 1]) : exp_lo(w[j >> 1]);
    const uint32_t hi = hb[min(e + 14u, 255u)];
    const uint32_t lo = e > 0 ? hb[e - 1] : 0u;
    key = max(key, ((hi - lo) << 8) | (255u - e));
  }
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
  wave_lds_sync();   // the bins are read before the next step clears them
  return 255u - (key & 0xFFu);
}

// Payload and escapes of one block, storage chunk c (positions 8c .. 8c+7) per lane and step.
// X: the block's values [P][D] (K: in memory, V: in LDS); bases: its bases in meta order (LDS). Escapes go to
// `inline_dst` as value | position << 16 entries or to `pool_dst` as values (whichever is
// non-null), starting at entry/element 0.
template <bool IsV, int D>
__device__ __forceinline__ void encode_block_wave(const uint16_t* X, const uint8_t* bases, int P, uint8_t* payload,
                                  uint32_t* inline_dst, uint16_t* pool_dst, int lane) {
  constexpr int G = D / kGroup;
  const int nchunks = P * D / 8;          // a multiple of 64: P is a multiple of 16, D of 64
  uint32_t rank = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 64) {
    const int c = c0 + lane;
    const int t = (8 * c) / (kTile * D), r = (8 * c) % (kTile * D);
    uint16_t xs[8];
    int b[8];
    if (!IsV) {
      // storage order is [token][dim] inside the tile: 8 consecutive dims of one token, one group
      const uint4 v = *reinterpret_cast<const uint4*>(X + (size_t)t * kTile * D + r);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xs[2 * j] = (uint16_t)(w[j] & 0xFFFFu);
        xs[2 * j + 1] = (uint16_t)(w[j] >> 16);
      }
      const int tok = r / D, g = (r % D) / kGroup;
      const int bb = bases[t * kTile * G + g * kTile + tok];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = bb;
    } else {
      // [dim][token] inside the tile: 8 consecutive tokens of one dim, bases consecutive in meta order
      const int d = r / kTile, tok0 = r % kTile;
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[j] = X[(size_t)(t * kTile + tok0 + j) * D + d];
      const uint2 bw = *reinterpret_cast<const uint2*>(bases + t * kTile * G + (d / kGroup) * kTile + tok0);
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = (int)(((j < 4 ? bw.x : bw.y) >> (8 * (j & 3))) & 0xFFu);
    }
    uint32_t word = 0, sm_lo = 0, sm_hi = 0, escmask = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint16_t x = xs[j];
      const int e = (x >> 7) & 0xFF;
      int off = e - b[j];
      if (off < 0 || off > 14) {
        off = kEscape;
        escmask |= 1u << j;
      }
      const int bit = (j & 1) ? (16 + 4 * (j >> 1)) : (4 * (j >> 1));
      word |= (uint32_t)off << bit;
      const uint32_t sm = ((x >> 8) & 0x80u) | (x & 0x7Fu);
      if (j < 4) sm_lo |= sm << (8 * j); else sm_hi |= sm << (8 * (j - 4));
    }
    uint8_t* tb = payload + (size_t)t * tile_bytes(D);
    *reinterpret_cast<uint2*>(tb + r) = make_uint2(sm_lo, sm_hi);
    *reinterpret_cast<uint32_t*>(tb + 16 * D + r / 2) = word;
    const uint32_t ne = (uint32_t)__builtin_popcount(escmask);
    const uint32_t inc = wave_incl_scan(ne);
    if (escmask && (inline_dst || pool_dst)) {
      uint32_t k = rank + inc - ne;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (escmask & (1u << j)) {
          if (inline_dst) inline_dst[k] = (uint32_t)xs[j] | ((uint32_t)(8 * c + j) << 16);
          else pool_dst[k] = xs[j];
          ++k;
        }
      }
    }
    rank += readlane(inc, 63);
  }
}

// Bases of one block's P G groups (group i = values [64 i, 64 i + 64) of X, in memory or in LDS),
// written to `bases` in meta order; returns the block's escape count (wave-uniform).
template <int D>
__device__ __forceinline__ uint32_t block_bases(const uint16_t* X, int P, uint8_t* bases, uint8_t* bins, int lane) {
  constexpr int G = D / kGroup;
  uint32_t esc = 0;   // this lane's escapes
  for (int q0 = 0; q0 < P * G; q0 += 8) {
    const int q = q0 + (lane >> 3);
    const uint4 v = reinterpret_cast<const uint4*>(X)[q * 8 + (lane & 7)];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t mn = 255u, mx = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mn = min(mn, min(exp_lo(w[j]), exp_hi(w[j])));
      mx = max(mx, max(exp_lo(w[j]), exp_hi(w[j])));
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
      mn = min(mn, (uint32_t)__shfl_xor((int)mn, m));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, m));
    }
    uint32_t b = mn;
    uint64_t slow = ballot((lane & 7) == 0 && mx - mn > 14u);   // bit 8j: group j of the step
    if (__builtin_popcountll(slow) >= 3) {
      const uint32_t bs = group_bases8(w, bins, lane);
      if (mx - mn > 14u) b = bs;
    } else {
      while (slow) {
        const int j = __builtin_ctzll(slow) >> 3;
        slow &= slow - 1;
        const uint32_t e = (uint32_t)(X[(q0 + j) * 64 + lane] >> 7) & 0xFFu;
        const uint32_t bs = group_base(e, reinterpret_cast<uint32_t*>(bins), lane);
        if ((lane >> 3) == j) b = bs;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) esc += (exp_lo(w[j]) - b > 14u) + (exp_hi(w[j]) - b > 14u);
    if ((lane & 7) == 0) {
      const int tok = q / G, g = q % G;
      bases[(tok / kTile) * kTile * G + g * kTile + (tok % kTile)] = (uint8_t)b;
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) esc += (uint32_t)__shfl_xor((int)esc, m);
  return uniform(esc);
}

// Compresses src_k, src_v ([P][D] token-major raw BF16) into `unit`; `lds` is the wave's own
// compress_wave_lds(P, D) bytes (16-byte aligned). Every lane of the wave calls it.
template <int D>
__device__ __forceinline__ void compress_unit_wave(const uint16_t* __restrict__ src_k, const uint16_t* __restrict__ src_v, int P,
                                   uint8_t* __restrict__ unit, uint16_t* __restrict__ pool, int64_t pool_cap,
                                   uint64_t* __restrict__ cursor, uint32_t* __restrict__ status, uint8_t* lds,
                                   int lane) {
  constexpr int G = D / kGroup;
  const int PD = P * D;
  uint16_t* sv = reinterpret_cast<uint16_t*>(lds);
  uint8_t* sbase = lds + 2 * (size_t)PD;
  uint8_t* bins = lds + 2 * (size_t)PD + ((size_t)2 * P * G + 15) / 16 * 16;
  // 1. stage V
  for (int i = lane; i < PD / 8; i += 64) reinterpret_cast<uint4*>(sv)[i] = reinterpret_cast<const uint4*>(src_v)[i];
  wave_lds_sync();
  // 2. bases, eight groups per step (a block has P G groups, a multiple of 16), K's from memory,
  // then V's from LDS
  const uint32_t kesc = block_bases<D>(src_k, P, sbase, bins, lane);
  const uint32_t vesc = block_bases<D>(sv, P, sbase + P * G, bins, lane);
  wave_lds_sync();
  // 3. where the escapes go
  const uint32_t kc = kesc, vc = vesc, total = kc + vc;
  const uint32_t hdr = hdr_offset(P, D);
  uint64_t dest = kInline;
  bool drop = false;
  if ((int)total > inline_capacity(P, D)) {
    uint64_t off = 0;
    if (lane == 0) off = atomicAdd((unsigned long long*)cursor, (unsigned long long)total);
    off = ((uint64_t)readlane((uint32_t)(off >> 32), 0) << 32) | readlane((uint32_t)off, 0);
    if (off + total > (uint64_t)pool_cap) {
      if (lane == 0) atomicOr(status, kStatusPoolFull);
      drop = true;
    } else {
      dest = off;
    }
  }
  uint32_t* inl = (!drop && dest == kInline) ? reinterpret_cast<uint32_t*>(unit + hdr + 16) : nullptr;
  uint16_t* pl = (!drop && dest != kInline) ? pool + dest : nullptr;
  // 4. payload and escapes
  encode_block_wave<false, D>(src_k, sbase, P, unit + kblock_offset(P, D), inl, pl, lane);
  encode_block_wave<true, D>(sv, sbase + P * G, P, unit + vblock_offset(P, D), inl ? inl + kc : nullptr,
                             pl ? pl + kc : nullptr, lane);
  // 5. meta: bases, header, zero tail of the inline area
  for (int i = lane; i < 2 * P * G; i += 64) unit[i] = sbase[i];
  const uint32_t used = inl ? 4 * total : 0;
  for (uint32_t i = hdr + 16 + used + lane; i < meta_bytes(P, D); i += 64) unit[i] = 0;
  if (lane == 0) {
    uint32_t* h = reinterpret_cast<uint32_t*>(unit + hdr);
    h[0] = drop ? 0 : kc;
    h[1] = drop ? 0 : vc;
    *reinterpret_cast<uint64_t*>(unit + hdr + 8) = dest;
  }
}

}  // namespace kvz
