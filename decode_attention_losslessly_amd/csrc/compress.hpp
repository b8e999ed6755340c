// Compression of one full page of one head into a unit (§III.B "Lossless KV Cache Format":
// exponents coded as offsets from a base, sign and fraction kept; §III.D: a page is compressed
// once it is full). Used by kvz_compress_pages and by kvz_append_token when a tail fills.
//
// One 256-thread workgroup per unit:
//   1. both source blocks [P][D] are staged in LDS;
//   2. each wave takes groups (64 values = 64 lanes): a histogram of the group's exponents in
//      the wave's LDS bins and its running sum give, for every lane's own exponent e, how many
//      group exponents fall in [e, e+14]; the largest count wins, the smallest exponent on
//      ties; escapes are counted;
//   3. the escape list goes inline when K + V escapes fit the meta region, else to the pool at
//      an atomically bumped cursor;
//   4. storage positions are encoded 8 per thread (one offset word, 8 sm bytes) in storage
//      order, with a workgroup scan giving each escape its rank.
// CH selects the channel groups (format 2): a group is a tile's 16 tokens over 4 adjacent dims
// instead of one token's 64 dims; its base is byte tile * D/4 + dim/4 of the block's base table.
#pragma once

#include "kvz_device.hpp"

namespace kvz {

constexpr int kCompressThreads = 256;

struct CompressShared {
  uint32_t esc_count[2];
  uint32_t wave_sum[kCompressThreads / 64];
  uint64_t dest;        // pool offset, kInline, or ~1 when the pool is full
  uint32_t drop;        // 1 when escapes are dropped (pool full)
  alignas(16) uint32_t bins[kCompressThreads / 64][256];   // per wave: exponent histogram, then its running sum
};

// Base of one group held one value per lane (exponent e): the exponent b among the lanes'
// that maximises #{j : b <= e_j <= b + 14}, the smallest on ties. With C[k] = #{j : e_j <= k}
// (the running sum of the group's exponent histogram), that count for b = e is
// C[min(e + 14, 255)] - C[e - 1].
__device__ __forceinline__ uint32_t group_base(uint32_t e, uint32_t* bins, int lane) {
  reinterpret_cast<uint4*>(bins)[lane] = make_uint4(0, 0, 0, 0);
  wave_lds_sync();
  atomicAdd(&bins[e], 1u);
  wave_lds_sync();
  const uint4 h = reinterpret_cast<const uint4*>(bins)[lane];   // bins 4l .. 4l+3
  const uint32_t s0 = h.x, s1 = s0 + h.y, s2 = s1 + h.z, s3 = s2 + h.w;
  const uint32_t before = wave_incl_scan(s3) - s3;
  wave_lds_sync();
  reinterpret_cast<uint4*>(bins)[lane] = make_uint4(before + s0, before + s1, before + s2, before + s3);
  wave_lds_sync();
  const uint32_t hi = bins[min(e + 14u, 255u)];
  const uint32_t lo = e > 0 ? bins[e - 1] : 0u;
  uint32_t key = ((hi - lo) << 8) | (255u - e);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
  wave_lds_sync();   // the bins are read before the next group clears them
  return 255u - (uniform(key) & 0xFFu);
}

// exclusive scan over the workgroup; returns this thread's prefix, *total gets the sum
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, CompressShared& sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sh.wave_sum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kCompressThreads / 64; ++w) {
    const uint32_t s = sh.wave_sum[w];
    before += (w < wave) ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// storage position s (within one block) -> token-major index tok*D + d (inlined where D is a
// compile-time constant, so that its divisions become shifts)
template <bool IsV>
__device__ __forceinline__ int storage_to_index(int s, int D) {
  const int t = s / (kTile * D), r = s % (kTile * D);
  int tok, d;
  if (IsV) { d = r / kTile; tok = r % kTile; } else { tok = r / D; d = r % D; }
  return (t * kTile + tok) * D + d;
}

// Index in a block's base table of the group holding (token tok, dim d).
template <bool CH>
__device__ __forceinline__ int base_index(int tok, int d, int D) {
  if (CH) return (tok / kTile) * (D / 4) + d / 4;
  return (tok / kTile) * kTile * (D / kGroup) + (d / kGroup) * kTile + (tok % kTile);
}

// Writes the block's payload; its escapes go to `inline_dst` as value | position << 16 entries
// or to `pool_dst` as values (whichever is non-null), starting at entry/element 0.
// DT: the head dim when fixed at compile time, 0 to take it from d_rt
template <bool IsV, int DT, bool CH = false>
__device__ void encode_block(const uint16_t* X, const uint8_t* bases_meta, int P, int d_rt,
                             uint8_t* payload, uint32_t* inline_dst, uint16_t* pool_dst, CompressShared& sh) {
  const int D = DT ? DT : d_rt;
  const int nchunks = P * D / 8;
  uint32_t rank = 0;
  for (int c0 = 0; c0 < nchunks; c0 += kCompressThreads) {
    const int c = c0 + (int)threadIdx.x;
    uint32_t word = 0, ne = 0;
    uint32_t sm_lo = 0, sm_hi = 0;
    uint16_t xs[8];
    uint32_t escmask = 0;
    if (c < nchunks) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = 8 * c + j;
        const int idx = storage_to_index<IsV>(s, D);
        const int tok = idx / D, d = idx % D;
        const uint16_t x = X[idx];
        xs[j] = x;
        const int b = bases_meta[base_index<CH>(tok, d, D)];
        const int e = (x >> 7) & 0xFF;
        int off = e - b;
        if (off < 0 || off > 14) { off = kEscape; escmask |= 1u << j; ++ne; }
        const int bit = (j & 1) ? (16 + 4 * (j >> 1)) : (4 * (j >> 1));
        word |= (uint32_t)off << bit;
        const uint32_t sm = ((x >> 8) & 0x80u) | (x & 0x7Fu);
        if (j < 4) sm_lo |= sm << (8 * j); else sm_hi |= sm << (8 * (j - 4));
      }
      const int t = (8 * c) / (kTile * D), r = (8 * c) % (kTile * D);
      uint8_t* tb = payload + (size_t)t * tile_bytes(D);
      *reinterpret_cast<uint2*>(tb + r) = make_uint2(sm_lo, sm_hi);
      *reinterpret_cast<uint32_t*>(tb + 16 * D + r / 2) = word;
    }
    uint32_t total;
    uint32_t pre = block_excl_scan(ne, sh, &total);
    if (escmask && (inline_dst || pool_dst)) {
      uint32_t k = rank + pre;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (escmask & (1u << j)) {
          if (inline_dst) inline_dst[k] = (uint32_t)xs[j] | ((uint32_t)(8 * c + j) << 16);
          else pool_dst[k] = xs[j];
          ++k;
        }
      }
    }
    rank += total;
  }
}

// Compresses src_k, src_v ([P][D] token-major raw BF16) into `unit`. DT: the head dim when fixed
// at compile time (64, 128), 0 to take it from d_rt.
template <int DT, bool CH = false>
__device__ void compress_unit(const uint16_t* __restrict__ src_k, const uint16_t* __restrict__ src_v, int P, int d_rt,
                              uint8_t* __restrict__ unit, uint16_t* __restrict__ pool, int64_t pool_cap,
                              uint64_t* __restrict__ cursor, uint32_t* __restrict__ status,
                              uint16_t* sh_x /* [2*P*D] */, uint8_t* sh_base /* [2*P*G] */, CompressShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = DT ? DT : d_rt;
  const int G = D / kGroup, PD = P * D;
  // 1. stage
  for (int i = tid; i < PD / 8; i += kCompressThreads) {
    reinterpret_cast<uint4*>(sh_x)[i] = reinterpret_cast<const uint4*>(src_k)[i];
    reinterpret_cast<uint4*>(sh_x + PD)[i] = reinterpret_cast<const uint4*>(src_v)[i];
  }
  if (tid < 2) sh.esc_count[tid] = 0;
  __syncthreads();
  // 2. bases, one group per wave at a time
  uint32_t cnt[2] = {0, 0};
  const int ngroups = 2 * P * G;
  for (int q = wave; q < ngroups; q += kCompressThreads / 64) {
    const int tensor = q / (P * G), rem = q % (P * G);
    int tok, d;   // this lane's value of the group
    if (CH) { tok = (rem / (D / 4)) * kTile + lane / 4; d = 4 * (rem % (D / 4)) + lane % 4; }
    else { tok = rem / G; d = (rem % G) * kGroup + lane; }
    const uint16_t x = sh_x[tensor * PD + tok * D + d];
    const uint32_t e = (x >> 7) & 0xFFu;
    const uint32_t b = group_base(e, sh.bins[wave], lane);
    const uint64_t escm = ballot((e - b) > 14u);
    cnt[tensor] += (uint32_t)__builtin_popcountll(escm);
    if (lane == 0) sh_base[tensor * P * G + base_index<CH>(tok, d, D)] = (uint8_t)b;
  }
  if (lane == 0) {
    atomicAdd(&sh.esc_count[0], cnt[0]);
    atomicAdd(&sh.esc_count[1], cnt[1]);
  }
  __syncthreads();
  // 3. where the escapes go
  const uint32_t kc = sh.esc_count[0], vc = sh.esc_count[1], total = kc + vc;
  const int cap = inline_capacity(P, D);
  const uint32_t hdr = hdr_offset(P, D);
  if (tid == 0) {
    sh.drop = 0;
    if ((int)total <= cap) {
      sh.dest = kInline;
    } else {
      const uint64_t off = atomicAdd((unsigned long long*)cursor, (unsigned long long)total);
      if (off + total > (uint64_t)pool_cap) {
        atomicOr(status, kStatusPoolFull);
        sh.drop = 1;
        sh.dest = kInline;
      } else {
        sh.dest = off;
      }
    }
  }
  __syncthreads();
  const uint64_t dest = sh.dest;
  const bool keep = sh.drop == 0;
  uint32_t* inl = (keep && dest == kInline) ? reinterpret_cast<uint32_t*>(unit + hdr + 16) : nullptr;
  uint16_t* pl = (keep && dest != kInline) ? pool + dest : nullptr;
  // 4. payload and escapes
  encode_block<false, DT, CH>(sh_x, sh_base, P, D, unit + kblock_offset(P, D), inl, pl, sh);
  encode_block<true, DT, CH>(sh_x + PD, sh_base + P * G, P, D, unit + vblock_offset(P, D), inl ? inl + kc : nullptr,
                             pl ? pl + kc : nullptr, sh);
  // 5. meta: bases, header, zero tail of the inline area
  for (int i = tid; i < 2 * P * G; i += kCompressThreads) unit[i] = sh_base[i];
  const uint32_t used = inl ? 4 * total : 0;
  for (uint32_t i = hdr + 16 + used + tid; i < meta_bytes(P, D); i += kCompressThreads) unit[i] = 0;
  if (tid == 0) {
    uint32_t* h = reinterpret_cast<uint32_t*>(unit + hdr);
    h[0] = keep ? kc : 0;
    h[1] = keep ? vc : 0;
    *reinterpret_cast<uint64_t*>(unit + hdr + 8) = dest;
  }
}

}  // namespace kvz
