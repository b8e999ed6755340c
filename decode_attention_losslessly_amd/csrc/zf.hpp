// ZipFusion's own block format (ZipFusion summary, §III.B "Lossless KV Cache Format"), the
// library's second cache format: a 512-value block is compressed when every exponent in it
// lies in [b, b + 15], b = its smallest exponent rounded down to even; a compressed value keeps
// its low byte (lowest exponent bit + 7 fraction bits) and a 4-bit code, sign << 3 | k with
// k = e/2 - b/2; the 512 low bytes come first, then the 256 code bytes (even position in the
// low nibble), 768 bytes in all. Other blocks are kept raw in the pool.
//
// Blocks are 512 consecutive storage positions of a 16-token tile, in the main format's storage
// order (K token-major, V dim-major), so a lane's loads have the same shape in both formats:
// a 16-value piece is 16 low bytes and 8 code bytes. Unit (one page of one head):
//   meta   block bytes (b/2, or 0xFF = raw), K blocks of every tile then V blocks, padded to 8
//          bytes; u64 pool offset of the unit's raw blocks (u16 elements, all ones if none);
//          zero padding to a multiple of 128 bytes
//   slots  one 768-byte slot per block in the same order; a raw block's slot is zero and its
//          512 values are in the pool at offset + 512 * (its rank among the unit's raw blocks)
#pragma once

#include "compress.hpp"
#include "kvz_lanes.hpp"

namespace kvz {

constexpr int kZfBlock = 512;
constexpr int kZfSlot = 768;
constexpr uint32_t kZfRaw = 0xFFu;

__host__ __device__ constexpr int zf_blocks_per_tile(int D) { return 16 * D / kZfBlock; }
__host__ __device__ constexpr int zf_nblocks(int P, int D) { return 2 * (P / kTile) * zf_blocks_per_tile(D); }
__host__ __device__ constexpr uint32_t zf_rawoff_offset(int P, int D) {
  return (uint32_t)((zf_nblocks(P, D) + 7) / 8 * 8);
}
__host__ __device__ constexpr uint32_t zf_meta_bytes(int P, int D) {
  return (zf_rawoff_offset(P, D) + 8 + 127) / 128 * 128;
}
__host__ __device__ constexpr uint32_t zf_unit_bytes(int P, int D) {
  return zf_meta_bytes(P, D) + (uint32_t)zf_nblocks(P, D) * kZfSlot;
}
// block index of (K or V, tile, block within tile)
__host__ __device__ constexpr int zf_block_index(bool is_v, int P, int D, int tile, int j) {
  return (is_v ? (P / kTile) * zf_blocks_per_tile(D) : 0) + tile * zf_blocks_per_tile(D) + j;
}

// ---------------------------------------------------------------- per-lane loads
// A lane's piece (16 storage positions starting at 16 * piece of the tile) of K or V: its low
// bytes, its codes and its block's meta byte.
struct ZPiece {
  uint4 low;
  uint2 code;
  uint32_t meta;
};

__device__ __forceinline__ void zf_load_piece(const uint8_t* unit, int P, int D, bool is_v, int tile, int piece,
                                              ZPiece& z) {
  const int j = (16 * piece) / kZfBlock, o = (16 * piece) % kZfBlock;
  const int idx = zf_block_index(is_v, P, D, tile, j);
  const uint8_t* slot = unit + zf_meta_bytes(P, D) + (size_t)idx * kZfSlot;
  z.low = stream16(slot + o);
  z.code = stream8(slot + kZfBlock + o / 2);
  z.meta = stream1(unit + idx);
}

// The grouped-query K layout (lane l: token l % 16, dims 32 (l / 16) .. + 31, i.e. the adjacent
// pieces 2c, 2c + 1 of chunk c = 4 (l % 16) + l / 16): 32 values of one block, 32 low bytes,
// 16 code bytes and the block's meta byte.
struct ZPair {
  uint4 low0, low1;
  uint4 code;
  uint32_t meta;
};

__device__ __forceinline__ void zf_load_pair(const uint8_t* unit, int P, int D, int tile, int piece0, ZPair& z) {
  const int j = (16 * piece0) / kZfBlock, o = (16 * piece0) % kZfBlock;
  const int idx = zf_block_index(false, P, D, tile, j);
  const uint8_t* slot = unit + zf_meta_bytes(P, D) + (size_t)idx * kZfSlot;
  z.low0 = stream16(slot + o);
  z.low1 = stream16(slot + o + 16);
  z.code = stream16(slot + kZfBlock + o / 2);
  z.meta = stream1(unit + idx);
}

// ---------------------------------------------------------------- rebuild
// 8 values from their low bytes (L0: values 0..3, L1: 4..7) and codes (W: value i in nibble i,
// the even value of each byte in its low nibble): high byte = sign << 7 | (b/2 + k), where
// b/2 + k = e/2 <= 127 never reaches bit 7, so four high bytes come from one 32-bit add (the
// sign is moved from bit 3 to bit 7 of its byte). out[k] = values 2k, 2k+1 as a BF16 pair.
__device__ __forceinline__ void zf_decode8(uint32_t L0, uint32_t L1, uint32_t W, uint32_t B, uint32_t* out) {
  const uint32_t ce = W & 0x0F0F0F0Fu, co = (W >> 4) & 0x0F0F0F0Fu;   // codes of values 0,2,4,6 / 1,3,5,7
  const uint32_t se = ce & 0x08080808u, so = co & 0x08080808u;
  const uint32_t he = ((ce ^ se) + B) | (se << 4);                     // high bytes of values 0,2,4,6
  const uint32_t ho = ((co ^ so) + B) | (so << 4);                     // high bytes of values 1,3,5,7
  const uint32_t h03 = __builtin_amdgcn_perm(ho, he, 0x05010400u);     // h0 h1 h2 h3
  const uint32_t h47 = __builtin_amdgcn_perm(ho, he, 0x07030602u);     // h4 h5 h6 h7
  out[0] = __builtin_amdgcn_perm(h03, L0, 0x05010400u);                // L0 h0 L1 h1
  out[1] = __builtin_amdgcn_perm(h03, L0, 0x07030602u);
  out[2] = __builtin_amdgcn_perm(h47, L1, 0x05010400u);
  out[3] = __builtin_amdgcn_perm(h47, L1, 0x07030602u);
}

// 16 values of one piece into 8 BF16 pairs (meta must not be kZfRaw)
__device__ __forceinline__ void zf_decode_piece(const ZPiece& z, uint32_t* pairs) {
  const uint32_t B = z.meta * 0x01010101u;
  zf_decode8(z.low.x, z.low.y, z.code.x, B, pairs);
  zf_decode8(z.low.z, z.low.w, z.code.y, B, pairs + 4);
}

// 32 values of a pair into 16 BF16 pairs (meta must not be kZfRaw)
__device__ __forceinline__ void zf_decode_pair(const ZPair& z, uint32_t* pairs) {
  const uint32_t B = z.meta * 0x01010101u;
  zf_decode8(z.low0.x, z.low0.y, z.code.x, B, pairs);
  zf_decode8(z.low0.z, z.low0.w, z.code.y, B, pairs + 4);
  zf_decode8(z.low1.x, z.low1.y, z.code.z, B, pairs + 8);
  zf_decode8(z.low1.z, z.low1.w, z.code.w, B, pairs + 12);
}

// the piece's 16 values straight from the pool (its block is raw); rank = the block's rank
// among the unit's raw blocks
__device__ __forceinline__ void zf_raw_piece(const uint16_t* pool, uint64_t off, uint32_t rank, int piece,
                                             uint32_t* pairs) {
  const uint4* src = reinterpret_cast<const uint4*>(pool + off + (size_t)rank * kZfBlock + (16 * piece) % kZfBlock);
  const uint4 a = src[0], b = src[1];
  pairs[0] = a.x; pairs[1] = a.y; pairs[2] = a.z; pairs[3] = a.w;
  pairs[4] = b.x; pairs[5] = b.y; pairs[6] = b.z; pairs[7] = b.w;
}

// A unit of at most 8 blocks keeps its blocks' meta bytes in bytes 0..7 and its raw-pool offset in
// bytes 8..15: its first 16 bytes (`head`) then give a raw block's pool offset and rank with no
// further load.
__host__ __device__ constexpr bool zf_head_holds_meta(int P, int D) { return zf_nblocks(P, D) <= 8; }

__device__ __forceinline__ uint64_t zf_head_offset(const uint4& head) {
  return (uint64_t)head.z | ((uint64_t)head.w << 32);
}

// bit i set when block i (< 8) is raw: meta bytes 0..7 of the head equal to kZfRaw
__device__ __forceinline__ uint32_t zf_head_raw_mask(const uint4& head) {
  const uint64_t e = ~((uint64_t)head.x | ((uint64_t)head.y << 32));   // raw bytes become zero
  const uint64_t hi = 0x8080808080808080ull, lo7 = 0x7F7F7F7F7F7F7F7Full;
  const uint64_t raw = ~((((e & lo7) + lo7) | e) & hi) & hi;          // bit 7 of each raw byte
  return (uint32_t)((raw * 0x0002040810204081ull) >> 56);            // gather bit 7 of byte i into bit i
}

// rank of block idx (< 8) among the unit's raw blocks, from the head's raw-block mask
__device__ __forceinline__ uint32_t zf_head_rank(uint32_t raw_mask, int idx) {
  return (uint32_t)__builtin_popcount(raw_mask & ((1u << idx) - 1u));
}

// rank of block idx among the raw blocks of the unit (counts meta bytes equal to kZfRaw below idx)
__device__ __forceinline__ uint32_t zf_raw_rank(const uint8_t* unit, int idx) {
  uint32_t r = 0;
  for (int i = 0; i < idx; ++i) r += unit[i] == kZfRaw ? 1u : 0u;
  return r;
}

// rank of block idx among the unit's raw blocks, from the head's mask when it holds the metas
__device__ __forceinline__ uint32_t zf_rank(uint32_t raw_mask, const uint8_t* unit, bool in_head, int idx) {
  return in_head ? zf_head_rank(raw_mask, idx) : zf_raw_rank(unit, idx);
}

__device__ __forceinline__ uint64_t zf_raw_offset(const uint8_t* unit, int P, int D) {
  return *reinterpret_cast<const uint64_t*>(unit + zf_rawoff_offset(P, D));
}

// ---------------------------------------------------------------- compression
// Compresses src_k, src_v ([P][D] token-major raw BF16) into one unit with a 256-thread
// workgroup: one wave per block finds the block's exponent range; the unit's raw blocks get
// one contiguous range of the pool (atomically bumped cursor); then each lane writes 8 values
// (8 low bytes, one code word) or copies them raw.
__device__ void compress_unit_zf(const uint16_t* __restrict__ src_k, const uint16_t* __restrict__ src_v, int P,
                                 int D, uint8_t* __restrict__ unit, uint16_t* __restrict__ pool, int64_t pool_cap,
                                 uint64_t* __restrict__ cursor, uint32_t* __restrict__ status,
                                 uint16_t* sh_x /* [2*P*D] */, uint8_t* sh_meta /* [nb] */,
                                 uint16_t* sh_rank /* [nb] */, CompressShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int PD = P * D, nb = zf_nblocks(P, D), half = nb / 2;
  for (int i = tid; i < PD / 8; i += kCompressThreads) {
    reinterpret_cast<uint4*>(sh_x)[i] = reinterpret_cast<const uint4*>(src_k)[i];
    reinterpret_cast<uint4*>(sh_x + PD)[i] = reinterpret_cast<const uint4*>(src_v)[i];
  }
  __syncthreads();
  // value i (< 8) of lane `lane` in block idx, as an index into sh_x
  auto src_index = [&](int idx, int i) {
    const bool is_v = idx >= half;
    const int s = (is_v ? idx - half : idx) * kZfBlock + 8 * lane + i;   // storage position in the tensor
    return (is_v ? PD : 0) + (is_v ? storage_to_index<true>(s, D) : storage_to_index<false>(s, D));
  };
  // 1. exponent range of every block
  for (int idx = wave; idx < nb; idx += kCompressThreads / 64) {
    uint32_t lo = 255, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t e = (sh_x[src_index(idx, i)] >> 7) & 0xFFu;
      lo = min(lo, e);
      hi = max(hi, e);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      lo = min(lo, (uint32_t)__shfl_xor((int)lo, m));
      hi = max(hi, (uint32_t)__shfl_xor((int)hi, m));
    }
    const uint32_t b = lo & ~1u;
    if (lane == 0) sh_meta[idx] = (uint8_t)(hi - b <= 15 ? (b >> 1) : kZfRaw);
  }
  __syncthreads();
  // 2. raw ranks and the unit's pool range
  if (tid == 0) {
    uint32_t n = 0;
    for (int idx = 0; idx < nb; ++idx) {
      sh_rank[idx] = (uint16_t)n;
      n += sh_meta[idx] == kZfRaw ? 1u : 0u;
    }
    sh.drop = 0;
    sh.dest = kInline;   // no raw block
    if (n) {
      const uint64_t need = (uint64_t)n * kZfBlock;
      const uint64_t off = atomicAdd((unsigned long long*)cursor, (unsigned long long)need);
      if (off + need > (uint64_t)pool_cap) {
        atomicOr(status, kStatusPoolFull);
        sh.drop = 1;
      } else {
        sh.dest = off;
      }
    }
  }
  __syncthreads();
  const uint64_t dest = sh.dest;
  const bool keep = sh.drop == 0;
  // 3. slots and raw copies
  const uint32_t mb = zf_meta_bytes(P, D);
  for (int idx = wave; idx < nb; idx += kCompressThreads / 64) {
    const uint32_t meta = sh_meta[idx];
    uint8_t* slot = unit + mb + (size_t)idx * kZfSlot;
    uint16_t x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = sh_x[src_index(idx, i)];
    if (meta == kZfRaw) {
      if (keep) {
        uint16_t* dst = pool + dest + (size_t)sh_rank[idx] * kZfBlock + 8 * lane;
        *reinterpret_cast<uint4*>(dst) = make_uint4(x[0] | (uint32_t)x[1] << 16, x[2] | (uint32_t)x[3] << 16,
                                                    x[4] | (uint32_t)x[5] << 16, x[6] | (uint32_t)x[7] << 16);
      }
      *reinterpret_cast<uint2*>(slot + 8 * lane) = make_uint2(0, 0);
      *reinterpret_cast<uint32_t*>(slot + kZfBlock + 4 * lane) = 0;
    } else {
      uint32_t lo0 = 0, lo1 = 0, code = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t e = (x[i] >> 7) & 0xFFu;
        const uint32_t c = ((uint32_t)(x[i] >> 15) << 3) | ((e >> 1) - meta);
        code |= c << (4 * i);
        if (i < 4) lo0 |= (uint32_t)(x[i] & 0xFFu) << (8 * i);
        else lo1 |= (uint32_t)(x[i] & 0xFFu) << (8 * (i - 4));
      }
      *reinterpret_cast<uint2*>(slot + 8 * lane) = make_uint2(lo0, lo1);
      *reinterpret_cast<uint32_t*>(slot + kZfBlock + 4 * lane) = code;
    }
  }
  // 4. meta
  for (uint32_t i = tid; i < mb; i += kCompressThreads) {
    uint8_t v = 0;
    if ((int)i < nb) v = sh_meta[i];
    unit[i] = v;
  }
  __syncthreads();
  if (tid == 0) *reinterpret_cast<uint64_t*>(unit + zf_rawoff_offset(P, D)) = (keep && dest != kInline) ? dest : kInline;
}

}  // namespace kvz
