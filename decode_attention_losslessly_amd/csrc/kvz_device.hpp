// Device-side building blocks shared by the kvz kernels (gfx950, wave64).
//
// The format (group of 64 values of one token row, sm byte = sign<<7 | mantissa, 4-bit
// exponent offset from a per-group base with 15 = escape, 16-token tiles, K token-major and
// V dim-major inside a tile, per-unit meta region) is documented in include/kvz.h. The pages
// fix only that the format is lossless and rebuilt with plain bit operations (ZipFusion
// summary, §II.A "KV Cache and BF16", §III.B "Lossless KV Cache Format", §III.C "Attention
// over the Compressed KV Cache"); everything below is this library's own design.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvz {

constexpr int kGroup = 64;
constexpr int kTile = 16;
constexpr int kEscape = 15;
constexpr uint64_t kInline = ~0ull;
constexpr uint32_t kStatusPoolFull = 1u, kStatusBadPage = 2u, kStatusSeqTooLong = 4u;

// ---------------------------------------------------------------- format geometry
__host__ __device__ constexpr uint32_t meta_bytes(int P, int D) {
  return (uint32_t)((2 * P * (D / kGroup) + 16 + 127) / 128 * 128);
}
__host__ __device__ constexpr uint32_t block_bytes(int P, int D) { return (uint32_t)(P * D * 3 / 2); }
__host__ __device__ constexpr uint32_t tile_bytes(int D) { return (uint32_t)(24 * D); }
__host__ __device__ constexpr uint32_t unit_bytes(int P, int D) {
  return meta_bytes(P, D) + 2 * block_bytes(P, D);
}
// inline escapes are 4-byte entries: value | (storage position in its block << 16)
__host__ __device__ constexpr int inline_capacity(int P, int D) {
  return (int)(meta_bytes(P, D) - 2 * P * (D / kGroup) - 16) / 4;
}
// byte offsets inside a unit
__host__ __device__ constexpr uint32_t hdr_offset(int P, int D) { return (uint32_t)(2 * P * (D / kGroup)); }
__host__ __device__ constexpr uint32_t kbase_offset(int D, int tile) { return (uint32_t)(tile * kTile * (D / kGroup)); }
__host__ __device__ constexpr uint32_t vbase_offset(int P, int D, int tile) {
  return (uint32_t)(P * (D / kGroup) + tile * kTile * (D / kGroup));
}
__host__ __device__ constexpr uint32_t kblock_offset(int P, int D) { return meta_bytes(P, D); }
__host__ __device__ constexpr uint32_t vblock_offset(int P, int D) {
  return meta_bytes(P, D) + block_bytes(P, D);
}

// ---------------------------------------------------------------- scalar (uniform) loads
// Loads through the constant address space so that a wave-uniform address becomes an
// s_load and the value lands in SGPRs. Only for memory no kernel writes while it runs.
template <typename T>
__device__ __forceinline__ T sload(const void* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(
      reinterpret_cast<uintptr_t>(p));
}

typedef uint32_t sgpr_u32x4 __attribute__((ext_vector_type(4)));
// 16-byte uniform load (16-byte aligned address)
__device__ __forceinline__ uint4 sload4(const void* p) {
  const sgpr_u32x4 v = sload<sgpr_u32x4>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ uint32_t readlane(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
__device__ __forceinline__ uint64_t ballot(bool b) { return __builtin_amdgcn_ballot_w64(b); }
__device__ __forceinline__ int lane_id() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
// v with lane `lane` replaced by val (val and lane wave-uniform)
__device__ __forceinline__ uint32_t writelane(uint32_t v, uint32_t val, int lane) {
  return lane_id() == lane ? val : v;
}

// ---------------------------------------------------------------- cross-lane arithmetic
// DPP controls (GCN/CDNA encoding)
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr3 = 0x113, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowShl4 = 0x104, kRowShl8 = 0x108;
constexpr int kRowHalfMirror = 0x141;   // lane j of each 8-lane half-row <- lane 7 - j
constexpr int kRowRor4 = 0x124, kRowRor8 = 0x128;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

template <int Ctrl, int RowMask = 0xF, int BankMask = 0xF, bool BoundZero = true>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), Ctrl,
                                                               RowMask, BankMask, BoundZero));
}
template <int Ctrl, int RowMask = 0xF, int BankMask = 0xF, bool BoundZero = true>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, Ctrl, RowMask, BankMask, BoundZero);
}

// sum over the 4 lanes of a quad, result in every lane of the quad
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_f<kQuadXor1>(v);
  v += dpp_f<kQuadXor2>(v);
  return v;
}

// sum over the 8 lanes of a half-row (lanes 8k .. 8k+7), result in every one of them: the quad
// sums, then each lane adds the other quad's sum through the half-row mirror
__device__ __forceinline__ float octet_sum(float v) {
  v = quad_sum(v);
  v += dpp_f<kRowHalfMirror>(v);
  return v;
}

// inclusive prefix sum over the 64 lanes in lane order (u32): Hillis-Steele inside each row
// of 16 lanes, then the row broadcasts carry rows 0 and 2 into rows 1 and 3, and lane 31 into
// rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_u<kRowShr1>(v);
  v += dpp_u<kRowShr2>(v);
  v += dpp_u<kRowShr4>(v);
  v += dpp_u<kRowShr8>(v);
  v += dpp_u<kRowBcast15, 0xA>(v);
  v += dpp_u<kRowBcast31, 0xC>(v);
  return v;
}

// LDS written by this wave becomes visible to this wave's later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// unsigned max over the 64 lanes, returned wave-uniform
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, k));
  return uniform(v);
}

// max over the 64 lanes, returned wave-uniform
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// ---------------------------------------------------------------- decode (§III.C)
// 16-bit field positions inside a packed pair of BF16 values: sign and mantissa come from the
// sm bytes, the exponent field (bits 7..14 and 23..30) from offset + base.
constexpr uint32_t kSmMask = 0x807F807Fu;

// Hides x from the optimiser (no instruction): after `x = W & m`, the compiler would otherwise
// rewrite (W & m) << s as (W << s) & (m << s), and the shift could no longer fuse with the add
// that follows it into one v_lshl_add_u32.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}

// Rebuilds the 8 values of one offset word: S0 holds the sm bytes of positions 0..3, S1 those
// of 4..7, W the offset word; bb[k] the base term of pair k. out[k] = (pos 2k, pos 2k+1) as a
// packed BF16 pair (low half = even position). An escaped position decodes to a placeholder
// whose exponent field is (base + 15) mod 256; callers patch it from the escape list.
__device__ __forceinline__ void decode8(uint32_t S0, uint32_t S1, uint32_t W, uint32_t bb0,
                                        uint32_t bb1, uint32_t bb2, uint32_t bb3, uint32_t* out) {
  const uint32_t x0 = __builtin_amdgcn_perm(S0, S0, 0x01010000u);   // [s0, s0, s1, s1]
  const uint32_t x1 = __builtin_amdgcn_perm(S0, S0, 0x03030202u);   // [s2, s2, s3, s3]
  const uint32_t x2 = __builtin_amdgcn_perm(S1, S1, 0x01010000u);
  const uint32_t x3 = __builtin_amdgcn_perm(S1, S1, 0x03030202u);
  // offsets of pair k at bits 0 and 16 (k even) or 4 and 20 (k odd) of W or W >> 8: a mask,
  // then one shift-and-add puts them at bits 7 and 23 on top of the base term
  const uint32_t W8 = W >> 8;
  const uint32_t e0 = (opaque(W & 0x000F000Fu) << 7) + bb0;
  const uint32_t e1 = (opaque(W & 0x00F000F0u) << 3) + bb1;
  const uint32_t e2 = (opaque(W8 & 0x000F000Fu) << 7) + bb2;
  const uint32_t e3 = (opaque(W8 & 0x00F000F0u) << 3) + bb3;
  out[0] = (x0 & kSmMask) | (e0 & ~kSmMask);
  out[1] = (x1 & kSmMask) | (e1 & ~kSmMask);
  out[2] = (x2 & kSmMask) | (e2 & ~kSmMask);
  out[3] = (x3 & kSmMask) | (e3 & ~kSmMask);
}

// Escape flags of an offset word: bit 4k+3 set iff the nibble at bits 4k..4k+3 is 15.
// Nibble k < 4 is position 2k of the word; nibble k >= 4 is position 2(k-4)+1.
__device__ __forceinline__ uint32_t escape_flags(uint32_t W) {
  return (((W & 0x77777777u) + 0x11111111u) & W) & 0x88888888u;
}
__host__ __device__ __forceinline__ uint32_t flag_bit(int pos) {
  return (pos & 1) ? (1u << (16 + 4 * (pos >> 1) + 3)) : (1u << (4 * (pos >> 1) + 3));
}

__device__ __forceinline__ uint32_t set_half(uint32_t v, int half, uint32_t x) {
  return half ? ((v & 0x0000FFFFu) | (x << 16)) : ((v & 0xFFFF0000u) | (x & 0xFFFFu));
}

// Sets half `half` of register `reg` of lane `lane` to x; reg, lane, half and x are
// wave-uniform, so the register is addressed through the GPR index mode, not a branch tree.
template <int N>
__device__ __forceinline__ void patch_one(uint32_t (&pairs)[N], int reg, int lane, int half, uint32_t x) {
  reg = (int)uniform((uint32_t)reg);
  const uint32_t keep = uniform(half ? 0x0000FFFFu : 0xFFFF0000u);
  const uint32_t put = uniform(half ? (x << 16) : (x & 0xFFFFu));
  const uint32_t old = pairs[reg];
  pairs[reg] = lane_id() == lane ? ((old & keep) | put) : old;
}

__device__ __forceinline__ uint32_t popc_flags(uint32_t f) { return (uint32_t)__builtin_popcount(f); }

// Escape flags with bit order = storage order: position j of the word goes to bit
// 4*(j/2) + (j%2), so that walking set bits from the lowest visits positions in list order.
__device__ __forceinline__ uint32_t flags_in_order(uint32_t f) {
  return ((f & 0x8888u) >> 3) | (((f >> 16) & 0x8888u) >> 2);
}
__device__ __forceinline__ int ordered_bit_to_pos(int b) { return 2 * (b >> 2) + (b & 1); }

// ---------------------------------------------------------------- BF16 helpers
__device__ __forceinline__ float bf16lo_to_f32(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t p) { return __builtin_bit_cast(float, p & 0xFFFF0000u); }

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// two floats -> packed BF16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

}  // namespace kvz
