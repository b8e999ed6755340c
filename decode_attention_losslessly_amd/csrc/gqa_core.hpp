// The grouped-query attention core shared by the kernels over both cache formats and the
// uncompressed baseline: the per-wave state, one token tile through the matrix cores (scores,
// online softmax, P.V), raw (uncompressed) tiles, and the start and end of a work item. The
// kernels differ only in how they load and rebuild K and V. See attn_gqa.hip for the layout.
#pragma once

#include "attn_common.hpp"
#include "kvz_lanes.hpp"

namespace kvz {

constexpr int kGqaRows = 8;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

struct GqaState {
  float m;          // running max of query row l%16 (log2 domain)
  float l;          // this lane's share of that row's denominator
  f32x4 o[8];       // output tile j: rows 4*(l/16)+i, dim 16j + l%16
  uint32_t q[16];   // B operand: query row l%16, dims 32*(l/16)..+31
};

// One token tile: kp = this lane's K pairs (token l%16, dims 32*(l/16)..), vdim[2]/vp[2][8] =
// V token pairs of two dims owned by this lane; `rows` valid tokens.
__device__ __forceinline__ void gqa_tile(GqaState& st, const uint32_t (&kp)[16], const int (&vdim)[2],
                                         const uint32_t (&vp)[2][8], int rows, float scale, uint32_t* vlds,
                                         int lane) {
  // scores S^T[token][row]
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 a = {kp[4 * c], kp[4 * c + 1], kp[4 * c + 2], kp[4 * c + 3]};
    const u32x4 b = {st.q[4 * c], st.q[4 * c + 1], st.q[4 * c + 2], st.q[4 * c + 3]};
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), sc,
                                                  0, 0, 0);
  }
  const int tok0 = 4 * (lane >> 4);
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = (tok0 + i < rows) ? sc[i] * scale : -INFINITY;
  // online softmax per query row (column l%16; the 4 lanes l%16 + 16k share it)
  const bool up = (s[0] > st.m) | (s[1] > st.m) | (s[2] > st.m) | (s[3] > st.m);
  if (ballot(up)) {
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(st.m, mx);
    const float alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(st.m - mn);
    st.l *= alpha;
    st.m = mn;
    // output rows of this lane are 4*(l/16)+i: fetch their alphas
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, tok0 + i);
#pragma unroll
      for (int j = 0; j < 8; ++j) st.o[j][i] *= ai;
    }
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = (s[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[i] - st.m);
  const uint32_t h01 = pack_bf16(p[0], p[1]), h23 = pack_bf16(p[2], p[3]);
  const float h[4] = {bf16lo_to_f32(h01), bf16hi_to_f32(h01), bf16lo_to_f32(h23), bf16hi_to_f32(h23)};
  const uint32_t l01 = pack_bf16(p[0] - h[0], p[1] - h[1]), l23 = pack_bf16(p[2] - h[2], p[3] - h[3]);
  st.l += (h[0] + bf16lo_to_f32(l01)) + (h[1] + bf16hi_to_f32(l01)) + (h[2] + bf16lo_to_f32(l23)) +
          (h[3] + bf16hi_to_f32(l23));
  const bool lo_row = (lane & 15) >= kGqaRows;
  const u32x2 pa = {lo_row ? l01 : h01, lo_row ? l23 : h23};
  // V -> LDS [dim][pair] (8 u32 per dim), then B operands: tokens 4q..4q+3 of dim 16j + l%16.
  // Dims with bit 3 set keep their two 16-byte halves in swapped places, so that dims d and d+8,
  // whose rows are 64 dwords apart, use different banks on the stores and on the reads.
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int sw = (vdim[g] >> 1) & 4;
    uint32_t* row = vlds + vdim[g] * 8;
    *reinterpret_cast<uint4*>(row + sw) = make_uint4(vp[g][0], vp[g][1], vp[g][2], vp[g][3]);
    *reinterpret_cast<uint4*>(row + (4 ^ sw)) = make_uint4(vp[g][4], vp[g][5], vp[g][6], vp[g][7]);
  }
  wave_lds_sync();
  const bf16x4 A = __builtin_bit_cast(bf16x4, pa);
  const int qg = lane >> 4;
  const int rd_off = (2 * qg) ^ ((lane >> 1) & 4);   // bit 3 of the dim is bit 3 of l%16
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint2 bv = *reinterpret_cast<const uint2*>(vlds + (16 * j + (lane & 15)) * 8 + rd_off);
    const u32x2 b = {bv.x, bv.y};
    st.o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(bf16x4, b), st.o[j], 0, 0, 0);
  }
  wave_lds_sync();
}

// ---------------------------------------------------------------- raw (dense / tail) source
// K: token l%16, dims 32*(l/16)..+31 (64 B); V: dims 2l, 2l+1 of all 16 tokens, regrouped into
// token pairs. Rows >= `rows` are read as zeros.
struct GqaRawStage {
  uint4 k[4];
  uint32_t v[16];
  int rows;
};

__device__ __forceinline__ void gqa_raw_load(GqaRawStage& st, const uint16_t* kpage, const uint16_t* vpage, int tok0,
                                             int rows, int lane) {
  st.rows = rows;
  const int tok = lane & 15;
  const bool ok = tok < rows;
  // K loads share cache lines with each other (cached); V rows are read whole (streamed)
  const uint4* kr = reinterpret_cast<const uint4*>(kpage + (size_t)(tok0 + (ok ? tok : 0)) * 128 + 32 * (lane >> 4));
#pragma unroll
  for (int j = 0; j < 4; ++j) st.k[j] = kr[j];
  const uint32_t* vr = reinterpret_cast<const uint32_t*>(vpage + (size_t)tok0 * 128) + lane;
#pragma unroll
  for (int t = 0; t < 16; ++t) st.v[t] = stream4(vr + (size_t)(t < rows ? t : 0) * 64);
}

__device__ __forceinline__ void gqa_raw_compute(GqaState& st, const GqaRawStage& stg, float scale, uint32_t* vlds,
                                                int lane) {
  const bool ok = (lane & 15) < stg.rows;
  uint32_t kp[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 x = ok ? stg.k[j] : make_uint4(0, 0, 0, 0);
    kp[4 * j] = x.x; kp[4 * j + 1] = x.y; kp[4 * j + 2] = x.z; kp[4 * j + 3] = x.w;
  }
  uint32_t raw[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) raw[t] = t < stg.rows ? stg.v[t] : 0u;
  uint32_t vp[2][8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    vp[0][k] = __builtin_amdgcn_perm(raw[2 * k + 1], raw[2 * k], 0x05040100u);
    vp[1][k] = __builtin_amdgcn_perm(raw[2 * k + 1], raw[2 * k], 0x07060302u);
  }
  const int vdim[2] = {2 * lane, 2 * lane + 1};
  gqa_tile(st, kp, vdim, vp, stg.rows, scale, vlds, lane);
}

__device__ __forceinline__ void gqa_raw_tile(GqaState& st, const uint16_t* kpage, const uint16_t* vpage, int tok0,
                                             int rows, float scale, uint32_t* vlds, int lane) {
  GqaRawStage stg;
  gqa_raw_load(stg, kpage, vpage, tok0, rows, lane);
  gqa_raw_compute(st, stg, scale, vlds, lane);
}

// ---------------------------------------------------------------- work item start and end
__device__ __forceinline__ void gqa_init(GqaState& st, const uint16_t* q, int r, int Hq, int hq0, int nq, int lane) {
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int row = (lane & 15) % kGqaRows;
  const bool ok = row < nq;
  const uint4* qr = reinterpret_cast<const uint4*>(q + ((size_t)r * Hq + hq0 + (ok ? row : 0)) * 128 + 32 * (lane >> 4));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 x = ok ? qr[j] : make_uint4(0, 0, 0, 0);
    st.q[4 * j] = x.x; st.q[4 * j + 1] = x.y; st.q[4 * j + 2] = x.z; st.q[4 * j + 3] = x.w;
  }
}

__device__ __forceinline__ void gqa_store(const GqaState& st, int r, int Hq, int hq0, int nq, int S, int s,
                                          float* ws_acc, float* ws_ml, int lane) {
  // denominators: row n = l%16 (< 8), summed over the 4 lane groups
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  // outputs: rows 4*(l/16)+i; add row + 8 (lanes l + 32) to rows < 8
  f32x4 o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[j][i] = st.o[j][i] + __shfl_xor(st.o[j][i], 32);
  }
  if (lane < 32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = 4 * (lane >> 4) + i;
      if (n < nq) {
        float* acc = ws_acc + (((size_t)r * Hq + hq0 + n) * S + s) * 128;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[16 * j + (lane & 15)] = o[j][i];
      }
    }
  }
  if (lane < nq) {
    float* ml = ws_ml + (((size_t)r * Hq + hq0 + lane) * S + s) * 2;
    ml[0] = st.m;
    ml[1] = l;
  }
}

}  // namespace kvz
