// Split-K merge: combines the (m, l, acc) partials of one (request, query head) into the output
// (the pages merge split results after attention and count the merge in its time: ZipFusion
// summary, §IV.B "Attention Kernel Performance").
//   M = max_s m_s,  w_s = 2^(m_s - M),  o = sum_s w_s acc_s / sum_s w_s l_s
// The plan pages per split that the split kernel used (or its chunk count, when it used the
// ranked schedule) and its plan pages per page of the table are read from where it recorded them.
// Output in BF16 (round to nearest even) and optionally in fp32; zeros when the request is empty.
//
// W waves per row: each takes the splits s = w, w + W, ... in one pass, eight at a time (all 8
// loads issued before the first is used), keeping its own running maximum, so a row costs one
// round trip per 8 of a wave's splits; the W partial results meet in LDS, rescaled to the
// largest maximum. Rows with at most 8 splits take one wave each (4 rows per
// workgroup); otherwise few rows (a small batch, where the splits are many) get 8 waves per
// row up to 64 splits and 16 beyond, and more rows 4.
#include "attn_common.hpp"

namespace kvz {

template <int D, int W, int R>
__global__ __launch_bounds__(64 * W * R) void merge_kernel(const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
                                                       const int32_t* __restrict__ seq_lens, int B, int Hq, int P,
                                                       int max_pages, int S, const int32_t* __restrict__ chosen,
                                                       int dense, uint16_t* __restrict__ out,
                                                       float* __restrict__ out_f32) {
  constexpr int NV = D / 64;
  __shared__ float sh_num[W][D];
  __shared__ float sh_den[W], sh_max[W];
  static_assert(W == 1 || R == 1, "several waves per row: one row per workgroup");
  const int lane = threadIdx.x & 63;
  const int wave = W == 1 ? 0 : (int)(threadIdx.x >> 6);
  const int row = (int)uniform(blockIdx.x * R + (R > 1 ? (threadIdx.x >> 6) : 0));
  if (row >= B * Hq) return;   // uniform per workgroup when W > 1 (R == 1 and the grid has one block per row)
  const int r = row / Hq;
  int L = sload<int32_t>(seq_lens + r);
  L = L < 0 ? 0 : min(L, max_pages * P);
  const int c = sload<int32_t>(chosen);   // < 0: the split kernel used -c ranked chunks
  const int tpp = max(1, sload<int32_t>(chosen + 1));   // plan pages per page of the table
  const int npages = dense ? (L + P - 1) / P : L / P * tpp;
  const int Sr = min(c < 0 ? -c : active_splits(npages, max(1, c)), S);
  const float* ml = ws_ml + (size_t)row * S * 2;
  const float* acc = ws_acc + (size_t)row * S * D;
  // One pass: the wave's splits s = wave + W * k, eight at a time (all loads of a batch issued
  // before the first is used), folded into a running maximum M, weight sum den and weighted
  // sum num; a batch that raises M rescales what came before by 2^(M_old - M_new).
  float M = -INFINITY, den = 0.f, num[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) num[i] = 0.f;
  for (int k0 = 0; wave + W * k0 < Sr; k0 += 8) {
    float m[8], l[8], a[8][NV];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = wave + W * (k0 + j);
      const int sc = s < Sr ? s : 0;
      m[j] = s < Sr ? ml[2 * sc] : -INFINITY;
      l[j] = ml[2 * sc + 1];
#pragma unroll
      for (int i = 0; i < NV; ++i) a[j][i] = acc[(size_t)sc * D + lane + 64 * i];
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < 8; ++j) mb = fmaxf(mb, m[j]);
    if (mb == -INFINITY) continue;   // nothing but empty splits so far
    const float f = __builtin_amdgcn_exp2f(M - mb);   // 0 while M is -inf
    den *= f;
#pragma unroll
    for (int i = 0; i < NV; ++i) num[i] *= f;
    M = mb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float wj = __builtin_amdgcn_exp2f(m[j] - M);   // 0 for an empty split or a padded slot
      den += wj * l[j];
#pragma unroll
      for (int i = 0; i < NV; ++i) num[i] += wj * a[j][i];
    }
  }
  float dsum = den;
  if constexpr (W > 1) {
#pragma unroll
    for (int i = 0; i < NV; ++i) sh_num[wave][lane + 64 * i] = num[i];
    if (lane == 0) {
      sh_den[wave] = den;
      sh_max[wave] = M;
    }
    __syncthreads();
    if (wave != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) Mt = fmaxf(Mt, sh_max[w]);
    float fw[W];
#pragma unroll
    for (int w = 0; w < W; ++w) fw[w] = Mt == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sh_max[w] - Mt);
    dsum = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) dsum += fw[w] * sh_den[w];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float n = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) n += fw[w] * sh_num[w][lane + 64 * i];
      num[i] = n;
    }
  }
  const float inv = dsum > 0.f ? 1.0f / dsum : 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float o = num[i] * inv;
    const size_t idx = (size_t)row * D + lane + 64 * i;
    out[idx] = (uint16_t)(pack_bf16(o, 0.f) & 0xFFFFu);
    if (out_f32) out_f32[idx] = o;
  }
}

int launch_merge(const float* ws_acc, const float* ws_ml, const int32_t* seq_lens, int B, int Hq, int D, int P,
                 int max_pages, int S, const int32_t* chosen, int dense, uint16_t* out, float* out_f32,
                 hipStream_t stream) {
  const int rows = B * Hq;
  // 0: a wave per row, 1: 4 waves, 2: 16 waves, 3: 8 waves (few rows of up to 64 splits: one batch
  // of eight loads per wave, half the workgroup of 16 to reduce; batch 1 at 4K, 64 splits a row:
  // the merge 6.3 -> 6.0 us and the step 16.4 -> 16.0 us)
  const int shape = S <= 8 ? 0 : (rows < 1024 ? (S <= 64 ? 3 : 2) : 1);
  const unsigned blocks = shape == 0 ? (unsigned)(rows + 3) / 4 : (unsigned)rows;
  const unsigned threads = shape == 2 ? 1024 : (shape == 3 ? 512 : 256);
#define KVZ_MERGE(DD, WW, RR)                                                                                  \
  hipLaunchKernelGGL((merge_kernel<DD, WW, RR>), dim3(blocks), dim3(threads), 0, stream, ws_acc, ws_ml, seq_lens, \
                     B, Hq, P, max_pages, S, chosen, dense, out, out_f32)
  if (D == 128) {
    if (shape == 0) KVZ_MERGE(128, 1, 4); else if (shape == 1) KVZ_MERGE(128, 4, 1);
    else if (shape == 3) KVZ_MERGE(128, 8, 1); else KVZ_MERGE(128, 16, 1);
  } else if (D == 64) {
    if (shape == 0) KVZ_MERGE(64, 1, 4); else if (shape == 1) KVZ_MERGE(64, 4, 1);
    else if (shape == 3) KVZ_MERGE(64, 8, 1); else KVZ_MERGE(64, 16, 1);
  } else {
    return -2;
  }
#undef KVZ_MERGE
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvz
