// Split-K merge: combines the (m, l, acc) partials of one (request, query head) into the output
// (the pages merge split results after attention and count the merge in its time: ZipFusion
// summary, §IV.B "Attention Kernel Performance").
//   M = max_s m_s,  w_s = 2^(m_s - M),  o = sum_s w_s acc_s / sum_s w_s l_s
// The pages per split that the split kernel used (or its chunk count, when it used the ranked
// schedule) are read from where it recorded them.
// Output in BF16 (round to nearest even) and optionally in fp32; zeros when the request is empty.
//
// W waves per row: every wave reads all the maxima (one vector load per 64 splits) and takes the
// splits s = w, w + W, ...; their acc rows are loaded 8 at a time, all 8 issued before the first
// is used, so a row with many splits costs a few round trips rather than one per split; the W
// partial sums meet in LDS. Rows with at most 8 splits take one wave each (4 rows per
// workgroup); otherwise few rows (a small batch, where the splits are many) get 16 waves per
// row, and more rows 4.
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
  __shared__ float sh_den[W];
  static_assert(W == 1 || R == 1, "several waves per row: one row per workgroup");
  const int lane = threadIdx.x & 63;
  const int wave = W == 1 ? 0 : (int)(threadIdx.x >> 6);
  const int row = (int)uniform(blockIdx.x * R + (R > 1 ? (threadIdx.x >> 6) : 0));
  if (row >= B * Hq) return;   // uniform per workgroup when W > 1 (R == 1 and the grid has one block per row)
  const int r = row / Hq;
  int L = sload<int32_t>(seq_lens + r);
  L = L < 0 ? 0 : min(L, max_pages * P);
  const int npages = dense ? (L + P - 1) / P : L / P;
  const int c = sload<int32_t>(chosen);   // < 0: the split kernel used -c ranked chunks
  const int Sr = min(c < 0 ? -c : active_splits(npages, max(1, c)), S);
  const float* ml = ws_ml + (size_t)row * S * 2;
  const float* acc = ws_acc + (size_t)row * S * D;
  float M = -INFINITY;
  for (int s0 = 0; s0 < Sr; s0 += 64)
    if (s0 + lane < Sr) M = fmaxf(M, ml[2 * (s0 + lane)]);
  M = wave_max(M);
  float num[NV], den = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) num[i] = 0.f;
  if (M != -INFINITY) {
    // this wave's splits s = wave + W * k, eight at a time
    for (int k0 = 0; wave + W * k0 < Sr; k0 += 8) {
      float wgt[8], a[8][NV];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = wave + W * (k0 + j);
        const bool ok = s < Sr;
        const int sc = ok ? s : 0;
        wgt[j] = ok ? __builtin_amdgcn_exp2f(ml[2 * sc] - M) : 0.f;
        den += ok ? wgt[j] * ml[2 * sc + 1] : 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) a[j][i] = acc[(size_t)sc * D + lane + 64 * i];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < NV; ++i) num[i] += wgt[j] * a[j][i];
    }
  }
  float dsum = den;
  if constexpr (W > 1) {
#pragma unroll
    for (int i = 0; i < NV; ++i) sh_num[wave][lane + 64 * i] = num[i];
    if (lane == 0) sh_den[wave] = den;
    __syncthreads();
    if (wave != 0) return;
    dsum = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) dsum += sh_den[w];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float n = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) n += sh_num[w][lane + 64 * i];
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
  const int shape = S <= 8 ? 0 : (rows < 1024 ? 2 : 1);   // 0: a wave per row, 1: 4 waves, 2: 16 waves
  const unsigned blocks = shape == 0 ? (unsigned)(rows + 3) / 4 : (unsigned)rows;
  const unsigned threads = shape == 2 ? 1024 : 256;
#define KVZ_MERGE(DD, WW, RR)                                                                                  \
  hipLaunchKernelGGL((merge_kernel<DD, WW, RR>), dim3(blocks), dim3(threads), 0, stream, ws_acc, ws_ml, seq_lens, \
                     B, Hq, P, max_pages, S, chosen, dense, out, out_f32)
  if (D == 128) {
    if (shape == 0) KVZ_MERGE(128, 1, 4); else if (shape == 1) KVZ_MERGE(128, 4, 1); else KVZ_MERGE(128, 16, 1);
  } else if (D == 64) {
    if (shape == 0) KVZ_MERGE(64, 1, 4); else if (shape == 1) KVZ_MERGE(64, 4, 1); else KVZ_MERGE(64, 16, 1);
  } else {
    return -2;
  }
#undef KVZ_MERGE
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvz
