// Split-K merge: combines the (m, l, acc) partials of one (request, query head) into the output
// (the pages merge split results after attention and count the merge in its time: ZipFusion
// summary, §IV.B "Attention Kernel Performance").
//   M = max_s m_s,  w_s = 2^(m_s - M),  o = sum_s w_s acc_s / sum_s w_s l_s
// Output in BF16 (round to nearest even) and optionally in fp32; zeros when the request is empty.
#include "attn_common.hpp"

namespace kvz {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
                                                    const int32_t* __restrict__ seq_lens, int B, int Hq, int P,
                                                    int max_pages, int S, int C, int dense,
                                                    uint16_t* __restrict__ out, float* __restrict__ out_f32) {
  const int lane = threadIdx.x & 63;
  const int row = (int)uniform(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (row >= B * Hq) return;
  const int r = row / Hq;
  int L = sload<int32_t>(seq_lens + r);
  L = L < 0 ? 0 : min(L, max_pages * P);
  const int npages = dense ? (L + P - 1) / P : L / P;
  const int Sr = active_splits(npages, C);
  const float* ml = ws_ml + (size_t)row * S * 2;
  const float* acc = ws_acc + (size_t)row * S * D;
  float M = -INFINITY;
  for (int s = 0; s < Sr; ++s) M = fmaxf(M, ml[2 * s]);
  constexpr int NV = D / 64;
  float num[NV], den = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) num[i] = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < Sr; ++s) {
      const float w = __builtin_amdgcn_exp2f(ml[2 * s] - M);
      den += w * ml[2 * s + 1];
#pragma unroll
      for (int i = 0; i < NV; ++i) num[i] += w * acc[(size_t)s * D + lane + 64 * i];
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float o = num[i] * inv;
    const size_t idx = (size_t)row * D + lane + 64 * i;
    out[idx] = (uint16_t)(pack_bf16(o, 0.f) & 0xFFFFu);
    if (out_f32) out_f32[idx] = o;
  }
}

int launch_merge(const float* ws_acc, const float* ws_ml, const int32_t* seq_lens, int B, int Hq, int D, int P,
                 int max_pages, int S, int C, int dense, uint16_t* out, float* out_f32, hipStream_t stream) {
  dim3 grid((unsigned)(B * Hq + 3) / 4), block(256);
  if (D == 128)
    hipLaunchKernelGGL((merge_kernel<128>), grid, block, 0, stream, ws_acc, ws_ml, seq_lens, B, Hq, P, max_pages, S,
                       C, dense, out, out_f32);
  else if (D == 64)
    hipLaunchKernelGGL((merge_kernel<64>), grid, block, 0, stream, ws_acc, ws_ml, seq_lens, B, Hq, P, max_pages, S,
                       C, dense, out, out_f32);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvz
