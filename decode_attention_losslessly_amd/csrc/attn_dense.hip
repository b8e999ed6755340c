// Decode attention over an uncompressed paged cache [num_pages][H][P][D] (raw BF16, token-major):
// the in-library baseline for the compressed kernels (the pages compare against production
// FlashInfer, ZipFusion summary §IV.B). Same split geometry, softmax and merge as the compressed
// kernels, so that the difference between the two is the bytes read and the rebuild.
//
//   * multi-head: one wave per (request, head, split); K tile: lane l holds 16*D/64 raw values
//     of token l/4 and dots them with q (v_dot2_f32_bf16 + quad DPP sum); V tile: lane l holds
//     dims 2l, 2l+1 (D = 128) of all 16 tokens, regroups them into token pairs with v_perm and
//     accumulates hi/lo probability dot products as the compressed kernel does.
#include "attn_common.hpp"
#include "kvz_lanes.hpp"

namespace kvz {

constexpr int kDenseWaves = 4;

template <int D>
struct DenseStage {
  const uint16_t* kpage;   // [P][D] of this head, nullptr when skipped
  const uint16_t* vpage;
  int tile, rows;          // valid rows of this tile (16 except in the last page)
  uint4 k[D / 64 * 2];     // D/4 raw values of token lane/4
  uint32_t v[16];          // token t: dims (2*lane, 2*lane+1) for D=128, lanes < 32 for D=64
};

template <int D>
__device__ __forceinline__ void dense_load(DenseStage<D>& st, const DenseStage<D>& prev, const uint16_t* k_pages,
                                           const uint16_t* v_pages, const int32_t* pt_row, int page, int tile,
                                           int rows, int H, int h, int P, int num_pages, int lane,
                                           uint32_t* status) {
  if (tile == 0) {
    const int pid = sload<int32_t>(pt_row + page);
    if (pid < 0 || pid >= num_pages) {
      if (lane == 0 && status) atomicOr(status, kStatusBadPage);
      st.kpage = nullptr;
      st.vpage = nullptr;
    } else {
      st.kpage = k_pages + ((size_t)pid * H + h) * P * D;
      st.vpage = v_pages + ((size_t)pid * H + h) * P * D;
    }
  } else {
    st.kpage = prev.kpage;
    st.vpage = prev.vpage;
  }
  st.tile = tile;
  st.rows = rows;
  if (!st.kpage) return;
  constexpr int VK = D / 4;
  const int tok = tile * kTile + lane / 4;
  // K: each load covers a quarter of every lane's 64-byte run, so the four loads share cache
  // lines and go through the caches normally; V rows are read whole and streamed.
  const uint4* kr = reinterpret_cast<const uint4*>(st.kpage + (size_t)tok * D + (lane & 3) * VK);
#pragma unroll
  for (int j = 0; j < VK / 8; ++j) st.k[j] = kr[j];
  const int dp = (D == 128) ? lane : (lane & 31);
  const uint32_t* vr = reinterpret_cast<const uint32_t*>(st.vpage + (size_t)tile * kTile * D) + dp;
#pragma unroll
  for (int t = 0; t < 16; ++t) st.v[t] = stream4(vr + (size_t)t * (D / 2));
}

struct DenseState {
  float m, l;
  float acc[2];   // dims 2*lane, 2*lane+1 (D=128) / lanes < 32 (D=64)
};

template <int D>
__device__ __forceinline__ void dense_compute(DenseState& st, const uint32_t (&q)[D / 8], const DenseStage<D>& stg,
                                              float scale, int lane) {
  if (!stg.kpage) return;
  const bool valid = (lane / 4) < stg.rows;
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    a0 = dot2_bf16(stg.k[j].x, q[4 * j + 0], a0);
    a1 = dot2_bf16(stg.k[j].y, q[4 * j + 1], a1);
    a0 = dot2_bf16(stg.k[j].z, q[4 * j + 2], a0);
    a1 = dot2_bf16(stg.k[j].w, q[4 * j + 3], a1);
  }
  float s = quad_sum(a0 + a1) * scale;
  s = valid ? s : -INFINITY;
  // softmax update (same arithmetic as the compressed multi-head kernel)
  if (ballot(s > st.m)) {
    const float mn = fmaxf(st.m, wave_max(s));
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
    st.l *= alpha;
    st.acc[0] *= alpha;
    st.acc[1] *= alpha;
    st.m = mn;
  }
  const float p = s == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s - st.m);
  const float pn = dpp_f<kRowShl4>(p);
  const uint32_t hi = pack_bf16(p, pn);
  const float h_own = bf16lo_to_f32(hi), h_nb = bf16hi_to_f32(hi);
  const uint32_t lo = pack_bf16(p - h_own, pn - h_nb);
  st.l += h_own + bf16lo_to_f32(lo);
  float x0 = st.acc[0], x1 = st.acc[1], y0 = 0.f, y1 = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t phi = readlane(hi, 8 * k), plo = readlane(lo, 8 * k);
    const bool ok_a = 2 * k < stg.rows, ok_b = 2 * k + 1 < stg.rows;
    const uint32_t ta = ok_a ? stg.v[2 * k] : 0u, tb = ok_b ? stg.v[2 * k + 1] : 0u;
    const uint32_t even = __builtin_amdgcn_perm(tb, ta, 0x05040100u);   // (ta.lo, tb.lo)
    const uint32_t odd = __builtin_amdgcn_perm(tb, ta, 0x07060302u);    // (ta.hi, tb.hi)
    x0 = dot2_bf16(even, phi, x0);
    y0 = dot2_bf16(even, plo, y0);
    x1 = dot2_bf16(odd, phi, x1);
    y1 = dot2_bf16(odd, plo, y1);
  }
  st.acc[0] = x0 + y0;
  st.acc[1] = x1 + y1;
}

template <int D>
__global__ __launch_bounds__(64 * kDenseWaves) void attn_dense_mha_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pages, const uint16_t* __restrict__ v_pages,
    const int32_t* __restrict__ page_table, int max_pages, const int32_t* __restrict__ seq_lens, int B, int H,
    int grp, int P, int num_pages, SplitPlan plan, float scale, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml, uint32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Hq = H * grp;   // query heads, one wave each; grp of them read each KV head
  WorkItem wi;
  if (!plan_work(plan, seq_lens, B, P, max_pages, true, Hq, (int)uniform(blockIdx.x * kDenseWaves + wave), lane, wi))
    return;
  const int S = plan.S, C = wi.C, s = wi.s, hq = wi.k, h = hq / grp, r = wi.r;
  int L = request_len(wi, seq_lens);
  if (L > max_pages * P || L < 0) {
    if (lane == 0 && s == 0 && hq == 0 && status) atomicOr(status, kStatusSeqTooLong);
    L = L < 0 ? 0 : max_pages * P;
  }
  const int npages = (L + P - 1) / P;
  const bool ranked = C < 0;   // chunks are shares of all the request's pages, the partial one included
  const int Sr = ranked ? -C : active_splits(npages, C);
  if (s >= Sr) return;
  int p0, p1;
  if (ranked) {
    rank_range(npages, s, plan.ranks, p0, p1);
  } else {
    p0 = s * C;
    p1 = min(p0 + C, npages);
  }
  uint32_t qv[D / 8];
  {
    const uint32_t* qrow = reinterpret_cast<const uint32_t*>(q + ((size_t)r * Hq + hq) * D + (lane & 3) * (D / 4));
#pragma unroll
    for (int j = 0; j < D / 8; ++j) qv[j] = qrow[j];
  }
  DenseState st;
  st.m = -INFINITY;
  st.l = 0.f;
  st.acc[0] = st.acc[1] = 0.f;
  const int32_t* pt_row = page_table + (size_t)r * max_pages;
  const int T = P / kTile;
  const int nsteps = (p1 > p0 ? p1 - p0 : 0) * T;
  auto rows_of = [&](int i) {
    const int tok0 = (p0 + i / T) * P + (i % T) * kTile;
    return min(kTile, L - tok0);
  };
  if (nsteps > 0) {
    DenseStage<D> a, b;
    dense_load<D>(a, a, k_pages, v_pages, pt_row, p0, 0, rows_of(0), H, h, P, num_pages, lane, status);
    for (int i = 0; i < nsteps; i += 2) {
      if (i + 1 < nsteps)
        dense_load<D>(b, a, k_pages, v_pages, pt_row, p0 + (i + 1) / T, (i + 1) % T, rows_of(i + 1), H, h, P,
                      num_pages, lane, status);
      if (a.rows > 0) dense_compute<D>(st, qv, a, scale, lane);
      if (i + 1 >= nsteps) break;
      if (i + 2 < nsteps)
        dense_load<D>(a, b, k_pages, v_pages, pt_row, p0 + (i + 2) / T, (i + 2) % T, rows_of(i + 2), H, h, P,
                      num_pages, lane, status);
      if (b.rows > 0) dense_compute<D>(st, qv, b, scale, lane);
    }
  }
  float lsum = (lane & 3) == 0 ? st.l : 0.f;
  lsum += __shfl_xor(lsum, 4);
  lsum += __shfl_xor(lsum, 8);
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  const size_t row = (size_t)r * Hq + hq;
  float* acc = ws_acc + (row * S + s) * D;
  if (D == 128 || lane < 32) {
    acc[2 * (D == 128 ? lane : (lane & 31)) + 0] = st.acc[0];
    acc[2 * (D == 128 ? lane : (lane & 31)) + 1] = st.acc[1];
  }
  if (lane == 0) {
    ws_ml[(row * S + s) * 2 + 0] = st.m;
    ws_ml[(row * S + s) * 2 + 1] = lsum;
  }
}

int launch_attn_dense_mha(const uint16_t* q, const uint16_t* k_pages, const uint16_t* v_pages, const int32_t* pt,
                          int max_pages, const int32_t* seq_lens, int B, int Hq, int H, int D, int P,
                          int num_pages, SplitPlan plan, float scale, float* ws_acc, float* ws_ml, uint32_t* status,
                          hipStream_t stream) {
  static int slots128[64], slots64[64];
  if (H <= 0 || Hq % H) return -2;
  const dim3 block(64 * kDenseWaves);
  if (D == 128) {
    plan.slots = resident_waves(attn_dense_mha_kernel<128>, block.x, slots128, 64);
  } else if (D == 64) {
    plan.slots = resident_waves(attn_dense_mha_kernel<64>, block.x, slots64, 64);
  } else {
    return -2;
  }
  rank_fit(plan, plan.slots, (long)B * Hq);
  if (plan.slots <= 0) plan.slots = B * Hq * plan.S;
  const dim3 grid(plan_blocks(plan, (long)B * Hq, kDenseWaves));
  if (D == 128)
    hipLaunchKernelGGL((attn_dense_mha_kernel<128>), grid, block, 0, stream, q, k_pages, v_pages, pt, max_pages,
                       seq_lens, B, H, Hq / H, P, num_pages, plan, scale, ws_acc, ws_ml, status);
  else
    hipLaunchKernelGGL((attn_dense_mha_kernel<64>), grid, block, 0, stream, q, k_pages, v_pages, pt, max_pages,
                       seq_lens, B, H, Hq / H, P, num_pages, plan, scale, ws_acc, ws_ml, status);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvz
