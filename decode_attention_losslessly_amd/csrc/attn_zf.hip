// Decode attention over a cache in ZipFusion's block format (zf.hpp), multi-head (one query head
// per KV head). Same organisation as the main multi-head kernel (attn_mha.hip): one wave per
// (request, head, split), lane l holding K pieces l + 64 i and V dims l + 64 s, the next tile's
// loads issued before the current tile is computed, scores / softmax / P.V from mha_core.hpp.
// Compressed blocks are rebuilt in registers (§III.C of the ZipFusion summary: four high bytes
// per 32-bit add, combined with the kept low bytes). A raw block's pieces are read from the pool
// when its tile is computed (the pages' format keeps such blocks uncompressed and uses them
// without a rebuild): a load that depends on the unit's meta, whose latency the other waves of
// the SIMD cover. Handling them in the main loop measured faster than a second sweep after it,
// because with this format most units hold some raw block.
//
// The grouped-query kernel over this format has the skeleton of the escape format's
// grouped-query kernel (attn_gqa.hip, gqa_core.hpp: S^T = K Q^T and P.V on the matrix cores) with
// this format's loads and rebuild: lane l rebuilds the 32 K values of token l % 16, dims
// 32 (l / 16) .. + 31 (the matrix-core A operand, the pages' Tensor-Core operand rebuild) from
// one block's low bytes and codes, and V dims l and l + 64 as in the multi-head kernel.
//
// Also the test kernel that writes the rebuilt values of whole units back out, in either K lane
// layout.
#include "gqa_core.hpp"
#include "mha_core.hpp"
#include "zf.hpp"

namespace kvz {

constexpr int kZfWaves = 4;

template <int D>
struct ZStage {
  const uint8_t* unit;
  int page, tile;
  bool ok;           // false when the page id was out of range: a stand-in unit was read
  uint32_t rawlo;    // low dword of the unit's raw-pool offset (a scalar load, read when the tile is
                     // computed): all ones when the unit has no raw block
  ZPiece k[D / 64];
  ZPiece v[D / 64];
};

// Unconditional loads of one (page, tile) step (see the main kernel for why).
template <int D>
__device__ __forceinline__ void zf_issue(ZStage<D>& st, const uint8_t* units, int pid, int page, int tile, int H,
                                         int h, int P, int num_pages, int lane) {
  st.ok = pid >= 0 && pid < num_pages;
  st.page = page;
  st.tile = tile;
  st.unit = units + ((size_t)(st.ok ? pid : 0) * H + h) * zf_unit_bytes(P, D);
  st.rawlo = sload<uint32_t>(st.unit + zf_rawoff_offset(P, D));
#pragma unroll
  for (int i = 0; i < D / 64; ++i) zf_load_piece(st.unit, P, D, false, tile, k_piece<D, false>(lane, i), st.k[i]);
#pragma unroll
  for (int s = 0; s < D / 64; ++s) zf_load_piece(st.unit, P, D, true, tile, lane + 64 * s, st.v[s]);
}

// Rebuilds this lane's K and V pairs; with RAW, raw blocks are read from the pool (bounds-checked
// against its capacity; a unit whose raw blocks were dropped reads zeros).
template <int D, bool RAW>
__device__ __forceinline__ void zf_rebuild(const ZStage<D>& stg, int P, const uint16_t* pool, int64_t pool_cap,
                                           int lane, uint32_t (&kp)[D / 8], uint32_t (&vp)[D / 8]) {
  // a unit of at most 8 blocks: one 16-byte scalar load gives the raw offset and every rank
  const bool in_head = zf_head_holds_meta(P, D);
  uint32_t raw_mask = 0;
  uint64_t off = 0;
  if constexpr (RAW) {
    if (in_head) {
      const uint4 head = sload4(stg.unit);
      off = zf_head_offset(head);
      raw_mask = zf_head_raw_mask(head);
    } else {
      off = zf_raw_offset(stg.unit, P, D);
    }
  }
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    if (RAW && stg.k[i].meta == kZfRaw) {
      const int pc = k_piece<D, false>(lane, i);
      const uint32_t rank = zf_rank(raw_mask, stg.unit, in_head, zf_block_index(false, P, D, stg.tile, (16 * pc) / kZfBlock));
      if (off != kInline && off + (uint64_t)(rank + 1) * kZfBlock <= (uint64_t)pool_cap)
        zf_raw_piece(pool, off, rank, pc, &kp[8 * i]);
      else
        for (int j = 0; j < 8; ++j) kp[8 * i + j] = 0;
    } else {
      zf_decode_piece(stg.k[i], &kp[8 * i]);
    }
  }
#pragma unroll
  for (int s = 0; s < D / 64; ++s) {
    if (RAW && stg.v[s].meta == kZfRaw) {
      const int d = lane + 64 * s;
      const uint32_t rank = zf_rank(raw_mask, stg.unit, in_head, zf_block_index(true, P, D, stg.tile, (16 * d) / kZfBlock));
      if (off != kInline && off + (uint64_t)(rank + 1) * kZfBlock <= (uint64_t)pool_cap)
        zf_raw_piece(pool, off, rank, d, &vp[8 * s]);
      else
        for (int j = 0; j < 8; ++j) vp[8 * s + j] = 0;
    } else {
      zf_decode_piece(stg.v[s], &vp[8 * s]);
    }
  }
}

template <int D>
__device__ __forceinline__ void zf_compute(MhaState<D>& st, const ZStage<D>& stg, int P, const uint16_t* pool,
                                           int64_t pool_cap, float scale, int lane) {
  if (!stg.ok) return;
  uint32_t kp[D / 8], vp[D / 8];
  if (uniform(stg.rawlo) == 0xFFFFFFFFu) zf_rebuild<D, false>(stg, P, pool, pool_cap, lane, kp, vp);
  else zf_rebuild<D, true>(stg, P, pool, pool_cap, lane, kp, vp);
  float sc[D / 64];
  mha_scores<D>(st, kp, scale, sc);
  uint32_t phi[8], plo[8];
  mha_softmax<D>(st, sc, phi, plo);
  mha_accumulate_v<D>(st, vp, phi, plo);
}

template <int D>
__global__ __launch_bounds__(64 * kZfWaves) void attn_zf_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ units, const uint16_t* __restrict__ pool,
    int64_t pool_cap, const uint16_t* __restrict__ k_tail, const uint16_t* __restrict__ v_tail,
    const int32_t* __restrict__ page_table, int max_pages, const int32_t* __restrict__ seq_lens, int B, int H,
    int grp, int P, int num_pages, SplitPlan plan, float scale, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml, uint32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Hq = H * grp;   // query heads, one wave each; grp of them read each KV head
  WorkItem wi;
  if (!plan_work(plan, seq_lens, B, P, max_pages, false, Hq, (int)uniform(blockIdx.x * kZfWaves + wave), lane, wi))
    return;
  const int S = plan.S, C = wi.C, s = wi.s, hq = wi.k, h = hq / grp, r = wi.r;
  int L = request_len(wi, seq_lens);
  if (L > max_pages * P || L < 0) {
    if (lane == 0 && s == 0 && hq == 0) atomicOr(status, kStatusSeqTooLong);
    L = L < 0 ? 0 : max_pages * P;
  }
  int nfull = L / P;
  const int rows = L % P;
  const int Sr = active_splits(nfull, C);   // as the merge counts them (see the escape-format kernel)
  if (num_pages <= 0 && nfull > 0) {
    if (lane == 0 && s == 0 && hq == 0) atomicOr(status, kStatusBadPage);
    nfull = 0;
  }
  if (s >= Sr) return;
  const int p0 = s * C, p1 = min(p0 + C, nfull);
  const size_t slot = ((size_t)r * Hq + hq) * S + s;

  MhaState<D> st;
  {
    const uint4* qrow = reinterpret_cast<const uint4*>(q + ((size_t)r * Hq + hq) * D + (16 * lane) % D);
    const uint4 a = qrow[0], b = qrow[1];
    st.q[0] = a.x; st.q[1] = a.y; st.q[2] = a.z; st.q[3] = a.w;
    st.q[4] = b.x; st.q[5] = b.y; st.q[6] = b.z; st.q[7] = b.w;
  }
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) st.acc[i] = 0.f;
  const int32_t* pt_row = page_table + (size_t)r * max_pages;
  const int T = P / kTile;
  const int nsteps = (p1 > p0 ? p1 - p0 : 0) * T;
  bool bad = false;
  if (nsteps > 0) {
    int ln = 0, lp = p0, lt = 0;
    const int last = nsteps - 1;
    auto advance = [&]() {
      if (ln < last) {
        ++ln;
        if (++lt == T) { lt = 0; ++lp; }
      }
    };
    ZStage<D> a, b;
    int pid = sload<int32_t>(pt_row + lp);
    zf_issue<D>(a, units, pid, lp, lt, H, h, P, num_pages, lane);
    advance();
    pid = sload<int32_t>(pt_row + lp);
    for (int i = 0; i < nsteps; i += 2) {
      zf_issue<D>(b, units, pid, lp, lt, H, h, P, num_pages, lane);
      advance();
      pid = sload<int32_t>(pt_row + lp);
      bad |= !a.ok;
      zf_compute<D>(st, a, P, pool, pool_cap, scale, lane);
      if (i + 1 >= nsteps) break;
      zf_issue<D>(a, units, pid, lp, lt, H, h, P, num_pages, lane);
      advance();
      pid = sload<int32_t>(pt_row + lp);
      bad |= !b.ok;
      zf_compute<D>(st, b, P, pool, pool_cap, scale, lane);
    }
  }
  if (bad && lane == 0) atomicOr(status, kStatusBadPage);
  if (s == Sr - 1 && rows > 0) {
    const size_t toff = ((size_t)r * H + h) * P * D;
    mha_tail<D>(st, k_tail + toff, v_tail + toff, rows, scale, lane);
  }
  constexpr int LPT = D / 16;
  float lsum = (lane % LPT) == 0 ? st.l : 0.f;
#pragma unroll
  for (int o = LPT; o < 64; o <<= 1) lsum += __shfl_xor(lsum, o);
  float* acc = ws_acc + slot * D;
#pragma unroll
  for (int g = 0; g < D / 64; ++g) acc[lane + 64 * g] = st.acc[g];
  if (lane == 0) {
    ws_ml[slot * 2 + 0] = st.m;
    ws_ml[slot * 2 + 1] = lsum;
  }
}

// ---------------------------------------------------------------- grouped queries
struct ZgStage {
  const uint8_t* unit;
  int tile;
  bool ok;           // false when the page id was out of range: a stand-in unit was read
  uint32_t rawlo;    // low dword of the unit's raw-pool offset: all ones when it has no raw block
  ZPair k;           // token l % 16, dims 32 (l / 16) .. + 31
  ZPiece v[2];       // dims l, l + 64
};

// HEAD (a unit of at most 8 blocks): the raw offset's low dword is a scalar load, read when the
// tile is computed (no vector register held for it while the stage is in flight)
template <bool HEAD = false>
__device__ __forceinline__ void zf_gqa_issue(ZgStage& st, const uint8_t* units, int pid, int tile, int H, int h, int P,
                                             int num_pages, int lane) {
  st.ok = pid >= 0 && pid < num_pages;
  st.tile = tile;
  st.unit = units + ((size_t)(st.ok ? pid : 0) * H + h) * zf_unit_bytes(P, 128);
  if constexpr (HEAD) st.rawlo = sload<uint32_t>(st.unit + zf_rawoff_offset(P, 128));
  else st.rawlo = stream4(st.unit + zf_rawoff_offset(P, 128));
  zf_load_pair(st.unit, P, 128, tile, k_piece<128, true>(lane, 0), st.k);
#pragma unroll
  for (int s = 0; s < 2; ++s) zf_load_piece(st.unit, P, 128, true, tile, lane + 64 * s, st.v[s]);
}

// Rebuilds this lane's K pairs (A-operand layout) and V pairs (dims l, l + 64); with RAW, raw
// blocks are read from the pool (bounds-checked against its capacity; a unit whose raw blocks
// were dropped reads zeros).
// HEAD: the unit has at most 8 blocks (its first 16 bytes give the raw offset and the ranks;
// a compile-time choice here, so that the kernel carries one raw path only).
template <bool RAW, bool HEAD>
__device__ __forceinline__ void zf_gqa_rebuild(const ZgStage& stg, int P, const uint16_t* pool, int64_t pool_cap,
                                               int lane, uint32_t (&kp)[16], uint32_t (&vp)[2][8]) {
  constexpr bool in_head = HEAD;
  uint32_t raw_mask = 0;
  uint64_t off = 0;
  if constexpr (RAW) {
    if constexpr (HEAD) {
      const uint4 head = sload4(stg.unit);
      off = zf_head_offset(head);
      raw_mask = zf_head_raw_mask(head);
    } else {
      off = zf_raw_offset(stg.unit, P, 128);
    }
  }
  if (RAW && stg.k.meta == kZfRaw) {
    const int pc = k_piece<128, true>(lane, 0);
    const uint32_t rank = zf_rank(raw_mask, stg.unit, in_head, zf_block_index(false, P, 128, stg.tile, (16 * pc) / kZfBlock));
    if (off != kInline && off + (uint64_t)(rank + 1) * kZfBlock <= (uint64_t)pool_cap) {
      zf_raw_piece(pool, off, rank, pc, &kp[0]);
      zf_raw_piece(pool, off, rank, pc + 1, &kp[8]);
    } else {
      for (int j = 0; j < 16; ++j) kp[j] = 0;
    }
  } else {
    zf_decode_pair(stg.k, kp);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (RAW && stg.v[s].meta == kZfRaw) {
      const int d = lane + 64 * s;
      const uint32_t rank = zf_rank(raw_mask, stg.unit, in_head, zf_block_index(true, P, 128, stg.tile, (16 * d) / kZfBlock));
      if (off != kInline && off + (uint64_t)(rank + 1) * kZfBlock <= (uint64_t)pool_cap)
        zf_raw_piece(pool, off, rank, d, vp[s]);
      else
        for (int j = 0; j < 8; ++j) vp[s][j] = 0;
    } else {
      zf_decode_piece(stg.v[s], vp[s]);
    }
  }
}

template <bool HEAD>
__device__ __forceinline__ void zf_gqa_compute(GqaState& st, const ZgStage& stg, int P, const uint16_t* pool,
                                               int64_t pool_cap, float scale, uint32_t* vlds, int lane) {
  if (!stg.ok) return;
  uint32_t kp[16], vp[2][8];
  if (uniform(stg.rawlo) == 0xFFFFFFFFu) zf_gqa_rebuild<false, HEAD>(stg, P, pool, pool_cap, lane, kp, vp);
  else zf_gqa_rebuild<true, HEAD>(stg, P, pool, pool_cap, lane, kp, vp);
  const int vdim[2] = {lane, lane + 64};
  gqa_tile(st, kp, vdim, vp, kTile, scale, vlds, lane);
}

// One wave per (request, KV head, chunk of up to 8 query heads, split), as the escape format's
// grouped-query kernel (3 waves per SIMD: see there), with the next tile's loads issued before
// the current tile is computed.
template <bool HEAD>
__global__ __launch_bounds__(64 * kZfWaves) __attribute__((amdgpu_waves_per_eu(3))) void attn_zf_gqa_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ units, const uint16_t* __restrict__ pool,
    int64_t pool_cap, const uint16_t* __restrict__ k_tail, const uint16_t* __restrict__ v_tail,
    const int32_t* __restrict__ page_table, int max_pages, const int32_t* __restrict__ seq_lens, int B, int Hq, int H,
    int P, int num_pages, SplitPlan plan, float scale, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    uint32_t* __restrict__ status) {
  __shared__ uint32_t vlds_all[kZfWaves][128 * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = Hq / H, nchunks = (grp + kGqaRows - 1) / kGqaRows;
  WorkItem wi;
  if (!plan_work(plan, seq_lens, B, P, max_pages, false, H * nchunks, (int)uniform(blockIdx.x * kZfWaves + wave),
                 lane, wi))
    return;
  const int S = plan.S, C = wi.C, s = wi.s, qc = wi.k % nchunks, h = wi.k / nchunks, r = wi.r;
  const int hq0 = h * grp + qc * kGqaRows, nq = min(kGqaRows, grp - qc * kGqaRows);
  int L = request_len(wi, seq_lens);
  if (L > max_pages * P || L < 0) {
    if (lane == 0 && s == 0 && h == 0 && qc == 0) atomicOr(status, kStatusSeqTooLong);
    L = L < 0 ? 0 : max_pages * P;
  }
  int nfull = L / P;
  const int rows = L % P;
  const int Sr = active_splits(nfull, C);   // as the merge counts them (see the escape-format kernels)
  if (num_pages <= 0 && nfull > 0) {
    if (lane == 0 && s == 0 && h == 0 && qc == 0) atomicOr(status, kStatusBadPage);
    nfull = 0;
  }
  if (s >= Sr) return;
  const int p0 = s * C, p1 = min(p0 + C, nfull);
  GqaState st;
  gqa_init(st, q, r, Hq, hq0, nq, lane);
  uint32_t* vlds = vlds_all[wave];
  const int32_t* pt_row = page_table + (size_t)r * max_pages;
  const int T = P / kTile;
  const int nsteps = (p1 > p0 ? p1 - p0 : 0) * T;
  bool bad = false;
  if (nsteps > 0) {
    int ln = 0, lp = p0, lt = 0;
    const int last = nsteps - 1;
    auto advance = [&]() {
      if (ln < last) {
        ++ln;
        if (++lt == T) { lt = 0; ++lp; }
      }
    };
    ZgStage a, b;
    int pid = sload<int32_t>(pt_row + lp);
    zf_gqa_issue<HEAD>(a, units, pid, lt, H, h, P, num_pages, lane);
    advance();
    pid = sload<int32_t>(pt_row + lp);
    for (int i = 0; i < nsteps; i += 2) {
      zf_gqa_issue<HEAD>(b, units, pid, lt, H, h, P, num_pages, lane);
      advance();
      pid = sload<int32_t>(pt_row + lp);
      bad |= !a.ok;
      zf_gqa_compute<HEAD>(st, a, P, pool, pool_cap, scale, vlds, lane);
      if (i + 1 >= nsteps) break;
      zf_gqa_issue<HEAD>(a, units, pid, lt, H, h, P, num_pages, lane);
      advance();
      pid = sload<int32_t>(pt_row + lp);
      bad |= !b.ok;
      zf_gqa_compute<HEAD>(st, b, P, pool, pool_cap, scale, vlds, lane);
    }
  }
  if (bad && lane == 0) atomicOr(status, kStatusBadPage);
  if (s == Sr - 1 && rows > 0) {
    const size_t toff = ((size_t)r * H + h) * P * 128;
    for (int t0 = 0; t0 < rows; t0 += kTile)
      gqa_raw_tile(st, k_tail + toff, v_tail + toff, t0, min(kTile, rows - t0), scale, vlds, lane);
  }
  gqa_store(st, r, Hq, hq0, nq, S, s, ws_acc, ws_ml, lane);
}

// Test kernel: one wave per (unit, head) writes the rebuilt K and V of whole units (the same
// loads and rebuild as the attention kernels, raw blocks from the pool), with the multi-head or
// (GQA) the grouped-query K lane layout.
template <int D, bool GQA>
__global__ __launch_bounds__(64) void decompress_zf_kernel(const uint8_t* __restrict__ units,
                                                           const uint16_t* __restrict__ pool, int64_t pool_cap,
                                                           const int32_t* __restrict__ page_ids, int H, int P,
                                                           int num_pages, uint16_t* __restrict__ k_dst,
                                                           uint16_t* __restrict__ v_dst, uint32_t* __restrict__ status) {
  const int lane = threadIdx.x;
  const int i = blockIdx.x / H, h = blockIdx.x % H;
  const int pid = sload<int32_t>(page_ids + i);
  if (pid < 0 || pid >= num_pages) {
    if (lane == 0) atomicOr(status, kStatusBadPage);
    return;
  }
  uint16_t* kd = k_dst + ((size_t)i * H + h) * P * D;
  uint16_t* vd = v_dst + ((size_t)i * H + h) * P * D;
  for (int t = 0; t < P / kTile; ++t) {
    uint32_t kp[D / 8], vp[D / 8];
    if constexpr (GQA) {
      ZgStage st;
      zf_gqa_issue(st, units, pid, t, H, h, P, num_pages, lane);
      uint32_t v2[2][8];
      if (zf_head_holds_meta(P, 128)) zf_gqa_rebuild<true, true>(st, P, pool, pool_cap, lane, kp, v2);
      else zf_gqa_rebuild<true, false>(st, P, pool, pool_cap, lane, kp, v2);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        vp[j] = v2[0][j];
        vp[8 + j] = v2[1][j];
      }
    } else {
      ZStage<D> st;
      zf_issue<D>(st, units, pid, 0, t, H, h, P, num_pages, lane);
      zf_rebuild<D, true>(st, P, pool, pool_cap, lane, kp, vp);
    }
#pragma unroll
    for (int p = 0; p < D / 64; ++p) {
      const int pc = k_piece<D, GQA>(lane, p);
      uint32_t* dst = reinterpret_cast<uint32_t*>(kd + (size_t)(t * kTile + piece_token<D>(pc)) * D + piece_dim<D>(pc));
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j] = kp[8 * p + j];
    }
#pragma unroll
    for (int s = 0; s < D / 64; ++s) {
      const int d = lane + 64 * s;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        vd[(size_t)(t * kTile + 2 * k) * D + d] = (uint16_t)(vp[8 * s + k] & 0xFFFFu);
        vd[(size_t)(t * kTile + 2 * k + 1) * D + d] = (uint16_t)(vp[8 * s + k] >> 16);
      }
    }
  }
}

int launch_attn_zf(const uint16_t* q, const uint8_t* units, const uint16_t* pool, int64_t pool_cap,
                   const uint16_t* k_tail, const uint16_t* v_tail, const int32_t* page_table, int max_pages,
                   const int32_t* seq_lens, int B, int Hq, int H, int D, int P, int num_pages, SplitPlan plan,
                   float scale, float* ws_acc, float* ws_ml, uint32_t* status, hipStream_t stream) {
  static int slots128[64], slots64[64];
  if (H <= 0 || Hq % H) return -2;
  const dim3 block(64 * kZfWaves);
  if (D == 128) {
    plan.slots = resident_waves(attn_zf_kernel<128>, block.x, slots128, 64);
  } else if (D == 64) {
    plan.slots = resident_waves(attn_zf_kernel<64>, block.x, slots64, 64);
  } else {
    return -2;
  }
  if (plan.slots <= 0) plan.slots = B * Hq * plan.S;
  const dim3 grid(plan_blocks(plan, (long)B * Hq, kZfWaves));
  if (D == 128)
    hipLaunchKernelGGL((attn_zf_kernel<128>), grid, block, 0, stream, q, units, pool, pool_cap, k_tail, v_tail,
                       page_table, max_pages, seq_lens, B, H, Hq / H, P, num_pages, plan, scale, ws_acc, ws_ml, status);
  else
    hipLaunchKernelGGL((attn_zf_kernel<64>), grid, block, 0, stream, q, units, pool, pool_cap, k_tail, v_tail,
                       page_table, max_pages, seq_lens, B, H, Hq / H, P, num_pages, plan, scale, ws_acc, ws_ml, status);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_attn_zf_gqa(const uint16_t* q, const uint8_t* units, const uint16_t* pool, int64_t pool_cap,
                       const uint16_t* k_tail, const uint16_t* v_tail, const int32_t* page_table, int max_pages,
                       const int32_t* seq_lens, int B, int Hq, int H, int D, int P, int num_pages, SplitPlan plan,
                       float scale, float* ws_acc, float* ws_ml, uint32_t* status, hipStream_t stream) {
  if (D != 128) return -2;
  static int slots_head[64], slots[64];
  const dim3 block(64 * kZfWaves);
  const long items = (long)B * H * ((Hq / H + kGqaRows - 1) / kGqaRows);
  const bool head = zf_head_holds_meta(P, 128);
  plan.slots = head ? resident_waves(attn_zf_gqa_kernel<true>, block.x, slots_head, 64)
                    : resident_waves(attn_zf_gqa_kernel<false>, block.x, slots, 64);
  plan.slots_pref = 2 * plan.slots / 3;   // two of its three waves per SIMD, as attn_gqa_kernel
  if (plan.slots <= 0) plan.slots = (int)(items * plan.S);
  if (head)
    hipLaunchKernelGGL(attn_zf_gqa_kernel<true>, dim3(plan_blocks(plan, items, kZfWaves)), block, 0, stream, q, units,
                       pool, pool_cap, k_tail, v_tail, page_table, max_pages, seq_lens, B, Hq, H, P, num_pages, plan,
                       scale, ws_acc, ws_ml, status);
  else
    hipLaunchKernelGGL(attn_zf_gqa_kernel<false>, dim3(plan_blocks(plan, items, kZfWaves)), block, 0, stream, q, units,
                       pool, pool_cap, k_tail, v_tail, page_table, max_pages, seq_lens, B, Hq, H, P, num_pages, plan,
                       scale, ws_acc, ws_ml, status);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_decompress_zf(const uint8_t* units, const uint16_t* pool, int64_t pool_cap, const int32_t* page_ids, int n,
                         int H, int P, int D, int num_pages, int lane_map, uint16_t* k_dst, uint16_t* v_dst,
                         uint32_t* status, hipStream_t stream) {
  dim3 grid((unsigned)n * H), block(64);
  if (D == 128 && lane_map == 1)
    hipLaunchKernelGGL((decompress_zf_kernel<128, true>), grid, block, 0, stream, units, pool, pool_cap, page_ids, H,
                       P, num_pages, k_dst, v_dst, status);
  else if (D == 128 && lane_map == 0)
    hipLaunchKernelGGL((decompress_zf_kernel<128, false>), grid, block, 0, stream, units, pool, pool_cap, page_ids, H,
                       P, num_pages, k_dst, v_dst, status);
  else if (D == 64 && lane_map == 0)
    hipLaunchKernelGGL((decompress_zf_kernel<64, false>), grid, block, 0, stream, units, pool, pool_cap, page_ids, H,
                       P, num_pages, k_dst, v_dst, status);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvz
