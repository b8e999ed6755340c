// Decode attention when several query heads share one KV head (grouped-query attention).
//
// With g query heads per KV head, a 16-token tile of K times the g query rows is a real small
// GEMM, so this path uses the CDNA4 matrix cores (the pages' kernel feeds H100 Tensor Cores from
// operands rebuilt in registers: ZipFusion summary, §III.C "Attention over the Compressed KV
// Cache"). One wave per (request, KV head, chunk of up to 8 query heads, split):
//
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: lane l rebuilds (or loads) 32 dims of token
//     l%16, which is the A-operand layout; Q^T is the B operand, query rows 8..15 repeat rows
//     0..7;
//   * the 16x16 result sits in lanes exactly as the A operand of the P.V product needs it
//     (lane l: query row l%16, tokens 4*(l/16)..+3), so probabilities never move between lanes;
//     rows 0..7 carry bf16(p) and rows 8..15 carry bf16(p - bf16(p)), which keeps the P.V
//     product accurate to ~2^-16 relative at no extra instruction;
//   * V is rebuilt with the multi-head lane layout (lane l: dims l, l+64, all 16 tokens as token
//     pairs), written to LDS as [dim][pair] and read back in the B-operand layout of
//     v_mfma_f32_16x16x16_bf16 (4 tokens of one dim per lane), 8 dim tiles per token tile;
//   * output rows r and r+8 are summed at the end.
#include "gqa_core.hpp"
#include "mha_pool.hpp"

namespace kvz {

constexpr int kGqaWaves = 4;

// ---------------------------------------------------------------- compressed source
struct GqaCStage {
  const uint8_t* unit;
  int page;         // index in the request's page table
  int tile;
  bool ok;          // false when the page id was out of range: a stand-in unit was read
  uint32_t meta;
  KRaw<128> k;
  VRaw<128> v;
};

// Issues the loads of one (page, tile) step, unconditionally (as in the multi-head kernel), so
// that the next step's loads stay in flight while the current step is computed.
// `live` is false for a stage issued past the last step: its loads read nothing.
template <bool CH>
__device__ __forceinline__ void gqa_c_issue(GqaCStage& st, const uint8_t* units, int pid, int page, int tile, int H,
                                            int h, int P, int num_pages, int lane, bool live = true) {
  st.ok = pid >= 0 && pid < num_pages;
  st.page = page;
  st.unit = units + ((size_t)(st.ok ? pid : 0) * H + h) * unit_bytes(P, 128);
  st.tile = tile;
  st.meta = load_meta(st.unit, P, 128, tile, lane, live);
  load_k<128, true, true, CH>(st.unit, P, tile, lane, st.k, live);
  load_v<128>(st.unit, P, tile, lane, st.v, live);
}

// Returns false, leaving the state untouched, when the unit's escapes are in the pool and POOL
// is off.
template <bool POOL, bool CH>
__device__ __forceinline__ bool gqa_c_compute(GqaState& st, const GqaCStage& stg, int P, uint32_t& krank,
                                              uint32_t& vrank, uint16_t* esc_lds, uint32_t* vlds,
                                              const uint16_t* pool, int64_t pool_cap, float scale, int lane) {
  if (!stg.ok) return true;
  UnitHeader hdr = header_from_meta<128>(stg.meta);
  if (!POOL && hdr.off != kInline) return false;
  if (POOL) clamp_to_pool(hdr, pool_cap);
  if (stg.tile == 0) { krank = 0; vrank = 0; }
  uint32_t kp[16];
  decode_k<128, CH>(stg.k, kp);
  if (hdr.kc) patch_k_tile<128, true, POOL>(kp, stg.k, stg.meta, hdr, P, stg.tile, krank, esc_lds, pool, pool_cap, lane);
  uint32_t vflat[16];
#pragma unroll
  for (int g = 0; g < 2; ++g) decode_v_seg(stg.v.seg[g], v_bases<128, CH>(stg.meta, g), &vflat[8 * g]);
  if (hdr.vc) patch_v_tile<128, POOL, 2>(vflat, stg.v, stg.meta, hdr, P, stg.tile, vrank, esc_lds, pool, pool_cap, lane);
  uint32_t vp[2][8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    vp[0][k] = vflat[k];
    vp[1][k] = vflat[8 + k];
  }
  const int vdim[2] = {lane, lane + 64};
  gqa_tile(st, kp, vdim, vp, kTile, scale, vlds, lane);
  return true;
}

// One tile of any unit for the pool-capable loop: `meta` is its meta window (loaded a step
// ahead); the payload and, for a pool unit, both escape windows go out in one round trip.
// krank / vrank are the block cursors, reset at tile 0.
template <bool CH>
__device__ __forceinline__ void gqa_any_tile(GqaState& st, const uint8_t* unit, uint32_t meta, int P, int tile,
                                             uint32_t& krank, uint32_t& vrank, uint16_t* lds, uint32_t* vlds,
                                             const uint16_t* pool, int64_t pool_cap, float scale, int lane) {
  UnitHeader hdr = header_from_meta<128>(meta);
  clamp_to_pool(hdr, pool_cap);
  if (tile == 0) { krank = 0; vrank = 0; }
  KRaw<128> k;
  VRaw<128> v;
  load_k<128, true, false>(unit, P, tile, lane, k);
  load_v<128>(unit, P, tile, lane, v);
  Window kw, vw;
  const bool in_pool = any_stage<128>(hdr, krank, vrank, lds, pool, pool_cap, kw, vw, lane);
  uint32_t kp[16];
  any_rebuild_k<128, true, CH>(kp, k, meta, hdr, in_pool, kw, P, tile, krank, lds, pool, pool_cap, lane);
  uint32_t vflat[16];
  any_rebuild_v<128, CH>(vflat, v, meta, hdr, in_pool, vw, P, tile, vrank, lds, pool, pool_cap, lane);
  if (in_pool) wave_lds_sync();   // the window reads are complete before the next staging writes
  uint32_t vp[2][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    vp[0][j] = vflat[j];
    vp[1][j] = vflat[8 + j];
  }
  const int vdim[2] = {lane, lane + 64};
  gqa_tile(st, kp, vdim, vp, kTile, scale, vlds, lane);
}

// ---------------------------------------------------------------- kernels
// Both grouped-query kernels ask for 3 waves per SIMD: the compiler then keeps the MFMA
// accumulators in architectural VGPRs and fits in 168 registers without spilling (left alone
// it moves them to AGPRs and lands at 2 waves per SIMD).
#define KVZ_GQA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(3)))

// One wave per (request, KV head, chunk of query heads, split). As in the multi-head kernel,
// the main loop skips units whose escapes are in the pool and the wave adds them after the
// loop, when the pipeline's registers are free; a split that meets mostly such units goes on
// in the pool-capable loop instead. CH: channel groups (format 2).
template <bool CH>
__global__ __launch_bounds__(64 * kGqaWaves) KVZ_GQA_OCCUPANCY void attn_gqa_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ units, const uint16_t* __restrict__ pool,
    int64_t pool_cap, const uint64_t* __restrict__ esc_cursor, const uint16_t* __restrict__ k_tail,
    const uint16_t* __restrict__ v_tail, const int32_t* __restrict__ page_table, int max_pages,
    const int32_t* __restrict__ seq_lens, int B, int Hq, int H, int P, int num_pages, SplitPlan plan, float scale,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, uint32_t* __restrict__ status) {
  __shared__ __align__(16) uint16_t esc_all[kGqaWaves][esc_lds_elems<128>()];
  __shared__ uint32_t vlds_all[kGqaWaves][128 * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = Hq / H, nchunks = (grp + kGqaRows - 1) / kGqaRows;
  WorkItem wi;
  if (!plan_work(plan, seq_lens, B, P, max_pages, false, H * nchunks, (int)uniform(blockIdx.x * kGqaWaves + wave),
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
  // the splits the plan and the merge count for this row; with no unit slots every full page is
  // a bad id and is skipped, but every counted split still writes its (empty) partial
  const int Sr = active_splits(nfull, C);
  if (num_pages <= 0 && nfull > 0) {
    if (lane == 0 && s == 0 && h == 0 && qc == 0) atomicOr(status, kStatusBadPage);
    nfull = 0;
  }
  if (s >= Sr) return;
  const int p0 = s * C, p1 = min(p0 + C, nfull);
  GqaState st;
  gqa_init(st, q, r, Hq, hq0, nq, lane);
  const int32_t* pt_row = page_table + (size_t)r * max_pages;
  const int T = P / kTile;
  uint32_t krank = 0, vrank = 0;
  uint16_t* esc_lds = esc_all[wave];
  uint32_t* vlds = vlds_all[wave];
  const int nsteps = (p1 > p0 ? p1 - p0 : 0) * T;
  int first_skip = -1, last_skip = -1;
  int nskip = 0;          // tiles skipped by the main loop
  int resume = -1;        // step from which the pool-capable loop takes over
  bool bad = false;
  // Records a skipped (pool) tile; the same rules as the multi-head kernel: most tiles so far in
  // the pool sends the wave to the pool-capable loop at the next page, from the split's first
  // step when every tile so far went there, and at once when the first unit has a quarter or
  // more of its values escaped.
  auto note = [&](const GqaCStage& stg, int done) {
    if (first_skip < 0) first_skip = stg.page;
    last_skip = stg.page;
    ++nskip;
    bool heavy = false;
    if (nskip == 1 && done == 1) {
      const UnitHeader hd = header_from_meta<128>(stg.meta);
      heavy = (uint64_t)hd.kc + hd.vc >= (uint64_t)P * 128 / 2;
    }
    if (heavy || (nskip >= 2 && 2 * nskip > done)) {
      if (nskip == done) {
        resume = 0;
        first_skip = last_skip = -1;
      } else {
        resume = (stg.page - p0 + 1) * T;
      }
    }
  };
  // an escape-heavy cache starts every split in the pool-capable loop (as in the multi-head kernel)
  if (nsteps > 0 && sload<uint64_t>(esc_cursor) >= (uint64_t)num_pages * H * (uint64_t)(P * 128 / 2)) resume = 0;
  if (nsteps > 0 && resume < 0) {
    // load cursor as in the multi-head kernel: stays on the last step once there
    int ln = 0, lp = p0, lt = 0;
    bool live = true;   // false once the cursor has passed the last step: those stages read nothing
    const int last = nsteps - 1;
    auto advance = [&]() {
      if (ln < last) {
        ++ln;
        if (++lt == T) { lt = 0; ++lp; }
      } else {
        live = false;
      }
    };
    GqaCStage a, b;
    int pid = sload<int32_t>(pt_row + lp);
    gqa_c_issue<CH>(a, units, pid, lp, lt, H, h, P, num_pages, lane);
    advance();
    pid = sload<int32_t>(pt_row + lp);
    for (int i = 0; i < nsteps; i += 2) {
      gqa_c_issue<CH>(b, units, pid, lp, lt, H, h, P, num_pages, lane, live);
      advance();
      pid = sload<int32_t>(pt_row + lp);
      bad |= !a.ok;
      if (!gqa_c_compute<false, CH>(st, a, P, krank, vrank, esc_lds, vlds, pool, pool_cap, scale, lane)) note(a, i + 1);
      if (i + 1 >= nsteps || resume >= 0) break;
      gqa_c_issue<CH>(a, units, pid, lp, lt, H, h, P, num_pages, lane, live);
      advance();
      pid = sload<int32_t>(pt_row + lp);
      bad |= !b.ok;
      if (!gqa_c_compute<false, CH>(st, b, P, krank, vrank, esc_lds, vlds, pool, pool_cap, scale, lane)) note(b, i + 2);
      if (resume >= 0) break;
    }
  }
  if (resume >= 0 && resume < nsteps) {
    // the rest of the split, every unit as it comes; the next tile's meta window is in flight
    // while a tile is computed
    auto unit_of = [&](int n, bool& ok) {
      const int pid = sload<int32_t>(pt_row + p0 + n / T);
      ok = pid >= 0 && pid < num_pages;
      return units + ((size_t)(ok ? pid : 0) * H + h) * unit_bytes(P, 128);
    };
    bool ok;
    const uint8_t* u = unit_of(resume, ok);
    uint32_t meta = load_meta(u, P, 128, resume % T, lane);
    for (int n = resume; n < nsteps; ++n) {
      bool nok = true;
      const uint8_t* nu = u;
      uint32_t nmeta = 0;
      if (n + 1 < nsteps) {
        nu = unit_of(n + 1, nok);
        nmeta = load_meta(nu, P, 128, (n + 1) % T, lane);
      }
      if (ok) gqa_any_tile<CH>(st, u, meta, P, n % T, krank, vrank, esc_lds, vlds, pool, pool_cap, scale, lane);
      bad |= !ok;
      u = nu;
      ok = nok;
      meta = nmeta;
    }
  }
  if (bad && lane == 0) atomicOr(status, kStatusBadPage);
  if (first_skip >= 0) {
    // units whose escapes are in the pool: the recorded pages, then any between them
    auto do_page = [&](int page) {
      const int pid = sload<int32_t>(pt_row + page);
      for (int t = 0; t < T; ++t) {
        GqaCStage a;
        gqa_c_issue<CH>(a, units, pid, page, t, H, h, P, num_pages, lane);
        gqa_c_compute<true, CH>(st, a, P, krank, vrank, esc_lds, vlds, pool, pool_cap, scale, lane);
      }
    };
    do_page(first_skip);
    if (last_skip != first_skip) do_page(last_skip);
    const uint32_t hdr_off = hdr_offset(P, 128) + 8;
    for (int c0 = first_skip + 1; c0 < last_skip; c0 += 64) {
      const int pg = c0 + lane;
      bool in_pool = false;
      if (pg < last_skip) {
        const int pid = pt_row[pg];
        if (pid >= 0 && pid < num_pages)
          in_pool = *reinterpret_cast<const uint64_t*>(units + ((size_t)pid * H + h) * unit_bytes(P, 128) + hdr_off) !=
                    kInline;
      }
      uint64_t todo = ballot(in_pool);
      while (todo) {
        const int page = c0 + __builtin_ctzll(todo);
        todo &= todo - 1;
        do_page(page);
      }
    }
  }
  if (s == Sr - 1 && rows > 0) {
    const size_t toff = ((size_t)r * H + h) * P * 128;
    for (int t0 = 0; t0 < rows; t0 += kTile)
      gqa_raw_tile(st, k_tail + toff, v_tail + toff, t0, min(kTile, rows - t0), scale, vlds, lane);
  }
  gqa_store(st, r, Hq, hq0, nq, S, s, ws_acc, ws_ml, lane);
}

__global__ __launch_bounds__(64 * kGqaWaves) KVZ_GQA_OCCUPANCY void attn_dense_gqa_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pages, const uint16_t* __restrict__ v_pages,
    const int32_t* __restrict__ page_table, int max_pages, const int32_t* __restrict__ seq_lens, int B, int Hq, int H,
    int P, int num_pages, SplitPlan plan, float scale, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    uint32_t* __restrict__ status) {
  __shared__ uint32_t vlds_all[kGqaWaves][128 * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = Hq / H, nchunks = (grp + kGqaRows - 1) / kGqaRows;
  WorkItem wi;
  if (!plan_work(plan, seq_lens, B, P, max_pages, true, H * nchunks, (int)uniform(blockIdx.x * kGqaWaves + wave),
                 lane, wi))
    return;
  const int S = plan.S, C = wi.C, s = wi.s, qc = wi.k % nchunks, h = wi.k / nchunks, r = wi.r;
  const int hq0 = h * grp + qc * kGqaRows, nq = min(kGqaRows, grp - qc * kGqaRows);
  int L = request_len(wi, seq_lens);
  if (L > max_pages * P || L < 0) {
    if (lane == 0 && s == 0 && h == 0 && qc == 0 && status) atomicOr(status, kStatusSeqTooLong);
    L = L < 0 ? 0 : max_pages * P;
  }
  int npages = (L + P - 1) / P;
  const int Sr = active_splits(npages, C);   // as the merge counts them (see the compressed kernel)
  if (num_pages <= 0 && npages > 0) {   // no pages: every page id is bad
    if (lane == 0 && s == 0 && h == 0 && qc == 0 && status) atomicOr(status, kStatusBadPage);
    npages = 0;
  }
  if (s >= Sr) return;
  const int p0 = s * C, p1 = min(p0 + C, npages);
  GqaState st;
  gqa_init(st, q, r, Hq, hq0, nq, lane);
  uint32_t* vlds = vlds_all[wave];
  const int32_t* pt_row = page_table + (size_t)r * max_pages;
  const int T = P / kTile;
  // steps of 16 tokens; the last page may end early (rows < 16, or no rows at all)
  const int nsteps = (p1 > p0 ? p1 - p0 : 0) * T;
  bool bad = false;
  if (nsteps > 0) {
    int ln = 0, lp = p0, lt = 0;
    bool live = true;   // false once the cursor has passed the last step
    const int last = nsteps - 1;
    auto advance = [&]() {
      if (ln < last) {
        ++ln;
        if (++lt == T) { lt = 0; ++lp; }
      } else {
        live = false;
      }
    };
    // loads of one step, unconditional: a bad page id reads page 0 and the step is skipped; a
    // stage past the last step (never computed) has no rows, so its loads all fall on one row
    auto issue = [&](GqaRawStage& stg, int pid, bool& ok) {
      ok = pid >= 0 && pid < num_pages;
      const size_t base = ((size_t)(ok ? pid : 0) * H + h) * P * 128;
      const int rows = live ? max(0, min(kTile, L - lp * P - lt * kTile)) : 0;
      gqa_raw_load(stg, k_pages + base, v_pages + base, lt * kTile, rows, lane);
    };
    GqaRawStage a, b;
    bool aok, bok;
    int pid = sload<int32_t>(pt_row + lp);
    issue(a, pid, aok);
    advance();
    pid = sload<int32_t>(pt_row + lp);
    for (int i = 0; i < nsteps; i += 2) {
      issue(b, pid, bok);
      advance();
      pid = sload<int32_t>(pt_row + lp);
      bad |= !aok;
      if (aok && a.rows > 0) gqa_raw_compute(st, a, scale, vlds, lane);
      if (i + 1 >= nsteps) break;
      issue(a, pid, aok);
      advance();
      pid = sload<int32_t>(pt_row + lp);
      bad |= !bok;
      if (bok && b.rows > 0) gqa_raw_compute(st, b, scale, vlds, lane);
    }
  }
  if (bad && lane == 0 && status) atomicOr(status, kStatusBadPage);
  gqa_store(st, r, Hq, hq0, nq, S, s, ws_acc, ws_ml, lane);
}

static int gqa_items(int B, int Hq, int H) { return B * H * ((Hq / H + kGqaRows - 1) / kGqaRows); }

int launch_attn_gqa(const uint16_t* q, const uint8_t* units, const uint16_t* pool, int64_t pool_cap,
                    const uint64_t* esc_cursor, const uint16_t* k_tail,
                    const uint16_t* v_tail, const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                    int B, int Hq, int H, int D, int P, int num_pages, SplitPlan plan, float scale, float* ws_acc,
                    float* ws_ml, uint32_t* status, bool channel, hipStream_t stream) {
  if (D != 128) return -2;
  static int slots[64], slots_c[64];
  const dim3 block(64 * kGqaWaves);
  auto kernel = channel ? attn_gqa_kernel<true> : attn_gqa_kernel<false>;
  plan.slots = resident_waves(kernel, block.x, channel ? slots_c : slots, 64);
  plan.slots_pref = 2 * plan.slots / 3;   // two of its three waves per SIMD (see plan_work)
  if (plan.slots <= 0) plan.slots = gqa_items(B, Hq, H) * plan.S;
  hipLaunchKernelGGL(kernel, dim3(plan_blocks(plan, gqa_items(B, Hq, H), kGqaWaves)), block, 0, stream, q, units,
                     pool, pool_cap, esc_cursor, k_tail, v_tail, page_table, max_pages, seq_lens, B, Hq, H, P, num_pages, plan, scale,
                     ws_acc, ws_ml, status);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_attn_dense_gqa(const uint16_t* q, const uint16_t* k_pages, const uint16_t* v_pages, const int32_t* pt,
                          int max_pages, const int32_t* seq_lens, int B, int Hq, int H, int D, int P, int num_pages,
                          SplitPlan plan, float scale, float* ws_acc, float* ws_ml, uint32_t* status,
                          hipStream_t stream) {
  if (D != 128) return -2;
  static int slots[64];
  const dim3 block(64 * kGqaWaves);
  plan.slots = resident_waves(attn_dense_gqa_kernel, block.x, slots, 64);
  plan.slots_pref = 2 * plan.slots / 3;   // as the compressed kernel (measured: as fast or faster)
  if (plan.slots <= 0) plan.slots = gqa_items(B, Hq, H) * plan.S;
  hipLaunchKernelGGL(attn_dense_gqa_kernel, dim3(plan_blocks(plan, gqa_items(B, Hq, H), kGqaWaves)), block, 0, stream,
                     q, k_pages, v_pages, pt, max_pages, seq_lens, B, Hq, H, P, num_pages, plan, scale, ws_acc, ws_ml,
                     status);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvz
