// Decode attention over the compressed cache, one query head per KV head (multi-head).
//
// The compressed blocks are read straight from HBM and rebuilt in registers with integer bit
// operations just before use; nothing is decompressed to memory (ZipFusion summary, §III.C
// "Attention over the Compressed KV Cache"). The pages' kernel is built for H100 Tensor Cores;
// this one is organised for CDNA4 wave64 VALU work, because with one query row per KV head the
// contraction is a matrix-vector product that does not fill a matrix core:
//
//   * one wave per (request, head, split), or per (request, head, chunk) under the ranked
//     schedule (attn_common.hpp); four independent waves per workgroup;
//   * K tile (16 tokens x D): lane l rebuilds the storage pieces l + 64 i (16 dims of one
//     token each: tokens l/8 and 8 + l/8 at D = 128, token l/4 at D = 64), so every load
//     instruction reads whole cache lines; it dots them with its 16 dims of q in
//     v_dot2_f32_bf16 and a DPP sum over the D/16 lanes that share a token gives the score;
//   * online softmax in the log2 domain; the wave-wide max is only taken when a score exceeds
//     the running maximum (the rescale is exact, it is just skipped when it would multiply by 1);
//   * probabilities are split into hi = bf16(p) and lo = bf16(p - hi), and token pairs of each
//     are broadcast to SGPRs with readlane;
//   * V tile: lane l rebuilds dims l (+64) for all 16 tokens as packed token pairs and
//     accumulates dot2(pair, hi) + dot2(pair, lo) in fp32, so every lane owns complete sums for
//     its dims and no cross-lane reduction of the output is needed;
//   * the next tile's compressed bytes are loaded before the current tile is computed.
#include "attn_common.hpp"
#include "kvz_lanes.hpp"
#include "mha_core.hpp"
#include "mha_pool.hpp"

namespace kvz {

constexpr int kWavesPerBlock = 4;

template <int D>
struct MhaStage {
  const uint8_t* unit;
  int page;        // index in the request's page table
  int tile;
  bool ok;         // false when the page id was out of range: a stand-in unit was read
  uint32_t meta;   // this lane's dword of the tile's meta window
  KRaw<D> k;
  VRaw<D> v;
};

// Issues the loads of one (page, tile) step. The loads are unconditional (a bad page id reads
// unit 0 instead and marks the stage), so that every path through the main loop has the same
// loads in flight and the next step's loads can overlap the current step's compute.
// `live` is false for a stage issued past the last step: its loads read nothing.
template <int D, bool CH>
__device__ __forceinline__ void mha_issue(MhaStage<D>& st, const uint8_t* units, int pid, int page, int tile, int H,
                                          int h, int P, int num_pages, int lane, bool live = true) {
  st.ok = pid >= 0 && pid < num_pages;
  st.page = page;
  st.unit = units + ((size_t)(st.ok ? pid : 0) * H + h) * unit_bytes(P, D);
  st.tile = tile;
  st.meta = load_meta(st.unit, P, D, tile, lane, live);
  load_k<D, false, true, CH>(st.unit, P, tile, lane, st.k, live);
  load_v<D>(st.unit, P, tile, lane, st.v, live);
}

// Returns false, leaving the state untouched, when the unit's escapes are in the pool and POOL
// is off.
template <int D, bool POOL, bool CH>
__device__ __forceinline__ bool mha_compute(MhaState<D>& st, const MhaStage<D>& stg, int P, uint32_t& krank,
                                            uint32_t& vrank, uint16_t* lds, const uint16_t* pool, int64_t pool_cap,
                                            float scale, int lane) {
  if (!stg.ok) return true;
  constexpr int VK = KRaw<D>::VK, NS = D / 64;
  UnitHeader hdr = header_from_meta<D>(stg.meta);
  if (!POOL && hdr.off != kInline) return false;
  if (POOL) clamp_to_pool(hdr, pool_cap);
  if (stg.tile == 0) { krank = 0; vrank = 0; }
  uint32_t kp[VK / 2];
  decode_k<D, CH>(stg.k, kp);
  if (hdr.kc) patch_k_tile<D, false, POOL>(kp, stg.k, stg.meta, hdr, P, stg.tile, krank, lds, pool, pool_cap, lane);
  float sc[D / 64];
  mha_scores<D>(st, kp, scale, sc);
  uint32_t phi[8], plo[8];
  mha_softmax<D>(st, sc, phi, plo);
  uint32_t vp[NS * 8];
#pragma unroll
  for (int g = 0; g < NS; ++g) decode_v_seg(stg.v.seg[g], v_bases<D, CH>(stg.meta, g), &vp[8 * g]);
  if (hdr.vc) patch_v_tile<D, POOL>(vp, stg.v, stg.meta, hdr, P, stg.tile, vrank, lds, pool, pool_cap, lane);
  mha_accumulate_v<D>(st, vp, phi, plo);
  return true;
}

// One wave per (request, head, split or chunk). The main loop handles units whose escapes are inline
// and skips a unit whose escapes are in the pool, remembering the first and last such page;
// after the loop (when the pipeline's registers are free again) the wave adds those two pages
// and any other pool unit between them, found by reading the unit headers 64 at a time. The
// pool path thus costs registers only outside the loop, and the rare pool unit costs only its
// own work. Four waves per SIMD is the register budget (128 VGPRs at D = 128): the streaming rate
// needs them, and the pool-capable loop is fitted into it. CH: channel groups (format 2).
template <int D, bool CH>
__global__ __launch_bounds__(64 * kWavesPerBlock) __attribute__((amdgpu_waves_per_eu(4))) void attn_mha_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ units, const uint16_t* __restrict__ pool,
    int64_t pool_cap, const uint64_t* __restrict__ esc_cursor, const uint16_t* __restrict__ k_tail,
    const uint16_t* __restrict__ v_tail, const int32_t* __restrict__ page_table, int max_pages,
    const int32_t* __restrict__ seq_lens, int B, int H, int grp, int P, int num_pages, SplitPlan plan, float scale,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, uint32_t* __restrict__ status) {
  __shared__ __align__(16) uint16_t lds_all[kWavesPerBlock][esc_lds_elems<D>()];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Hq = H * grp;   // query heads: grp of them read each KV head (one wave each)
  WorkItem wi;
  if (!plan_work(plan, seq_lens, B, P, max_pages, false, Hq, (int)uniform(blockIdx.x * kWavesPerBlock + wave), lane, wi))
    return;
  const int S = plan.S, C = wi.C, s = wi.s, hq = wi.k, h = hq / grp, r = wi.r;
  uint16_t* lds = lds_all[wave];
  int L = request_len(wi, seq_lens);
  if (L > max_pages * P || L < 0) {
    if (lane == 0 && s == 0 && hq == 0) atomicOr(status, kStatusSeqTooLong);
    L = L < 0 ? 0 : max_pages * P;
  }
  int nfull = L / P;
  const int rows = L % P;
  const int T = P / kTile;
  const int tpp = plan.tpp;   // plan pages per page: 1, or T when the splits count tiles
  // the splits the plan and the merge count for this row; with no unit slots every full page is
  // a bad id and is skipped, but every counted split still writes its (empty) partial
  const int Sr = C < 0 ? -C : active_splits(nfull * tpp, C);
  if (num_pages <= 0 && nfull > 0) {
    if (lane == 0 && s == 0 && hq == 0) atomicOr(status, kStatusBadPage);
    nfull = 0;
  }
  const bool ranked = C < 0;
  if (s >= Sr) return;
  int p0, p1;   // plan pages
  if (ranked) {
    rank_range(nfull * tpp, s, plan.ranks, p0, p1);
  } else {
    p0 = s * C;
    p1 = min(p0 + C, nfull * tpp);
  }
  // the split's tiles [a0, a1), counted over the request's full pages
  const int a0 = p0 * (T / tpp), a1 = max(p0, p1) * (T / tpp);
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
  const int nsteps = a1 - a0;
  // escape cursors of the split's first tile: 0 at a unit's start, else the escapes of the
  // unit's tiles before it
  uint32_t krank0 = 0, vrank0 = 0;
  if (nsteps > 0 && a0 % T != 0) {
    const int pid = sload<int32_t>(pt_row + a0 / T);
    if (pid >= 0 && pid < num_pages)
      escapes_before<D>(units + ((size_t)pid * H + h) * unit_bytes(P, D), P, a0 % T, lane, krank0, vrank0);
  }
  uint32_t krank = krank0, vrank = vrank0;
  int first_skip = -1, last_skip = -1;
  int nskip = 0;          // tiles skipped by the main loop
  int resume = -1;        // step from which the pool-capable loop takes over
  bool bad = false;
  // Records a skipped (pool) tile. When most tiles so far went to the pool, the wave leaves the
  // pipelined loop at the next page and walks the rest with the pool-capable loop, which loads
  // a tile's escapes with its payload instead of reloading the unit after the main loop. When
  // every tile so far went to the pool, that loop starts over from the first step and nothing is
  // left for after it. A first unit with a quarter or more of its values escaped starts it at
  // once: that marks an escape-heavy cache (a unit goes to the pool as soon as its escapes
  // outgrow the few inline entries).
  auto note = [&](const MhaStage<D>& stg, int done) {
    if (first_skip < 0) first_skip = stg.page;
    last_skip = stg.page;
    ++nskip;
    bool heavy = false;
    if (nskip == 1 && done == 1) {
      const UnitHeader hd = header_from_meta<D>(stg.meta);
      heavy = (uint64_t)hd.kc + hd.vc >= (uint64_t)P * D / 2;
    }
    if (heavy || (nskip >= 2 && 2 * nskip > done)) {
      if (nskip == done) {
        resume = 0;
        first_skip = last_skip = -1;
      } else {
        resume = (stg.page + 1) * T - a0;
      }
    }
  };
  // An escape-heavy cache (its pool holds, averaged over the unit slots, a quarter of a unit's
  // values or more) sends every split to the pool-capable loop from its first step: otherwise
  // the pipelined loop would load a split's first two tiles only to find them in the pool, and
  // the pool-capable loop would load them again.
  if (nsteps > 0 && sload<uint64_t>(esc_cursor) >= (uint64_t)num_pages * H * (uint64_t)(P * D / 2)) resume = 0;
  if (nsteps > 0 && resume < 0) {
    // load cursor: step ln = (page lp, tile lt); it stays on the last step once there, and the
    // stages issued past the end (never computed) read nothing (`live` false)
    int ln = 0, lp = a0 / T, lt = a0 % T;
    bool live = true;
    const int last = nsteps - 1;
    auto advance = [&]() {
      if (ln < last) {
        ++ln;
        if (++lt == T) { lt = 0; ++lp; }
      } else {
        live = false;
      }
    };
    MhaStage<D> a, b;
    int pid = sload<int32_t>(pt_row + lp);
    mha_issue<D, CH>(a, units, pid, lp, lt, H, h, P, num_pages, lane);
    advance();
    pid = sload<int32_t>(pt_row + lp);   // one step ahead of its use
    for (int i = 0; i < nsteps; i += 2) {
      mha_issue<D, CH>(b, units, pid, lp, lt, H, h, P, num_pages, lane, live);
      advance();
      pid = sload<int32_t>(pt_row + lp);
      bad |= !a.ok;
      if (!mha_compute<D, false, CH>(st, a, P, krank, vrank, lds, pool, pool_cap, scale, lane)) note(a, i + 1);
      if (i + 1 >= nsteps || resume >= 0) break;
      mha_issue<D, CH>(a, units, pid, lp, lt, H, h, P, num_pages, lane, live);
      advance();
      pid = sload<int32_t>(pt_row + lp);
      bad |= !b.ok;
      if (!mha_compute<D, false, CH>(st, b, P, krank, vrank, lds, pool, pool_cap, scale, lane)) note(b, i + 2);
      if (resume >= 0) break;
    }
  }
  if (resume >= 0 && resume < nsteps) {
    // the rest of the split, every unit as it comes; the next tile's meta window is in flight
    // while a tile is computed
    auto unit_of = [&](int n, bool& ok) {
      const int pid = sload<int32_t>(pt_row + (a0 + n) / T);
      ok = pid >= 0 && pid < num_pages;
      return units + ((size_t)(ok ? pid : 0) * H + h) * unit_bytes(P, D);
    };
    if (resume == 0) {   // from the split's first tile again
      krank = krank0;
      vrank = vrank0;
    }
    bool ok;
    const uint8_t* u = unit_of(resume, ok);
    uint32_t meta = load_meta(u, P, D, (a0 + resume) % T, lane);
    for (int n = resume; n < nsteps; ++n) {
      bool nok = true;
      const uint8_t* nu = u;
      uint32_t nmeta = 0;
      if (n + 1 < nsteps) {
        nu = unit_of(n + 1, nok);
        nmeta = load_meta(nu, P, D, (a0 + n + 1) % T, lane);
      }
      if (ok) mha_any_tile<D, CH>(st, u, meta, P, (a0 + n) % T, krank, vrank, lds, pool, pool_cap, scale, lane);
      bad |= !ok;
      u = nu;
      ok = nok;
      meta = nmeta;
    }
  }
  if (bad && lane == 0) atomicOr(status, kStatusBadPage);
  if (first_skip >= 0) {
    // units whose escapes are in the pool: the recorded pages, then any between them (the
    // split's tiles of each: its first page may begin and its last end inside the unit)
    auto do_page = [&](int page) {
      const int pid = sload<int32_t>(pt_row + page);
      const int tb = max(0, a0 - page * T), te = min(T, a1 - page * T);
      if (tb > 0) {
        krank = krank0;
        vrank = vrank0;
      }
      for (int t = tb; t < te; ++t) {
        MhaStage<D> a;
        mha_issue<D, CH>(a, units, pid, page, t, H, h, P, num_pages, lane);
        mha_compute<D, true, CH>(st, a, P, krank, vrank, lds, pool, pool_cap, scale, lane);
      }
    };
    do_page(first_skip);
    if (last_skip != first_skip) do_page(last_skip);
    const uint32_t hdr_off = hdr_offset(P, D) + 8;
    for (int c0 = first_skip + 1; c0 < last_skip; c0 += 64) {
      const int pg = c0 + lane;
      bool in_pool = false;
      if (pg < last_skip) {
        const int pid = pt_row[pg];
        if (pid >= 0 && pid < num_pages)
          in_pool = *reinterpret_cast<const uint64_t*>(units + ((size_t)pid * H + h) * unit_bytes(P, D) + hdr_off) !=
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
    const size_t toff = ((size_t)r * H + h) * P * D;
    mha_tail<D>(st, k_tail + toff, v_tail + toff, rows, scale, lane);
  }
  // partials: l summed over one lane per token group (the D/16 lanes of a token hold the
  // same terms)
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

int launch_attn_mha(const uint16_t* q, const uint8_t* units, const uint16_t* pool, int64_t pool_cap,
                    const uint64_t* esc_cursor, const uint16_t* k_tail,
                    const uint16_t* v_tail, const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                    int B, int Hq, int H, int D, int P, int num_pages, SplitPlan plan, float scale, float* ws_acc,
                    float* ws_ml, uint32_t* status, bool channel, hipStream_t stream) {
  static int slots128[64], slots64[64], slots128c[64], slots64c[64];
  if (H <= 0 || Hq % H) return -2;
  const dim3 block(64 * kWavesPerBlock);
  if (D == 128) {
    plan.slots = channel ? resident_waves(attn_mha_kernel<128, true>, block.x, slots128c, 64)
                         : resident_waves(attn_mha_kernel<128, false>, block.x, slots128, 64);
  } else if (D == 64) {
    plan.slots = channel ? resident_waves(attn_mha_kernel<64, true>, block.x, slots64c, 64)
                         : resident_waves(attn_mha_kernel<64, false>, block.x, slots64, 64);
  } else {
    return -2;
  }
  // The ranked schedule's big ranks: one round of the resident waves. The split schedule aims
  // at two waves per resident slot: waves on one SIMD run at different speeds, and a second
  // round lets the slots of early finishers take new work (measured 1-1.5% faster at 8K and 32K
  // contexts, ragged or not; the grouped-query kernel, measured the same way, does best with
  // two thirds of one round). Query groups (head dim 64 only) make one item per query head.
  rank_fit(plan, plan.slots, (long)B * Hq);
  plan.slots = plan.slots > 0 ? 2 * plan.slots : B * Hq * plan.S;
  const dim3 grid(plan_blocks(plan, (long)B * Hq, kWavesPerBlock));
  auto kernel = D == 128 ? (channel ? attn_mha_kernel<128, true> : attn_mha_kernel<128, false>)
                         : (channel ? attn_mha_kernel<64, true> : attn_mha_kernel<64, false>);
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, q, units, pool, pool_cap, esc_cursor, k_tail, v_tail, page_table,
                     max_pages, seq_lens, B, H, Hq / H, P, num_pages, plan, scale, ws_acc, ws_ml, status);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvz
