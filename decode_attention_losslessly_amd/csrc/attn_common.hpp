// Pieces shared by the decode-attention kernels: split geometry, partial results, merge.
//
// Split-K over the sequence (flash-decoding): work item (request r, head, split s) covers the
// full pages [s*C, min((s+1)*C, L/P)) of the request, or under the ranked schedule below a
// chunk whose pages are a share of the request's; the last split or chunk also covers the
// L mod P tail rows. It leaves (m, l, acc[D]):
// the running maximum of the log2-domain scores, the sum of exp2(score - m) and the weighted
// sum of values. A second kernel merges the partials (the pages count this merge inside
// attention's cost: ZipFusion summary, §IV.B "Attention Kernel Performance").
#pragma once

#include "kvz_device.hpp"

namespace kvz {

constexpr float kLog2e = 1.4426950408889634f;

// number of splits request r needs: at least one, so that an empty request still writes a
// (m = -inf, l = 0) partial and the merge can produce zeros
__device__ __forceinline__ int active_splits(int nfull, int C) { return nfull > 0 ? (nfull + C - 1) / C : 1; }

// ---------------------------------------------------------------- split schedule
// How one call's work is cut. Request r holds `ipr` work items (its KV heads, times the chunks
// of query heads in the grouped-query kernels), each over the request's np_r pages (its full
// pages; every page for the uncompressed baseline), and an item is cut into splits of C pages.
// C is chosen on the device from the sequence lengths: the smallest C in [C_lo, C_hi] whose
// splits, over the whole batch, fit the waves the kernel keeps resident at once (`slots`), so
// that a batch of uneven lengths still fills the GPU in one pass rather than leaving waves idle
// behind its longest requests. C_lo bounds the splits of one item (the workspace holds S of
// them); C_lo == C_hi fixes C. The launch's first wave records C after the partials, where the
// merge reads it, and the plan's tiles per page after it.
//
// A plan page is normally one page of the table. The compressed multi-head kernel can also count
// its splits in 16-token tiles (tpp = P / 16 plan pages per page of the table), so that a batch
// of few, large pages is not left to one wave per page walking its tiles in a row: a split may
// then start and end inside a unit.
struct SplitPlan {
  int S;           // partial slots per (request, query head)
  int C_lo, C_hi;  // bounds on the pages per split
  int slots;       // waves of the kernel resident at once on the device
  int slots_pref;  // > 0: a smaller wave count to aim for first (see plan_work)
  int ranks;       // > 0: the ranked schedule below may be used, with this many big ranks
  int rank_min;    // ... when a big chunk holds at least this many pages on average (0: always)
  int tpp;         // plan pages per page of the table: 1, or P / 16 (splits counted in tiles)
  int* chosen;     // [0]: the plan pages per split used (or minus the chunks per item when
                   // ranked), [1]: tpp; written by the launch's first wave
};

__device__ __forceinline__ void plan_record(const SplitPlan& pl, int C) {
  pl.chosen[0] = C;
  pl.chosen[1] = pl.tpp;
}

constexpr int kLenUnknown = -2147483647 - 1;

struct WorkItem {
  int r;    // request
  int k;    // item within the request
  int s;    // split of the item (the chunk's rank when ranked)
  int C;    // pages per split; minus the chunks per item when ranked
  int L;    // seq_lens[r] as read by the plan, or kLenUnknown when the plan did not read it
};

// the request's length: from the plan's registers when it read them, else one scalar load
__device__ __forceinline__ int request_len(const WorkItem& w, const int32_t* seq_lens) {
  return w.L != kLenUnknown ? w.L : sload<int32_t>(seq_lens + w.r);
}

// ---------------------------------------------------------------- ranked schedule
// A wave's speed depends on its age on its SIMD (the issue arbiter favours the oldest wave), so
// waves given equal work finish far apart, and the end of a launch runs with too few waves to
// keep HBM busy. The ranked schedule cuts every item into (1 + kRankTailPer) R chunks and
// numbers the waves rank by rank (every item's chunk 0, then every item's chunk 1, ...), so the
// hardware starts them in that order: the first R ranks (one round of resident waves when
// R = resident waves / items) take 80% of each item's pages in equal chunks, and the
// kRankTailPer R tail ranks take the rest in chunks that shrink linearly to a fifth of the
// first, which fill the slots of early finishers and end close together. Chunks are
// proportional to each request's own length, so the schedule suits batches of nearly even
// lengths (the plan checks that); the multi-head kernels use it, the grouped-query ones keep
// their split schedule.
constexpr uint32_t kRankOne = 1u << 20;                 // shares are in units of 2^-20
constexpr uint32_t kRankBig = kRankOne / 5 * 4;         // share of the first R ranks
constexpr int kRankTaper = 5;                           // first / last tail chunk
constexpr int kRankTailPer = 1;                         // tail ranks per big rank

// chunks per item with R big ranks
__host__ __device__ constexpr int rank_chunks(int R) { return (1 + kRankTailPer) * R; }

// share of an item's pages in its chunks before rank k (k in [0, rank_chunks(R)])
__device__ __forceinline__ uint32_t rank_share(int k, int R) {
  if (k <= R) return (uint32_t)((uint64_t)kRankBig * k / R);
  // with T tail ranks, tail chunk i weighs (taper - 1)(T - 1 - i) + (T - 1); n of them weigh
  // wsum(n)
  const int T = kRankTailPer * R;
  const uint64_t i = (uint64_t)(k - R), c = (uint64_t)(T - 1), a = kRankTaper - 1;
  const uint64_t rest = kRankOne - kRankBig;
  if (c == 0) return kRankBig + (uint32_t)(rest * i);   // one tail chunk
  auto wsum = [&](uint64_t n) { return a * (n * c - n * (n - 1) / 2) + n * c; };
  return kRankBig + (uint32_t)(rest * wsum(i) / wsum((uint64_t)T));
}

// pages [p0, p1) of chunk k of an item with np pages
__device__ __forceinline__ void rank_range(int np, int k, int R, int& p0, int& p1) {
  p0 = (int)(((uint64_t)np * rank_share(k, R)) >> 20);
  p1 = (int)(((uint64_t)np * rank_share(k + 1, R)) >> 20);
}

// plan pages of a request of length L: its pages (every page for the uncompressed baseline,
// the full ones for the compressed kernels), tpp plan pages to each full page
__device__ __forceinline__ int plan_pages(int32_t L, int P, int max_pages, bool dense, int tpp = 1) {
  L = L < 0 ? 0 : min(L, max_pages * P);
  return dense ? (L + P - 1) / P : L / P * tpp;
}

// Pages of the requests, read once: up to kPlanRegs requests per lane are held in registers
// (a batch of up to 256), larger batches are re-read from memory at every use.
constexpr int kPlanRegs = 4;
struct PlanPages {
  int np[kPlanRegs];
  int len[kPlanRegs];   // the lengths as read, so that a wave need not load its own again
  bool held;
  int tpp;              // plan pages per page of the table
};

__device__ __forceinline__ PlanPages plan_load(const int32_t* seq_lens, int B, int P, int max_pages, bool dense,
                                               int lane, int tpp = 1) {
  PlanPages pp;
  pp.held = B <= 64 * kPlanRegs;
  pp.tpp = tpp;
#pragma unroll
  for (int j = 0; j < kPlanRegs; ++j) {
    const int r = 64 * j + lane;
    const bool in = pp.held && r < B;
    pp.len[j] = in ? seq_lens[r] : 0;
    pp.np[j] = in ? plan_pages(pp.len[j], P, max_pages, dense, tpp) : -1;
  }
  return pp;
}

// length of request r (wave-uniform) from the registers, or kLenUnknown (one readlane per
// register, then a scalar select: a select among the vector registers themselves became a
// dynamically indexed array in scratch memory)
__device__ __forceinline__ int plan_len(const PlanPages& pp, int r) {
  if (!pp.held) return kLenUnknown;
  int v = (int)readlane((uint32_t)pp.len[0], r & 63);
#pragma unroll
  for (int j = 1; j < kPlanRegs; ++j) {
    const int x = (int)readlane((uint32_t)pp.len[j], r & 63);
    v = (r >> 6) == j ? x : v;
  }
  return v;
}

// splits of request r's item at C pages per split (0 past the batch)
__device__ __forceinline__ uint32_t plan_splits(const PlanPages& pp, const int32_t* seq_lens, int B, int P,
                                                int max_pages, bool dense, int r, int j, int C) {
  if (r >= B) return 0u;
  const int np = pp.held ? pp.np[j] : plan_pages(seq_lens[r], P, max_pages, dense, pp.tpp);
  return (uint32_t)active_splits(np, C);
}

// splits of all requests at C pages per split (one item each), wave-uniform
__device__ __forceinline__ uint64_t plan_total(const PlanPages& pp, const int32_t* seq_lens, int B, int P,
                                               int max_pages, bool dense, int C, int lane) {
  if (pp.held) {
    uint32_t n = 0;
#pragma unroll
    for (int j = 0; j < kPlanRegs; ++j) n += pp.np[j] >= 0 ? (uint32_t)active_splits(pp.np[j], C) : 0u;
    return readlane(wave_incl_scan(n), 63);
  }
  uint64_t t = 0;
  for (int b0 = 0; b0 < B; b0 += 64) t += readlane(wave_incl_scan(plan_splits(pp, seq_lens, B, P, max_pages, dense,
                                                                               b0 + lane, 0, C)), 63);
  return t;
}

// pages of all requests in the batch (wave-uniform)
__device__ __forceinline__ uint64_t plan_page_sum(const PlanPages& pp, const int32_t* seq_lens, int B, int P,
                                                  int max_pages, bool dense, int lane) {
  uint64_t npg = 0;
  if (pp.held) {
    uint32_t n = 0;
#pragma unroll
    for (int j = 0; j < kPlanRegs; ++j) n += pp.np[j] > 0 ? (uint32_t)pp.np[j] : 0u;
    npg = readlane(wave_incl_scan(n), 63);
  } else {
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int r = b0 + lane;
      npg += readlane(wave_incl_scan(r < B ? (uint32_t)plan_pages(seq_lens[r], P, max_pages, dense, pp.tpp) : 0u),
                      63);
    }
  }
  return npg;
}

// most pages of one request in the batch (wave-uniform)
__device__ __forceinline__ uint32_t plan_page_max(const PlanPages& pp, const int32_t* seq_lens, int B, int P,
                                                  int max_pages, bool dense, int lane) {
  uint32_t m = 0;
  if (pp.held) {
#pragma unroll
    for (int j = 0; j < kPlanRegs; ++j) m = max(m, pp.np[j] > 0 ? (uint32_t)pp.np[j] : 0u);
  } else {
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int r = b0 + lane;
      m = max(m, r < B ? (uint32_t)plan_pages(seq_lens[r], P, max_pages, dense, pp.tpp) : 0u);
    }
  }
  return wave_max_u32(m);
}

// This wave's split; false when the wave has none. Waves are numbered request by request, then,
// for the compressed kernels, split by split and item by item: the four waves of a workgroup
// then take the same split of four items of one request, which have the same length, so they
// end together and free their workgroup's slots at once (a workgroup's slots are given back
// only when all its waves are done). On a batch of uneven lengths with 32 heads this was 3.9%
// faster; the uncompressed baseline measured 2.3% slower with it and keeps item by item.
__device__ __forceinline__ bool plan_work(const SplitPlan& pl, const int32_t* seq_lens, int B, int P, int max_pages,
                                          bool dense, int ipr, int wave_id, int lane, WorkItem& w) {
  const uint64_t items = (uint64_t)B * ipr, slots = (uint64_t)pl.slots;
  if (pl.ranks > 0) {
    // ranked when forced, or when the lengths are nearly even (the longest request at most
    // 5/4 of the mean: chunks are shares of each request's pages, so in a ragged batch the
    // longest requests' chunks would be the longest waves, where the split schedule cuts all
    // work into equal splits) and a big chunk holds at least rank_min pages on average:
    // big share * pages of the batch / (B * R) >= rank_min
    const PlanPages pp = plan_load(seq_lens, B, P, max_pages, dense, lane, pl.tpp);
    bool use = pl.rank_min <= 0;
    if (!use) {
      const uint64_t npg = plan_page_sum(pp, seq_lens, B, P, max_pages, dense, lane);
      const uint64_t mx = plan_page_max(pp, seq_lens, B, P, max_pages, dense, lane);
      use = 4 * mx * (uint64_t)B <= 5 * npg &&
            npg * kRankBig >= (uint64_t)pl.rank_min * B * pl.ranks * kRankOne;
    }
    if (use) {
      const int n = rank_chunks(pl.ranks);
      if (wave_id == 0 && lane == 0) plan_record(pl, -n);
      if ((uint64_t)wave_id >= items * n) return false;
      const int j = (int)((uint64_t)wave_id % items);
      w.s = (int)((uint64_t)wave_id / items);
      w.r = j / ipr;
      w.k = j % ipr;
      w.C = -n;
      w.L = plan_len(pp, w.r);
      return true;
    }
  }
  int C = pl.C_lo;
  if (pl.C_hi > pl.C_lo && items >= slots) C = pl.C_hi;   // no split fits: one per item
  if (C >= max_pages * pl.tpp) {
    // every request has exactly one split (an empty one too): numbering is direct
    if (wave_id == 0 && lane == 0) plan_record(pl, C);
    if ((uint64_t)wave_id >= items) return false;
    w.r = wave_id / ipr;
    w.k = wave_id % ipr;
    w.s = 0;
    w.C = C;
    w.L = kLenUnknown;
    return true;
  }
  const PlanPages pp = plan_load(seq_lens, B, P, max_pages, dense, lane, pl.tpp);
  if (pl.C_hi > pl.C_lo && C < pl.C_hi) {
    // With N = ipr * (pages of the batch) and `items` = ipr * B, the splits at C lie between
    // N / C and N / C + items (the total only falls as C grows): no C below N / s fits s waves,
    // and every C from N / (s - items) on does. Search between the two.
    const uint64_t N = plan_page_sum(pp, seq_lens, B, P, max_pages, dense, lane) * (uint64_t)ipr;
    auto smallest_fit = [&](uint64_t s) {
      int lo = (int)min((uint64_t)pl.C_hi, max((uint64_t)pl.C_lo, (N + s - 1) / s));
      int hi = pl.C_hi;
      if (s > items) hi = (int)min((uint64_t)hi, max((uint64_t)lo, (N + s - items - 1) / (s - items)));
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (plan_total(pp, seq_lens, B, P, max_pages, dense, mid, lane) * ipr <= s) hi = mid;
        else lo = mid + 1;
      }
      return lo;
    };
    // A kernel may prefer fewer waves than it can hold (slots_pref: the grouped-query kernel
    // streams faster at two waves per SIMD than at three, measured): that target is kept when
    // its splits come to at least 7/8 of it, else the batch's items divide it badly (96 requests
    // of 8 KV heads: 1,536 waves) and the full count is used.
    bool done = false;
    const uint64_t pref = (uint64_t)pl.slots_pref;
    if (pref > items && pref < slots) {
      const int Cp = smallest_fit(pref);
      if (8 * plan_total(pp, seq_lens, B, P, max_pages, dense, Cp, lane) * ipr >= 7 * pref) {
        C = Cp;
        done = true;
      }
    }
    if (!done) C = smallest_fit(slots);
  }
  if (wave_id == 0 && lane == 0) plan_record(pl, C);
  // find the request whose splits hold this wave's number, 64 requests at a time
  uint64_t base = 0;
  auto visit = [&](int b0, uint32_t sr) -> bool {
    const uint32_t cnt = sr * (uint32_t)ipr;
    const uint32_t incl = wave_incl_scan(cnt);
    const uint64_t hit = ballot(base + incl > (uint64_t)wave_id);
    if (!hit) {
      base += readlane(incl, 63);
      return false;
    }
    const int l = __builtin_ctzll(hit);
    const uint32_t local = (uint32_t)((uint64_t)wave_id - base) - readlane(incl - cnt, l);
    const uint32_t n = readlane(sr, l);
    w.r = b0 + l;
    if (dense) {   // item by item, split by split
      w.k = (int)(local / n);
      w.s = (int)(local % n);
    } else {       // split by split, item by item
      w.s = (int)(local / (uint32_t)ipr);
      w.k = (int)(local % (uint32_t)ipr);
    }
    w.C = C;
    w.L = plan_len(pp, w.r);
    return true;
  };
  if (pp.held) {
#pragma unroll
    for (int j = 0; j < kPlanRegs; ++j) {
      if (64 * j >= B) break;
      if (visit(64 * j, pp.np[j] >= 0 ? (uint32_t)active_splits(pp.np[j], C) : 0u)) return true;
    }
    return false;
  }
  for (int b0 = 0; b0 < B; b0 += 64)
    if (visit(b0, plan_splits(pp, seq_lens, B, P, max_pages, dense, b0 + lane, 0, C))) return true;
  return false;
}

// waves of `kernel` (launched with `threads` per workgroup) resident at once on the current
// device, cached per device in `cache`; 0 when the runtime cannot say
template <typename F>
inline int resident_waves(F kernel, int threads, int* cache, int ncache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= ncache) return 0;
  if (cache[dev] > 0) return cache[dev];
  int blocks = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, threads, 0) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  cache[dev] = blocks * (threads / 64) * cus;
  return cache[dev];
}

// Big ranks from the waves the kernel keeps resident (one round of them takes the big chunks),
// unless the caller fixed them; never more chunks than the workspace's S slots.
inline void rank_fit(SplitPlan& pl, int resident, long items) {
  if (pl.ranks <= 0) return;
  long R = pl.ranks;
  if (pl.rank_min > 0 && resident > 0) R = resident / items > 1 ? resident / items : 1;
  while (R > 0 && rank_chunks((int)R) > pl.S) --R;
  pl.ranks = (int)R;   // 0 when the workspace holds too few slots: the schedule is not used
}

// workgroups to launch: every split the plan can produce gets a wave. No item has more than S
// splits or chunks (C >= C_lo; rank_fit keeps the chunks within S), so a small batch, whose
// splits cannot fill the slots, launches no waves that would only exit.
inline unsigned plan_blocks(const SplitPlan& pl, long items, int waves_per_block) {
  const long fixed = items * pl.S;                                   // C fixed: at most S per item
  long waves = pl.C_hi > pl.C_lo ? (pl.slots > items ? (long)pl.slots : items) : fixed;
  if (pl.ranks > 0 && items * rank_chunks(pl.ranks) > waves) waves = items * rank_chunks(pl.ranks);
  if (waves > fixed) waves = fixed;
  return (unsigned)((waves + waves_per_block - 1) / waves_per_block);
}

struct Partials {
  float* acc;   // [rows][S][D]
  float* ml;    // [rows][S][2]
};

__device__ __forceinline__ Partials partials(void* ws, int rows, int S, int D) {
  Partials p;
  p.acc = reinterpret_cast<float*>(ws);
  p.ml = p.acc + (size_t)rows * S * D;
  return p;
}

}  // namespace kvz
