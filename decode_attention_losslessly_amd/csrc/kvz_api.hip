// C ABI of libkvz: argument validation, split sizing and kernel launches. The library never
// allocates device memory and never synchronises; every call enqueues on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kvz.h"
#include "attn_common.hpp"
#include "zf.hpp"

namespace kvz {
int launch_decompress(const uint8_t* units, const uint16_t* pool, int64_t pool_cap, const int32_t* page_ids, int n, int H, int P,
                      int D, int num_pages, int lane_map, uint16_t* k_dst, uint16_t* v_dst, uint32_t* status,
                      bool channel, hipStream_t stream);
int launch_compress(const uint16_t* k_src, const uint16_t* v_src, const int32_t* ids, int n, int H, int P, int D,
                    int num_pages, uint8_t* units, uint16_t* pool, int64_t pool_cap, uint64_t* cursor,
                    uint32_t* status, int format, hipStream_t stream);
int launch_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* page_table, int max_pages,
                  int32_t* seq_lens, int B, int H, int P, int D, int num_pages, uint8_t* units, uint16_t* pool,
                  int64_t pool_cap, uint64_t* cursor, uint16_t* k_tail, uint16_t* v_tail, uint32_t* status,
                  int format, hipStream_t stream);
int launch_attn_zf(const uint16_t* q, const uint8_t* units, const uint16_t* pool, int64_t pool_cap,
                   const uint16_t* k_tail, const uint16_t* v_tail, const int32_t* page_table, int max_pages,
                   const int32_t* seq_lens, int B, int Hq, int H, int D, int P, int num_pages, SplitPlan plan,
                   float scale, float* ws_acc, float* ws_ml, uint32_t* status, hipStream_t stream);
int launch_attn_zf_gqa(const uint16_t* q, const uint8_t* units, const uint16_t* pool, int64_t pool_cap,
                       const uint16_t* k_tail, const uint16_t* v_tail, const int32_t* page_table, int max_pages,
                       const int32_t* seq_lens, int B, int Hq, int H, int D, int P, int num_pages, SplitPlan plan,
                       float scale, float* ws_acc, float* ws_ml, uint32_t* status, hipStream_t stream);
int launch_decompress_zf(const uint8_t* units, const uint16_t* pool, int64_t pool_cap, const int32_t* page_ids, int n,
                         int H, int P, int D, int num_pages, int lane_map, uint16_t* k_dst, uint16_t* v_dst,
                         uint32_t* status, hipStream_t stream);
int launch_attn_mha(const uint16_t* q, const uint8_t* units, const uint16_t* pool, int64_t pool_cap,
                    const uint64_t* esc_cursor, const uint16_t* k_tail,
                    const uint16_t* v_tail, const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                    int B, int Hq, int H, int D, int P, int num_pages, SplitPlan plan, float scale, float* ws_acc,
                    float* ws_ml, uint32_t* status, bool channel, hipStream_t stream);
int launch_attn_gqa(const uint16_t* q, const uint8_t* units, const uint16_t* pool, int64_t pool_cap,
                    const uint64_t* esc_cursor, const uint16_t* k_tail,
                    const uint16_t* v_tail, const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                    int B, int Hq, int Hkv, int D, int P, int num_pages, SplitPlan plan, float scale, float* ws_acc,
                    float* ws_ml, uint32_t* status, bool channel, hipStream_t stream);
int launch_attn_dense_mha(const uint16_t* q, const uint16_t* k_pages, const uint16_t* v_pages, const int32_t* pt,
                          int max_pages, const int32_t* seq_lens, int B, int Hq, int H, int D, int P,
                          int num_pages, SplitPlan plan, float scale, float* ws_acc, float* ws_ml, uint32_t* status,
                          hipStream_t stream);
int launch_attn_dense_gqa(const uint16_t* q, const uint16_t* k_pages, const uint16_t* v_pages, const int32_t* pt,
                          int max_pages, const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int P,
                          int num_pages, SplitPlan plan, float scale, float* ws_acc, float* ws_ml, uint32_t* status,
                          hipStream_t stream);
int launch_compact_pool(uint8_t* units, const uint16_t* pool, int64_t pool_cap, const int32_t* page_ids, int n, int H,
                        int P, int D, int num_pages, int format, uint16_t* new_pool, int64_t new_cap,
                        uint64_t* new_cursor, uint32_t* status, hipStream_t stream);
int launch_merge(const float* ws_acc, const float* ws_ml, const int32_t* seq_lens, int B, int Hq, int D, int P,
                 int max_pages, int S, const int32_t* chosen, int dense, uint16_t* out, float* out_f32,
                 hipStream_t stream);
}  // namespace kvz

namespace {

constexpr int kTargetItems = 4096;   // splits aimed for: ~16 waves per CU on 256 CUs
constexpr int kGqaRows = 8;          // query heads per grouped-query wave

// waves per split of the batch: one per (request, KV head, chunk of up to 8 query heads) in the
// grouped-query kernels (head dim 128), one per (request, query head) in the multi-head ones
int64_t work_items_per_split(int B, int Hq, int Hkv, int D) {
  const int grp = Hq / Hkv;
  if (grp > 1 && D != 128) return (int64_t)B * Hq;
  const int64_t chunks = grp > 1 ? ((int64_t)grp + kGqaRows - 1) / kGqaRows : 1;
  return (int64_t)B * Hkv * chunks;
}

// Pages per split: `pps` when the caller fixes it, else the smallest the kernels may choose.
// The kernels pick the split size per call from the sequence lengths (the smallest one whose
// splits fit their resident waves); this lower bound keeps the splits of one item, and so the
// workspace, to about twice the split count that would fill kTargetItems waves with the batch's
// items, and a split to at least 64 tokens.
int pages_per_split(int B, int Hq, int Hkv, int D, int P, int max_pages, int pps) {
  if (pps > 0) return pps;   // (pps < 0 asks for the ranked schedule; this bound is then unused by it)
  const int64_t items = work_items_per_split(B, Hq, Hkv, D);
  const int64_t s_cap = items >= 2 * kTargetItems ? 1 : (2 * kTargetItems + items - 1) / items;
  const int min_c = P >= 64 ? 1 : 64 / P;
  int64_t c = ((int64_t)max_pages + s_cap - 1) / s_cap;
  if (c < min_c) c = min_c;
  if (c < 1) c = 1;
  return (int)c;
}

int split_count(int max_pages, int C) { return max_pages > 0 ? (int)(((int64_t)max_pages + C - 1) / C) : 1; }

// Big ranks R of the ranked schedule (0: not used), which the multi-head kernels over the
// escape format and the uncompressed baseline may use: the first round of kTargetItems
// waves takes R chunks of every item, and the rest R chunks more (the launch lowers R to its
// own resident waves). The kernel uses it only when a big chunk averages kRankMinPages pages or
// more over the call's actual lengths and the lengths are nearly even; pps < 0 forces it with
// -pps big ranks. (The grouped-query kernel, whose splits each write the partials of up to 8
// query heads, measured slower with it, 3% to 35%, and so did the ZipFusion-format kernel, which
// reads raw blocks from the pool: 925 -> 1114 us on the 8K batch of 32; both keep the split
// schedule.)
constexpr int kRankMinPages = 5;    // measured: ranked won at 6.4 pages per big chunk, lost at 3.2
constexpr int kMaxForcedRanks = 4096;
// No ranked slots are reserved when even requests of the table's full width would give big
// chunks of less than half kRankMinPages pages (the launch sizes R from its own resident waves,
// which may differ from kTargetItems by that much): the grid and the workspace then hold the
// split schedule's waves only.
int rank_count(int B, int Hq, int Hkv, int max_pages, int pps) {
  if (pps < 0) return -pps;
  if (pps > 0 || Hq != Hkv) return 0;
  const int64_t items = (int64_t)B * Hkv;
  if (items >= 2 * kTargetItems) return 0;
  const int R = items >= kTargetItems ? 1 : (int)(kTargetItems / items);
  if ((uint64_t)max_pages * kvz::kRankBig * 2 < (uint64_t)kRankMinPages * R * kvz::kRankOne) return 0;
  return R;
}

constexpr int64_t kTileSplitWaves = 2048;

// Tiles per plan page of the compressed multi-head kernel. With pages of more than one tile and
// a batch whose items, even at the table's full width, hold fewer than kTileSplitWaves pages,
// splits of whole pages would leave most of the GPU idle while each wave walks a page's tiles in
// a row (256-token pages: 16 tiles). That kernel can start and end a split inside a unit, so
// there its splits are counted in 16-token tiles. The other kernels, a fixed split size
// (pps > 0) and the ranked schedule keep whole pages, and so does a batch with pages enough
// (1 x 32 heads x 4K tokens in 64-token pages: 2,048 splits of one page, 12.2 us, against
// 12.6 us counted in tiles, whose split-size search then only costs time).
int split_tiles(int B, int Hq, int Hkv, int D, int P, int max_pages, int pps) {
  if (pps != 0 || P <= kvz::kTile || (Hq != Hkv && D == 128)) return 1;
  if (work_items_per_split(B, Hq, Hkv, D) * (int64_t)max_pages >= kTileSplitWaves) return 1;
  return P / kvz::kTile;
}

// Smallest split, in tiles, when splits are counted in tiles: the fewest tiles whose splits,
// over the batch's items at the table's full width, come to at most kTileSplitWaves. A split
// that starts inside a unit first counts the escapes of the unit's earlier tiles (their offset
// codes: a third of their bytes), so short splits cost extra reads as well as their start-up.
// Measured (whole decode step, 1 x 2 heads x one 256-token page, and 1 x 32 heads x 4K tokens in
// 256-token pages): 1 tile 11.9 and 38.1 us, 2 tiles 12.9 and 30.6, 4 tiles 16.1 and 28.1 (the
// second with whole pages per split: 52.5); the best of each is the one with at most 2,048 waves.
int tile_split_min(int B, int Hq, int Hkv, int D, int max_pages, int tpp) {
  const int64_t tiles = work_items_per_split(B, Hq, Hkv, D) * (int64_t)max_pages * tpp;
  const int64_t c = (tiles + kTileSplitWaves - 1) / kTileSplitWaves;
  return (int)(c < 1 ? 1 : c);
}

// split slots per (request, query head): the dynamic schedule's bound (in pages, or in tiles
// where the multi-head kernel counts tiles), and the ranked one's chunks per row
int slot_count(int B, int Hq, int Hkv, int D, int P, int max_pages, int pps) {
  int S = split_count(max_pages, pages_per_split(B, Hq, Hkv, D, P, max_pages, pps));
  const int n = kvz::rank_chunks(rank_count(B, Hq, Hkv, max_pages, pps));
  if (n > S) S = n;
  const int t = split_tiles(B, Hq, Hkv, D, P, max_pages, pps);
  if (t > 1) {
    const int St = split_count(max_pages * t, tile_split_min(B, Hq, Hkv, D, max_pages, t));
    if (St > S) S = St;
  }
  return S;
}

// the format's shapes: an inline escape keeps its storage position in 16 bits, so a block holds at
// most 65536 values
bool shape_ok(int P, int D) {
  return P > 0 && P % 16 == 0 && D > 0 && D % 64 == 0 && (int64_t)P * D <= 65536;
}

// Compression stages a unit's values in LDS (160 KB per workgroup): the wave compressor (first
// format, head dim 64 or 128) holds the V block, up to the format's largest block of 65536
// values; the workgroup compressor (other head dims, the block format, channel groups) holds K
// and V, half that.
bool compress_fits(const kvz_cache* c) {
  const int64_t n = (int64_t)c->page_size * c->head_dim;
  const bool wave = c->format == KVZ_FORMAT_ESCAPE && (c->head_dim == 64 || c->head_dim == 128);
  return n <= (wave ? 65536 : 32768);
}

// the kernels hold a request's length, at most max_pages * P tokens, in 32 bits
bool table_fits(int max_pages, int P) { return (int64_t)max_pages * P <= INT32_MAX; }

bool cache_ok(const kvz_cache* c) {
  // a cache without unit slots (every request shorter than a page) may have no unit array
  return c && (c->units || c->num_pages == 0) && c->status && shape_ok(c->page_size, c->head_dim) &&
         c->num_kv_heads > 0 &&
         c->num_pages >= 0 && c->max_batch >= 0 && c->esc_capacity >= 0 && c->esc_cursor &&
         (c->format == KVZ_FORMAT_ESCAPE || c->format == KVZ_FORMAT_ZIPFUSION || c->format == KVZ_FORMAT_CHANNEL);
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

// ---------------------------------------------------------------- allocation-free attention
// The split partials of kvz_decode_attention_noalloc: a file-scope device array, one copy on every
// GPU the library runs on, held until the process ends. In host code its name is only a stand-in
// for the symbol, not a device address: each GPU's copy has its own address, which
// hipGetSymbolAddress gives once per device (with that device current) and which is kept here.
static __device__ __align__(256) uint8_t scratch[KVZ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`; nullptr when the runtime cannot give its address.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

size_t kvz_unit_bytes(int32_t P, int32_t D) { return shape_ok(P, D) ? kvz::unit_bytes(P, D) : 0; }
size_t kvz_unit_bytes_for(int32_t format, int32_t P, int32_t D) {
  if (!shape_ok(P, D)) return 0;
  if (format == KVZ_FORMAT_ESCAPE || format == KVZ_FORMAT_CHANNEL) return kvz::unit_bytes(P, D);
  if (format == KVZ_FORMAT_ZIPFUSION) return kvz::zf_unit_bytes(P, D);
  return 0;
}
size_t kvz_payload_bytes(int32_t P, int32_t D) { return shape_ok(P, D) ? kvz::block_bytes(P, D) : 0; }
size_t kvz_meta_bytes(int32_t P, int32_t D) { return shape_ok(P, D) ? kvz::meta_bytes(P, D) : 0; }
int32_t kvz_inline_capacity(int32_t P, int32_t D) { return shape_ok(P, D) ? kvz::inline_capacity(P, D) : 0; }

int32_t kvz_num_splits(int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t P, int32_t max_pages_per_seq,
                       int32_t pps) {
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv || !shape_ok(P, D) || max_pages_per_seq < 0) return 0;
  if (pps < -kMaxForcedRanks) return 0;
  return slot_count(B, H_q, H_kv, D, P, max_pages_per_seq, pps);
}

// workspace: per (request, query head, split) acc[D] and (m, l) as float, then one 16-byte slot
// where the split kernel records the pages per split it used. ws_bytes is 0 when the size does
// not fit in size_t (arguments validated by the caller: all positive).
static size_t ws_partial_bytes(int B, int Hq, int S, int D) { return (size_t)B * Hq * S * (D + 2) * sizeof(float); }
static size_t ws_bytes(int B, int Hq, int S, int D) {
  size_t n = (size_t)B;
  if (__builtin_mul_overflow(n, (size_t)Hq, &n) || __builtin_mul_overflow(n, (size_t)S, &n) ||
      __builtin_mul_overflow(n, (size_t)(D + 2) * sizeof(float), &n) || __builtin_add_overflow(n, (size_t)16, &n))
    return 0;
  return n;
}
static int32_t* ws_chosen(void* ws, int B, int Hq, int S, int D) {
  return reinterpret_cast<int32_t*>(static_cast<char*>(ws) + ws_partial_bytes(B, Hq, S, D));
}
static kvz::SplitPlan make_plan(int C, int S, int max_pages, bool fixed, int32_t* chosen) {
  kvz::SplitPlan p;
  p.S = S;
  p.C_lo = C;
  p.C_hi = fixed ? C : (max_pages > C ? max_pages : C);
  p.slots = 0;   // filled in by the launch from the kernel's occupancy
  p.slots_pref = 0;
  p.ranks = 0;   // the ranked schedule: set only for the kernel that implements it
  p.rank_min = 0;
  p.tpp = 1;
  p.chosen = chosen;
  return p;
}

size_t kvz_workspace_bytes(int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t P, int32_t max_pages_per_seq,
                           int32_t pps) {
  const int S = kvz_num_splits(B, H_q, H_kv, D, P, max_pages_per_seq, pps);
  return S > 0 ? ws_bytes(B, H_q, S, D) : 0;
}

int kvz_compress_pages(const kvz_cache* c, const uint16_t* k_src, const uint16_t* v_src, const int32_t* ids,
                       int32_t n, void* stream) {
  if (!cache_ok(c) || n < 0 || (n > 0 && (!k_src || !v_src || !ids))) return KVZ_ERR_INVALID_ARG;
  if (!compress_fits(c)) return KVZ_ERR_UNSUPPORTED;
  if (n == 0) return KVZ_OK;
  return kvz::launch_compress(k_src, v_src, ids, n, c->num_kv_heads, c->page_size, c->head_dim, c->num_pages,
                              c->units, c->esc_pool, c->esc_capacity, c->esc_cursor, c->status, c->format,
                              as_stream(stream));
}

int kvz_append_token(const kvz_cache* c, const uint16_t* k_new, const uint16_t* v_new, const int32_t* page_table,
                     int32_t max_pages, int32_t* seq_lens, int32_t B, void* stream) {
  if (!cache_ok(c) || B < 0 || max_pages < 0 || !c->k_tail || !c->v_tail) return KVZ_ERR_INVALID_ARG;
  if (!table_fits(max_pages, c->page_size)) return KVZ_ERR_UNSUPPORTED;
  if (B > 0 && (!k_new || !v_new || !page_table || !seq_lens)) return KVZ_ERR_INVALID_ARG;
  if (B > c->max_batch) return KVZ_ERR_INVALID_ARG;
  if (!compress_fits(c)) return KVZ_ERR_UNSUPPORTED;
  if (B == 0) return KVZ_OK;
  return kvz::launch_append(k_new, v_new, page_table, max_pages, seq_lens, B, c->num_kv_heads, c->page_size,
                            c->head_dim, c->num_pages, c->units, c->esc_pool, c->esc_capacity, c->esc_cursor,
                            c->k_tail, c->v_tail, c->status, c->format, as_stream(stream));
}

static int check_attention_shape(int B, int Hq, int Hkv, int D, int P, int max_pages) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || max_pages < 0) return KVZ_ERR_INVALID_ARG;
  if (!shape_ok(P, D) || Hq % Hkv || !table_fits(max_pages, P)) return KVZ_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return KVZ_ERR_UNSUPPORTED;
  return KVZ_OK;
}

int kvz_decode_attention_splits(const uint16_t* q, const kvz_cache* c, const int32_t* page_table, int32_t max_pages,
                                const int32_t* seq_lens, int32_t B, int32_t H_q, float sm_scale, int32_t pps,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!cache_ok(c)) return KVZ_ERR_INVALID_ARG;
  const int H = c->num_kv_heads, D = c->head_dim, P = c->page_size;
  int rc = check_attention_shape(B, H_q, H, D, P, max_pages);
  if (rc) return rc;
  if (B == 0) return KVZ_OK;
  if (!q || !page_table || !seq_lens || !workspace || !c->k_tail || !c->v_tail || pps < -kMaxForcedRanks)
    return KVZ_ERR_INVALID_ARG;
  if (B > c->max_batch) return KVZ_ERR_INVALID_ARG;
  const int C = pages_per_split(B, H_q, H, D, P, max_pages, pps);
  const int S = slot_count(B, H_q, H, D, P, max_pages, pps);
  if (ws_bytes(B, H_q, S, D) == 0) return KVZ_ERR_INVALID_ARG;
  if (workspace_bytes < ws_bytes(B, H_q, S, D)) return KVZ_ERR_WORKSPACE;
  float* ws_acc = reinterpret_cast<float*>(workspace);
  float* ws_ml = ws_acc + (size_t)B * H_q * S * D;
  const float scale = sm_scale * 1.4426950408889634f;
  kvz::SplitPlan plan = make_plan(C, S, max_pages, pps > 0, ws_chosen(workspace, B, H_q, S, D));
  // grouped queries go to the MFMA kernels at head dim 128; at head dim 64 the multi-head kernels
  // take one wave per query head (each reads its KV head's units)
  const bool gqa = H_q != H && D == 128;
  if (c->format == KVZ_FORMAT_ZIPFUSION && gqa) {
    rc = kvz::launch_attn_zf_gqa(q, c->units, c->esc_pool, c->esc_capacity, c->k_tail, c->v_tail, page_table,
                                 max_pages, seq_lens, B, H_q, H, D, P, c->num_pages, plan, scale, ws_acc, ws_ml,
                                 c->status, as_stream(stream));
  } else if (c->format == KVZ_FORMAT_ZIPFUSION) {
    rc = kvz::launch_attn_zf(q, c->units, c->esc_pool, c->esc_capacity, c->k_tail, c->v_tail, page_table, max_pages,
                             seq_lens, B, H_q, H, D, P, c->num_pages, plan, scale, ws_acc, ws_ml, c->status,
                             as_stream(stream));
  } else if (!gqa) {
    const int tpp = split_tiles(B, H_q, H, D, P, max_pages, pps);
    if (tpp > 1) {   // splits counted in tiles
      plan = make_plan(tile_split_min(B, H_q, H, D, max_pages, tpp), S, max_pages * tpp, false,
                       ws_chosen(workspace, B, H_q, S, D));
      plan.tpp = tpp;
    } else {
      plan.ranks = rank_count(B, H_q, H, max_pages, pps);
      plan.rank_min = pps < 0 ? 0 : kRankMinPages;
    }
    rc = kvz::launch_attn_mha(q, c->units, c->esc_pool, c->esc_capacity, c->esc_cursor, c->k_tail, c->v_tail,
                              page_table, max_pages, seq_lens, B, H_q, H, D, P, c->num_pages, plan, scale, ws_acc,
                              ws_ml, c->status, c->format == KVZ_FORMAT_CHANNEL, as_stream(stream));
  } else {
    rc = kvz::launch_attn_gqa(q, c->units, c->esc_pool, c->esc_capacity, c->esc_cursor, c->k_tail, c->v_tail, page_table, max_pages, seq_lens, B,
                              H_q, H, D, P, c->num_pages, plan, scale, ws_acc, ws_ml, c->status,
                              c->format == KVZ_FORMAT_CHANNEL, as_stream(stream));
  }
  return rc ? (rc == -2 ? KVZ_ERR_UNSUPPORTED : KVZ_ERR_HIP) : KVZ_OK;
}

int kvz_decode_attention_dense_splits(const uint16_t* q, const uint16_t* k_pages, const uint16_t* v_pages,
                                      int32_t num_pages, int32_t H, int32_t D, int32_t P, const int32_t* page_table,
                                      int32_t max_pages, const int32_t* seq_lens, int32_t B, int32_t H_q,
                                      float sm_scale, int32_t pps, void* workspace, size_t workspace_bytes,
                                      uint32_t* status, void* stream) {
  int rc = check_attention_shape(B, H_q, H, D, P, max_pages);
  if (rc) return rc;
  if (B == 0) return KVZ_OK;
  // pages may be absent only when there are none (every page id is then bad and skipped)
  if (!q || (num_pages > 0 && (!k_pages || !v_pages)) || !page_table || !seq_lens || !workspace || num_pages < 0 ||
      pps < -kMaxForcedRanks)
    return KVZ_ERR_INVALID_ARG;
  const int C = pages_per_split(B, H_q, H, D, P, max_pages, pps);
  const int S = slot_count(B, H_q, H, D, P, max_pages, pps);
  if (ws_bytes(B, H_q, S, D) == 0) return KVZ_ERR_INVALID_ARG;
  if (workspace_bytes < ws_bytes(B, H_q, S, D)) return KVZ_ERR_WORKSPACE;
  float* ws_acc = reinterpret_cast<float*>(workspace);
  float* ws_ml = ws_acc + (size_t)B * H_q * S * D;
  const float scale = sm_scale * 1.4426950408889634f;
  kvz::SplitPlan plan = make_plan(C, S, max_pages, pps > 0, ws_chosen(workspace, B, H_q, S, D));
  if (H_q == H || D != 128) {   // as the compressed path: grouped queries at head dim 64 one query head per wave
    plan.ranks = rank_count(B, H_q, H, max_pages, pps);   // the baseline gets the same schedule as the compressed kernel
    plan.rank_min = pps < 0 ? 0 : kRankMinPages;
    rc = kvz::launch_attn_dense_mha(q, k_pages, v_pages, page_table, max_pages, seq_lens, B, H_q, H, D, P, num_pages,
                                    plan, scale, ws_acc, ws_ml, status, as_stream(stream));
  } else {
    rc = kvz::launch_attn_dense_gqa(q, k_pages, v_pages, page_table, max_pages, seq_lens, B, H_q, H, D, P, num_pages,
                                    plan, scale, ws_acc, ws_ml, status, as_stream(stream));
  }
  return rc ? (rc == -2 ? KVZ_ERR_UNSUPPORTED : KVZ_ERR_HIP) : KVZ_OK;
}

int kvz_merge_splits(const void* workspace, size_t workspace_bytes, const int32_t* seq_lens, int32_t B, int32_t H_q,
                     int32_t H, int32_t D, int32_t P, int32_t max_pages, int32_t pps, int32_t dense, uint16_t* out,
                     float* out_f32, void* stream) {
  int rc = check_attention_shape(B, H_q, H, D, P, max_pages);
  if (rc) return rc;
  if (B == 0) return KVZ_OK;
  if (!workspace || !seq_lens || !out || pps < -kMaxForcedRanks) return KVZ_ERR_INVALID_ARG;
  const int S = slot_count(B, H_q, H, D, P, max_pages, pps);
  if (ws_bytes(B, H_q, S, D) == 0) return KVZ_ERR_INVALID_ARG;
  if (workspace_bytes < ws_bytes(B, H_q, S, D)) return KVZ_ERR_WORKSPACE;
  const float* ws_acc = reinterpret_cast<const float*>(workspace);
  const float* ws_ml = ws_acc + (size_t)B * H_q * S * D;
  rc = kvz::launch_merge(ws_acc, ws_ml, seq_lens, B, H_q, D, P, max_pages, S,
                         ws_chosen(const_cast<void*>(workspace), B, H_q, S, D), dense ? 1 : 0, out, out_f32,
                         as_stream(stream));
  return rc ? KVZ_ERR_HIP : KVZ_OK;
}

int kvz_decode_attention(const uint16_t* q, const kvz_cache* c, const int32_t* page_table, int32_t max_pages,
                         const int32_t* seq_lens, int32_t B, int32_t H_q, float sm_scale, int32_t pps,
                         uint16_t* out, float* out_f32, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cache_ok(c)) return KVZ_ERR_INVALID_ARG;
  if (B > 0 && !out) return KVZ_ERR_INVALID_ARG;
  int rc = kvz_decode_attention_splits(q, c, page_table, max_pages, seq_lens, B, H_q, sm_scale, pps, workspace,
                                       workspace_bytes, stream);
  if (rc || B == 0) return rc;
  return kvz_merge_splits(workspace, workspace_bytes, seq_lens, B, H_q, c->num_kv_heads, c->head_dim, c->page_size,
                          max_pages, pps, 0, out, out_f32, stream);
}

int kvz_decode_attention_noalloc(const uint16_t* q, const kvz_cache* c, const int32_t* page_table,
                                 int32_t max_pages, const int32_t* seq_lens, int32_t B, int32_t H_q, float sm_scale,
                                 int32_t pps, uint16_t* out, float* out_f32, void* stream) {
  if (!cache_ok(c)) return KVZ_ERR_INVALID_ARG;
  const int rc = check_attention_shape(B, H_q, c->num_kv_heads, c->head_dim, c->page_size, max_pages);
  if (rc) return rc;
  if (pps < -kMaxForcedRanks) return KVZ_ERR_INVALID_ARG;
  if (B == 0) return KVZ_OK;
  const size_t need = kvz_workspace_bytes(B, H_q, c->num_kv_heads, c->head_dim, c->page_size, max_pages, pps);
  if (need == 0) return KVZ_ERR_INVALID_ARG;
  if (need > KVZ_NOALLOC_SCRATCH_BYTES) return KVZ_ERR_SCRATCH;
  void* ws = scratch_on_current_device();
  if (!ws) return KVZ_ERR_HIP;
  return kvz_decode_attention(q, c, page_table, max_pages, seq_lens, B, H_q, sm_scale, pps, out, out_f32, ws,
                              KVZ_NOALLOC_SCRATCH_BYTES, stream);
}

int kvz_decode_attention_dense(const uint16_t* q, const uint16_t* k_pages, const uint16_t* v_pages, int32_t num_pages,
                               int32_t H, int32_t D, int32_t P, const int32_t* page_table, int32_t max_pages,
                               const int32_t* seq_lens, int32_t B, int32_t H_q, float sm_scale, int32_t pps,
                               uint16_t* out, float* out_f32, void* workspace, size_t workspace_bytes,
                               uint32_t* status, void* stream) {
  if (B > 0 && !out) {
    const int rc = check_attention_shape(B, H_q, H, D, P, max_pages);
    return rc ? rc : KVZ_ERR_INVALID_ARG;
  }
  int rc = kvz_decode_attention_dense_splits(q, k_pages, v_pages, num_pages, H, D, P, page_table, max_pages, seq_lens,
                                             B, H_q, sm_scale, pps, workspace, workspace_bytes, status, stream);
  if (rc || B == 0) return rc;
  return kvz_merge_splits(workspace, workspace_bytes, seq_lens, B, H_q, H, D, P, max_pages, pps, 1, out, out_f32,
                          stream);
}

int kvz_decompress_pages(const kvz_cache* c, const int32_t* page_ids, int32_t n, int32_t lane_map, uint16_t* k_dst,
                         uint16_t* v_dst, void* stream) {
  if (!cache_ok(c) || n < 0 || (n > 0 && (!page_ids || !k_dst || !v_dst))) return KVZ_ERR_INVALID_ARG;
  if (lane_map < 0 || lane_map > 3) return KVZ_ERR_INVALID_ARG;
  const int D = c->head_dim;
  if ((D != 64 && D != 128) || ((lane_map & 1) && D != 128)) return KVZ_ERR_UNSUPPORTED;
  if (n == 0) return KVZ_OK;
  if (c->format == KVZ_FORMAT_ZIPFUSION) {
    if (lane_map > 1) return KVZ_ERR_UNSUPPORTED;   // the format has no escape routes
    const int rc = kvz::launch_decompress_zf(c->units, c->esc_pool, c->esc_capacity, page_ids, n, c->num_kv_heads,
                                             c->page_size, D, c->num_pages, lane_map, k_dst, v_dst, c->status,
                                             as_stream(stream));
    return rc == -2 ? KVZ_ERR_UNSUPPORTED : (rc ? KVZ_ERR_HIP : KVZ_OK);
  }
  const int rc = kvz::launch_decompress(c->units, c->esc_pool, c->esc_capacity, page_ids, n, c->num_kv_heads, c->page_size, D,
                                        c->num_pages, lane_map, k_dst, v_dst, c->status,
                                        c->format == KVZ_FORMAT_CHANNEL, as_stream(stream));
  return rc == -2 ? KVZ_ERR_UNSUPPORTED : (rc ? KVZ_ERR_HIP : KVZ_OK);
}

int kvz_compact_pool(const kvz_cache* c, const int32_t* page_ids, int32_t n, uint16_t* new_pool,
                     int64_t new_capacity, uint64_t* new_cursor, void* stream) {
  if (!cache_ok(c) || n < 0 || new_capacity < 0 || !new_cursor) return KVZ_ERR_INVALID_ARG;
  if (n > 0 && (!page_ids || !new_pool || !c->esc_pool)) return KVZ_ERR_INVALID_ARG;
  if (n == 0) return KVZ_OK;
  const int rc = kvz::launch_compact_pool(c->units, c->esc_pool, c->esc_capacity, page_ids, n, c->num_kv_heads,
                                          c->page_size, c->head_dim, c->num_pages, c->format, new_pool, new_capacity,
                                          new_cursor, c->status, as_stream(stream));
  return rc ? KVZ_ERR_HIP : KVZ_OK;
}

const char* kvz_strerror(int code) {
  switch (code) {
    case KVZ_OK: return "ok";
    case KVZ_ERR_INVALID_ARG: return "invalid argument";
    case KVZ_ERR_UNSUPPORTED: return "unsupported shape";
    case KVZ_ERR_WORKSPACE: return "workspace too small";
    case KVZ_ERR_HIP: return "HIP runtime error";
    case KVZ_ERR_SCRATCH: return "call needs more scratch than the library's own array holds";
    default: return "unknown error";
  }
}

}  // extern "C"
