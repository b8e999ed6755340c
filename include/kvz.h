/*
 * kvz — single-token decode attention over a paged BF16 KV cache kept in a lossless
 * compressed form, for AMD Instinct MI355X (gfx950). C ABI.
 *
 * The method (ZipFusion: Fusing Lossless KV Decompression with Attention for Efficient LLM
 * Decoding, paperlayer.ai summary of arXiv 2610.33719v1):
 *   - the cache format is lossless: every BF16 bit pattern comes back (§II.A "KV Cache and
 *     BF16"; §III.B "Lossless KV Cache Format");
 *   - attention reads the compressed blocks and rebuilds each value in registers with plain
 *     bit operations, with no separate decompression pass and no uncompressed copy in device
 *     memory (§III.C "Attention over the Compressed KV Cache");
 *   - partially filled pages stay uncompressed so decoding can append to them, and a page is
 *     compressed once it is full (§III.D "KV Cache Management and Scheduling");
 *   - split results are merged by a second reduction and that merge is part of attention's
 *     cost (§IV.B "Attention Kernel Performance").
 *
 * Format (this library's own layout). P = page size in tokens (multiple of 16), D = head
 * dimension (multiple of 64), P * D at most 65536 (a storage position fits in 16 bits),
 * G = D / 64, H = number of KV heads. The size functions return 0 for other shapes.
 *   group     the 64 values of one token row of one head, dims [64g, 64g + 64)
 *   sm byte   (sign << 7) | 7-bit mantissa, kept for every value
 *   base      per group: the group exponent with the most group exponents in [base, base+14],
 *             the smallest such exponent on ties
 *   offset    4 bits: exponent - base when 0..14, else 15 = escape; the value's raw 16 bits
 *             then sit in the block's escape list
 *   tile      16 consecutive tokens of a page; storage position inside a tile is
 *             tok*D + d for K (token-major) and d*16 + tok for V (dim-major)
 *   block     one (page, head, K or V): per tile, 16*D sm bytes in storage order, then 2*D
 *             little-endian u32 offset words; word w holds position 8w+2k in bits 4k..4k+3
 *             and position 8w+2k+1 in bits 16+4k..16+4k+3 (k = 0..3)
 *   escapes   a block's escaped values, in storage order
 *   unit      one (page, head), kvz_unit_bytes(P, D) bytes at offset (page*H + head) * that:
 *             meta region of kvz_meta_bytes(P, D) bytes, then the K block, then the V block
 *   meta      [0, P*G)         K bases, byte tile*16*G + g*16 + tok
 *             [P*G, 2*P*G)     V bases, same order
 *             [2PG, 2PG+4)     u32 number of K escapes
 *             [2PG+4, 2PG+8)   u32 number of V escapes
 *             [2PG+8, 2PG+16)  u64 offset (in u16 elements) of the unit's escapes in the pool,
 *                              or all ones when they are inline
 *             [2PG+16, end)    inline escapes, K's then V's, when all of them fit
 *                              (kvz_inline_capacity): one u32 each, the raw BF16 value in
 *                              bits 0..15 and its storage position in its block in bits
 *                              16..31; unused bytes are zero
 *             the meta region is 2PG+16 bytes rounded up to a multiple of 128
 *   pool      u16 raw values only: a unit's K escapes then its V escapes, contiguous
 *   tail      per request row r and head h, P raw BF16 rows [P][D] (token-major, K and V
 *             alike) holding the L mod P newest tokens
 *
 * Second format, kvz_cache.format = KVZ_FORMAT_ZIPFUSION: ZipFusion's own block format
 * (§III.B), for comparison with the pages' design; multi-head and grouped-query attention.
 *   block     512 consecutive storage positions of a tile (same storage order as above: K
 *             token-major, V dim-major); compressed when every exponent lies in [b, b+15],
 *             b = the block's smallest exponent rounded down to even, else kept raw
 *   value     low byte (lowest exponent bit + 7 mantissa bits) and a 4-bit code
 *             sign << 3 | (e/2 - b/2); compressed block = 512 low bytes then 256 code bytes
 *             (even position in the low nibble), 768 bytes
 *   unit      kvz_unit_bytes_for(KVZ_FORMAT_ZIPFUSION, P, D) bytes: block bytes (b/2, or 0xFF =
 *             raw) for K's blocks of every tile then V's, padded to 8 bytes; u64 pool offset (u16
 *             elements) of the unit's raw blocks, all ones if none; zero padding to a multiple of
 *             128; then one 768-byte slot per block in the same order (zero for a raw block)
 *   pool      esc_pool holds raw blocks, 512 values each, a unit's raw blocks contiguous in
 *             block order; esc_cursor must start at a multiple of 8
 *
 * Third format, kvz_cache.format = KVZ_FORMAT_CHANNEL: the first format with channel groups
 * (§III.B fixes a block's exponent range, not which values share a base). A group is the 16
 * tokens of one tile over 4 adjacent dims [4j, 4j+4), still 64 values, so units, pool and sizes
 * are those of the first format (kvz_unit_bytes); only the base table changes: the base of tile
 * t's group j is byte t*16G + j of the K (or V) base bytes. Channels carry their own scales, so
 * these groups escape less often (about a third as often on K with outlier channels). Head dims
 * 64 and 128 for attention; compression and appends use the workgroup compressor.
 *
 * Conventions for every entry point:
 *   - pointers are device pointers unless marked (host); the caller owns all memory;
 *   - calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL = the default
 *     stream); the library never allocates device memory and never synchronises;
 *   - a negative return value means nothing was enqueued; see kvz_strerror;
 *   - device-side conditions set sticky bits in *status with atomic OR and leave the
 *     affected outputs unspecified: KVZ_STATUS_* below;
 *   - calls on different streams must not write the same memory.
 */
#ifndef KVZ_H
#define KVZ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KVZ_OK = 0,
  KVZ_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad stride */
  KVZ_ERR_UNSUPPORTED = -2, /* shape outside what the kernels handle (see each call) */
  KVZ_ERR_WORKSPACE = -3,   /* workspace smaller than kvz_workspace_bytes(...) */
  KVZ_ERR_HIP = -4,         /* a HIP runtime call failed */
  KVZ_ERR_SCRATCH = -5      /* kvz_decode_attention_noalloc: the call needs more than
                               KVZ_NOALLOC_SCRATCH_BYTES of scratch */
};

enum {
  KVZ_FORMAT_ESCAPE = 0,     /* exponent offsets with escapes (the format described above) */
  KVZ_FORMAT_ZIPFUSION = 1,  /* ZipFusion's block format (see above) */
  KVZ_FORMAT_CHANNEL = 2     /* the first format with channel groups (see above) */
};

enum {
  KVZ_STATUS_ESC_POOL_FULL = 1u,  /* a unit's escapes did not fit the pool; its escaped
                                     values decode to unspecified values */
  KVZ_STATUS_BAD_PAGE_ID = 2u,    /* a page id outside [0, num_pages) was met and skipped */
  KVZ_STATUS_SEQ_TOO_LONG = 4u    /* seq_len > max_pages_per_seq * P (clamped) */
};

/* Host-side description of a compressed cache; read at call time, not kept. */
typedef struct kvz_cache {
  int32_t page_size;     /* P: multiple of 16 */
  int32_t num_kv_heads;  /* H */
  int32_t head_dim;      /* D: multiple of 64 */
  int32_t num_pages;     /* unit slots per head */
  int32_t max_batch;     /* tail rows */
  int32_t format;        /* KVZ_FORMAT_* of the units and the pool */
  uint8_t* units;        /* [num_pages][H][kvz_unit_bytes(P, D)], 256-byte aligned; may be
                            null when num_pages is 0 (tails only) */
  uint16_t* esc_pool;    /* escape pool, esc_capacity u16 elements */
  int64_t esc_capacity;
  uint64_t* esc_cursor;  /* [1] u16 elements of the pool in use; bumped by the library */
  uint16_t* k_tail;      /* [max_batch][H][P][D] raw BF16 */
  uint16_t* v_tail;      /* [max_batch][H][P][D] raw BF16 */
  uint32_t* status;      /* [1] sticky KVZ_STATUS_* bits */
} kvz_cache;

/* Sizes of the format (host functions, no device work; 0 for an unsupported shape). Every value
 * keeps 12 bits (sign/mantissa byte and offset nibble, §III.B: the retained bits and a small code
 * per value), so
 *   kvz_payload_bytes   one block's sm bytes and offset words: 1.5 * P * D
 *   kvz_meta_bytes      the unit's meta region (bases, header, inline escapes)
 *   kvz_unit_bytes      kvz_meta_bytes + 2 * kvz_payload_bytes (meta, then the K and V blocks)
 *   kvz_inline_capacity escapes a unit's meta region holds inline */
size_t kvz_payload_bytes(int32_t P, int32_t D);
size_t kvz_unit_bytes(int32_t P, int32_t D);
/* unit size in the given format (0 for an unsupported shape or format) */
size_t kvz_unit_bytes_for(int32_t format, int32_t P, int32_t D);
size_t kvz_meta_bytes(int32_t P, int32_t D);
int32_t kvz_inline_capacity(int32_t P, int32_t D);

/* Bytes of scratch kvz_decode_attention / kvz_decode_attention_dense need: split partials
 * (acc[D], m, l) in float for every (request, query head, split slot), then 16 bytes where the
 * split kernel records, for the merge, the plan pages per split it used (or minus its chunks per
 * row, below) and the plan pages per page of the table (int32 each). Its content needs no
 * initialisation. A plan page is a page of the table, except where the multi-head kernel over
 * the compressed cache (KVZ_FORMAT_ESCAPE, KVZ_FORMAT_CHANNEL; not grouped queries at head dim
 * 128) counts its splits in 16-token tiles: with P > 16, pages_per_split = 0, and fewer than
 * 2048 pages over the batch's (request, query head) rows at the table's full width, a plan page
 * is a tile (P / 16 to a page), splits may start and end inside a unit, and the smallest split
 * is the fewest tiles whose splits at full width come to at most 2048 (a split that starts
 * inside a unit first counts the escapes of the unit's earlier tiles, which locate its own).
 *   pages_per_split > 0  fixes the pages per split.
 *   pages_per_split = 0  lets the kernels choose per call from the sequence lengths: the
 *                        smallest split, no smaller than a bound the library sets from the
 *                        shapes, whose splits over the whole batch fit the waves the kernel
 *                        keeps resident, so that batches of uneven lengths fill the GPU in one
 *                        pass (the resident waves come from the runtime's occupancy query,
 *                        made on the host once per device and kernel at the first call). The
 *                        multi-head kernels (compressed and uncompressed) instead use a
 *                        ranked schedule when the call's lengths are nearly even (the longest
 *                        at most 5/4 of the mean) and make its chunks large (on average at
 *                        least 5 pages): each row is cut into 2R chunks, R = max(1, the
 *                        kernel's resident waves / (B H)), at most max(1, 4096 / (B H)); the
 *                        first R take 80% of the request's pages in equal parts and run first,
 *                        the last R take the rest in shrinking parts, so that the waves, whose
 *                        speeds differ with their age on the SIMD, end together. The workspace
 *                        holds slots for those chunks only when requests as long as the page
 *                        table is wide could make big chunks of 2.5 pages or more (R counted
 *                        from 4096 waves); otherwise these calls take the split schedule.
 *   pages_per_split < 0  asks the multi-head kernels for the ranked schedule with
 *                        R = -pages_per_split (at most 4096); the grouped-query kernels then
 *                        choose as with 0.
 * The same value must be passed to the attention call. Returns 0 when B = 0 (an attention call
 * over an empty batch reads no workspace), for arguments the attention calls reject (B < 0, H_q
 * or H_kv not positive, H_q not a multiple of H_kv, an unsupported P or D, max_pages_per_seq < 0,
 * pages_per_split < -4096), and when the size does not fit in size_t, which the attention calls
 * reject with KVZ_ERR_INVALID_ARG. */
size_t kvz_workspace_bytes(int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t P,
                           int32_t max_pages_per_seq, int32_t pages_per_split);

/* Split slots per (request, query head) in the workspace: the most splits an attention call
 * with these arguments can use (host function); 0 for B = 0 and for rejected arguments, as
 * kvz_workspace_bytes. */
int32_t kvz_num_splits(int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t P,
                       int32_t max_pages_per_seq, int32_t pages_per_split);

/* Compresses n full dense pages into units (the format above; §III.B, §III.D: a page is
 * encoded once it is full).
 *   k_src, v_src   [n][H][P][D] raw BF16, token-major
 *   dst_page_ids   [n] unit slots to write, each in [0, num_pages)
 * Escapes that do not fit inline are appended to the pool at *esc_cursor (bumped atomically,
 * so their place in the pool depends on scheduling; everything else is deterministic).
 * Supported: P * D up to 65536 (the format's limit) for the first format at D = 64 or 128,
 * up to 32768 otherwise (the block format, channel groups, other head dims): a unit's values
 * are staged in on-chip memory. Errors: KVZ_ERR_INVALID_ARG, KVZ_ERR_UNSUPPORTED. Device status:
 * ESC_POOL_FULL, BAD_PAGE_ID. */
int kvz_compress_pages(const kvz_cache* cache, const uint16_t* k_src, const uint16_t* v_src,
                       const int32_t* dst_page_ids, int32_t n, void* stream);

/* Appends one token to each of B requests (§III.D: decoding appends to the uncompressed
 * partial page). For request row r with L = seq_lens[r]: writes k_new[r], v_new[r] into tail
 * row L mod P of row r; when that fills the tail (L mod P == P-1) the tail is compressed into
 * unit page_table[r][L / P] (which the caller has set to a free slot); then seq_lens[r] = L+1.
 *   k_new, v_new   [B][H][D] raw BF16
 *   page_table     [B][max_pages_per_seq]
 *   seq_lens       [B], updated on the device
 * B must not exceed max_batch; max_pages_per_seq * P must fit in int32 (a request's length is
 * held in 32 bits) and P * D within the limits of kvz_compress_pages, else KVZ_ERR_UNSUPPORTED. Errors: KVZ_ERR_INVALID_ARG, KVZ_ERR_UNSUPPORTED.
 * Device status: ESC_POOL_FULL, BAD_PAGE_ID, SEQ_TOO_LONG (no write). */
int kvz_append_token(const kvz_cache* cache, const uint16_t* k_new, const uint16_t* v_new,
                     const int32_t* page_table, int32_t max_pages_per_seq, int32_t* seq_lens,
                     int32_t B, void* stream);

/* Decode attention over the compressed cache (§III.C: values rebuilt in registers inside the
 * kernel; §IV.B: split partials merged by a second kernel).
 *   q            [B][H_q][D] BF16; query head h reads KV head h / (H_q / H)
 *   page_table   [B][max_pages_per_seq]; entries i < seq_lens[r] / P are units
 *   seq_lens     [B] tokens per request: full pages, then seq_lens[r] mod P tail rows of row r
 *   out          [B][H_q][D] BF16 (round to nearest even); a request with no token gets zeros
 *   out_f32      nullable [B][H_q][D] float, the same result before rounding
 *   workspace    >= kvz_workspace_bytes(B, H_q, H, D, P, max_pages_per_seq, pages_per_split)
 * Supported: D in {64, 128}, any H_q multiple of H. Grouped queries (H_q > H) at D = 128: a wave
 * takes up to 8 query heads of one KV head; with up to 16, or 25 to 32, query heads per KV head a
 * unit's waves share one workgroup, other group sizes spread them over workgroups that may each
 * read the unit. At D = 64 each query head has its own wave, which reads its KV head's units;
 * max_pages_per_seq * P within int32 (as for kvz_append_token).
 * Errors: KVZ_ERR_INVALID_ARG, KVZ_ERR_UNSUPPORTED, KVZ_ERR_WORKSPACE. Device status:
 * BAD_PAGE_ID, SEQ_TOO_LONG. */
int kvz_decode_attention(const uint16_t* q, const kvz_cache* cache, const int32_t* page_table,
                         int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t B,
                         int32_t H_q, float sm_scale, int32_t pages_per_split, uint16_t* out,
                         float* out_f32, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the scratch array the library holds on each GPU for kvz_decode_attention_noalloc. */
#define KVZ_NOALLOC_SCRATCH_BYTES (32u << 20)

/* kvz_decode_attention without the workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The workspace this call needs (kvz_workspace_bytes of its arguments: the split partials and the
 * slot where the split kernel records its split size) is a scratch array of
 * KVZ_NOALLOC_SCRATCH_BYTES in device memory that the library holds on every GPU it runs on until
 * the process ends. The call allocates nothing and calls no allocating routine; the caller still
 * passes every input and output. All calls on one GPU share that GPU's array, which keeps the last
 * call's contents (a call needs none of them: it writes every partial it reads). Calls that
 * overlap on one GPU (on different streams or from different host threads) race on the array and
 * give unspecified results; calls on one stream are ordered and safe.
 * Arguments, results, errors and status as kvz_decode_attention, and KVZ_ERR_SCRATCH (nothing
 * enqueued) when kvz_workspace_bytes(B, H_q, H, D, P, max_pages_per_seq, pages_per_split) exceeds
 * KVZ_NOALLOC_SCRATCH_BYTES; KVZ_ERR_HIP when the runtime cannot give the array's address. */
int kvz_decode_attention_noalloc(const uint16_t* q, const kvz_cache* cache, const int32_t* page_table,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t B, int32_t H_q,
                                 float sm_scale, int32_t pages_per_split, uint16_t* out, float* out_f32,
                                 void* stream);

/* The same attention over an uncompressed paged cache: the baseline the compressed path is
 * measured against (the pages compare with production FlashInfer, §IV.B).
 *   k_pages, v_pages  [num_pages][H][P][D] raw BF16, token-major (may be null when num_pages is 0)
 *   page_table        [B][max_pages_per_seq]; the first ceil(seq_lens[r] / P) entries are used
 *   status            nullable [1] sticky bits (BAD_PAGE_ID, SEQ_TOO_LONG)
 * Other arguments as kvz_decode_attention. Supported: D in {64, 128}, any H_q multiple of H. */
int kvz_decode_attention_dense(const uint16_t* q, const uint16_t* k_pages,
                               const uint16_t* v_pages, int32_t num_pages, int32_t H,
                               int32_t D, int32_t P, const int32_t* page_table,
                               int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t B,
                               int32_t H_q, float sm_scale, int32_t pages_per_split,
                               uint16_t* out, float* out_f32, void* workspace,
                               size_t workspace_bytes, uint32_t* status, void* stream);

/* The two phases of kvz_decode_attention / kvz_decode_attention_dense as separate calls, for
 * callers that schedule them apart (and for timing the split kernel alone).
 *   kvz_decode_attention_splits        the compressed split kernel: partials into workspace
 *   kvz_decode_attention_dense_splits  the dense split kernel: partials into workspace
 *   kvz_merge_splits                   merges the partials of either into out / out_f32;
 *                                      dense = 1 when they came from the dense kernel
 * Arguments mean what they mean in the one-call forms; B, H_q, H, D, P, max_pages_per_seq and
 * pages_per_split must be the same in both phases, and the workspace must not change between
 * them (the merge reads the split size the split kernel recorded there). Errors and status as
 * the one-call forms. */
int kvz_decode_attention_splits(const uint16_t* q, const kvz_cache* cache, const int32_t* page_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t B,
                                int32_t H_q, float sm_scale, int32_t pages_per_split,
                                void* workspace, size_t workspace_bytes, void* stream);
int kvz_decode_attention_dense_splits(const uint16_t* q, const uint16_t* k_pages,
                                      const uint16_t* v_pages, int32_t num_pages, int32_t H,
                                      int32_t D, int32_t P, const int32_t* page_table,
                                      int32_t max_pages_per_seq, const int32_t* seq_lens,
                                      int32_t B, int32_t H_q, float sm_scale,
                                      int32_t pages_per_split, void* workspace,
                                      size_t workspace_bytes, uint32_t* status, void* stream);
int kvz_merge_splits(const void* workspace, size_t workspace_bytes, const int32_t* seq_lens,
                     int32_t B, int32_t H_q, int32_t H, int32_t D, int32_t P,
                     int32_t max_pages_per_seq, int32_t pages_per_split, int32_t dense,
                     uint16_t* out, float* out_f32, void* stream);

/* Test entry point: runs the attention kernels' own in-register decode on n units and writes
 * the rebuilt values, so that decode can be compared bit for bit (§II.A, §III.B: every BF16 bit
 * pattern comes back; §III.C: values rebuilt with bit operations inside the kernel).
 *   page_ids      [n]
 *   lane_map      which of the kernels' decode routes runs:
 *                 0  multi-head lane layout; escapes as the main loops and the per-unit path
 *                    after them patch them (inline list, or a pool list staged whole)
 *                 1  the same route with the grouped-query kernel's K layout (D = 128 only)
 *                 2  multi-head lane layout through the pool-capable loop's route (a pool
 *                    unit's escape windows staged with the payload, every offset word patched
 *                    from them)
 *                 3  the route of 2 with the grouped-query kernel's K layout (D = 128 only)
 *   k_dst, v_dst  [n][H][P][D] raw BF16, token-major
 * Supported: D in {64, 128}; lane maps 0 and 1 only for KVZ_FORMAT_ZIPFUSION (it has no
 * escapes). Errors: KVZ_ERR_INVALID_ARG (lane_map outside 0..3), KVZ_ERR_UNSUPPORTED. Device
 * status: BAD_PAGE_ID. */
int kvz_decompress_pages(const kvz_cache* cache, const int32_t* page_ids, int32_t n,
                         int32_t lane_map, uint16_t* k_dst, uint16_t* v_dst, void* stream);

/* Moves the pool data of the listed units (their escape lists, or raw blocks in the ZipFusion
 * format) into a new pool and points the units at it, so that the pool space of units that are
 * no longer used can be released: the caller then installs new_pool / new_capacity /
 * new_cursor in its kvz_cache and frees the old pool (§III.D: memory given back for reuse).
 *   page_ids      [n] distinct unit slots to keep (every head of each); units not listed keep
 *                 pointing into the old pool and must not be used with the new one
 *   new_pool      u16 [new_capacity], must not overlap the old pool
 *   new_cursor    [1] u16 elements of new_pool in use, bumped atomically (0 for an empty pool;
 *                 a multiple of 8 for the ZipFusion format)
 * Placement in the new pool depends on scheduling; contents and results do not. Must not run
 * concurrently with other calls on the same cache. Errors: KVZ_ERR_INVALID_ARG. Device status:
 * BAD_PAGE_ID, ESC_POOL_FULL (new pool too small, or a header pointing outside the old pool:
 * that unit's pool data is dropped, as when compression finds the pool full). */
int kvz_compact_pool(const kvz_cache* cache, const int32_t* page_ids, int32_t n, uint16_t* new_pool,
                     int64_t new_capacity, uint64_t* new_cursor, void* stream);

const char* kvz_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* KVZ_H */
