/*
 * kvz_bench — measurement kernels that sit beside libkvz (built as libkvz_bench.so). Not part of
 * the decode-attention path: they give the references its kernels are measured against.
 *
 * Decode attention re-reads every cached key and value at every step and is bound by memory
 * bandwidth (ZipFusion summary, §IV.B "Attention Kernel Performance"; the FlashSVD review's
 * background on decode attention). The attention kernels' rate is therefore compared with the
 * rate at which this device can stream the same bytes in the same pattern.
 *
 * Conventions as in kvz.h: device pointers, caller-owned memory, asynchronous on `stream`,
 * nothing allocated, negative return = nothing enqueued (KVZ_ERR_* values of kvz.h).
 */
#ifndef KVZ_BENCH_H
#define KVZ_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming-read ceiling of the compressed attention kernels. Reads exactly the unit bytes an
 * attention call over the escape-format cache reads: for every request r and KV head h, the
 * units of the full pages i < seq_lens[r] / P, found through page_table[r][i], and those page
 * table entries; nothing else. The access pattern is theirs: one wave walks a chunk of one
 * (request, head) row's pages in page-table order, each unit read whole with 16-byte
 * non-temporal loads, the next unit's loads issued before the current unit's data is used.
 * The data is only folded into one word per lane, written to sink.
 *   units            [num_pages][H][unit_bytes] (kvz_unit_bytes), read only
 *   unit_bytes       a multiple of 16, at most 16384
 *   page_table       [B][max_pages_per_seq]; entries outside [0, num_pages) are read as 0
 *   chunks_per_row   waves per (request, head) row: B * H * chunks_per_row waves in all, each
 *                    over ceil(pages / chunks_per_row) consecutive pages of its row
 *   sink             [B * H * chunks_per_row * 64] u32, written
 * Bytes read per call: (sum over r of seq_lens[r] / P) * H * (unit_bytes + 4).
 * Errors: KVZ_ERR_INVALID_ARG, KVZ_ERR_HIP. */
int kvzb_read_units(const uint8_t* units, int32_t num_pages, size_t unit_bytes, const int32_t* page_table,
                    int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t B, int32_t H, int32_t P,
                    int32_t chunks_per_row, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVZ_BENCH_H */
