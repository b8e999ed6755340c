// kvz_compress_pages and kvz_append_token kernels, for the three cache formats (0: exponent
// offsets with escapes, compress.hpp; 1: ZipFusion blocks, zf.hpp; 2: format 0 with channel
// groups, compress.hpp). Units of format 0 with head dim 64 or 128 are compressed one wave per
// unit (compress_wave.hpp); the workgroup compressor serves the other head dims and formats.
#include "compress.hpp"
#include "compress_wave.hpp"
#include "zf.hpp"

namespace kvz {

// one unit of either format; smem holds 2*P*D u16 of staged values, then the per-group (or
// per-block) bytes
__device__ __forceinline__ void compress_any(const uint16_t* k, const uint16_t* v, int P, int D, uint8_t* units,
                                             int pid, int H, int h, uint16_t* pool, int64_t pool_cap,
                                             uint64_t* cursor, uint32_t* status, uint8_t* smem, CompressShared& sh,
                                             int format) {
  const size_t blk = (size_t)P * D;
  uint16_t* sx = reinterpret_cast<uint16_t*>(smem);
  if (format == 1) {
    const int nb = zf_nblocks(P, D);
    compress_unit_zf(k, v, P, D, units + ((size_t)pid * H + h) * zf_unit_bytes(P, D), pool, pool_cap, cursor, status,
                     sx, smem + 4 * blk, reinterpret_cast<uint16_t*>(smem + 4 * blk + (nb + 1) / 2 * 2), sh);
  } else if (format == 2) {
    uint8_t* unit = units + ((size_t)pid * H + h) * unit_bytes(P, D);
    if (D == 128) compress_unit<128, true>(k, v, P, D, unit, pool, pool_cap, cursor, status, sx, smem + 4 * blk, sh);
    else if (D == 64) compress_unit<64, true>(k, v, P, D, unit, pool, pool_cap, cursor, status, sx, smem + 4 * blk, sh);
    else compress_unit<0, true>(k, v, P, D, unit, pool, pool_cap, cursor, status, sx, smem + 4 * blk, sh);
  } else {
    uint8_t* unit = units + ((size_t)pid * H + h) * unit_bytes(P, D);
    if (D == 128) compress_unit<128>(k, v, P, D, unit, pool, pool_cap, cursor, status, sx, smem + 4 * blk, sh);
    else if (D == 64) compress_unit<64>(k, v, P, D, unit, pool, pool_cap, cursor, status, sx, smem + 4 * blk, sh);
    else compress_unit<0>(k, v, P, D, unit, pool, pool_cap, cursor, status, sx, smem + 4 * blk, sh);
  }
}

__global__ __launch_bounds__(kCompressThreads) void compress_pages_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, const int32_t* __restrict__ dst_ids,
    int H, int P, int D, int num_pages, uint8_t* __restrict__ units, uint16_t* __restrict__ pool, int64_t pool_cap,
    uint64_t* __restrict__ cursor, uint32_t* __restrict__ status, int format) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ CompressShared sh;
  const int i = blockIdx.x / H, h = blockIdx.x % H;
  const int pid = dst_ids[i];
  if (pid < 0 || pid >= num_pages) {
    if (threadIdx.x == 0) atomicOr(status, kStatusBadPage);
    return;
  }
  const size_t blk = (size_t)P * D;
  compress_any(k_src + ((size_t)i * H + h) * blk, v_src + ((size_t)i * H + h) * blk, P, D, units, pid, H, h, pool,
               pool_cap, cursor, status, smem, sh, format);
}

// One workgroup per (request, head): write the new row into the tail; if that fills the tail,
// compress it into the unit named by the page table.
__global__ __launch_bounds__(kCompressThreads) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, const int32_t* __restrict__ page_table,
    int max_pages, const int32_t* __restrict__ seq_lens, int H, int P, int D, int num_pages,
    uint8_t* __restrict__ units, uint16_t* __restrict__ pool, int64_t pool_cap, uint64_t* __restrict__ cursor,
    uint16_t* __restrict__ k_tail, uint16_t* __restrict__ v_tail, uint32_t* __restrict__ status, int format) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ CompressShared sh;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  const int L = seq_lens[r];
  if (L < 0 || L >= max_pages * P) {
    if (threadIdx.x == 0 && h == 0) atomicOr(status, kStatusSeqTooLong);
    return;
  }
  const int slot = L % P;
  const size_t blk = (size_t)P * D;
  uint16_t* tk = k_tail + ((size_t)r * H + h) * blk;
  uint16_t* tv = v_tail + ((size_t)r * H + h) * blk;
  const uint16_t* kn = k_new + ((size_t)r * H + h) * D;
  const uint16_t* vn = v_new + ((size_t)r * H + h) * D;
  for (int d = threadIdx.x; d < D; d += kCompressThreads) {
    tk[(size_t)slot * D + d] = kn[d];
    tv[(size_t)slot * D + d] = vn[d];
  }
  if (slot != P - 1) return;
  __threadfence_block();
  __syncthreads();
  const int pid = page_table[(size_t)r * max_pages + L / P];
  if (pid < 0 || pid >= num_pages) {
    if (threadIdx.x == 0) atomicOr(status, kStatusBadPage);
    return;
  }
  compress_any(tk, tv, P, D, units, pid, H, h, pool, pool_cap, cursor, status, smem, sh, format);
}

// One wave per unit (first format, head dim D = 64 or 128).
template <int D>
__global__ __launch_bounds__(64) void compress_pages_wave_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, const int32_t* __restrict__ dst_ids, int H,
    int P, int num_pages, uint8_t* __restrict__ units, uint16_t* __restrict__ pool, int64_t pool_cap,
    uint64_t* __restrict__ cursor, uint32_t* __restrict__ status) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int i = blockIdx.x / H, h = blockIdx.x % H;
  const int pid = dst_ids[i];
  if (pid < 0 || pid >= num_pages) {
    if (threadIdx.x == 0) atomicOr(status, kStatusBadPage);
    return;
  }
  const size_t blk = (size_t)P * D;
  compress_unit_wave<D>(k_src + ((size_t)i * H + h) * blk, v_src + ((size_t)i * H + h) * blk, P,
                        units + ((size_t)pid * H + h) * unit_bytes(P, D), pool, pool_cap, cursor, status, smem,
                        (int)threadIdx.x);
}

// One wave per (request, head): the new row into the tail; a tail it fills is compressed by the
// same wave.
template <int D>
__global__ __launch_bounds__(64) void append_wave_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, const int32_t* __restrict__ page_table,
    int max_pages, const int32_t* __restrict__ seq_lens, int H, int P, int num_pages, uint8_t* __restrict__ units,
    uint16_t* __restrict__ pool, int64_t pool_cap, uint64_t* __restrict__ cursor, uint16_t* __restrict__ k_tail,
    uint16_t* __restrict__ v_tail, uint32_t* __restrict__ status) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  const int L = seq_lens[r];
  if (L < 0 || L >= max_pages * P) {
    if (threadIdx.x == 0 && h == 0) atomicOr(status, kStatusSeqTooLong);
    return;
  }
  const int slot = L % P;
  const size_t blk = (size_t)P * D;
  uint16_t* tk = k_tail + ((size_t)r * H + h) * blk;
  uint16_t* tv = v_tail + ((size_t)r * H + h) * blk;
  const uint16_t* kn = k_new + ((size_t)r * H + h) * D;
  const uint16_t* vn = v_new + ((size_t)r * H + h) * D;
  for (int d = threadIdx.x; d < D; d += 64) {
    tk[(size_t)slot * D + d] = kn[d];
    tv[(size_t)slot * D + d] = vn[d];
  }
  if (slot != P - 1) return;
  __threadfence_block();
  __syncthreads();
  const int pid = page_table[(size_t)r * max_pages + L / P];
  if (pid < 0 || pid >= num_pages) {
    if (threadIdx.x == 0) atomicOr(status, kStatusBadPage);
    return;
  }
  compress_unit_wave<D>(tk, tv, P, units + ((size_t)pid * H + h) * unit_bytes(P, D), pool, pool_cap, cursor, status,
                        smem, (int)threadIdx.x);
}

__global__ void bump_lens_kernel(int32_t* __restrict__ seq_lens, int B, int limit) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < B) {
    const int L = seq_lens[r];
    if (L >= 0 && L < limit) seq_lens[r] = L + 1;
  }
}

static size_t compress_smem(int P, int D) { return 4 * (size_t)P * D + 2 * (size_t)P * (D / kGroup); }

// Dynamic LDS beyond 64 KB must be opted into per kernel. Below that nothing is called, so that
// the usual page sizes launch with stream operations only (a caller may capture them in a graph).
static bool allow_smem(const void* kernel, size_t smem) {
  if (smem <= 65536) return true;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) == hipSuccess;
}

int launch_compress(const uint16_t* k_src, const uint16_t* v_src, const int32_t* ids, int n, int H, int P, int D,
                    int num_pages, uint8_t* units, uint16_t* pool, int64_t pool_cap, uint64_t* cursor,
                    uint32_t* status, int format, hipStream_t stream) {
  if (format == 0 && (D == 64 || D == 128)) {
    const size_t lds = compress_wave_lds(P, D);
    const void* kern = D == 128 ? (const void*)compress_pages_wave_kernel<128> : (const void*)compress_pages_wave_kernel<64>;
    if (!allow_smem(kern, lds)) return -4;
    if (D == 128)
      hipLaunchKernelGGL(compress_pages_wave_kernel<128>, dim3((unsigned)n * H), dim3(64), lds, stream, k_src, v_src, ids,
                         H, P, num_pages, units, pool, pool_cap, cursor, status);
    else
      hipLaunchKernelGGL(compress_pages_wave_kernel<64>, dim3((unsigned)n * H), dim3(64), lds, stream, k_src, v_src, ids,
                         H, P, num_pages, units, pool, pool_cap, cursor, status);
    return hipGetLastError() == hipSuccess ? 0 : -4;
  }
  const size_t smem = compress_smem(P, D);
  if (!allow_smem((const void*)compress_pages_kernel, smem)) return -4;
  hipLaunchKernelGGL(compress_pages_kernel, dim3((unsigned)n * H), dim3(kCompressThreads), smem, stream, k_src,
                     v_src, ids, H, P, D, num_pages, units, pool, pool_cap, cursor, status, format);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* page_table, int max_pages,
                  int32_t* seq_lens, int B, int H, int P, int D, int num_pages, uint8_t* units, uint16_t* pool,
                  int64_t pool_cap, uint64_t* cursor, uint16_t* k_tail, uint16_t* v_tail, uint32_t* status,
                  int format, hipStream_t stream) {
  if (format == 0 && (D == 64 || D == 128)) {
    const size_t lds = compress_wave_lds(P, D);
    const void* kern = D == 128 ? (const void*)append_wave_kernel<128> : (const void*)append_wave_kernel<64>;
    if (!allow_smem(kern, lds)) return -4;
    if (D == 128)
      hipLaunchKernelGGL(append_wave_kernel<128>, dim3((unsigned)B * H), dim3(64), lds, stream, k_new, v_new, page_table,
                         max_pages, seq_lens, H, P, num_pages, units, pool, pool_cap, cursor, k_tail, v_tail, status);
    else
      hipLaunchKernelGGL(append_wave_kernel<64>, dim3((unsigned)B * H), dim3(64), lds, stream, k_new, v_new, page_table,
                         max_pages, seq_lens, H, P, num_pages, units, pool, pool_cap, cursor, k_tail, v_tail, status);
  } else {
    const size_t smem = compress_smem(P, D);
    if (!allow_smem((const void*)append_kernel, smem)) return -4;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)B * H), dim3(kCompressThreads), smem, stream, k_new, v_new,
                       page_table, max_pages, seq_lens, H, P, D, num_pages, units, pool, pool_cap, cursor, k_tail,
                       v_tail, status, format);
  }
  if (hipGetLastError() != hipSuccess) return -4;
  hipLaunchKernelGGL(bump_lens_kernel, dim3((unsigned)(B + 255) / 256), dim3(256), 0, stream, seq_lens, B,
                     max_pages * P);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvz
