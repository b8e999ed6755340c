// kvz_compact_pool: copies the pool data of the listed units (escape lists in the escape format,
// raw blocks in the ZipFusion format) into a new pool and repoints the units at it, so that the
// space of freed units can be given back (the pages reassign memory released by compression and
// by finished requests: ZipFusion summary, §III.D "KV Cache Management and Scheduling"; here the
// caller then swaps the new pool in and frees the old one).
//
// One 256-thread workgroup per (unit, head): read the unit's pool extent from its header, take
// that many elements of the new pool at an atomically bumped cursor, copy, rewrite the header.
#include "compress.hpp"
#include "zf.hpp"

namespace kvz {

constexpr int kCompactThreads = 256;

__global__ __launch_bounds__(kCompactThreads) void compact_pool_kernel(
    uint8_t* __restrict__ units, const uint16_t* __restrict__ pool, int64_t pool_cap,
    const int32_t* __restrict__ page_ids, int H, int P, int D, int num_pages, int format,
    uint16_t* __restrict__ new_pool, int64_t new_cap, uint64_t* __restrict__ new_cursor,
    uint32_t* __restrict__ status) {
  __shared__ uint64_t sh_dest;
  __shared__ int sh_ok;
  const int i = blockIdx.x / H, h = blockIdx.x % H, tid = threadIdx.x;
  const int pid = page_ids[i];
  if (pid < 0 || pid >= num_pages) {
    if (tid == 0) atomicOr(status, kStatusBadPage);
    return;
  }
  uint8_t* unit;
  uint64_t* off_field;
  uint64_t count;   // pool elements the unit owns
  if (format == 1) {
    unit = units + ((size_t)pid * H + h) * zf_unit_bytes(P, D);
    off_field = reinterpret_cast<uint64_t*>(unit + zf_rawoff_offset(P, D));
    uint32_t n = 0;
    for (int b = 0; b < zf_nblocks(P, D); ++b) n += unit[b] == kZfRaw ? 1u : 0u;
    count = (uint64_t)n * kZfBlock;
  } else {
    unit = units + ((size_t)pid * H + h) * unit_bytes(P, D);
    const uint32_t* hdr = reinterpret_cast<const uint32_t*>(unit + hdr_offset(P, D));
    off_field = reinterpret_cast<uint64_t*>(unit + hdr_offset(P, D) + 8);
    count = (uint64_t)hdr[0] + hdr[1];
  }
  const uint64_t off = *off_field;
  if (off == kInline || count == 0) return;   // nothing in the pool (uniform for the workgroup)
  __syncthreads();                            // every wave has read the header before it changes
  if (tid == 0) {
    sh_ok = 0;
    if (off + count <= (uint64_t)pool_cap) {
      const uint64_t dest = atomicAdd((unsigned long long*)new_cursor, (unsigned long long)count);
      if (dest + count <= (uint64_t)new_cap) {
        sh_dest = dest;
        sh_ok = 1;
      }
    }
    if (!sh_ok) {
      // no room (or a header outside the old pool): drop the unit's pool data, as compression
      // does when its pool is full, so that nothing ever reads past a pool
      atomicOr(status, kStatusPoolFull);
      *off_field = kInline;
      if (format != 1) {
        uint32_t* hdr = reinterpret_cast<uint32_t*>(unit + hdr_offset(P, D));
        hdr[0] = 0;
        hdr[1] = 0;
      }
    }
  }
  __syncthreads();
  if (!sh_ok) return;
  const uint64_t dest = sh_dest;
  for (uint64_t e = tid; e < count; e += kCompactThreads) new_pool[dest + e] = pool[off + e];
  __syncthreads();
  if (tid == 0) *off_field = dest;
}

int launch_compact_pool(uint8_t* units, const uint16_t* pool, int64_t pool_cap, const int32_t* page_ids, int n, int H,
                        int P, int D, int num_pages, int format, uint16_t* new_pool, int64_t new_cap,
                        uint64_t* new_cursor, uint32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(compact_pool_kernel, dim3((unsigned)n * H), dim3(kCompactThreads), 0, stream, units, pool, pool_cap,
                     page_ids, H, P, D, num_pages, format, new_pool, new_cap, new_cursor, status);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvz
