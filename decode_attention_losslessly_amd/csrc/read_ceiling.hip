// The streaming-read ceiling of the compressed attention kernels (include/kvz_bench.h): the same
// unit bytes, read in the same pattern (a wave walks one (request, head) row's pages in
// page-table order; a unit is one burst of 16-byte non-temporal loads through a buffer resource
// whose extent is the unit; the next unit's loads go out before the current unit is used), with
// no decode and no arithmetic beyond one XOR per loaded dword.
#include <hip/hip_runtime.h>

#include "kvz.h"
#include "kvz_bench.h"
#include "kvz_lanes.hpp"

namespace kvz {

constexpr int kReadWaves = 4;   // waves per workgroup, as the attention kernels

template <int NL>   // 16-byte loads per lane per unit: ceil(unit bytes / 1024)
__global__ __launch_bounds__(64 * kReadWaves) void read_units_kernel(const uint8_t* __restrict__ units, int num_pages,
                                                                    uint32_t U, const int32_t* __restrict__ pt,
                                                                    int max_pages, const int32_t* __restrict__ seq_lens,
                                                                    int B, int H, int P, int chunks,
                                                                    uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wid = (int)uniform(blockIdx.x * kReadWaves + (threadIdx.x >> 6));
  const int row = wid / chunks, c = wid % chunks;
  if (row >= B * H) return;
  const int r = row / H, h = row % H;
  int L = sload<int32_t>(seq_lens + r);
  L = L < 0 ? 0 : min(L, max_pages * P);
  const int np = L / P, per = (np + chunks - 1) / chunks;
  const int p0 = min(np, c * per), p1 = min(np, p0 + per);
  const int32_t* row_pt = pt + (size_t)r * max_pages;
  auto unit_of = [&](int p) {
    const int pid = sload<int32_t>(row_pt + p);
    return units + ((size_t)(pid >= 0 && pid < num_pages ? pid : 0) * H + h) * U;
  };
  uint32_t acc = 0;
  if (p0 < p1) {
    uint4 cur[NL], nxt[NL];
    {
      const UnitRsrc u = unit_rsrc(unit_of(p0), U);
#pragma unroll
      for (int j = 0; j < NL; ++j) cur[j] = uload16(u, 16 * lane + 1024 * j, 0);
    }
    for (int p = p0; p < p1; ++p) {
      // the next unit (a stand-in of extent 0 past the chunk's end, which reads nothing)
      const bool live = p + 1 < p1;
      const UnitRsrc u = unit_rsrc(unit_of(live ? p + 1 : p), live ? U : 0u);
#pragma unroll
      for (int j = 0; j < NL; ++j) nxt[j] = uload16(u, 16 * lane + 1024 * j, 0);
#pragma unroll
      for (int j = 0; j < NL; ++j) acc ^= cur[j].x ^ cur[j].y ^ cur[j].z ^ cur[j].w;
#pragma unroll
      for (int j = 0; j < NL; ++j) cur[j] = nxt[j];
    }
  }
  sink[(size_t)wid * 64 + lane] = acc;
}

}  // namespace kvz

extern "C" int kvzb_read_units(const uint8_t* units, int32_t num_pages, size_t unit_bytes, const int32_t* page_table,
                               int32_t max_pages, const int32_t* seq_lens, int32_t B, int32_t H, int32_t P,
                               int32_t chunks, uint32_t* sink, void* stream) {
  if (!units || !page_table || !seq_lens || !sink || num_pages <= 0 || B < 0 || H <= 0 || P <= 0 || max_pages < 0 ||
      chunks <= 0 || unit_bytes == 0 || unit_bytes % 16 || unit_bytes > 16384 || (long)max_pages * P > INT32_MAX)
    return KVZ_ERR_INVALID_ARG;
  const long waves = (long)B * H * chunks;
  if (waves == 0) return KVZ_OK;
  if (waves > (1l << 30)) return KVZ_ERR_INVALID_ARG;
  const dim3 grid((unsigned)((waves + kvz::kReadWaves - 1) / kvz::kReadWaves)), block(64 * kvz::kReadWaves);
  const int nl = (int)((unit_bytes + 1023) / 1024);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint32_t U = (uint32_t)unit_bytes;
#define KVZB_READ(n)                                                                                           \
  hipLaunchKernelGGL((kvz::read_units_kernel<n>), grid, block, 0, s, units, num_pages, U, page_table, max_pages, \
                     seq_lens, B, H, P, chunks, sink)
  switch (nl) {
    case 1: KVZB_READ(1); break;
    case 2: KVZB_READ(2); break;
    case 3: KVZB_READ(3); break;
    case 4: KVZB_READ(4); break;
    case 5: KVZB_READ(5); break;
    case 6: KVZB_READ(6); break;
    case 7: KVZB_READ(7); break;
    case 8: KVZB_READ(8); break;
    default: {
      if (nl <= 12) KVZB_READ(12); else KVZB_READ(16);
    }
  }
#undef KVZB_READ
  return hipGetLastError() == hipSuccess ? KVZ_OK : KVZ_ERR_HIP;
}
