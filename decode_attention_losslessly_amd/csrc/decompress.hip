// Test-only kernel: the attention kernels' in-register decode of K and V, written back as raw
// BF16 so that it can be compared bit for bit with the source of the compressed pages.
// One wave per (unit, head); per tile: load, rebuild, patch escapes, store. Two routes, each in
// both lane layouts (GQA: the grouped-query kernel's K layout):
//   WIN false  the main loops and the per-unit path after them: inline lists patched by a
//              wave-uniform walk, pool lists staged whole and patched through a copy of the
//              pairs in LDS (patch_k_tile / patch_v_tile);
//   WIN true   the pool-capable loops: a pool unit's escape windows staged with the payload and
//              every offset word patched from them (any_stage / any_rebuild_k / any_rebuild_v).
// CH: channel groups (format 2).
#include "kvz_lanes.hpp"
#include "mha_pool.hpp"

namespace kvz {

template <int D, bool GQA, bool WIN, bool CH>
__global__ __launch_bounds__(64) void decompress_kernel(const uint8_t* __restrict__ units,
                                                        const uint16_t* __restrict__ pool, int64_t pool_cap,
                                                        const int32_t* __restrict__ page_ids, int H,
                                                        int P, int num_pages, uint16_t* __restrict__ k_dst,
                                                        uint16_t* __restrict__ v_dst,
                                                        uint32_t* __restrict__ status) {
  __shared__ __align__(16) uint16_t lds[esc_lds_elems<D>()];
  const int lane = threadIdx.x;
  const int i = blockIdx.x / H, h = blockIdx.x % H;
  const int pid = sload<int32_t>(page_ids + i);
  if (pid < 0 || pid >= num_pages) {
    if (lane == 0) atomicOr(status, kStatusBadPage);
    return;
  }
  const uint8_t* unit = units + ((size_t)pid * H + h) * unit_bytes(P, D);
  uint16_t* kd = k_dst + ((size_t)i * H + h) * P * D;
  uint16_t* vd = v_dst + ((size_t)i * H + h) * P * D;
  uint32_t krank = 0, vrank = 0;
  for (int t = 0; t < P / kTile; ++t) {
    const uint32_t meta = load_meta(unit, P, D, t, lane);
    UnitHeader hdr = header_from_meta<D>(meta);
    clamp_to_pool(hdr, pool_cap);
    KRaw<D> kr;
    VRaw<D> vr;
    uint32_t kp[KRaw<D>::VK / 2];
    constexpr int NS = D / 64;
    uint32_t vp[NS * 8];
    if constexpr (WIN) {
      load_k<D, GQA, false>(unit, P, t, lane, kr);
      load_v<D>(unit, P, t, lane, vr);
      Window kw, vw;
      const bool in_pool = any_stage<D>(hdr, krank, vrank, lds, pool, pool_cap, kw, vw, lane);
      any_rebuild_k<D, GQA, CH>(kp, kr, meta, hdr, in_pool, kw, P, t, krank, lds, pool, pool_cap, lane);
      any_rebuild_v<D, CH>(vp, vr, meta, hdr, in_pool, vw, P, t, vrank, lds, pool, pool_cap, lane);
      if (in_pool) wave_lds_sync();
    } else {
      load_k<D, GQA, true, CH>(unit, P, t, lane, kr);
      decode_k<D, CH>(kr, kp);
      if (hdr.kc) patch_k_tile<D, GQA>(kp, kr, meta, hdr, P, t, krank, lds, pool, pool_cap, lane);
      load_v<D>(unit, P, t, lane, vr);
#pragma unroll
      for (int s = 0; s < NS; ++s) decode_v_seg(vr.seg[s], v_bases<D, CH>(meta, s), &vp[8 * s]);
      if (hdr.vc) patch_v_tile<D>(vp, vr, meta, hdr, P, t, vrank, lds, pool, pool_cap, lane);
    }
#pragma unroll
    for (int i = 0; i < KRaw<D>::NP; ++i) {
      const int pc = k_piece<D, GQA>(lane, i);
      uint32_t* dst = reinterpret_cast<uint32_t*>(kd + (size_t)(t * kTile + piece_token<D>(pc)) * D + piece_dim<D>(pc));
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j] = kp[8 * i + j];
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int d = lane + 64 * s;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        vd[(size_t)(t * kTile + 2 * k) * D + d] = (uint16_t)(vp[8 * s + k] & 0xFFFFu);
        vd[(size_t)(t * kTile + 2 * k + 1) * D + d] = (uint16_t)(vp[8 * s + k] >> 16);
      }
    }
  }
}

int launch_decompress(const uint8_t* units, const uint16_t* pool, int64_t pool_cap, const int32_t* page_ids, int n, int H,
                      int P, int D, int num_pages, int lane_map, uint16_t* k_dst, uint16_t* v_dst,
                      uint32_t* status, bool channel, hipStream_t stream) {
  // lane_map: 0 / 1 = multi-head / grouped-query layout through the main loops' route,
  //           2 / 3 = the same layouts through the pool-capable loops' route
  const dim3 grid((unsigned)n * H), block(64);
#define KVZ_DECOMPRESS(d, gqa, win)                                                                          \
  hipLaunchKernelGGL((channel ? decompress_kernel<d, gqa, win, true> : decompress_kernel<d, gqa, win, false>), grid, \
                     block, 0, stream, units, pool, pool_cap, page_ids, H, P, num_pages, k_dst, v_dst, status)
  if (D == 128) {
    switch (lane_map) {
      case 0: KVZ_DECOMPRESS(128, false, false); break;
      case 1: KVZ_DECOMPRESS(128, true, false); break;
      case 2: KVZ_DECOMPRESS(128, false, true); break;
      case 3: KVZ_DECOMPRESS(128, true, true); break;
      default: return -2;
    }
  } else if (D == 64) {
    switch (lane_map) {
      case 0: KVZ_DECOMPRESS(64, false, false); break;
      case 2: KVZ_DECOMPRESS(64, false, true); break;
      default: return -2;
    }
  } else {
    return -2;
  }
#undef KVZ_DECOMPRESS
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvz
