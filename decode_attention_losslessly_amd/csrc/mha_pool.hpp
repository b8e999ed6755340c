// The path for caches whose units mostly keep their escapes in the pool (too many for the
// unit's inline area; the escape lists then live in the pool, values only, in storage order:
// the pages' format has no escapes, so this is the build's own part of the format). The
// multi-head kernel's tile is here; the window staging, the word patch and the V patch also
// serve the grouped-query kernel, whose V lanes are laid out the same way.
//
// A wave that meets mostly pool units leaves the pipelined loop and walks the rest of its split
// (all of it, when every tile so far went to the pool) one tile at a time here. A tile's meta
// window is loaded one step ahead, so that its header (pool offset and escape counts) is known
// when the tile's payload loads are issued: the K and V escape windows that can hold the tile's
// escapes (from each block's cursor, at most a tile's worth) are then copied in the same round
// trip, side by side, into the wave's LDS area, and every lane patches its own escaped positions
// from there with fixed register indices.
#pragma once

#include "kvz_lanes.hpp"
#include "mha_core.hpp"

namespace kvz {

// u16 elements of one staged window: a tile's list (at most kTile*D values) from a 16-byte
// aligned start (up to 7 elements before it). Two windows fill esc_lds_elems<D>().
template <int D>
constexpr int win_elems() { return kTile * D + 8; }
static_assert(2 * win_elems<128>() == esc_lds_elems<128>(), "K and V windows fill the wave's LDS area");
static_assert(2 * win_elems<64>() == esc_lds_elems<64>(), "K and V windows fill the wave's LDS area");

struct Window {
  uint32_t mis;     // the list's first element sits at window[mis]
};

template <int D>
constexpr int win_chunks() { return (win_elems<D>() / 8 + 63) / 64; }   // 16-byte chunks per lane

// One 16-byte chunk of the pool at element e0 (8 elements), read element by element where it
// would cross the end of the pool.
__device__ __forceinline__ uint4 pool_chunk(const uint16_t* pool, int64_t pool_cap, uint64_t e0) {
  if (e0 + 8 <= (uint64_t)pool_cap) return *reinterpret_cast<const uint4*>(pool + e0);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e0 + e < (uint64_t)pool_cap) w[e >> 1] |= (uint32_t)pool[e0 + e] << (16 * (e & 1));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Loads the pool ranges [kfirst, kfirst + kn) and [vfirst, vfirst + vn) into lds[0 ..) and
// lds[win_elems ..). Windows clear of the pool's end (all but the last few of a pool) go
// straight from memory to LDS, 16 bytes per lane, with no registers held; a window that
// reaches the end is read chunk by chunk, element by element at the end, through registers.
// The wave-local fence at the end waits for the copies (they count as memory loads): the
// compiler does not order a later LDS read after such a copy by itself.
template <int D>
__device__ __forceinline__ void stage_windows(const uint16_t* pool, int64_t pool_cap, uint64_t kfirst, uint32_t kn,
                                              uint64_t vfirst, uint32_t vn, uint16_t* lds, Window& kw, Window& vw,
                                              int lane) {
  constexpr int NC = win_chunks<D>();
  const uint64_t ka = kfirst & ~7ull, va = vfirst & ~7ull;
  kw.mis = (uint32_t)(kfirst - ka);
  vw.mis = (uint32_t)(vfirst - va);
  const uint32_t knch = kn ? (kw.mis + kn + 7) / 8 : 0u, vnch = vn ? (vw.mis + vn + 7) / 8 : 0u;
  uint16_t* vl = lds + win_elems<D>();
  // chunk ch = lane + 64 c is pool element base + 8 ch and lands at window element 8 ch: a
  // wave-uniform base per row c plus the lane's own 8 * lane
  const uint16_t* kb = pool + ka;
  const uint16_t* vb = pool + va;
  const uint32_t lo = 8u * (uint32_t)lane;
  if (ka + 8ull * knch <= (uint64_t)pool_cap && va + 8ull * vnch <= (uint64_t)pool_cap) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if ((uint32_t)lane + 64u * c < knch)
        __builtin_amdgcn_global_load_lds(kb + 512 * c + lo, (__attribute__((address_space(3))) void*)(lds + 512 * c), 16, 0,
                                         0);
      if ((uint32_t)lane + 64u * c < vnch)
        __builtin_amdgcn_global_load_lds(vb + 512 * c + lo, (__attribute__((address_space(3))) void*)(vl + 512 * c), 16, 0,
                                         0);
    }
  } else {
    // K's window, then V's (one tensor's chunks in registers at a time)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint64_t a0 = t ? va : ka;
      const uint32_t nch = t ? vnch : knch;
      uint16_t* dst = t ? vl : lds;
      uint4 x[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint32_t ch = (uint32_t)lane + 64u * c;
        x[c] = ch < nch ? pool_chunk(pool, pool_cap, a0 + 8ull * ch) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if ((uint32_t)lane + 64u * c < nch) *reinterpret_cast<uint4*>(dst + 512 * c + lo) = x[c];
    }
  }
  wave_lds_sync();
}

// Patches the escaped positions of one offset word (8 positions: out[k] holds positions 2k,
// 2k+1) from a staged window; r0 is the list rank of the word's first escape. A word's escapes
// are consecutive in the window from there, so every position reads the slot given by the
// escapes before it (all eight reads issued together), and a per-half mask made from the
// escape flags keeps the window value for an escaped position and the rebuilt value otherwise.
// An index counts only the tile's own offset nibbles, so it stays below mis + kTile * D, inside
// the window, whatever the data; slots past the staged list (a damaged unit whose escape
// counts disagree with its offset codes) hold stale values.
__device__ __forceinline__ void patch_word(uint32_t W, uint32_t r0, const uint16_t* win, const Window& w,
                                          uint32_t* out) {
  const uint32_t f = escape_flags(W);   // position 2k: bit 4k + 3; position 2k + 1: bit 4k + 19
  const char* p = reinterpret_cast<const char*>(win + w.mis + r0);
  int e[8];        // -1 where the position is escaped, else 0
  uint32_t x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    e[j] = __builtin_amdgcn_sbfe((int)f, 4 * (j >> 1) + 3 + 16 * (j & 1), 1);
    x[j] = *reinterpret_cast<const uint16_t*>(p);
    p += __mul24(e[j], -2);   // the next slot follows an escaped position
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // low half from position 2k's flag, high half from position 2k + 1's
    const uint32_t m = __builtin_amdgcn_perm((uint32_t)e[2 * k + 1], (uint32_t)e[2 * k], 0x07060100u);
    const uint32_t val = x[2 * k] | (x[2 * k + 1] << 16);
    out[k] = (val & m) | (out[k] & ~m);
  }
}

// K tile (multi-head lane layout: lane l holds pieces l + 64 i): ranks in storage order, then
// every lane patches its pieces. Returns the tile's escape count.
template <int D>
__device__ __forceinline__ uint32_t win_patch_k(uint32_t (&pairs)[KRaw<D>::VK / 2], const KRaw<D>& raw,
                                                const uint16_t* win, const Window& w) {
  constexpr int NP = KRaw<D>::NP;
  uint32_t total = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    // piece i of every lane precedes piece i + 1 of any lane
    const uint32_t c0 = popc_flags(escape_flags(raw.nib[2 * i])), c1 = popc_flags(escape_flags(raw.nib[2 * i + 1]));
    const uint32_t inc = wave_incl_scan(c0 + c1);
    const uint32_t r = total + inc - (c0 + c1);
    total += readlane(inc, 63);
    patch_word(raw.nib[2 * i], r, win, w, &pairs[8 * i]);
    patch_word(raw.nib[2 * i + 1], r + c0, win, w, &pairs[8 * i + 4]);
  }
  return total;
}

// V tile (lane l holds dims l + 64 s, storage order segment-major then lane). Returns the
// tile's escape count.
template <int D>
__device__ __forceinline__ uint32_t win_patch_v(uint32_t (&pairs)[D / 8], const VRaw<D>& raw, const uint16_t* win,
                                                const Window& w) {
  constexpr int NS = D / 64;
  uint32_t total = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint32_t c0 = popc_flags(escape_flags(raw.seg[s].nib.x)), c1 = popc_flags(escape_flags(raw.seg[s].nib.y));
    const uint32_t inc = wave_incl_scan(c0 + c1);
    const uint32_t r = total + inc - (c0 + c1);
    total += readlane(inc, 63);
    patch_word(raw.seg[s].nib.x, r, win, w, &pairs[8 * s]);
    patch_word(raw.seg[s].nib.y, r + c0, win, w, &pairs[8 * s + 4]);
  }
  return total;
}

// K tile of a pool unit in the grouped-query lane layout (D = 128; lane l holds the adjacent
// storage pieces 2c, 2c + 1, c = 4 (l % 16) + l / 16): ranks in storage order from one scan in
// chunk order, then every lane patches its four offset words from the staged window. Returns
// the tile's escape count.
__device__ __forceinline__ uint32_t win_patch_k_gqa(uint32_t (&pairs)[16], const KRaw<128>& raw, const uint16_t* win,
                                                    const Window& w, int lane) {
  uint32_t c0[2], c1[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    c0[i] = popc_flags(escape_flags(raw.nib[2 * i]));
    c1[i] = popc_flags(escape_flags(raw.nib[2 * i + 1]));
  }
  const uint32_t cl = c0[0] + c1[0] + c0[1] + c1[1];
  const uint32_t c_ord = (uint32_t)__shfl((int)cl, 16 * (lane & 3) + (lane >> 2));   // chunk `lane`'s count
  const uint32_t inc = wave_incl_scan(c_ord);
  const uint32_t total = readlane(inc, 63);
  uint32_t r = (uint32_t)__shfl((int)(inc - c_ord), 4 * (lane & 15) + (lane >> 4));  // this lane's chunk
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    patch_word(raw.nib[2 * i], r, win, w, &pairs[8 * i]);
    patch_word(raw.nib[2 * i + 1], r + c0[i], win, w, &pairs[8 * i + 4]);
    r += c0[i] + c1[i];
  }
  return total;
}

// ---------------------------------------------------------------- one tile of any unit
// The steps of the pool-capable loops (multi-head and grouped-query), shared with the test
// decode so that the rebuilt values can be checked bit for bit. The tile's payload loads are
// issued first; for a pool unit, both escape windows (from the block cursors krank / vrank, at
// most a tile's worth each) are then staged in the same round trip. Returns whether the unit's
// escapes are in the pool.
template <int D>
__device__ __forceinline__ bool any_stage(const UnitHeader& hdr, uint32_t krank, uint32_t vrank, uint16_t* lds,
                                          const uint16_t* pool, int64_t pool_cap, Window& kw, Window& vw, int lane) {
  const bool in_pool = hdr.off != kInline;
  kw.mis = 0;
  vw.mis = 0;
  if (in_pool) {
    const uint32_t kr = uniform(krank), vr = uniform(vrank);
    const uint32_t kn = hdr.kc > kr ? min((uint32_t)(kTile * D), hdr.kc - kr) : 0u;
    const uint32_t vn = hdr.vc > vr ? min((uint32_t)(kTile * D), hdr.vc - vr) : 0u;
    stage_windows<D>(pool, pool_cap, hdr.off + kr, kn, hdr.off + hdr.kc + vr, vn, lds, kw, vw, lane);
  }
  return in_pool;
}

// Rebuilds the tile's K pairs in the given lane layout (k loaded without its bases, which come
// from the meta window) and patches its escapes: from the staged K window for a pool unit, else
// from the inline list.
template <int D, bool GQA, bool CH = false>
__device__ __forceinline__ void any_rebuild_k(uint32_t (&kp)[KRaw<D>::VK / 2], KRaw<D>& k, uint32_t meta,
                                              const UnitHeader& hdr, bool in_pool, const Window& kw, int P, int tile,
                                              uint32_t& krank, uint16_t* lds, const uint16_t* pool, int64_t pool_cap,
                                              int lane) {
  k_bases_from_meta<D, GQA, CH>(k, meta, lane);
  decode_k<D, CH>(k, kp);
  if (hdr.kc) {
    if (in_pool) {
      if constexpr (GQA) krank = uniform(krank) + win_patch_k_gqa(kp, k, lds, kw, lane);
      else krank = uniform(krank) + win_patch_k<D>(kp, k, lds, kw);
    } else {
      patch_k_tile<D, GQA, false>(kp, k, meta, hdr, P, tile, krank, lds, pool, pool_cap, lane);
    }
  }
}

// Rebuilds the tile's V pairs (lane l: dims l + 64 s, token pairs) and patches its escapes: from
// the staged V window for a pool unit, else from the inline list.
template <int D, bool CH = false>
__device__ __forceinline__ void any_rebuild_v(uint32_t (&vp)[D / 8], const VRaw<D>& v, uint32_t meta,
                                              const UnitHeader& hdr, bool in_pool, const Window& vw, int P, int tile,
                                              uint32_t& vrank, uint16_t* lds, const uint16_t* pool, int64_t pool_cap,
                                              int lane) {
#pragma unroll
  for (int g = 0; g < D / 64; ++g) decode_v_seg(v.seg[g], v_bases<D, CH>(meta, g), &vp[8 * g]);
  if (hdr.vc) {
    if (in_pool) vrank = uniform(vrank) + win_patch_v<D>(vp, v, lds + win_elems<D>(), vw);
    else patch_v_tile<D, false>(vp, v, meta, hdr, P, tile, vrank, lds, pool, pool_cap, lane);
  }
}

// One tile of any unit: `meta` is its meta window (already loaded); the payload and, for a
// pool unit, both escape windows are loaded in one round trip. krank / vrank are the block
// cursors (escapes in the unit's earlier tiles), reset at tile 0.
template <int D, bool CH = false>
__device__ __forceinline__ void mha_any_tile(MhaState<D>& st, const uint8_t* unit, uint32_t meta, int P, int tile,
                                             uint32_t& krank, uint32_t& vrank, uint16_t* lds, const uint16_t* pool,
                                             int64_t pool_cap, float scale, int lane) {
  constexpr int VK = KRaw<D>::VK, NS = D / 64;
  UnitHeader hdr = header_from_meta<D>(meta);
  clamp_to_pool(hdr, pool_cap);
  if (tile == 0) { krank = 0; vrank = 0; }
  KRaw<D> k;
  VRaw<D> v;
  load_k<D, false, false>(unit, P, tile, lane, k);
  load_v<D>(unit, P, tile, lane, v);
  Window kw, vw;
  const bool in_pool = any_stage<D>(hdr, krank, vrank, lds, pool, pool_cap, kw, vw, lane);
  uint32_t kp[VK / 2];
  any_rebuild_k<D, false, CH>(kp, k, meta, hdr, in_pool, kw, P, tile, krank, lds, pool, pool_cap, lane);
  float sc[D / 64];
  mha_scores<D>(st, kp, scale, sc);
  uint32_t phi[8], plo[8];
  mha_softmax<D>(st, sc, phi, plo);
  uint32_t vp[NS * 8];
  any_rebuild_v<D, CH>(vp, v, meta, hdr, in_pool, vw, P, tile, vrank, lds, pool, pool_cap, lane);
  mha_accumulate_v<D>(st, vp, phi, plo);
  if (in_pool) wave_lds_sync();   // the windows are read before the next tile's staging writes
}

}  // namespace kvz
