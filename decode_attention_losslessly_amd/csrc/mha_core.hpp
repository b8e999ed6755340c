// Per-wave state and arithmetic of the multi-head decode-attention kernels (one query head per
// KV head), shared by the kernels of both cache formats: scores from rebuilt K pieces, the online
// softmax in the log2 domain, and the P.V accumulation from rebuilt V token pairs. The K lane
// layout is the multi-head one of kvz_lanes.hpp (lane l: pieces l + 64 i).
#pragma once

#include "attn_common.hpp"
#include "kvz_lanes.hpp"

namespace kvz {

template <int D>
struct MhaState {
  float m;          // running max, log2 domain (wave-uniform)
  float l;          // this lane's share of the denominator (its tokens' terms)
  float acc[D / 64];
  uint32_t q[8];    // dims 16*l % D .. +16 of the query, as bf16 pairs
};

// lanes that hold pieces of one token, and the score of that token in all of them
template <int D>
__device__ __forceinline__ float token_sum(float v) {
  if constexpr (D == 128) return octet_sum(v);
  else return quad_sum(v);
}

// Softmax update for one tile given this lane's scores s[i] (token of piece i; with MASKED,
// -inf for a token past the end); returns the hi/lo probability pairs of the 8 token pairs as
// wave-uniform values.
template <int D, bool MASKED = false>
__device__ __forceinline__ void mha_softmax(MhaState<D>& st, const float (&s)[D / 64], uint32_t (&phi)[8],
                                            uint32_t (&plo)[8]) {
  constexpr int NP = D / 64, LPT = D / 16;   // pieces per lane, lanes per token
  float smax = s[0];
#pragma unroll
  for (int i = 1; i < NP; ++i) smax = fmaxf(smax, s[i]);
  if (ballot(smax > st.m)) {
    const float mt = wave_max(smax);
    const float mn = fmaxf(st.m, mt);
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) st.acc[i] *= alpha;
    st.m = mn;
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    // piece i holds tokens (64 / LPT) i + l / LPT; the next token sits LPT lanes up
    // a masked token's p is 0 even while the running max is still -inf
    const float p = (MASKED && s[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[i] - st.m);
    const float pn = dpp_f<LPT == 8 ? kRowShl8 : kRowShl4>(p);
    const uint32_t hi = pack_bf16(p, pn);
    const float h_own = bf16lo_to_f32(hi), h_nb = bf16hi_to_f32(hi);
    const uint32_t lo = pack_bf16(p - h_own, pn - h_nb);
    st.l += h_own + bf16lo_to_f32(lo);
#pragma unroll
    for (int k = 0; k < 8 / NP; ++k) {
      phi[(8 / NP) * i + k] = readlane(hi, 2 * LPT * k);
      plo[(8 / NP) * i + k] = readlane(lo, 2 * LPT * k);
    }
  }
}

template <int D>
__device__ __forceinline__ void mha_accumulate_v(MhaState<D>& st, const uint32_t (&vp)[D / 8],
                                                 const uint32_t (&phi)[8], const uint32_t (&plo)[8]) {
#pragma unroll
  for (int s = 0; s < D / 64; ++s) {
    float a = st.acc[s], b = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a = dot2_bf16(vp[8 * s + k], phi[k], a);
      b = dot2_bf16(vp[8 * s + k], plo[k], b);
    }
    st.acc[s] = a + b;
  }
}

// scores of this lane's pieces from their rebuilt (or raw) K pairs
template <int D>
__device__ __forceinline__ void mha_scores(const MhaState<D>& st, const uint32_t (&kp)[D / 8], float scale,
                                           float (&s)[D / 64]) {
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      a0 = dot2_bf16(kp[8 * i + j], st.q[j], a0);
      a1 = dot2_bf16(kp[8 * i + j + 1], st.q[j + 1], a1);
    }
    s[i] = token_sum<D>(a0 + a1) * scale;
  }
}

// The uncompressed tail rows (at most P-1 tokens) of one request and head, one 16-token tile at
// a time, in the same lane layout as the compressed K; rows >= `rows` are masked.
template <int D>
__device__ __forceinline__ void mha_tail(MhaState<D>& st, const uint16_t* tk, const uint16_t* tv, int rows,
                                         float scale, int lane) {
  constexpr int NP = D / 64, NS = D / 64;
  for (int t0 = 0; t0 < rows; t0 += kTile) {
    uint32_t kp[D / 8];
    bool valid[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pc = k_piece<D, false>(lane, i);
      const int tok = t0 + piece_token<D>(pc);
      valid[i] = tok < rows;
      const uint4* krow = reinterpret_cast<const uint4*>(tk + (size_t)(valid[i] ? tok : 0) * D + piece_dim<D>(pc));
      const uint4 a = krow[0], b = krow[1];
      kp[8 * i] = a.x; kp[8 * i + 1] = a.y; kp[8 * i + 2] = a.z; kp[8 * i + 3] = a.w;
      kp[8 * i + 4] = b.x; kp[8 * i + 5] = b.y; kp[8 * i + 6] = b.z; kp[8 * i + 7] = b.w;
    }
    float sc[NP];
    mha_scores<D>(st, kp, scale, sc);
#pragma unroll
    for (int i = 0; i < NP; ++i) sc[i] = valid[i] ? sc[i] : -INFINITY;
    uint32_t phi[8], plo[8];
    mha_softmax<D, true>(st, sc, phi, plo);
    uint32_t vp[NS * 8];
#pragma unroll
    for (int g = 0; g < NS; ++g) {
      const int d = lane + 64 * g;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int t_a = t0 + 2 * k, t_b = t_a + 1;
        const uint32_t va = t_a < rows ? tv[(size_t)t_a * D + d] : 0u;
        const uint32_t vb = t_b < rows ? tv[(size_t)t_b * D + d] : 0u;
        vp[8 * g + k] = va | (vb << 16);
      }
    }
    mha_accumulate_v<D>(st, vp, phi, plo);
  }
}

}  // namespace kvz
