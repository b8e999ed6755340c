// Pieces shared by the decode-attention kernels: split geometry, partial results, merge.
//
// Split-K over the sequence (flash-decoding): work item (request r, head, split s) covers the
// full pages [s*C, min((s+1)*C, L/P)) of the request; the split that holds the last full page
// (split 0 when there is none) also covers the L mod P tail rows. It leaves (m, l, acc[D]):
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
