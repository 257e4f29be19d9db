// Pieces shared by the split-K decode kernels: locating a chunk in the plan,
// and the log-sum-exp merge of a unit's chunk partials.
#pragma once

#include "dms_internal.h"

namespace dms {

struct ChunkInfo {
  int unit, b, h;
  int first, nch;      // the unit's chunks: [first, first + nch)
  int s_begin, s_end;  // slots of this chunk
  int t;               // query position seq_len[b] - 1
  int nclean;
};

// false if this workgroup has no chunk (grid is sized for the maximum count)
__device__ __forceinline__ bool locate_chunk(int c, int hkv, const int32_t *plan, const int32_t *n_slots,
                                             const int32_t *n_clean, const int32_t *seq_len,
                                             const PlanLayout &L, ChunkInfo &ci) {
  if (c >= plan[L.hdr + 0]) return false;
  const int C = plan[L.hdr + 1];
  ci.unit = plan[L.chunk_unit + c];
  ci.b = ci.unit / hkv;
  ci.h = ci.unit % hkv;
  ci.first = plan[L.first_chunk + ci.unit];
  ci.nch = plan[L.first_chunk + ci.unit + 1] - ci.first;
  ci.s_begin = (c - ci.first) * C;
  ci.s_end = min(n_slots[ci.unit], ci.s_begin + C);
  ci.t = seq_len[ci.b] - 1;
  ci.nclean = n_clean[ci.unit];
  return true;
}

// Merge rule for chunk partials in log2 units:
//   M = max_c m_c,  L = sum_c l_c 2^(m_c - M),  out = sum_c o_c 2^(m_c - M) / L
// over the chunks [first, first + nch) of unit u; out is [unit][G][D].
__device__ inline void merge_chunks(int u, int first, int nch, int G, int D, const float2 *part_ml,
                                    const float *part_o, float *out) {
  for (int x = threadIdx.x; x < G * D; x += blockDim.x) {
    const int g = x / D;
    float M = -INFINITY;
    for (int i = 0; i < nch; ++i) M = fmaxf(M, part_ml[size_t(first + i) * G + g].x);
    float Ls = 0.f, Os = 0.f;
    if (M != -INFINITY) {
      for (int i = 0; i < nch; ++i) {
        const float2 ml = part_ml[size_t(first + i) * G + g];
        if (ml.x == -INFINITY) continue;
        const float f = exp2f(ml.x - M);
        Ls = fmaf(ml.y, f, Ls);
        Os = fmaf(part_o[size_t(first + i) * G * D + x], f, Os);
      }
    }
    out[size_t(u) * G * D + x] = Ls > 0.f ? Os / Ls : 0.f;
  }
}

}  // namespace dms
