// Pieces shared by the split-K decode kernels: locating a chunk in the plan,
// and the fused log-sum-exp merge of a unit's chunk partials.
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

// ---------------------------------------------------------------------------
// Merge of a unit's chunk partials (split-K).  Two ways to order the partial
// stores of the chunks before the reads of the merge:
//
// * Deferred (plans of fewer than kTargetChunks units, which split units by
//   design): the decode launch only writes the partials, and a separate merge
//   launch on the same stream combines them (k_merge_partials); stream order
//   makes every partial happen before the merge.  No fences in either kernel.
// * Fused (kTargetChunks units or more, split only when the lengths are
//   ragged): the last chunk of a unit to finish merges inside the decode
//   launch (count_and_merge).  Partials are published with agent-scope atomic
//   stores; after a workgroup barrier (every thread's stores happen before
//   it) one thread counts the chunk in with an agent-scope release
//   increment, and the workgroup whose increment completes the count takes an
//   agent-scope acquire fence: every other chunk's release increment heads a
//   release sequence its increment read from, so all partials happen before
//   its reads.  On gfx950 each such release writes back the XCD's L2
//   (buffer_wbl2), a fixed cost per chunk, which is why plans that split by
//   design take the deferred merge.
//
// Merge rule in log2 units:
//   M = max_c m_c,  w_c = 2^(m_c - M),  out = sum_c o_c w_c / sum_c l_c w_c
// ---------------------------------------------------------------------------
__device__ __forceinline__ void publish(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float fetch(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kMergeLds = 2048;  // (chunk, head) weights kept in LDS

// Where column x / D (query head col % G of query col / G) of a unit's output
// goes: base + (col / G) * query_stride + (col % G) * D + d.  For one query
// per sequence this is the [B][Hq][D] layout (base = unit * G * D).
struct OutMap {
  size_t base, query_stride;
  int G, D;
  __device__ __forceinline__ size_t at(int x) const {
    const int col = x / D, d = x - col * D;
    return base + size_t(col / G) * query_stride + size_t(col % G) * D + d;
  }
};

// Combine the partials of chunks first .. first + nch - 1 of one unit into its
// output, by the whole workgroup.  G here is the number of output columns of
// the unit (query heads times queries); `om` places them.
__device__ inline void merge_unit(int first, int nch, int G, int D, const float2 *part_ml,
                                  const float *part_o, float *out, const OutMap &om) {
  __shared__ float s_w[kMergeLds];
  __shared__ float s_inv[16];
  const float *ml = reinterpret_cast<const float *>(part_ml);
  if (nch * G <= kMergeLds) {
    // w[i][g] = 2^(m_ig - M_g); 1 / L_g
    for (int x = threadIdx.x; x < nch * G; x += blockDim.x)
      s_w[x] = fetch(ml + 2 * (size_t(first) * G + x));
    __syncthreads();
    if (threadIdx.x < G) {
      const int g = threadIdx.x;
      float M = -INFINITY;
      for (int i = 0; i < nch; ++i) M = fmaxf(M, s_w[i * G + g]);
      float Ls = 0.f;
      for (int i = 0; i < nch; ++i) {
        const float m = s_w[i * G + g];
        const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
        s_w[i * G + g] = w;
        Ls = fmaf(fetch(ml + 2 * (size_t(first + i) * G + g) + 1), w, Ls);
      }
      s_inv[g] = Ls > 0.f ? 1.f / Ls : 0.f;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < G * D; x += blockDim.x) {
      const int g = x / D;
      float acc = 0.f;
      for (int i = 0; i < nch; ++i)
        acc = fmaf(fetch(part_o + size_t(first + i) * G * D + x), s_w[i * G + g], acc);
      out[om.at(x)] = acc * s_inv[g];
    }
  } else {  // very many chunks: the plain two-pass loop
    for (int x = threadIdx.x; x < G * D; x += blockDim.x) {
      const int g = x / D;
      float M = -INFINITY;
      for (int i = 0; i < nch; ++i) M = fmaxf(M, fetch(ml + 2 * (size_t(first + i) * G + g)));
      float Ls = 0.f, Os = 0.f;
      if (M != -INFINITY) {
        for (int i = 0; i < nch; ++i) {
          const float m = fetch(ml + 2 * (size_t(first + i) * G + g));
          if (m == -INFINITY) continue;
          const float w = exp2f(m - M);
          Ls = fmaf(fetch(ml + 2 * (size_t(first + i) * G + g) + 1), w, Ls);
          Os = fmaf(fetch(part_o + size_t(first + i) * G * D + x), w, Os);
        }
      }
      out[om.at(x)] = Ls > 0.f ? Os / Ls : 0.f;
    }
  }
}

// The fused merge: called by every thread of the workgroup after it has
// published its share of this chunk's partials.  Returns after the unit is
// merged (if this workgroup was the last of its unit) or at once.
__device__ inline void count_and_merge(const ChunkInfo &ci, int G, int D, int32_t *merge_count,
                                       const float2 *part_ml, const float *part_o, float *out,
                                       const OutMap &om) {
  __shared__ int s_last;
  __syncthreads();  // every thread's partial stores happen before the increment
  if (threadIdx.x == 0) {
    const bool last = __hip_atomic_fetch_add(&merge_count[ci.unit], 1, __ATOMIC_RELEASE,
                                             __HIP_MEMORY_SCOPE_AGENT) == ci.nch - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  merge_unit(ci.first, ci.nch, G, D, part_ml, part_o, out, om);
  if (threadIdx.x == 0)
    __hip_atomic_store(&merge_count[ci.unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Which merge a plan of `units` units takes (see above).
__host__ __device__ inline bool fused_merge(int units) { return units >= kTargetChunks; }

}  // namespace dms
