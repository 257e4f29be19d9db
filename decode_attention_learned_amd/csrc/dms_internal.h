// Internal declarations shared by the libdms translation units.
// Target: gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dms.h"

namespace dms {

constexpr int kPage = DMS_PAGE_SIZE;   // slots per page
constexpr int kWave = 64;              // CDNA wavefront width
// Target number of split-K chunks per decode call: 8 per CU on a 256-CU part.
constexpr int kTargetChunks = 2048;

inline int units_of(const dms_shape &s) { return s.batch * s.kv_heads; }

// Decode workspace: every region starts on a 256-byte boundary.
struct DecodeWorkspace {
  size_t hdr;          // int32[16]: [0] chunk count, [1] slots per chunk
  size_t first_chunk;  // int32[units + 1]: first chunk of each unit (prefix sum)
  size_t chunk_unit;   // int32[max_chunks]: owning unit of each chunk
  size_t part_ml;      // float2[max_chunks * G]: running max and sum per chunk and head
  size_t part_o;       // float[max_chunks * G * D]: unnormalised partial outputs
  size_t bytes;
  int max_chunks;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline DecodeWorkspace decode_workspace_layout(int units, int group, int head_dim) {
  DecodeWorkspace w;
  w.max_chunks = units + kTargetChunks;
  size_t off = 0;
  w.hdr = off;         off = align256(off + 16 * sizeof(int32_t));
  w.first_chunk = off; off = align256(off + size_t(units + 1) * sizeof(int32_t));
  w.chunk_unit = off;  off = align256(off + size_t(w.max_chunks) * sizeof(int32_t));
  w.part_ml = off;     off = align256(off + size_t(w.max_chunks) * group * 2 * sizeof(float));
  w.part_o = off;      off = align256(off + size_t(w.max_chunks) * group * head_dim * sizeof(float));
  w.bytes = off;
  return w;
}

// ---- launchers (each defined in the translation unit holding its kernels) ----
hipError_t launch_reset(const dms_shape &s, const dms_cache &c, hipStream_t st);
hipError_t launch_append(const dms_shape &s, const dms_cache &c, const void *k_new,
                         const void *v_new, const float *logit, int n_new, hipStream_t st);
hipError_t launch_compact(const dms_shape &s, const dms_cache &c, hipStream_t st);
hipError_t launch_decode(const dms_shape &s, const dms_cache &c, const void *q, float *out,
                         float sm_scale, void *ws, hipStream_t st);
hipError_t launch_prefill(const dms_shape &s, const void *q, const void *k, const void *v,
                          const float *logit, int seq_len, float sm_scale, float *out,
                          hipStream_t st);

// ---- wave64 helpers -------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// number of set bits of `mask` below this lane
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (l >= o) x += y;
  }
  return x;
}

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

}  // namespace dms
