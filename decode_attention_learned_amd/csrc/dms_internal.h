// Internal declarations shared by the libdms translation units.
// Target: gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <stddef.h>
#include <stdint.h>

#include "dms.h"

namespace dms {

constexpr int kPage = DMS_PAGE_SIZE;   // slots per page
constexpr int kWave = 64;              // CDNA wavefront width
// Split-K chunks per decode call.  kTargetChunks is one round of resident
// decode workgroups (8 waves each, 2 per CU on the 256 CUs).  Units of even
// length fill one round: with at least that many units every unit is one
// chunk (no merge), with fewer they are split.  Units of ragged length
// (longest > twice the mean) are split into up to three rounds' worth, so that
// workgroups that finish early take more chunks.  Measured on the Qwen3-8B (CR 8 and 1), ragged Qwen2.5-32B and
// Llama-1B decode workloads.
#ifndef DMS_TARGET_CHUNKS
#define DMS_TARGET_CHUNKS 512
#endif
constexpr int kTargetChunks = DMS_TARGET_CHUNKS;
constexpr int kRaggedRounds = 3;
// Even lengths are not split into chunks shorter than this many slots: below
// it the split's extra workgroups and merge cost more than the parallelism
// gains (Llama-3.2-1B-shaped heads, 128 units of ~1100 slots: 25.2 -> 23.3 us
// per decode step unsplit).  A multiple of the page size.
constexpr int kMinEvenChunk = 2048;

// The largest chunk count of a plan for `units` units.  build_plan gives one
// chunk per unit when units >= its budget (kTargetChunks, or kRaggedRounds *
// kTargetChunks for ragged lengths), and at most the budget otherwise, so the
// count never exceeds max(units, kRaggedRounds * kTargetChunks).
__host__ __device__ inline int max_chunks_of(int units) {
  return units > kRaggedRounds * kTargetChunks ? units : kRaggedRounds * kTargetChunks;
}

inline int units_of(const dms_shape &s) { return s.batch * s.kv_heads; }

// Split plan, kept in cache state (dms_cache.plan, int32 words).  Rebuilt from
// n_slots by every call that changes n_slots (reset, append, compact), so
// decode reads it without a planning launch of its own.
// Besides the plan, the same buffer holds per unit the position of the last
// token at its last compaction (compact_pos, -1 before any): a chunk of
// queries appended at positions >= p0 can be answered only if no compaction
// ran after position p0 (a later one may have dropped keys the chunk's
// earlier queries still see, or moved chunk tokens into the clean prefix).
struct PlanLayout {
  size_t hdr;          // [16]: [0] chunk count, [1] slots per chunk
  size_t first_chunk;  // [units + 1]: first chunk of each unit (prefix sum)
  size_t chunk_unit;   // [max_chunks]: owning unit of each chunk
  size_t merge_count;  // [units]: chunks of the unit finished in the running decode
  size_t compact_pos;  // [units]: position t of the unit's last compaction, -1 if none
  size_t words;
  int max_chunks;
};

__host__ __device__ inline PlanLayout plan_layout(int units) {
  PlanLayout p;
  p.max_chunks = max_chunks_of(units);
  p.hdr = 0;
  p.first_chunk = 16;
  p.chunk_unit = p.first_chunk + size_t(units) + 1;
  p.merge_count = p.chunk_unit + size_t(p.max_chunks);
  p.compact_pos = p.merge_count + size_t(units);
  p.words = p.compact_pos + size_t(units);
  return p;
}

// Decode workspace: partial results of the split-K chunks.
struct DecodeWorkspace {
  size_t part_ml;  // float2[max_chunks * G]: running max and sum per chunk and head
  size_t part_o;   // float[max_chunks * G * D]: unnormalised partial outputs
  size_t bytes;
  int max_chunks;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline DecodeWorkspace decode_workspace_layout(int units, int group, int head_dim) {
  DecodeWorkspace w;
  w.max_chunks = max_chunks_of(units);
  size_t off = 0;
  w.part_ml = off; off = align256(off + size_t(w.max_chunks) * group * 2 * sizeof(float));
  w.part_o = off;  off = align256(off + size_t(w.max_chunks) * group * head_dim * sizeof(float));
  w.bytes = off;
  return w;
}

// Split-K of the tiled chunk kernel (chunks of 32 queries or more).  Its
// grid is one workgroup per 32 queries and (sequence, KV head, group of 4
// query heads); three run per CU.  When that fills at most half of one
// resident round (3 x 256), each workgroup's tiles are dealt round-robin
// into `splits` parts (at most 4, all still in one round) whose partials a
// merge launch combines.  Measured: 512 queries of 4 sequences (512 workgroups, two
// thirds of a round) took 0.132 ms split 3 ways against 0.069 ms unsplit,
// the partials' traffic outweighing the extra third of the chip.
constexpr int kChunkResident = 3 * 256;
inline int chunk_splits(const dms_shape &s, int n_query) {
  const long wgs = long((n_query + 31) / 32) * s.batch * s.kv_heads * ((s.group + 3) / 4);
  if (wgs <= 0 || 2 * wgs > kChunkResident) return 1;
  const long f = kChunkResident / wgs;
  return f > 4 ? 4 : int(f);
}
// Partials of the splits: per split and output row (B * n_query * Hq rows),
// (reference, row sum) and D floats of unnormalised output.
struct ChunkSplitLayout {
  size_t rows, part_ml, part_o, bytes;
};
inline ChunkSplitLayout chunk_split_layout(const dms_shape &s, int n_query, int splits) {
  ChunkSplitLayout L;
  L.rows = size_t(s.batch) * size_t(n_query) * size_t(s.kv_heads) * size_t(s.group);
  L.part_ml = 0;
  L.part_o = align256(size_t(splits) * L.rows * 2 * sizeof(float));
  L.bytes = L.part_o + align256(size_t(splits) * L.rows * size_t(s.head_dim) * sizeof(float));
  return L;
}
inline size_t chunk_split_bytes(const dms_shape &s, int n_query, int splits) {
  return splits > 1 ? chunk_split_layout(s, n_query, splits).bytes : 0;
}

// ---- launchers (each defined in the translation unit holding its kernels) ----
hipError_t launch_reset(const dms_shape &s, const dms_cache &c, hipStream_t st);
hipError_t launch_append(const dms_shape &s, const dms_cache &c, const void *k_new,
                         const void *v_new, const float *logit, int n_new, hipStream_t st);
// the two parts of launch_append: slots, pages and counts; then decisions and K/V
hipError_t launch_append_alloc(const dms_shape &s, const dms_cache &c, int n_new, hipStream_t st);
hipError_t launch_append_write(const dms_shape &s, const dms_cache &c, const void *k_new,
                               const void *v_new, const float *logit, int n_new, hipStream_t st);
// The token that launch_append_alloc(n_new = 1) reserved in every unit, for a
// decode launch to write (decision, K, V) before it attends.
struct DecodeFill {
  const void *k_new, *v_new;  // [B][1][Hkv][D]
  const float *logit;         // [B][1][Hkv]
};
hipError_t launch_compact(const dms_shape &s, const dms_cache &c, hipStream_t st);
// device address of the static scratch array on the GPU of `stream` (decode_scratch.hip)
hipError_t scratch_address(hipStream_t stream, void **ptr);
hipError_t launch_export(const dms_shape &s, const dms_cache &c, int all_slots, int max_out,
                         int32_t *count_out, int32_t *pos_out, uint8_t *alpha_out, void *k_out,
                         void *v_out, hipStream_t st);
hipError_t launch_plan(const dms_shape &s, const dms_cache &c, hipStream_t st);
hipError_t launch_decode(const dms_shape &s, const dms_cache &c, const void *q, float *out,
                         float sm_scale, void *ws, hipStream_t st, const DecodeFill *fill = nullptr);
hipError_t launch_share(const dms_shape &s, const dms_cache &c, int src, int dst_first, int n_dst,
                        hipStream_t st);
hipError_t launch_release(const dms_shape &s, const dms_cache &c, int first, int n, hipStream_t st);
hipError_t launch_chunk_attn(const dms_shape &s, const dms_cache &c, const void *q, int n_query,
                             float *out, float sm_scale, void *ws, size_t ws_bytes, hipStream_t st);
hipError_t launch_decode_multi(const dms_shape &s, const dms_cache &c, const void *q, int n_query,
                               float *out, float sm_scale, void *ws, size_t ws_bytes, hipStream_t st);
// the deferred split-K merge after a decode launch (nothing for plans that merge in the launch)
hipError_t launch_merge(const dms_shape &s, const dms_cache &c, const DecodeWorkspace &w, char *ws,
                        float *out, int ncol, int c0, int C, hipStream_t st);
// temperature <= 0: the hard rule; > 0: the relaxed mask (noise may be null)
hipError_t launch_prefill(const dms_shape &s, const void *q, const void *k, const void *v,
                          const float *logit, const float *noise, float temperature, int seq_len,
                          float sm_scale, float *out, void *ws, hipStream_t st);
// float32 caches, chunks of 32 queries or more (prefill_f32.hip); no workspace
hipError_t launch_chunk_f32(const dms_shape &s, const dms_cache &c, const void *q, int n_query,
                            float *out, float sm_scale, hipStream_t st);
// float32 inputs, every prefill method (prefill_f32.hip); no workspace
hipError_t launch_prefill_f32(const dms_shape &s, const void *q, const void *k, const void *v,
                              const float *logit, const float *noise, float temperature,
                              int seq_len, float sm_scale, float *out, hipStream_t st);
hipError_t launch_prefill_gathered(const dms_shape &s, const void *q, const void *k, const void *v,
                                   const float *logit, int seq_len, float sm_scale, float *out,
                                   void *ws, hipStream_t st);

// Prefill workspace: per (b, h, 32-key tile) the key and value fragments
// (64 D bytes each, bf16: 8 KB each at D = 128) and 32 floats of additive mask.
inline size_t prefill_workspace_bytes(int batch, int kv_heads, int seq_len, int head_dim) {
  const size_t tiles = size_t(batch) * kv_heads * ((size_t(seq_len) + 31) / 32);
  const size_t tile_bytes = size_t(128) * head_dim;
  // packed tiles, their masks, packed tiles with masked keys zero (far use)
  return align256(tiles * tile_bytes) + align256(tiles * 32 * sizeof(float)) +
         align256(tiles * tile_bytes);
}

// Gathered-key prefill workspace: packed tiles as in the dense prefill
// workspace, of which only the value half is written (band tiles read their
// keys straight from K), the per-key masks, the same tile layout for the
// gathered kept keys plus their positions, and per unit the kept positions in
// order, kept counts before each tile and each tile's kept-key bits.  Byte
// offsets of each region.
struct PrefillGatheredLayout {
  size_t dense_mask, gathered, gathered_pos, gpos, tile_cnt, keptw, total;
};
inline PrefillGatheredLayout prefill_gathered_layout(int batch, int kv_heads, int seq_len,
                                                     int head_dim) {
  const size_t units = size_t(batch) * kv_heads;
  const size_t nt = (size_t(seq_len) + 31) / 32;
  const size_t tiles = units * nt;
  const size_t tile_bytes = size_t(128) * head_dim;
  PrefillGatheredLayout L;
  L.dense_mask = align256(tiles * tile_bytes);
  L.gathered = L.dense_mask + align256(tiles * 32 * sizeof(float));
  L.gathered_pos = L.gathered + align256(tiles * tile_bytes);
  L.gpos = L.gathered_pos + align256(tiles * 32 * sizeof(int32_t));
  L.tile_cnt = L.gpos + align256(units * size_t(seq_len) * sizeof(int32_t));
  L.keptw = L.tile_cnt + align256(units * (nt + 1) * sizeof(int32_t));
  L.total = L.keptw + align256(tiles * sizeof(uint32_t));
  return L;
}

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

// Chunk plan from n_slots, run by one workgroup of kPlanThreads threads.
// Every thread reads only the n_slots entries it is the sole writer of in a
// caller that updated them (unit u = base + threadIdx.x), so a caller that
// has just written n_slots needs nothing beyond a workgroup barrier.
// Chunk size C (slots, a multiple of the page size), chunks(u) = max(1, ceil(n_u / C)),
// with a budget of R * kTargetChunks chunks, R = kRaggedRounds if the longest
// unit holds more than twice the mean (max_u n_u > 2 * total / units), else 1:
//   units >= budget:  C = 64 * ceil(max_u n_u / 64)   (one chunk per unit)
//   otherwise:        C = 64 * max(1, ceil(total / (64 * (budget - units))))
// so that sum_u chunks(u) <= total / C + units <= budget; for even lengths C
// is at least kMinEvenChunk (fewer chunks still).
constexpr int kPlanThreads = 1024;

// `count(u)` returns n_slots of unit u.
template <typename Count>
__device__ inline void build_plan(int units, Count count, int32_t *plan) {
  const PlanLayout L = plan_layout(units);
  int32_t *hdr = plan + L.hdr;
  int32_t *first_chunk = plan + L.first_chunk;
  int32_t *chunk_unit = plan + L.chunk_unit;
  int32_t *merge_count = plan + L.merge_count;
  __shared__ unsigned long long s_total;
  __shared__ int s_max;
  __shared__ int s_tmp[kPlanThreads / kWave];
  if (threadIdx.x == 0) {
    s_total = 0ull;
    s_max = 0;
  }
  __syncthreads();
  long long part = 0;
  int mx = 0;
  for (int u = threadIdx.x; u < units; u += kPlanThreads) {
    const int n = count(u);
    part += n;
    mx = max(mx, n);
  }
  for (int o = 32; o > 0; o >>= 1) {
    part += __shfl_xor(part, o, kWave);
    mx = max(mx, __shfl_xor(mx, o, kWave));
  }
  if (lane_id() == 0) {
    atomicAdd(&s_total, (unsigned long long)part);
    atomicMax(&s_max, mx);
  }
  __syncthreads();
  const long long total = (long long)s_total;
  const bool ragged = (long long)s_max * units > 2 * total;
  const int budget = (ragged ? kRaggedRounds : 1) * kTargetChunks;
  long long per;
  if (units >= budget) {
    per = (s_max + kPage - 1) / kPage;
  } else {
    const long long room = (long long)kPage * (budget - units);
    per = (total + room - 1) / room;
  }
  const int C = max(ragged ? kPage : kMinEvenChunk, kPage * int(per < 1 ? 1 : per));
  int carry = 0;
  for (int base = 0; base < units; base += kPlanThreads) {
    const int u = base + threadIdx.x;
    int nch = 0;
    if (u < units) {
      const int n = count(u);
      nch = n > 0 ? (n + C - 1) / C : 1;
    }
    const int w = threadIdx.x / kWave, l = lane_id();
    int incl = wave_inclusive_scan(nch);
    if (l == kWave - 1) s_tmp[w] = incl;
    __syncthreads();
    if (w == 0) {
      int v = (l < kPlanThreads / kWave) ? s_tmp[l] : 0;
      v = wave_inclusive_scan(v);
      if (l < kPlanThreads / kWave) s_tmp[l] = v;
    }
    __syncthreads();
    incl += (w > 0 ? s_tmp[w - 1] : 0) + carry;
    const int blk_total = s_tmp[kPlanThreads / kWave - 1];
    __syncthreads();
    if (u < units) {
      const int first = incl - nch;
      first_chunk[u] = first;
      merge_count[u] = 0;
      for (int i = 0; i < nch; ++i) chunk_unit[first + i] = u;
    }
    carry += blk_total;
  }
  if (threadIdx.x == 0) {
    first_chunk[units] = carry;
    hdr[0] = carry;
    hdr[1] = C;
  }
}

// ---- page layout ----------------------------------------------------------
// A page holds 64 slots of one unit as two groups of 32 slots; each group
// stores its keys in 32*D elements and its values in 32*D elements, ordered so
// that every operand fragment of the decode kernel's matrix products is one
// contiguous 1 KB block (64 lanes x 16 bytes for bf16):
//   key   (slot j, dim d): fragment (t, ks) of 16 slots x 32 dims, lane q*16 + r
//         holds dims ks*32 + q*8 .. +8 of the slot at tile row r, where slot
//         js = j % 32 sits in tile t = (js % 8) / 4 at row r = 4*(js / 8) + js % 4
//   value (slot j, dim d): fragment dt of 16 dims x 32 slots, lane q*16 + (d % 16)
//         holds slots 8q .. 8q + 7 of the group for dim d
// Within a fragment, element e of lane l is at l*8 + e.  Eight consecutive dims
// of a key, and eight consecutive slots of a value dim, are contiguous.
__host__ __device__ inline int key_index(int j, int d, int D) {
  const int grp = j >> 5, js = j & 31;
  const int t = (js & 7) >> 2, r = 4 * (js >> 3) + (js & 3);
  const int ks = d >> 5, q = (d >> 3) & 3, e = d & 7;
  return grp * 32 * D + (((t * (D >> 5) + ks) * 4 + q) * 16 + r) * 8 + e;
}

__host__ __device__ inline int value_index(int j, int d, int D) {
  const int grp = j >> 5, js = j & 31;
  const int q = js >> 3, e = js & 7;
  const int dt = d >> 4, rr = d & 15;
  return grp * 32 * D + ((dt * 4 + q) * 16 + rr) * 8 + e;
}

// The decision: marked for eviction iff logit > 0 (+0, -0, NaN and negatives
// keep).  Tested on the bits so that no floating-point compile flag can
// change how NaN is treated: the positive floats, +inf included, are exactly
// the bit patterns 0x00000001 .. 0x7f800000.
__device__ __forceinline__ bool evict_decision(float logit) {
  const uint32_t u = __float_as_uint(logit);
  return u - 1u < 0x7f800000u;
}

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

}  // namespace dms
