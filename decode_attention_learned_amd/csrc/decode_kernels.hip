// Decode attention over the retained entries: generic split-K kernel and the
// launch path shared with the MFMA kernel.
//
// Method: atlas.scime.ai summary of "Inference-Time Hyper-Scaling with KV
// Cache Compression", section "Approach": attention reads only the entries a
// head has not evicted; a marked entry stays readable for the delay window.
// zhaoyang97 Paper-Notes, motivation section: each decode step reads the whole
// (retained) cache, so the step is bound by memory bandwidth.
//
// For query head hq = h*G + g of sequence b at t = seq_len[b] - 1:
//   out = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m),  s_j = scale * <q, k_j>,
// over the slots j of unit (b, h) alive at t.  A slot below n_clean is alive
// by construction; above it, alive iff !alpha or t - pos < w.
//
// Split-K: the plan (kept in cache state, see build_plan) cuts each unit's
// slot list into chunks of C slots; each chunk produces (m, l, o) per head,
// and a unit split into several chunks is merged with the log-sum-exp rule:
// by a merge launch right after the decode launch for plans of fewer than
// kTargetChunks units, else by the unit's last chunk to finish inside the
// decode launch (decode_common.h).  Scores are
// kept in log2 units (scale * log2 e folded into the score) so that every
// exponential is exp2.
#include "decode_common.h"

namespace dms {

// ---------------------------------------------------------------------------
// generic split-K decode (VALU, float32 arithmetic, either element type)
//
// The reference path of the test build (libdms_generic.so routes one-query
// decode of bf16 caches here), against which tests check the matrix-core
// kernels; the product library reaches it only for shapes those kernels
// refuse.  One workgroup per chunk.  Tiles of 32 slots are staged in LDS as float32;
// scores are formed per (head, slot), each head's online softmax is advanced
// by one wave, and each thread accumulates its (head, d) outputs.  One query
// per sequence: query cq of a chunk of C tokens just appended, at position
// seq_len - C + cq (decode: C = 1, cq = 0); slots above n_clean are seen when
// their position is at most the query's and they are alive there.
// `chunk_status` (chunk queries only, else null): as in the matrix-core kernel.
// ---------------------------------------------------------------------------
constexpr int kGenTile = 32;

template <typename E>
__device__ __forceinline__ float load_elem(const E *p);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float load_elem<uint32_t>(const uint32_t *p) { return __uint_as_float(*p); }

template <typename E, int D, int G>
__global__ __launch_bounds__(256) void k_decode_generic(
    int units, int hkv, int window, int maxp, float scale_log2, int C, int cq,
    const E *__restrict__ q, const E *__restrict__ k_pages, const E *__restrict__ v_pages,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ slot_pos,
    const uint8_t *__restrict__ slot_alpha, const int32_t *__restrict__ n_slots,
    const int32_t *__restrict__ n_clean_arr, const int32_t *__restrict__ seq_len,
    int32_t *__restrict__ plan, uint32_t *__restrict__ chunk_status, float2 *__restrict__ part_ml,
    float *__restrict__ part_o, float *__restrict__ out) {
  constexpr int OPT = (G * D + 255) / 256;  // outputs per thread
  const PlanLayout L = plan_layout(units);
  const int c = blockIdx.x;
  ChunkInfo ci;
  if (!locate_chunk(c, hkv, plan, n_slots, n_clean_arr, seq_len, L, ci)) return;
  const int u = ci.unit, b = ci.b, h = ci.h;
  const int s_begin = ci.s_begin, s_end = ci.s_end, nclean = ci.nclean;
  const int t = ci.t - (C - 1) + cq;  // the query's position
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  if (chunk_status != nullptr && cq == 0 && c == ci.first && tid == 0) {
    const int p0 = ci.t - (C - 1);  // the chunk's first position
    if (p0 < 0 || plan[L.compact_pos + u] > p0) atomicOr(chunk_status, DMS_STATUS_CHUNK_INVALID);
  }
  // output of column x / D (query head h * G + x / D)
  const OutMap om{((size_t(b) * C + cq) * hkv * G + size_t(h) * G) * D, size_t(hkv) * G * D, G, D};

  __shared__ float s_q[G][D];
  __shared__ float s_k[kGenTile][D + 1];
  __shared__ float s_v[D][kGenTile + 1];
  __shared__ float s_p[G][kGenTile];
  __shared__ float s_m[G], s_l[G], s_corr[G];

  for (int x = tid; x < G * D; x += 256) {
    const int g = x / D, d = x % D;
    s_q[g][d] = load_elem<E>(q + ((size_t(b) * C + cq) * hkv * G + h * G + g) * D + d);
  }
  if (tid < G) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  float acc[OPT];
#pragma unroll
  for (int r = 0; r < OPT; ++r) acc[r] = 0.f;
  __syncthreads();

  for (int s0 = s_begin; s0 < s_end; s0 += kGenTile) {
    const int page = page_table[size_t(u) * maxp + s0 / kPage];
    const int off0 = s0 % kPage;  // 0 or 32
    const int nt = min(kGenTile, s_end - s0);
    for (int x = tid; x < kGenTile * D; x += 256) {
      const int j = x / D, d = x % D;
      s_k[j][d] = j < nt ? load_elem<E>(k_pages + size_t(page) * kPage * D + key_index(off0 + j, d, D)) : 0.f;
    }
    for (int x = tid; x < D * kGenTile; x += 256) {
      const int d = x / kGenTile, j = x % kGenTile;
      s_v[d][j] = j < nt ? load_elem<E>(v_pages + size_t(page) * kPage * D + value_index(off0 + j, d, D)) : 0.f;
    }
    __syncthreads();
    for (int x = tid; x < G * kGenTile; x += 256) {
      const int g = x / kGenTile, j = x % kGenTile;
      float s = -INFINITY;
      if (j < nt) {
        const int slot = s0 + j;
        bool live = slot < nclean;
        if (!live) {
          const size_t m = size_t(page) * kPage + off0 + j;
          const int pos = slot_pos[m];
          live = pos <= t && (slot_alpha[m] == 0 || (t - pos) < window);
        }
        if (live) {
          float dot = 0.f;
#pragma unroll 8
          for (int d = 0; d < D; ++d) dot = fmaf(s_q[g][d], s_k[j][d], dot);
          s = dot * scale_log2;  // score in log2 units
        }
      }
      s_p[g][j] = s;
    }
    __syncthreads();
    for (int g = wave; g < G; g += 4) {
      const float s = lane < kGenTile ? s_p[g][lane] : -INFINITY;
      const float m_old = s_m[g];
      const float m_new = fmaxf(m_old, wave_max(s));
      float p = 0.f, corr = 1.f;
      if (m_new != -INFINITY) {
        p = (s == -INFINITY) ? 0.f : exp2f(s - m_new);
        corr = (m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new);
      }
      const float psum = wave_sum(p);
      if (lane < kGenTile) s_p[g][lane] = p;
      if (lane == 0) {
        s_l[g] = s_l[g] * corr + psum;
        s_m[g] = m_new;
        s_corr[g] = corr;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < OPT; ++r) {
      const int x = tid + r * 256;
      if (x < G * D) {
        const int g = x / D, d = x % D;
        float a = acc[r] * s_corr[g];
#pragma unroll 8
        for (int j = 0; j < kGenTile; ++j) a = fmaf(s_p[g][j], s_v[d][j], a);
        acc[r] = a;
      }
    }
    __syncthreads();
  }

  if (ci.nch == 1) {
#pragma unroll
    for (int r = 0; r < OPT; ++r) {
      const int x = tid + r * 256;
      if (x < G * D) {
        const int g = x / D;
        const float l = s_l[g];
        out[om.at(x)] = l > 0.f ? acc[r] / l : 0.f;
      }
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < OPT; ++r) {
    const int x = tid + r * 256;
    if (x < G * D) publish(part_o + size_t(c) * G * D + x, acc[r]);
  }
  if (tid < G) {
    publish(reinterpret_cast<float *>(part_ml + size_t(c) * G + tid), s_m[tid]);
    publish(reinterpret_cast<float *>(part_ml + size_t(c) * G + tid) + 1, s_l[tid]);
  }
  if (!fused_merge(units)) return;  // merged by k_merge_partials
  count_and_merge(ci, G, D, plan + L.merge_count, part_ml, part_o, out, om);
}

// ---------------------------------------------------------------------------
// Deferred merge (plans of fewer than kTargetChunks units): one workgroup per
// unit combines the partials its chunks wrote in the decode launch before it
// on the stream.  Units of one chunk were written by the decode launch itself.
// Output columns ncol = queries x G of the launch; c0 and C place them as in
// the decode launch (one query: c0 = 0, C = 1).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_merge_partials(int units, int hkv, int ncol, int G, int D,
                                                        int c0, int C, const int32_t *__restrict__ plan,
                                                        const float2 *__restrict__ part_ml,
                                                        const float *__restrict__ part_o,
                                                        float *__restrict__ out) {
  const PlanLayout L = plan_layout(units);
  const int u = blockIdx.x;
  const int first = plan[L.first_chunk + u];
  const int nch = plan[L.first_chunk + u + 1] - first;
  if (nch <= 1) return;
  const int b = u / hkv, h = u % hkv;
  const OutMap om{((size_t(b) * C + c0) * hkv * G + size_t(h) * G) * D, size_t(hkv) * G * D, G, D};
  merge_unit(first, nch, ncol, D, part_ml, part_o, out, om);
}

hipError_t launch_merge(const dms_shape &s, const dms_cache &c, const DecodeWorkspace &w, char *ws,
                        float *out, int ncol, int c0, int C, hipStream_t st) {
  if (fused_merge(units_of(s))) return hipSuccess;
  hipLaunchKernelGGL(k_merge_partials, dim3(units_of(s)), dim3(256), 0, st, units_of(s), s.kv_heads,
                     ncol, s.group, s.head_dim, c0, C, c.plan,
                     reinterpret_cast<const float2 *>(ws + w.part_ml),
                     reinterpret_cast<const float *>(ws + w.part_o), out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
// query cq of a chunk of C (decode: C = 1, cq = 0); chunk_status only for chunk queries
template <typename E, int D, int G>
static void launch_generic_t(const dms_shape &s, const dms_cache &c, const E *q, float *out,
                             float scale_log2, const DecodeWorkspace &w, char *ws, hipStream_t st,
                             int C, int cq, uint32_t *chunk_status) {
  hipLaunchKernelGGL((k_decode_generic<E, D, G>), dim3(w.max_chunks), dim3(256), 0, st,
                     units_of(s), s.kv_heads, s.window, s.max_pages_per_unit, scale_log2, C, cq, q,
                     static_cast<const E *>(c.k_pages), static_cast<const E *>(c.v_pages),
                     c.page_table, c.slot_pos, c.slot_alpha, c.n_slots, c.n_clean, c.seq_len,
                     c.plan, chunk_status, reinterpret_cast<float2 *>(ws + w.part_ml),
                     reinterpret_cast<float *>(ws + w.part_o), out);
}

template <typename E, int D>
static bool dispatch_group(const dms_shape &s, const dms_cache &c, const E *q, float *out,
                           float scale_log2, const DecodeWorkspace &w, char *ws, hipStream_t st,
                           int C = 1, int cq = 0, uint32_t *chunk_status = nullptr) {
  switch (s.group) {
#define DMS_G(GG)                                                                       \
  case GG:                                                                              \
    launch_generic_t<E, D, GG>(s, c, q, out, scale_log2, w, ws, st, C, cq, chunk_status); \
    return true;
    DMS_G(1) DMS_G(2) DMS_G(3) DMS_G(4) DMS_G(5) DMS_G(6) DMS_G(7) DMS_G(8)
    DMS_G(9) DMS_G(10) DMS_G(11) DMS_G(12) DMS_G(13) DMS_G(14) DMS_G(15) DMS_G(16)
#undef DMS_G
    default: return false;
  }
}

bool launch_decode_mfma(const dms_shape &s, const dms_cache &c, const void *q, float *out,
                        float scale_log2, const DecodeWorkspace &w, char *ws, hipStream_t st,
                        int n_query, const DecodeFill *fill, bool chunk);
bool launch_decode_f32(const dms_shape &s, const dms_cache &c, const void *q, float *out,
                       float scale_log2, const DecodeWorkspace &w, char *ws, hipStream_t st, int nq,
                       int c0, int C, uint32_t *chunk_status);

// The decode grid has one workgroup per possible chunk (max_chunks_of(units));
// workgroups past the plan's chunk count exit at once.  Plans of fewer than
// kTargetChunks units are merged by a second launch (launch_merge).  bf16
// caches run the bf16 matrix-core kernel, float32 caches the float32 one
// (decode_f32.hip); the vector kernel serves the test build that routes bf16
// decode to it.  With `fill`, the bf16 matrix-core kernel writes the reserved
// token itself; the other kernels take it from a write launch ahead of them.
hipError_t launch_decode(const dms_shape &s, const dms_cache &c, const void *q, float *out,
                         float sm_scale, void *wsv, hipStream_t st, const DecodeFill *fill) {
  const DecodeWorkspace w = decode_workspace_layout(units_of(s), s.group, s.head_dim);
  char *ws = static_cast<char *>(wsv);
  const float scale_log2 = sm_scale * 1.4426950408889634f;  // exp(x) = exp2(x * log2 e)
  bool done = false;
  if (s.kv_dtype == DMS_KV_BF16)
    done = launch_decode_mfma(s, c, q, out, scale_log2, w, ws, st, 1, fill, false);
  const bool mfma = done;
  if (!done && fill) {
    const hipError_t e = launch_append_write(s, c, fill->k_new, fill->v_new, fill->logit, 1, st);
    if (e != hipSuccess) return e;
  }
  if (s.kv_dtype == DMS_KV_BF16) {
    if (!done)
      done = s.head_dim == 64
                 ? dispatch_group<uint16_t, 64>(s, c, static_cast<const uint16_t *>(q), out, scale_log2, w, ws, st)
                 : dispatch_group<uint16_t, 128>(s, c, static_cast<const uint16_t *>(q), out, scale_log2, w, ws, st);
  } else {
    done = launch_decode_f32(s, c, q, out, scale_log2, w, ws, st, 1, 0, 1, nullptr);
  }
  if (!done) return hipErrorInvalidValue;
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the matrix-core launcher merges after each of its launches itself
  if (s.kv_dtype == DMS_KV_BF16 && mfma) return hipSuccess;
  return launch_merge(s, c, w, ws, out, s.group, 0, 1, st);
}

// Queries of a chunk of n_query tokens just appended.  Long chunks (32
// queries or more) run a tiled chunk kernel, one pass over the cache per 32
// queries (bf16: matrix cores in bf16; float32: the float32 matrix
// instruction).  Shorter ones run the split-K decode kernel of the cache's
// dtype in launches of at most 16 / G queries (the matrix products' 16
// columns), each merged after it.  The workspace holds partials for 16
// columns.
constexpr int kChunkKernelMin = 32;

hipError_t launch_decode_multi(const dms_shape &s, const dms_cache &c, const void *q, int n_query,
                               float *out, float sm_scale, void *wsv, size_t ws_bytes, hipStream_t st) {
  const DecodeWorkspace w = decode_workspace_layout(units_of(s), 16, s.head_dim);
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  if (s.kv_dtype == DMS_KV_F32 && n_query >= kChunkKernelMin)
    return launch_chunk_f32(s, c, q, n_query, out, sm_scale, st);
  if (s.kv_dtype == DMS_KV_F32) {
    char *ws = static_cast<char *>(wsv);
    const int per = 16 / s.group;  // queries per launch
    for (int c0 = 0; c0 < n_query; c0 += per) {
      const int nq = n_query - c0 < per ? n_query - c0 : per;
      if (!launch_decode_f32(s, c, q, out, scale_log2, w, ws, st, nq, c0, n_query, c.status))
        return hipErrorInvalidValue;
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const hipError_t m = launch_merge(s, c, w, ws, out, nq * s.group, c0, n_query, st);
      if (m != hipSuccess) return m;
    }
    return hipSuccess;
  }
  if (n_query >= kChunkKernelMin && s.group <= 16)
    return launch_chunk_attn(s, c, q, n_query, out, sm_scale, wsv, ws_bytes, st);
  if (!launch_decode_mfma(s, c, q, out, scale_log2, w, static_cast<char *>(wsv), st, n_query,
                          nullptr, true))
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dms
