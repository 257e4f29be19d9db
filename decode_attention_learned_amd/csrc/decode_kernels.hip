// Decode attention over the retained entries: split plan, split-K kernels,
// log-sum-exp merge.
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
// Split-K: the plan kernel cuts each unit's slot list into chunks of C slots
// (C a multiple of the page size, chosen from the total live length so that
// about kTargetChunks chunks exist), each chunk produces (m, l, o) per head,
// and the merge kernel combines them:
//   M = max_c m_c,  L = sum_c l_c e^(m_c - M),  out = sum_c o_c e^(m_c - M) / L.
#include "dms_internal.h"

namespace dms {

// ---------------------------------------------------------------------------
// plan (one workgroup)
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void k_decode_plan(int units,
                                                              const int32_t *__restrict__ n_slots,
                                                              int32_t *__restrict__ hdr,
                                                              int32_t *__restrict__ first_chunk,
                                                              int32_t *__restrict__ chunk_unit) {
  __shared__ long long s_total;
  __shared__ int s_tmp[kPlanThreads / kWave];
  if (threadIdx.x == 0) s_total = 0;
  __syncthreads();
  long long part = 0;
  for (int u = threadIdx.x; u < units; u += kPlanThreads) part += n_slots[u];
  // wave reduce then one atomic per wave
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, kWave);
  if (lane_id() == 0) atomicAdd(reinterpret_cast<unsigned long long *>(&s_total),
                                (unsigned long long)part);
  __syncthreads();
  const long long total = s_total;
  const long long per = (total + (long long)kPage * kTargetChunks - 1) / ((long long)kPage * kTargetChunks);
  const int C = kPage * int(per < 1 ? 1 : per);

  int carry = 0;
  for (int base = 0; base < units; base += kPlanThreads) {
    const int u = base + threadIdx.x;
    int nch = 0;
    if (u < units) {
      const int n = n_slots[u];
      nch = n > 0 ? (n + C - 1) / C : 1;
    }
    // block inclusive scan
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

// ---------------------------------------------------------------------------
// generic split-K decode (VALU, float32 arithmetic, either element type)
//
// One workgroup per chunk.  Tiles of 32 slots are staged in LDS as float32;
// scores are formed per (head, slot), each head's online softmax is advanced
// by one wave, and each thread accumulates its (head, d) outputs.
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
    int hkv, int window, int maxp, float scale_log2, const E *__restrict__ q,
    const E *__restrict__ k_pages, const E *__restrict__ v_pages,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ slot_pos,
    const uint8_t *__restrict__ slot_alpha, const int32_t *__restrict__ n_slots,
    const int32_t *__restrict__ n_clean_arr, const int32_t *__restrict__ seq_len,
    const int32_t *__restrict__ hdr, const int32_t *__restrict__ first_chunk,
    const int32_t *__restrict__ chunk_unit, float2 *__restrict__ part_ml,
    float *__restrict__ part_o, float *__restrict__ out) {
  constexpr int OPT = (G * D + 255) / 256;  // outputs per thread
  const int c = blockIdx.x;
  if (c >= hdr[0]) return;
  const int C = hdr[1];
  const int u = chunk_unit[c];
  const int b = u / hkv, h = u % hkv;
  const int first = first_chunk[u];
  const int nch = first_chunk[u + 1] - first;
  const int n = n_slots[u];
  const int s_begin = (c - first) * C;
  const int s_end = min(n, s_begin + C);
  const int t = seq_len[b] - 1;
  const int nclean = n_clean_arr[u];
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();

  __shared__ float s_q[G][D];
  __shared__ float s_k[kGenTile][D + 1];
  __shared__ float s_v[D][kGenTile + 1];
  __shared__ float s_p[G][kGenTile];
  __shared__ float s_m[G], s_l[G], s_corr[G];

  for (int x = tid; x < G * D; x += 256) {
    const int g = x / D, d = x % D;
    s_q[g][d] = load_elem<E>(q + (size_t(b) * hkv * G + h * G + g) * D + d);
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
      s_k[j][d] = j < nt ? load_elem<E>(k_pages + (size_t(page) * kPage + off0 + j) * D + d) : 0.f;
    }
    for (int x = tid; x < D * kGenTile; x += 256) {
      const int d = x / kGenTile, j = x % kGenTile;
      s_v[d][j] = j < nt ? load_elem<E>(v_pages + (size_t(page) * D + d) * kPage + off0 + j) : 0.f;
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
          live = slot_alpha[m] == 0 || (t - slot_pos[m]) < window;
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

  if (nch == 1) {
#pragma unroll
    for (int r = 0; r < OPT; ++r) {
      const int x = tid + r * 256;
      if (x < G * D) {
        const int g = x / D, d = x % D;
        const float l = s_l[g];
        out[(size_t(b) * hkv * G + h * G + g) * D + d] = l > 0.f ? acc[r] / l : 0.f;
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < OPT; ++r) {
      const int x = tid + r * 256;
      if (x < G * D) part_o[size_t(c) * G * D + x] = acc[r];
    }
    if (tid < G) part_ml[size_t(c) * G + tid] = make_float2(s_m[tid], s_l[tid]);
  }
}

// ---------------------------------------------------------------------------
// merge: one workgroup per unit with more than one chunk
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_decode_merge(int hkv, int G, int D,
                                                      const int32_t *__restrict__ first_chunk,
                                                      const float2 *__restrict__ part_ml,
                                                      const float *__restrict__ part_o,
                                                      float *__restrict__ out) {
  const int u = blockIdx.x;
  const int first = first_chunk[u];
  const int nch = first_chunk[u + 1] - first;
  if (nch <= 1) return;
  const int b = u / hkv, h = u % hkv;
  for (int x = threadIdx.x; x < G * D; x += blockDim.x) {
    const int g = x / D;
    float M = -INFINITY;
    for (int i = 0; i < nch; ++i) M = fmaxf(M, part_ml[size_t(first + i) * G + g].x);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int i = 0; i < nch; ++i) {
        const float2 ml = part_ml[size_t(first + i) * G + g];
        if (ml.x == -INFINITY) continue;
        const float w = exp2f(ml.x - M);
        L = fmaf(ml.y, w, L);
        O = fmaf(part_o[size_t(first + i) * G * D + x], w, O);
      }
    }
    out[(size_t(b) * hkv * G + h * G) * D + x] = L > 0.f ? O / L : 0.f;
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <typename E, int D, int G>
static void launch_generic_t(const dms_shape &s, const dms_cache &c, const E *q, float *out,
                             float scale_log2, const DecodeWorkspace &w, char *ws, hipStream_t st) {
  hipLaunchKernelGGL((k_decode_generic<E, D, G>), dim3(w.max_chunks), dim3(256), 0, st, s.kv_heads,
                     s.window, s.max_pages_per_unit, scale_log2, q, static_cast<const E *>(c.k_pages),
                     static_cast<const E *>(c.v_pages), c.page_table, c.slot_pos, c.slot_alpha,
                     c.n_slots, c.n_clean, c.seq_len, reinterpret_cast<const int32_t *>(ws + w.hdr),
                     reinterpret_cast<const int32_t *>(ws + w.first_chunk),
                     reinterpret_cast<const int32_t *>(ws + w.chunk_unit),
                     reinterpret_cast<float2 *>(ws + w.part_ml), reinterpret_cast<float *>(ws + w.part_o),
                     out);
}

template <typename E, int D>
static bool dispatch_group(const dms_shape &s, const dms_cache &c, const E *q, float *out,
                           float scale_log2, const DecodeWorkspace &w, char *ws, hipStream_t st) {
  switch (s.group) {
#define DMS_G(GG) case GG: launch_generic_t<E, D, GG>(s, c, q, out, scale_log2, w, ws, st); return true;
    DMS_G(1) DMS_G(2) DMS_G(3) DMS_G(4) DMS_G(5) DMS_G(6) DMS_G(7) DMS_G(8)
    DMS_G(9) DMS_G(10) DMS_G(11) DMS_G(12) DMS_G(13) DMS_G(14) DMS_G(15) DMS_G(16)
#undef DMS_G
    default: return false;
  }
}

bool launch_decode_mfma(const dms_shape &s, const dms_cache &c, const void *q, float *out,
                        float scale_log2, const DecodeWorkspace &w, char *ws, hipStream_t st);

hipError_t launch_decode(const dms_shape &s, const dms_cache &c, const void *q, float *out,
                         float sm_scale, void *wsv, hipStream_t st) {
  const int units = units_of(s);
  const DecodeWorkspace w = decode_workspace_layout(units, s.group, s.head_dim);
  char *ws = static_cast<char *>(wsv);
  hipLaunchKernelGGL(k_decode_plan, dim3(1), dim3(kPlanThreads), 0, st, units, c.n_slots,
                     reinterpret_cast<int32_t *>(ws + w.hdr),
                     reinterpret_cast<int32_t *>(ws + w.first_chunk),
                     reinterpret_cast<int32_t *>(ws + w.chunk_unit));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale_log2 = sm_scale * 1.4426950408889634f;  // exp(x) = exp2(x * log2 e)
  bool done = false;
  if (s.kv_dtype == DMS_KV_BF16) {
    done = launch_decode_mfma(s, c, q, out, scale_log2, w, ws, st);
    if (!done)
      done = s.head_dim == 64
                 ? dispatch_group<uint16_t, 64>(s, c, static_cast<const uint16_t *>(q), out, scale_log2, w, ws, st)
                 : dispatch_group<uint16_t, 128>(s, c, static_cast<const uint16_t *>(q), out, scale_log2, w, ws, st);
  } else {
    done = s.head_dim == 64
               ? dispatch_group<uint32_t, 64>(s, c, static_cast<const uint32_t *>(q), out, scale_log2, w, ws, st)
               : dispatch_group<uint32_t, 128>(s, c, static_cast<const uint32_t *>(q), out, scale_log2, w, ws, st);
  }
  if (!done) return hipErrorInvalidValue;
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_merge, dim3(units), dim3(256), 0, st, s.kv_heads, s.group, s.head_dim,
                     reinterpret_cast<const int32_t *>(ws + w.first_chunk),
                     reinterpret_cast<const float2 *>(ws + w.part_ml),
                     reinterpret_cast<const float *>(ws + w.part_o), out);
  return hipGetLastError();
}

}  // namespace dms
