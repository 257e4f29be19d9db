// Masked prefill attention for float32 inputs, on the vector units.
//
// Method and visibility rule as in prefill.hip: atlas.scime.ai summary of
// "Inference-Time Hyper-Scaling with KV Cache Compression", section
// "Approach" (binary per-head decision, eviction carried out after a delay
// window) and table "Measured effects reported in the paper" (16-token
// window).  Query row i of head hq sees key j of KV head hq / G iff
//   j <= i  and  not (alpha_j and i - j >= w),   alpha_j = logit_j > 0,
// and out = softmax_j(scale * <q_i, k_j>) v_j over the visible keys.  The
// relaxed (training-form) rule replaces the exclusion by the additive term
// log(1 - sigmoid((logit_j + noise_j) / tau)) for i - j >= w.
//
// The matrix cores of gfx950 take bf16 operands for this contraction at
// full rate; float32 inputs are kept exact here and take the vector units:
// products and sums in float32, the softmax in exp2 form with an exact
// running maximum.
//
// Work decomposition.  A workgroup of 256 threads takes 32 query rows of one
// query head.  Key tiles of 32 keys (keys, values and each key's decision or
// relaxed term) are staged in LDS with the query rows.  Eight consecutive
// lanes serve one query row: for the scores each takes 4 keys of the tile,
// for the output D / 8 consecutive dims.  Under the hard rule a tile whose
// keys are all marked and all at least w behind every query of the block
// adds nothing and is skipped, so the work follows the visible keys.
#include "dms_internal.h"

namespace dms {

namespace {

constexpr int FQB = 32;   // query rows per workgroup
constexpr int FKT = 32;   // keys per tile
constexpr int FNT = 256;  // threads per workgroup (8 per query row)
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__global__ __launch_bounds__(FNT) void k_prefill_f32(int S, int hkv, int G, int window,
                                                     float scale_log2, int relaxed, float inv_tau,
                                                     const float *__restrict__ q,
                                                     const float *__restrict__ k,
                                                     const float *__restrict__ v,
                                                     const float *__restrict__ logit,
                                                     const float *__restrict__ noise,
                                                     float *__restrict__ out) {
  constexpr int D4 = D / 4;   // float4 per row
  constexpr int RP = D4 + 1;  // padded row (float4), against bank conflicts between rows
  constexpr int OD4 = D4 / 8; // output float4 per thread
  const int qb = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int h = hq / G, Hq = hkv * G;
  const int i0 = qb * FQB;
  const int tid = threadIdx.x;
  const int r = tid >> 3, sub = tid & 7;  // query row in the block, lane within the row
  const int i = i0 + r;
  const int i_last = min(S, i0 + FQB) - 1;

  __shared__ float4 sQ[FQB][RP];
  __shared__ float4 sK[FKT][RP];
  __shared__ float4 sV[FKT][RP];
  __shared__ float sP[FQB][FKT + 1];
  __shared__ float sB[FKT];  // per key: additive term (log2 units) for i - j >= w

  for (int x = tid; x < FQB * D4; x += FNT) {
    const int rr = x / D4, c = x % D4;
    const int ii = i0 + rr;
    sQ[rr][c] = ii < S ? reinterpret_cast<const float4 *>(q + ((size_t(b) * S + ii) * Hq + hq) * D)[c]
                       : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  float4 o[OD4];
#pragma unroll
  for (int x = 0; x < OD4; ++x) o[x] = make_float4(0.f, 0.f, 0.f, 0.f);
  float m_run = -INFINITY, l_run = 0.f;  // l_run: this lane's share of the row sum

  for (int j0 = 0; j0 <= i_last; j0 += FKT) {
    // sB is rewritten here: every thread is past the previous tile's scores
    // (the barrier before its PV product)
    const bool far = j0 + FKT - 1 + window <= i0;  // every key >= w behind every query
    bool live = false;
    if (tid < FKT) {
      const int j = j0 + tid;
      float bias = 0.f;
      live = j < S;
      if (j < S) {
        const size_t at = (size_t(b) * S + j) * hkv + h;
        if (relaxed) {
          // log(1 - sigmoid(x)) = -softplus(x), in log2 units
          const float x = (logit[at] + (noise ? noise[at] : 0.f)) * inv_tau;
          bias = -(fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)))) * kLog2e;
        } else if (evict_decision(logit[at])) {
          bias = -INFINITY;
          live = !far;
        }
      }
      sB[tid] = bias;
    }
    // hard rule: a tile whose keys are all marked and out of every query's
    // window is skipped (the barrier also publishes sB and, first time, sQ)
    if (!__syncthreads_or(live)) continue;
    for (int x = tid; x < FKT * D4; x += FNT) {
      const int jj = x / D4, c = x % D4;
      const int j = j0 + jj;
      const size_t row = ((size_t(b) * S + j) * hkv + h) * D;
      sK[jj][c] = j < S ? reinterpret_cast<const float4 *>(k + row)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      sV[jj][c] = j < S ? reinterpret_cast<const float4 *>(v + row)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();

    // scores of row r for keys j0 + 4 sub .. + 3
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int c = 0; c < D4; ++c) {
      const float4 qv = sQ[r][c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 kv = sK[4 * sub + e][c];
        acc[e] = fmaf(qv.x, kv.x, acc[e]);
        acc[e] = fmaf(qv.y, kv.y, acc[e]);
        acc[e] = fmaf(qv.z, kv.z, acc[e]);
        acc[e] = fmaf(qv.w, kv.w, acc[e]);
      }
    }
    float s[4];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jj = 4 * sub + e, j = j0 + jj;
      const float add = i - j >= window ? sB[jj] : 0.f;
      s[e] = (j <= i && i < S) ? fmaf(acc[e], scale_log2, add) : -INFINITY;
      mx = fmaxf(mx, s[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 2, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 4, kWave));
    const float m_new = fmaxf(m_run, mx);
    // corr rescales what was accumulated against m_run; nothing visible yet: 0
    const float corr = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
    const float m_sub = m_new == -INFINITY ? 0.f : m_new;
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = exp2f(s[e] - m_sub);
      sP[r][4 * sub + e] = p;
      lsum += p;
    }
    l_run = fmaf(l_run, corr, lsum);
    m_run = m_new;
    __syncthreads();  // the row's weights are in LDS

    // output dims 4 (sub * OD4 + x) .. + 3 of row r
#pragma unroll
    for (int x = 0; x < OD4; ++x) {
      o[x].x *= corr;
      o[x].y *= corr;
      o[x].z *= corr;
      o[x].w *= corr;
    }
    for (int jj = 0; jj < FKT; ++jj) {
      const float p = sP[r][jj];
#pragma unroll
      for (int x = 0; x < OD4; ++x) {
        const float4 vv = sV[jj][sub * OD4 + x];
        o[x].x = fmaf(p, vv.x, o[x].x);
        o[x].y = fmaf(p, vv.y, o[x].y);
        o[x].z = fmaf(p, vv.z, o[x].z);
        o[x].w = fmaf(p, vv.w, o[x].w);
      }
    }
  }
  float l = l_run;
  l += __shfl_xor(l, 1, kWave);
  l += __shfl_xor(l, 2, kWave);
  l += __shfl_xor(l, 4, kWave);
  if (i >= S) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float4 *dst = reinterpret_cast<float4 *>(out + ((size_t(b) * S + i) * Hq + hq) * D) + sub * OD4;
#pragma unroll
  for (int x = 0; x < OD4; ++x)
    dst[x] = make_float4(o[x].x * inv, o[x].y * inv, o[x].z * inv, o[x].w * inv);
}

template <int D>
hipError_t launch_t(const dms_shape &s, const float *q, const float *k, const float *v,
                    const float *logit, const float *noise, float temperature, int seq_len,
                    float sm_scale, float *out, hipStream_t st) {
  const int hq = s.kv_heads * s.group;
  if (hq > 65535 || s.batch > 65535) return hipErrorInvalidValue;  // grid y, z
  const dim3 grid((seq_len + FQB - 1) / FQB, hq, s.batch);
  const int relaxed = temperature > 0.f;
  hipLaunchKernelGGL(k_prefill_f32<D>, grid, dim3(FNT), 0, st, seq_len, s.kv_heads, s.group,
                     s.window, sm_scale * kLog2e, relaxed, relaxed ? 1.f / temperature : 0.f, q, k, v,
                     logit, noise, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const dms_shape &s, const void *q, const void *k, const void *v,
                              const float *logit, const float *noise, float temperature,
                              int seq_len, float sm_scale, float *out, hipStream_t st) {
  const float *qf = static_cast<const float *>(q), *kf = static_cast<const float *>(k),
              *vf = static_cast<const float *>(v);
  if (s.head_dim == 128)
    return launch_t<128>(s, qf, kf, vf, logit, noise, temperature, seq_len, sm_scale, out, st);
  if (s.head_dim == 64)
    return launch_t<64>(s, qf, kf, vf, logit, noise, temperature, seq_len, sm_scale, out, st);
  return hipErrorInvalidValue;
}

}  // namespace dms
