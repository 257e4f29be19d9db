// Masked prefill attention for float32 inputs, on the gfx950 matrix cores.
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
// Float32 inputs keep float32 products: the contraction runs on
// v_mfma_f32_16x16x4_f32 (float32 operands and accumulation) with the
// softmax in float32 exp2 form and an exact running maximum.
//
// Work decomposition, as in the bf16 kernel: a workgroup of four waves
// takes 32 query positions of one KV head, wave w serving query head
// 4 hg + w of the group; key tiles of 32 are staged once per workgroup in
// LDS and serve all four heads.  Per tile and wave
//   S^T [32 keys x 16 queries] = K [32 x D] . Q^T [D x 16]   (x2 query tiles)
//   O^T [D x 16 queries]      += V^T [D x 32 keys] . P^T [32 x 16]
// Operand layouts of v_mfma_f32_16x16x4_f32 (lane l, q = l / 16): A holds
// element (l % 16, q), B element (q, l % 16), the result rows 4q .. 4q + 3 of
// column l % 16.  The reduction index of the QK product is permuted: k-step
// ks of lane group q takes dim q * D/4 + ks, so that a lane's key and query
// dims are consecutive (one 16-byte LDS read feeds four products).  In the
// PV product k-step i of a 16-key half takes key 4q + i from lane group q:
// the key whose score that lane already holds, so P needs no lane exchange;
// values are staged transposed for it.  Under the hard rule a tile whose
// keys are all marked and out of every query's window is skipped.  The next
// tile's keys, values and logits are requested before the current one is
// computed.
#include "dms_internal.h"

namespace dms {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int FQB = 32;   // query positions per workgroup
constexpr int FKT = 32;   // keys per tile
constexpr int FHW = 4;    // query heads (waves) per workgroup
constexpr int FNT = FHW * kWave;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// QK product of one staged tile for both query tiles: s[qt][t][r] is the
// score of key 16 t + 4 quad + r for query 16 qt + col (raw units).  sK holds
// the tile's keys row-major, rows of D + 4 floats; qf the Q^T operand.
template <int D>
__device__ __forceinline__ void f32_scores(const float *sK, const float4 (&qf)[2][D / 16], int col,
                                           int quad, floatx4 (&s)[2][2]) {
  constexpr int DQ = D / 4, KR = D + 4;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int t = 0; t < 2; ++t) s[qt][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < DQ / 4; ++m) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float4 ka = *reinterpret_cast<const float4 *>(&sK[(16 * t + col) * KR + quad * DQ + 4 * m]);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        s[qt][t] = mfma4(ka.x, qf[qt][m].x, s[qt][t]);
        s[qt][t] = mfma4(ka.y, qf[qt][m].y, s[qt][t]);
        s[qt][t] = mfma4(ka.z, qf[qt][m].z, s[qt][t]);
        s[qt][t] = mfma4(ka.w, qf[qt][m].w, s[qt][t]);
      }
    }
  }
}

// Online softmax over one tile: s holds each pair's score in log2 units (or
// -inf where the key is hidden from the query) and becomes the weights p;
// the running maximum is exact, and the accumulators are rescaled when it
// moves.  l_run is this lane's share of the row sum.
template <int D>
__device__ __forceinline__ void f32_softmax(floatx4 (&s)[2][2], float (&m_run)[2], float (&l_run)[2],
                                            floatx4 (&o)[D / 16][2]) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[qt][t][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run[qt], mx);
    const float corr = m_run[qt] == -INFINITY ? 0.f : exp2f(m_run[qt] - m_new);
    const float m_sub = m_new == -INFINITY ? 0.f : m_new;
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(s[qt][t][r] - m_sub);
        s[qt][t][r] = p;
        lsum += p;
      }
    l_run[qt] = fmaf(l_run[qt], corr, lsum);
    m_run[qt] = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt][qt] *= corr;
  }
}

// PV product of one staged tile: k-step i of half t takes key 16 t + 4 quad
// + i, whose weight this lane holds in p[qt][t][i].  sVt holds the tile's
// values transposed, rows of 32 + 4 floats.
template <int D>
__device__ __forceinline__ void f32_pv(const float *sVt, const floatx4 (&p)[2][2], int col, int quad,
                                       floatx4 (&o)[D / 16][2]) {
  constexpr int VR = 32 + 4;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float4 va = *reinterpret_cast<const float4 *>(&sVt[(16 * dt + col) * VR + 16 * t + 4 * quad]);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        o[dt][qt] = mfma4(va.x, p[qt][t][0], o[dt][qt]);
        o[dt][qt] = mfma4(va.y, p[qt][t][1], o[dt][qt]);
        o[dt][qt] = mfma4(va.z, p[qt][t][2], o[dt][qt]);
        o[dt][qt] = mfma4(va.w, p[qt][t][3], o[dt][qt]);
      }
    }
  }
}

// Normalised output of query tile qt to row dst[qt] (null: not a query):
// o[dt][qt][r] is dim 16 dt + 4 quad + r of query 16 qt + col.
template <int D>
__device__ __forceinline__ void f32_store(const floatx4 (&o)[D / 16][2], const float (&l_run)[2],
                                          float *const (&dst)[2], int quad) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float l = l_run[qt];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (dst[qt] == nullptr) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const floatx4 x = o[dt][qt] * inv;
      *reinterpret_cast<float4 *>(dst[qt] + 16 * dt + 4 * quad) = make_float4(x[0], x[1], x[2], x[3]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(FNT, 2) void k_prefill_f32(int batch, int S, int hkv, int G, int window,
                                                        float scale_log2, int relaxed, float inv_tau,
                                                        const float *__restrict__ q,
                                                        const float *__restrict__ k,
                                                        const float *__restrict__ v,
                                                        const float *__restrict__ logit,
                                                        const float *__restrict__ noise,
                                                        float *__restrict__ out) {
  constexpr int DQ = D / 4;       // dims per lane group; k-steps of a QK product
  constexpr int DT = D / 16;      // 16-dim blocks of the output
  constexpr int KR = D + 4;       // sK row (floats): 16-byte rows, rotating banks
  constexpr int VR = FKT + 4;     // sVt row (floats)
  constexpr int NPT = FKT * D / 4 / FNT;  // float4 of keys (and of values) each thread stages
  const int ngh = (G + FHW - 1) / FHW;
  // Workgroup -> (b, h, hg, query block) as in the bf16 kernel: consecutive
  // ids go to different XCDs, so all query blocks of one (b, h, hg) get ids of
  // one residue modulo 8 and share an L2; the latest (longest) blocks first.
  const int nqb = (S + FQB - 1) / FQB;
  const int npairs = batch * hkv * ngh;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int pair = (slot / nqb) * 8 + xcd;
  if (pair >= npairs) return;
  const int qb = nqb - 1 - slot % nqb;
  const int b = pair / (hkv * ngh), h = (pair / ngh) % hkv, hg = pair % ngh;
  const int Hq = hkv * G;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave, col = lane & 15, quad = lane >> 4;
  const int g = hg * FHW + wave;
  const bool active = g < G;
  const int hq = h * G + (active ? g : 0);
  const int i0 = qb * FQB;
  const int i_last = min(S, i0 + FQB) - 1;

  __shared__ __align__(16) float sK[FKT * KR];   // keys, row-major
  __shared__ __align__(16) float sVt[D * VR];    // values, transposed: [dim][key]
  // per key: additive term (log2 units) once i - j >= w; two buffers by tile
  // parity, since a wave may write the next tile's while another still reads
  // this one's
  __shared__ float sB[2][FKT];

  // Q^T operand of query tile qt: query i0 + 16 qt + col, dims quad * DQ .. + DQ
  float4 qf[2][DQ / 4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int i = i0 + 16 * qt + col;
    const float4 *src = reinterpret_cast<const float4 *>(q + ((size_t(b) * S + i) * Hq + hq) * D + quad * DQ);
#pragma unroll
    for (int m = 0; m < DQ / 4; ++m)
      qf[qt][m] = active && i < S ? src[m] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  floatx4 o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) o[dt][qt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  // staging registers: float4 e = tid + x * FNT of the tile is key e / (D/4),
  // dims 4 (e % (D/4)) .. + 3
  float4 nk[NPT], nv[NPT];
  float n_logit = 0.f, n_noise = 0.f;
  auto fetch = [&](int j0) {
#pragma unroll
    for (int x = 0; x < NPT; ++x) {
      const int e = tid + x * FNT;
      const int jj = e / (D / 4), c4 = e % (D / 4);
      const int j = j0 + jj;
      const size_t row = ((size_t(b) * S + j) * hkv + h) * D;
      nk[x] = j < S ? reinterpret_cast<const float4 *>(k + row)[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
      nv[x] = j < S ? reinterpret_cast<const float4 *>(v + row)[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < FKT && j0 + tid < S) {
      const size_t at = (size_t(b) * S + j0 + tid) * hkv + h;
      n_logit = logit[at];
      n_noise = relaxed && noise ? noise[at] : 0.f;
    }
  };
  fetch(0);

  for (int j0 = 0; j0 <= i_last; j0 += FKT) {
    float *sb = sB[(j0 / FKT) & 1];
    const bool far = j0 + FKT - 1 + window <= i0;  // every key >= w behind every query
    bool live = false;
    if (tid < FKT) {
      const int j = j0 + tid;
      float bias = 0.f;
      live = j < S;
      if (j < S) {
        if (relaxed) {
          // log(1 - sigmoid(x)) = -softplus(x), in log2 units
          const float x = (n_logit + n_noise) * inv_tau;
          bias = -(fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)))) * kLog2e;
        } else if (evict_decision(n_logit)) {
          bias = -INFINITY;
          live = !far;
        }
      }
      sb[tid] = bias;
    }
    // every wave is done with the previous tile; a tile no query sees is skipped
    const bool any = __syncthreads_or(live);
    if (any) {
#pragma unroll
      for (int x = 0; x < NPT; ++x) {
        const int e = tid + x * FNT;
        const int jj = e / (D / 4), c4 = e % (D / 4);
        *reinterpret_cast<float4 *>(&sK[jj * KR + 4 * c4]) = nk[x];
        sVt[(4 * c4 + 0) * VR + jj] = nv[x].x;
        sVt[(4 * c4 + 1) * VR + jj] = nv[x].y;
        sVt[(4 * c4 + 2) * VR + jj] = nv[x].z;
        sVt[(4 * c4 + 3) * VR + jj] = nv[x].w;
      }
    }
    if (j0 + FKT <= i_last) fetch(j0 + FKT);
    if (!any) continue;
    __syncthreads();
    if (!active) continue;

    floatx4 s[2][2];
    f32_scores<D>(sK, qf, col, quad, s);
    // the rule: causal, and the key's term once it is w or more behind the query
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int i = i0 + 16 * qt + col;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int jj = 16 * t + 4 * quad + r, j = j0 + jj;
          const float add = i - j >= window ? sb[jj] : 0.f;
          s[qt][t][r] = (j <= i && i < S) ? fmaf(s[qt][t][r], scale_log2, add) : -INFINITY;
        }
    }
    f32_softmax<D>(s, m_run, l_run, o);
    f32_pv<D>(sVt, s, col, quad, o);
  }
  if (!active) return;
  float *const dst[2] = {
      i0 + col < S ? out + ((size_t(b) * S + i0 + col) * Hq + hq) * D : nullptr,
      i0 + 16 + col < S ? out + ((size_t(b) * S + i0 + 16 + col) * Hq + hq) * D : nullptr};
  f32_store<D>(o, l_run, dst, quad);
}

template <int D>
hipError_t launch_t(const dms_shape &s, const float *q, const float *k, const float *v,
                    const float *logit, const float *noise, float temperature, int seq_len,
                    float sm_scale, float *out, hipStream_t st) {
  const long pairs = long(s.batch) * s.kv_heads * ((s.group + FHW - 1) / FHW);
  const long nqb = (seq_len + FQB - 1) / FQB;
  const long blocks = (pairs + 7) / 8 * nqb * 8;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  const int relaxed = temperature > 0.f;
  hipLaunchKernelGGL(k_prefill_f32<D>, dim3(unsigned(blocks)), dim3(FNT), 0, st, s.batch, seq_len,
                     s.kv_heads, s.group,
                     s.window, sm_scale * kLog2e, relaxed, relaxed ? 1.f / temperature : 0.f, q, k, v,
                     logit, noise, out);
  return hipGetLastError();
}

// Chunk queries over a float32 cache (the last C appended tokens of every
// sequence, each at its own position; the rule of dms_decode_attn_multi):
// the products above, with key tiles of 32 slots (half a page) staged from
// the page layout, whose runs of 8 consecutive dims of a key and of 8
// consecutive slots of a value dim land as they are in the row-major keys
// and the transposed values in LDS.  Slots below n_clean are seen by every
// query; above it slot j is seen by position t iff it is in use, pos_j <= t,
// and it is unmarked or t - pos_j < w.  Slots past n_slots in the last tile
// (a recycled page may hold anything there) are staged as zeros.  Grid
// (ceil(C / 32), units * ceil(G / 4)); a sequence shorter than the chunk, or
// compacted after the chunk's first position, is flagged
// DMS_STATUS_CHUNK_INVALID.
template <int D>
__global__ __launch_bounds__(FNT, 2) void k_chunk_f32(
    int hkv, int G, int window, int maxp, int C, float scale_log2, const float *__restrict__ q,
    const float *__restrict__ k_pages, const float *__restrict__ v_pages,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ slot_pos,
    const uint8_t *__restrict__ slot_alpha, const int32_t *__restrict__ n_slots,
    const int32_t *__restrict__ n_clean, const int32_t *__restrict__ seq_len,
    const int32_t *__restrict__ compact_pos, uint32_t *__restrict__ status,
    float *__restrict__ out) {
  constexpr int DQ = D / 4, DT = D / 16, KR = D + 4, VR = FKT + 4;
  constexpr int NRUN = FKT * D / 8 / FNT;  // 8-element runs of keys (and of values) per thread
  const int ngh = (G + FHW - 1) / FHW;
  const int u = blockIdx.y / ngh, hg = blockIdx.y % ngh;
  const int b = u / hkv, h = u % hkv;
  const int Hq = hkv * G;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave, col = lane & 15, quad = lane >> 4;
  const int g = hg * FHW + wave;
  const bool active = g < G;
  const int hq = h * G + (active ? g : 0);
  const int c0 = blockIdx.x * FQB;             // first chunk query of the workgroup
  const int t_first = seq_len[b] - C + c0;     // its position
  const int ns = n_slots[u], nc = n_clean[u];
  const int32_t *row = page_table + size_t(u) * maxp;
  // the chunk's tokens are the unit's last C slots, so query c0 + 31 sits in
  // slot ns - C + c0 + 31 and later slots are hidden from the workgroup
  const int last_slot = ns - C + min(c0 + FQB - 1, C - 1);
  const int nt = last_slot < 0 ? 0 : min((ns + FKT - 1) / FKT, last_slot / FKT + 1);
  if (blockIdx.x == 0 && hg == 0 && tid == 0) {
    const int p0 = seq_len[b] - C;  // the chunk's first position
    if (p0 < 0 || compact_pos[u] > p0) atomicOr(status, DMS_STATUS_CHUNK_INVALID);
  }

  __shared__ __align__(16) float sK[FKT * KR];
  __shared__ __align__(16) float sVt[D * VR];
  __shared__ int sPos[FKT];
  __shared__ int sMark[FKT];

  float4 qf[2][DQ / 4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int cq = c0 + 16 * qt + col;
    const float4 *src =
        reinterpret_cast<const float4 *>(q + ((size_t(b) * C + cq) * Hq + hq) * D + quad * DQ);
#pragma unroll
    for (int m = 0; m < DQ / 4; ++m)
      qf[qt][m] = active && cq < C ? src[m] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  floatx4 o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) o[dt][qt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  // staging registers: run e = tid + x * FNT of the tile is, for keys, slot
  // e / (D/8) dims 8 (e % (D/8)) .. + 7, and for values, dim e / 4 slots
  // 8 (e % 4) .. + 7
  float4 nk[NRUN][2], nv[NRUN][2];
  int n_pos = 0, n_mark = 0;
  auto fetch = [&](int t) {
    const int page = row[t >> 1];
    const int j0 = (t & 1) * FKT;           // first slot of the tile within its page
    const size_t pbase = size_t(page) * kPage * D;
    const int valid = ns - t * FKT;          // slots in use in this tile (>= 1)
#pragma unroll
    for (int x = 0; x < NRUN; ++x) {
      const int e = tid + x * FNT;
      const int js = e / (D / 8), c8 = e % (D / 8);
      const float4 *kp = reinterpret_cast<const float4 *>(k_pages + pbase + key_index(j0 + js, 8 * c8, D));
      const bool used = js < valid;
      nk[x][0] = used ? kp[0] : make_float4(0.f, 0.f, 0.f, 0.f);
      nk[x][1] = used ? kp[1] : make_float4(0.f, 0.f, 0.f, 0.f);
      const int d = e / 4, r8 = e % 4;
      const float4 *vp = reinterpret_cast<const float4 *>(v_pages + pbase + value_index(j0 + 8 * r8, d, D));
      float4 a = vp[0], bb = vp[1];
      const int s0 = 8 * r8;                 // slots s0 .. s0 + 7 of the tile
      a.x = s0 + 0 < valid ? a.x : 0.f;
      a.y = s0 + 1 < valid ? a.y : 0.f;
      a.z = s0 + 2 < valid ? a.z : 0.f;
      a.w = s0 + 3 < valid ? a.w : 0.f;
      bb.x = s0 + 4 < valid ? bb.x : 0.f;
      bb.y = s0 + 5 < valid ? bb.y : 0.f;
      bb.z = s0 + 6 < valid ? bb.z : 0.f;
      bb.w = s0 + 7 < valid ? bb.w : 0.f;
      nv[x][0] = a;
      nv[x][1] = bb;
    }
    if (tid < FKT) {
      n_pos = slot_pos[size_t(page) * kPage + j0 + tid];
      n_mark = slot_alpha[size_t(page) * kPage + j0 + tid];
    }
  };
  if (nt > 0) fetch(0);

  for (int t = 0; t < nt; ++t) {
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int x = 0; x < NRUN; ++x) {
      const int e = tid + x * FNT;
      const int js = e / (D / 8), c8 = e % (D / 8);
      *reinterpret_cast<float4 *>(&sK[js * KR + 8 * c8]) = nk[x][0];
      *reinterpret_cast<float4 *>(&sK[js * KR + 8 * c8 + 4]) = nk[x][1];
      const int d = e / 4, r8 = e % 4;
      *reinterpret_cast<float4 *>(&sVt[d * VR + 8 * r8]) = nv[x][0];
      *reinterpret_cast<float4 *>(&sVt[d * VR + 8 * r8 + 4]) = nv[x][1];
    }
    if (tid < FKT) {
      sPos[tid] = n_pos;
      sMark[tid] = n_mark;
    }
    if (t + 1 < nt) fetch(t + 1);
    __syncthreads();
    if (!active) continue;

    floatx4 s[2][2];
    f32_scores<D>(sK, qf, col, quad, s);
    // liveness of each slot for this column's query position
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int cq = c0 + 16 * qt + col;
      const int tq = t_first + 16 * qt + col;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int js = 16 * t2 + 4 * quad + r, slot = t * FKT + js;
          const int pos = sPos[js];
          const bool live = (cq < C) & (slot < ns) &
                            ((slot < nc) | ((pos <= tq) & ((sMark[js] == 0) | (tq - pos < window))));
          s[qt][t2][r] = live ? s[qt][t2][r] * scale_log2 : -INFINITY;
        }
    }
    f32_softmax<D>(s, m_run, l_run, o);
    f32_pv<D>(sVt, s, col, quad, o);
  }
  if (!active) return;
  float *const dst[2] = {
      c0 + col < C ? out + ((size_t(b) * C + c0 + col) * Hq + hq) * D : nullptr,
      c0 + 16 + col < C ? out + ((size_t(b) * C + c0 + 16 + col) * Hq + hq) * D : nullptr};
  f32_store<D>(o, l_run, dst, quad);
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

hipError_t launch_chunk_f32(const dms_shape &s, const dms_cache &c, const void *q, int n_query,
                            float *out, float sm_scale, hipStream_t st) {
  const long gy = long(s.batch) * s.kv_heads * ((s.group + FHW - 1) / FHW);
  if (gy > 65535) return hipErrorInvalidValue;  // grid y
  const dim3 grid(unsigned((n_query + FQB - 1) / FQB), unsigned(gy));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(FNT), 0, st, s.kv_heads, s.group, s.window,
                       s.max_pages_per_unit, n_query, sm_scale * kLog2e, static_cast<const float *>(q),
                       static_cast<const float *>(c.k_pages), static_cast<const float *>(c.v_pages),
                       c.page_table, c.slot_pos, c.slot_alpha, c.n_slots, c.n_clean, c.seq_len,
                       c.plan + plan_layout(units_of(s)).compact_pos, c.status, out);
  };
  if (s.head_dim == 128) go(k_chunk_f32<128>);
  else if (s.head_dim == 64) go(k_chunk_f32<64>);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dms
