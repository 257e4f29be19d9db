// Masked prefill attention under the DMS visibility rule, on the gfx950
// matrix cores.
//
// Method: atlas.scime.ai summary of "Inference-Time Hyper-Scaling with KV
// Cache Compression", section "Approach" (binary per-head decision, eviction
// carried out after a delay window) and table "Measured effects reported in
// the paper" (16-token window).  Applied to a whole prompt, query row i of
// head hq sees key j of KV head hq / G iff
//   j <= i  and  not (alpha_j and i - j >= w),   alpha_j = logit_j > 0.
// out = softmax_j(scale * <q_i, k_j>) v_j over the visible keys, fp32.
//
// Work decomposition.  A workgroup of 8 waves takes 64 query positions of
// one KV head: wave w serves query head g = 4*hg + (w % 4) of the group and
// query positions i0 + 32*(w / 4) .. +32.  Keys are consumed in tiles of 32
// from position 0 up to the causal end of the block.  Each key tile (keys
// and values) is loaded once per workgroup into LDS, in the order of the
// matrix-core operand fragments, and serves all four heads; the next tile's
// global loads are in flight while the current tile is computed.
//
// Per tile and wave the two products are the ones of the decode kernel, with
// query positions in place of heads:
//   S^T [32 keys x 16 queries] = K [32 x 128] . Q^T [128 x 16]   (x2 query tiles)
//   O^T [128 x 16 queries]    += V^T [128 x 32 keys] . P^T [32 x 16]
// on v_mfma_f32_16x16x32_bf16 with fp32 accumulation and an fp32 online
// softmax in exp2 form; the two 16-key tiles take their rows from the slot
// permutation (row 4a + r -> key 8a + r, or 8a + 4 + r) so that each lane's
// scores are exactly the eight keys it supplies to the PV product.
#include "dms_internal.h"

namespace dms {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int PD = 128;            // head dimension
constexpr int PBN = 32;            // keys per tile
constexpr int PBM = 64;            // query positions per workgroup
constexpr int PWAVES = 8;          // waves per workgroup
constexpr int PHPW = 4;            // query heads per workgroup
constexpr int PKS = PD / 32;       // QK products per 16-key tile
constexpr int PDT = PD / 16;       // PV products per tile
constexpr int PFRAG = 64;          // uint4 per operand fragment (64 lanes x 16 bytes)
constexpr int PK_FRAGS = 2 * PKS;  // key fragments per tile
constexpr int PV_FRAGS = PDT;      // value fragments per tile

__device__ __forceinline__ floatx4 mfma(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return uint32_t(__builtin_bit_cast(uint16_t, (__bf16)lo)) |
         (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)hi)) << 16);
}

// The tile's global pieces held by one thread between load and LDS store:
// thread t covers the 16-byte piece t of K and of V (512 pieces per tile):
// key t / 16, dims (t % 16) * 8 .. +8.
struct TilePieces {
  uint4 k, v;
  uint32_t alpha;  // threads 0..31: decision of key j0 + t
};

}  // namespace

__global__ __launch_bounds__(PWAVES * 64, 2) void k_prefill(
    int batch, int S, int hkv, int G, int window, float scale_log2, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, const float *__restrict__ logit,
    float *__restrict__ out) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int col = lane & 15, quad = lane >> 4;
  const int Hq = hkv * G;
  const int ngh = (G + PHPW - 1) / PHPW;
  const int nqb = (S + PBM - 1) / PBM;

  // Workgroup -> (b, h, hg, query block).  Consecutive ids go to different
  // XCDs (round-robin), so all query blocks of one (b, h, hg) are given ids of
  // the same residue modulo 8 and share an L2; within that, the longest
  // (latest) query blocks start first.
  const int nbh = batch * hkv * ngh;
  const int id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  const int per_xcd_pairs = (nbh + 7) / 8;
  const int pair_in_xcd = slot / nqb;
  const int qb = nqb - 1 - slot % nqb;
  const int pair = pair_in_xcd * 8 + xcd;
  if (pair_in_xcd >= per_xcd_pairs || pair >= nbh) return;
  const int b = pair / (hkv * ngh);
  const int h = (pair / ngh) % hkv;
  const int hg = pair % ngh;

  const int g = hg * PHPW + (wave % PHPW);
  const bool active = g < G;
  const int hq = h * G + (active ? g : 0);
  const int qi0 = qb * PBM + (wave / PHPW) * 32;  // this wave's first query position
  const int i_end = min(S, qb * PBM + PBM);       // workgroup's causal key end

  __shared__ uint4 sK[2][PK_FRAGS * PFRAG];
  __shared__ uint4 sV[2][PV_FRAGS * PFRAG];
  __shared__ uint32_t sA[2];

  // Q^T operand for two query tiles: query qi0 + 16*qt + col, dims ks*32 + quad*8
  uint4 qf[2][PKS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int i = qi0 + 16 * qt + col;
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) {
      qf[qt][ks] = make_uint4(0, 0, 0, 0);
      if (active && i < S)
        qf[qt][ks] = *reinterpret_cast<const uint4 *>(
            q + ((size_t(b) * S + i) * Hq + hq) * PD + ks * 32 + quad * 8);
    }
  }

  floatx4 o[PDT][2];
#pragma unroll
  for (int dt = 0; dt < PDT; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) o[dt][qt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  const size_t kv_row = size_t(hkv) * PD;  // elements between consecutive positions
  const uint16_t *kb0 = k + (size_t(b) * S * hkv + h) * PD;
  const uint16_t *vb0 = v + (size_t(b) * S * hkv + h) * PD;
  const float *lb0 = logit + size_t(b) * S * hkv + h;

  auto fetch_tile = [&](TilePieces &tp, int j0) {
    const int jj = tid >> 4, dc = tid & 15;
    const int j = j0 + jj;
    tp.k = make_uint4(0, 0, 0, 0);
    tp.v = make_uint4(0, 0, 0, 0);
    if (j < S) {
      tp.k = *reinterpret_cast<const uint4 *>(kb0 + size_t(j) * kv_row + dc * 8);
      tp.v = *reinterpret_cast<const uint4 *>(vb0 + size_t(j) * kv_row + dc * 8);
    }
    tp.alpha = 0u;
    if (tid < PBN && j0 + tid < S) tp.alpha = lb0[size_t(j0 + tid) * hkv] > 0.0f ? 1u : 0u;
  };

  auto store_tile = [&](const TilePieces &tp, int st) {
    const int jj = tid >> 4, dc = tid & 15;
    // key fragment (t, ks), lane qd*16 + row
    const int t = (jj & 7) >> 2, row = 4 * (jj >> 3) + (jj & 3);
    const int ks = dc >> 2, qd = dc & 3;
    sK[st][(t * PKS + ks) * PFRAG + qd * 16 + row] = tp.k;
    // value fragment dt = d / 16, lane (jj / 8)*16 + d % 16, element jj % 8
    uint16_t *vb = reinterpret_cast<uint16_t *>(&sV[st][0]);
    const uint16_t *el = reinterpret_cast<const uint16_t *>(&tp.v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = dc * 8 + e;
      vb[(((d >> 4) * 4 + (jj >> 3)) * 16 + (d & 15)) * 8 + (jj & 7)] = el[e];
    }
    if (wave == 0) {
      const uint64_t m = __ballot(lane < PBN && tp.alpha != 0u);
      if (lane == 0) sA[st] = uint32_t(m);
    }
  };

  const int ntiles = (i_end + PBN - 1) / PBN;
  TilePieces tp;
  fetch_tile(tp, 0);
  store_tile(tp, 0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int st = kt & 1;
    const int j0 = kt * PBN;
    if (kt + 1 < ntiles) fetch_tile(tp, j0 + PBN);  // in flight during the compute below

    // this wave's queries are qi0 .. qi0 + 31; the tile is needed if j0 <= qi0 + 31
    if (active && j0 <= qi0 + 31) {
      floatx4 s[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) s[t][qt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < PKS; ++ks) {
        const uint4 a0 = sK[st][(0 * PKS + ks) * PFRAG + lane];
        const uint4 a1 = sK[st][(1 * PKS + ks) * PFRAG + lane];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          s[0][qt] = mfma(a0, qf[qt][ks], s[0][qt]);
          s[1][qt] = mfma(a1, qf[qt][ks], s[1][qt]);
        }
      }
      const uint32_t abits = sA[st] >> (8 * quad);
      uint4 pb[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int i = qi0 + 16 * qt + col;
        float sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + 8 * quad + e;
          const bool marked = (abits >> e) & 1u;
          const bool vis = (j < S) & (j <= i) & (!marked | (i - j < window));
          const float raw = (e < 4 ? s[0][qt][e] : s[1][qt][e - 4]) * scale_log2;
          sv[e] = vis ? raw : -INFINITY;
        }
        float mx = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const float m_new = fmaxf(m_run[qt], mx);
        float p[8];
        float corr = 1.f;
        if (m_new == -INFINITY) {
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = 0.f;
        } else {
          corr = m_run[qt] == -INFINITY ? 0.f : exp2f(m_run[qt] - m_new);
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = exp2f(sv[e] - m_new);
        }
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ps += p[e];
        l_run[qt] = l_run[qt] * corr + ps;
        m_run[qt] = m_new;
        if (__ballot(corr != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < PDT; ++dt) o[dt][qt] *= corr;
        }
        pb[qt] = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
      }
#pragma unroll
      for (int dt = 0; dt < PDT; ++dt) {
        const uint4 va = sV[st][dt * PFRAG + lane];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) o[dt][qt] = mfma(va, pb[qt], o[dt][qt]);
      }
    }

    if (kt + 1 < ntiles) store_tile(tp, st ^ 1);
    __syncthreads();
  }

  if (!active) return;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float l = l_run[qt];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int i = qi0 + 16 * qt + col;
    if (i < S) {
      float *op = out + ((size_t(b) * S + i) * Hq + hq) * PD + quad * 4;
#pragma unroll
      for (int dt = 0; dt < PDT; ++dt)
        *reinterpret_cast<floatx4 *>(op + dt * 16) = o[dt][qt] * inv;
    }
  }
}

hipError_t launch_prefill(const dms_shape &s, const void *q, const void *k, const void *v,
                          const float *logit, int seq_len, float sm_scale, float *out,
                          hipStream_t st) {
  const int ngh = (s.group + PHPW - 1) / PHPW;
  const int nbh = s.batch * s.kv_heads * ngh;
  const int nqb = (seq_len + PBM - 1) / PBM;
  const int per_xcd_pairs = (nbh + 7) / 8;
  const long blocks = long(per_xcd_pairs) * nqb * 8;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_prefill, dim3(unsigned(blocks)), dim3(PWAVES * 64), 0, st, s.batch, seq_len,
                     s.kv_heads, s.group, s.window, sm_scale * 1.4426950408889634f,
                     static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                     static_cast<const uint16_t *>(v), logit, out);
  return hipGetLastError();
}

}  // namespace dms
