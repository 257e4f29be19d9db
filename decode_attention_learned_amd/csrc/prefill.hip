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
// Two kernels.  k_prefill_pack re-lays keys and values out once, per (b, h,
// 32-key tile), in the order of the matrix-core operand fragments (values
// transposed), with one decision word per tile, into the caller's workspace.
// k_prefill then only copies whole fragments into LDS.
//
// Work decomposition.  A workgroup of 8 waves takes 64 query positions of
// one KV head: wave w serves query head g = 4*hg + (w % 4) of the group and
// query positions i0 + 32*(w / 4) .. +32.  Keys are consumed in tiles of 32
// from position 0 up to the causal end of the block.  Each key tile (keys
// and values) is loaded once per workgroup into LDS, in the order of the
// matrix-core operand fragments, and serves all four heads; the next tile's
// global loads are in flight while the current tile is computed.  Tiles that
// lie wholly `w` or more positions behind every query of a wave need only the
// decision bits; the tiles on the diagonal band test the full rule.
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

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{lo, hi}, bf16x2v));
}

constexpr int PTILE_U4 = (PK_FRAGS + PV_FRAGS) * PFRAG;  // uint4 per packed tile (16 KB)

// One packed tile per (b, h, tile): [key fragments (8 x 1 KB) | value fragments (8 x 1 KB)].
__device__ __forceinline__ size_t tile_index(int b, int h, int tile, int hkv, int ntiles) {
  return (size_t(b) * hkv + h) * ntiles + tile;
}

}  // namespace

// ---------------------------------------------------------------------------
// pack: one workgroup (512 threads) per (tile, h, b)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void k_prefill_pack(int S, int hkv, int ntiles,
                                                      const uint16_t *__restrict__ k,
                                                      const uint16_t *__restrict__ v,
                                                      const float *__restrict__ logit,
                                                      uint4 *__restrict__ packed,
                                                      uint32_t *__restrict__ alpha_words) {
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x;
  const int j0 = tile * PBN;
  const size_t T = tile_index(b, h, tile, hkv, ntiles);
  uint4 *kdst = packed + T * PTILE_U4;
  uint4 *vdst = kdst + PK_FRAGS * PFRAG;
  __shared__ __align__(16) uint16_t sv[PBN][PD + 8];  // row-major values, padded rows

  // thread t: key jj = t / 16, dims dc*8 .. +8
  const int jj = t >> 4, dc = t & 15;
  const int j = j0 + jj;
  uint4 kp = make_uint4(0, 0, 0, 0), vp = make_uint4(0, 0, 0, 0);
  if (j < S) {
    const size_t off = ((size_t(b) * S + j) * hkv + h) * PD + dc * 8;
    kp = *reinterpret_cast<const uint4 *>(k + off);
    vp = *reinterpret_cast<const uint4 *>(v + off);
  }
  // key fragment (tt, ks), lane qd*16 + row (tile row from the slot permutation)
  const int tt = (jj & 7) >> 2, row = 4 * (jj >> 3) + (jj & 3);
  const int ks = dc >> 2, qd = dc & 3;
  kdst[(tt * PKS + ks) * PFRAG + qd * 16 + row] = kp;
  *reinterpret_cast<uint4 *>(&sv[jj][dc * 8]) = vp;
  if (t < kWave) {
    const bool marked = t < PBN && j0 + t < S && evict_decision(logit[(size_t(b) * S + j0 + t) * hkv + h]);
    const uint64_t m = __ballot(marked);
    if (t == 0) alpha_words[T] = uint32_t(m);
  }
  __syncthreads();
  // value fragment dt = t / 64, lane l = t % 64: dim dt*16 + l % 16, keys 8*(l/16) .. +8
  const int dt = t >> 6, l = t & 63;
  const int d = dt * 16 + (l & 15), k0 = 8 * (l >> 4);
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = uint32_t(sv[k0 + 2 * e][d]) | (uint32_t(sv[k0 + 2 * e + 1][d]) << 16);
  vdst[t] = make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(PWAVES * 64, 2) void k_prefill(
    int batch, int S, int hkv, int G, int window, float scale_log2, const uint16_t *__restrict__ q,
    const uint4 *__restrict__ packed, const uint32_t *__restrict__ alpha_words,
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

  const int ntiles_all = (S + PBN - 1) / PBN;
  const uint4 *pk = packed + tile_index(b, h, 0, hkv, ntiles_all) * PTILE_U4;
  const uint32_t *pa = alpha_words + tile_index(b, h, 0, hkv, ntiles_all);

  // thread t copies uint4 t and t + 512 of the 16 KB packed tile (keys, then values)
  uint4 ta = pk[tid], tb = pk[tid + PWAVES * 64];
  uint32_t talpha = pa[0];
  sK[0][tid] = ta;
  sV[0][tid] = tb;
  if (tid == 0) sA[0] = talpha;
  __syncthreads();

  // Lazy rescaling: a query's reference maximum m_run (raw score units) moves
  // only when a tile's maximum exceeds it by more than kLazy/c, so p <= 2^kLazy.
  // The result is unchanged (numerator and denominator share the reference),
  // and the rescale of the accumulators becomes rare after the first tiles.
  constexpr float kLazy = 8.0f;
  const float c = scale_log2;
  const float lazy_raw = kLazy / c;
  const int ntiles = (i_end + PBN - 1) / PBN;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int st = kt & 1;
    const int j0 = kt * PBN;
    const bool more = kt + 1 < ntiles;
    if (more) {  // next tile's loads are in flight during the compute below
      const uint4 *src = pk + size_t(kt + 1) * PTILE_U4;
      ta = src[tid];
      tb = src[tid + PWAVES * 64];
      talpha = pa[kt + 1];
    }

    // this wave's queries are qi0 .. qi0 + 31; the tile is needed if j0 <= qi0 + 31
    if (active && j0 <= qi0 + 31) {
      floatx4 s0[2], s1[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        s0[qt] = floatx4{0.f, 0.f, 0.f, 0.f};
        s1[qt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ks = 0; ks < PKS; ++ks) {
        const uint4 a0 = sK[st][(0 * PKS + ks) * PFRAG + lane];
        const uint4 a1 = sK[st][(1 * PKS + ks) * PFRAG + lane];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          s0[qt] = mfma(a0, qf[qt][ks], s0[qt]);
          s1[qt] = mfma(a1, qf[qt][ks], s1[qt]);
        }
      }
      // decision bits of this lane's eight keys j0 + 8*quad + e
      const uint32_t abits = sA[st] >> (8 * quad);
      // far: every key is >= window behind every query of this wave, and inside S
      const bool far = (qi0 - (j0 + PBN - 1) >= window) && (j0 + PBN <= S);
      float madd[8];  // 0 for a visible key, -inf otherwise (far tiles: decision only)
#pragma unroll
      for (int e = 0; e < 8; ++e) madd[e] = ((abits >> e) & 1u) ? -INFINITY : 0.f;
      uint4 pb[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float sv[8] = {s0[qt][0], s0[qt][1], s0[qt][2], s0[qt][3],
                       s1[qt][0], s1[qt][1], s1[qt][2], s1[qt][3]};
        if (far) {
#pragma unroll
          for (int e = 0; e < 8; ++e) sv[e] += madd[e];
        } else {
          const int i = qi0 + 16 * qt + col;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = j0 + 8 * quad + e;
            const bool vis = (j < S) & (j <= i) & ((madd[e] == 0.f) | (i - j < window));
            sv[e] = vis ? sv[e] : -INFINITY;
          }
        }
        float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        float m_ref = m_run[qt];
        if (__ballot(mx > m_ref + lazy_raw)) {  // some query of the tile needs a new reference
          const float m_new = mx > m_ref + lazy_raw ? mx : m_ref;
          const float corr = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
          l_run[qt] *= corr;
#pragma unroll
          for (int dt = 0; dt < PDT; ++dt) o[dt][qt] *= corr;
          m_ref = m_new;
          m_run[qt] = m_new;
        }
        // arguments are <= kLazy and finite or -inf: the plain hardware exp2 needs no range reduction
        float p[8];
        const float mc = m_ref == -INFINITY ? 0.f : m_ref * c;
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], c, -mc));
        l_run[qt] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        pb[qt] = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
      }
#pragma unroll
      for (int dt = 0; dt < PDT; ++dt) {
        const uint4 va = sV[st][dt * PFRAG + lane];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) o[dt][qt] = mfma(va, pb[qt], o[dt][qt]);
      }
    }

    if (more) {
      sK[st ^ 1][tid] = ta;
      sV[st ^ 1][tid] = tb;
      if (tid == 0) sA[st ^ 1] = talpha;
    }
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
                          const float *logit, int seq_len, float sm_scale, float *out, void *ws,
                          hipStream_t st) {
  const int ntiles = (seq_len + PBN - 1) / PBN;
  if (s.kv_heads > 65535 || s.batch > 65535) return hipErrorInvalidValue;  // pack grid y, z
  const size_t tiles = size_t(s.batch) * s.kv_heads * ntiles;
  uint4 *packed = static_cast<uint4 *>(ws);
  uint32_t *alpha_words = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + align256(tiles * 16384));
  hipLaunchKernelGGL(k_prefill_pack, dim3(ntiles, s.kv_heads, s.batch), dim3(512), 0, st, seq_len,
                     s.kv_heads, ntiles, static_cast<const uint16_t *>(k),
                     static_cast<const uint16_t *>(v), logit, packed, alpha_words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ngh = (s.group + PHPW - 1) / PHPW;
  const int nbh = s.batch * s.kv_heads * ngh;
  const int nqb = (seq_len + PBM - 1) / PBM;
  const int per_xcd_pairs = (nbh + 7) / 8;
  const long blocks = long(per_xcd_pairs) * nqb * 8;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_prefill, dim3(unsigned(blocks)), dim3(PWAVES * 64), 0, st, s.batch, seq_len,
                     s.kv_heads, s.group, s.window, sm_scale * 1.4426950408889634f,
                     static_cast<const uint16_t *>(q), packed, alpha_words, out);
  return hipGetLastError();
}

}  // namespace dms
