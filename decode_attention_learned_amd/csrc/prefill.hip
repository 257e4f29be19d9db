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
// transposed), plus an additive mask per key (0, or -inf for a key marked
// for eviction), into the caller's workspace.  k_prefill then only copies
// whole fragments into LDS.
//
// Work decomposition.  A workgroup of four waves takes 32 query positions of
// one KV head: wave w serves query head g = 4*hg + w of the group.  Keys are
// consumed in tiles of 32 from position 0 up to the causal end of the block.
// Each key tile is copied once per workgroup into LDS and serves all four
// heads.  Three workgroups share a CU (at most 168 VGPRs and 49.5 KB of LDS
// each), so every SIMD interleaves three waves.
//
// Tile ring.  Three LDS buffers, each its own array; tile t lives in buffer
// t % 3.  The load unit copies a packed tile from global memory straight
// into LDS (global_load_lds, 16 bytes per lane, no registers involved): the
// copy of tile k + 1 is issued at the start of iteration k into the buffer
// of tile k - 2, whose last reader (the PV product of iteration k - 1) every
// wave has passed at the barrier ending iteration k - 1.  Each wave waits
// for its own copies before the barrier that ends iteration k.
//
// Per tile and wave the two products are the ones of the decode kernel, with
// query positions in place of heads:
//   S^T [32 keys x 16 queries] = K [32 x 128] . Q^T [128 x 16]   (x2 query tiles)
//   O^T [128 x 16 queries]    += V^T [128 x 32 keys] . P^T [32 x 16]
// on v_mfma_f32_16x16x32_bf16 with fp32 accumulation and an fp32 online
// softmax in exp2 form; the two 16-key tiles take their rows from the slot
// permutation (row 4a + r -> key 8a + r, or 8a + 4 + r) so that each lane's
// scores are exactly the eight keys it supplies to the PV product.
//
// Two phases per tile.  Phase 1 (matrix cores) computes the scores of tile k
// and the PV product of tile k-1; phase 2 (vector unit) masks, checks and
// exponentiates the scores of tile k.  The waves of a SIMD come from
// different workgroups and interleave freely.
//
// Far and near tiles.  A tile whose keys all lie `w` or more positions behind
// every query of the workgroup ("far") is masked by the decision alone, which
// depends on the key only: the QK product starts from the additive mask as
// its accumulator, so such a tile costs no mask arithmetic.  Far tiles are
// read from a second packed copy in which the keys the hard rule masks out
// have zero rows (they are invisible there; zero operands cost the matrix
// cores less power).  The few tiles on the diagonal band ("near") come from
// the plain copy and apply the full rule per element in phase 2.  Far
// tiles from tile 1 on run, in whole rounds of three (one per buffer), in a
// loop of their own whose body has no test on the tile index; tile 0 and
// the tiles after the last whole round take the general path.
//
// Output.  After the last tile each wave stages its 32 fp32 output rows in
// the (then idle) ring buffers, so that one store instruction writes two
// whole 512-byte rows.
//
// Softmax reference.  Each query keeps a reference m (raw score units) that
// moves only when a score exceeds it by more than kLazy / c (c = scale *
// log2 e), so every exponent is at most kLazy.  The result does not depend on
// m (numerator and denominator share it); the check is a per-lane compare
// and a ballot, and the cross-lane maximum and the rescale of the
// accumulators run only when some score crosses the threshold.  The row sums
// add the same bf16-rounded p values that enter the PV product.
#include "dms_internal.h"

namespace dms {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));

constexpr int PBN = 32;            // keys per tile
constexpr int PHPW = 4;            // query heads per workgroup
constexpr int PFRAG = 64;          // uint4 per operand fragment (64 lanes x 16 bytes)
constexpr int PNT = 256;           // threads per workgroup of the prefill kernels
// Sizes that follow from the head dimension D (64 or 128): QK products per
// 16-key tile, PV products per tile, key fragments per tile, uint4 per packed
// tile (D*8: 16 KB at D = 128).  Every kernel and helper below is a template
// on D and names them by these short local constants.
#define PDIMS(D)                          \
  constexpr int PD = (D);                 \
  constexpr int PKS = PD / 32;            \
  constexpr int PDT = PD / 16;            \
  constexpr int PK_FRAGS = 2 * PKS;       \
  constexpr int PV_FRAGS = PDT;           \
  constexpr int PTILE_U4 = (PK_FRAGS + PV_FRAGS) * PFRAG;  \
  (void)PKS; (void)PDT; (void)PK_FRAGS; (void)PV_FRAGS; (void)PTILE_U4
constexpr float kLazy = 8.0f;      // largest exponent (log2 units) before the reference moves

__device__ __forceinline__ floatx4 mfma(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{lo, hi}, bf16x2v));
}

// acc + lo + hi of a packed bf16 pair, in one v_dot2c_f32_bf16
__device__ __forceinline__ float add_pair(uint32_t pair, float acc) {
  const bf16x2v one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pair), one, acc, false);
}

// One packed tile per (b, h, tile): [key fragments (8 x 1 KB) | value fragments (8 x 1 KB)],
// and separately 32 floats of additive mask.
__device__ __forceinline__ size_t tile_index(int b, int h, int tile, int hkv, int ntiles) {
  return (size_t(b) * hkv + h) * ntiles + tile;
}

// Per-query softmax state of one wave (two query tiles; lane holds column l % 16).
struct Softmax {
  float m[2];    // reference, raw score units (-inf until the first visible key)
  float nmc[2];  // -m * c (0 while m = -inf)
  float thr[2];  // m + kLazy / c: a score above it moves the reference
  float l[2];    // running sum of p over this lane's keys
};

// QK product of one tile for both query tiles, starting from `init`.
// The key fragments are read one 16-key half at a time (16 VGPRs).
template <int D>
__device__ __forceinline__ void qk_tile(const uint4 *__restrict__ sk, const floatx4 (&init)[2],
                                        const uint4 (&qf)[2][D / 32], int lane, floatx4 (&s)[2][2]) {
  PDIMS(D);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint4 ka[PKS];
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) ka[ks] = sk[(t * PKS + ks) * PFRAG + lane];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      floatx4 acc = init[t];
#pragma unroll
      for (int ks = 0; ks < PKS; ++ks) acc = mfma(ka[ks], qf[qt][ks], acc);
      s[qt][t] = acc;
    }
  }
}

__device__ __forceinline__ float lane_max(const floatx4 (&s)[2]) {
  return fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
               fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
}

// Does any score of this lane cross its query's threshold?
__device__ __forceinline__ bool crosses(const floatx4 (&s)[2][2], const Softmax &sm) {
  return (lane_max(s[0]) > sm.thr[0]) | (lane_max(s[1]) > sm.thr[1]);
}

// Rare path: move the reference of every query whose tile maximum crossed the
// threshold, and rescale its accumulators.
template <int D>
__device__ __forceinline__ void move_reference(const floatx4 (&s)[2][2], Softmax &sm,
                                               floatx4 (&o)[D / 16][2], float c) {
  PDIMS(D);
  const float lazy_raw = kLazy / c;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float mx = lane_max(s[qt]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    // branch-free: queries whose maximum stays under the threshold get factor 1
    const bool move = mx > sm.thr[qt];  // uniform over the four lanes of a query
    const float m_old = sm.m[qt];
    const float corr =
        move ? (m_old == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_old - mx) * c)) : 1.f;
    sm.l[qt] *= corr;
#pragma unroll
    for (int dt = 0; dt < PDT; ++dt) o[dt][qt] *= corr;
    sm.m[qt] = move ? mx : m_old;
    sm.nmc[qt] = move ? -mx * c : sm.nmc[qt];
    sm.thr[qt] = move ? mx + lazy_raw : sm.thr[qt];
  }
}

// p = 2^(s c - m c) for both query tiles, packed to bf16 in PV operand order,
// and added to the row sums.
__device__ __forceinline__ void exponentials(const floatx4 (&s)[2][2], Softmax &sm, float c,
                                             uint4 (&pb)[2]) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      p[e] = __builtin_amdgcn_exp2f(fmaf(s[qt][e >> 2][e & 3], c, sm.nmc[qt]));
    pb[qt] = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
    float l = sm.l[qt];
    l = add_pair(pb[qt].x, l);
    l = add_pair(pb[qt].y, l);
    l = add_pair(pb[qt].z, l);
    l = add_pair(pb[qt].w, l);
    sm.l[qt] = l;
  }
}

// PV product of one tile; the value fragments are read four at a time.
template <int D>
__device__ __forceinline__ void pv_tile(const uint4 *__restrict__ sv, const uint4 (&pb)[2], int lane,
                                        floatx4 (&o)[D / 16][2]) {
  PDIMS(D);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    uint4 va[PDT / 2];
#pragma unroll
    for (int d = 0; d < PDT / 2; ++d) va[d] = sv[(hh * PDT / 2 + d) * PFRAG + lane];
#pragma unroll
    for (int d = 0; d < PDT / 2; ++d) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        o[hh * PDT / 2 + d][qt] = mfma(va[d], pb[qt], o[hh * PDT / 2 + d][qt]);
    }
  }
}

// PV product of a cache tile whose slots from `valid` on (0..31) are unused:
// their value rows may hold anything a recycled page held (even NaN), so they
// are cleared in the operand (their weights are already zero).
template <int D>
__device__ __forceinline__ void pv_tile_tail(const uint4 *__restrict__ sv, const uint4 (&pb)[2],
                                             int lane, int valid, floatx4 (&o)[D / 16][2]) {
  PDIMS(D);
  const int quad = lane >> 4;
  uint32_t keep[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 8 * quad + 2 * e;  // this lane's slots j, j + 1 of the tile
    keep[e] = (j < valid ? 0xffffu : 0u) | (j + 1 < valid ? 0xffff0000u : 0u);
  }
#pragma unroll
  for (int dt = 0; dt < PDT; ++dt) {
    uint4 va = sv[dt * PFRAG + lane];
    va.x &= keep[0];
    va.y &= keep[1];
    va.z &= keep[2];
    va.w &= keep[3];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) o[dt][qt] = mfma(va, pb[qt], o[dt][qt]);
  }
}

// Write a wave's output (32 query rows of one head, o / l) through LDS so that
// each store instruction covers whole rows (two 512-byte rows at D = 128, four
// 256-byte rows at D = 64).  `stage` holds 16 rows of D floats for this wave;
// row r is rotated by 4 r floats so that the sixteen rows of a write land in
// different banks.
template <int D>
__device__ __forceinline__ void store_rows(const floatx4 (&o)[D / 16][2], const Softmax &sm,
                                           float *stage, float *out, size_t row0, size_t rstride,
                                           int i0, int S, int lane, bool normalize = true) {
  PDIMS(D);
  constexpr int LPR = D / 4;      // lanes per row (four floats each)
  constexpr int RPI = 64 / LPR;   // rows per store instruction
  const int col = lane & 15, quad = lane >> 4;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float l = sm.l[qt];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const float inv = normalize ? (l > 0.f ? 1.f / l : 0.f) : 1.f;
#pragma unroll
    for (int dt = 0; dt < PDT; ++dt)
      *reinterpret_cast<floatx4 *>(stage + col * D + ((dt * 16 + quad * 4 + 4 * col) & (D - 1))) =
          o[dt][qt] * inv;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int sub = lane / LPR, c4 = (lane % LPR) * 4;
#pragma unroll
    for (int r = 0; r < 16; r += RPI) {
      const int row = r + sub;
      const int i = i0 + 16 * qt + row;
      const floatx4 v = *reinterpret_cast<const floatx4 *>(stage + row * D + ((c4 + 4 * row) & (D - 1)));
      // nontemporal: the output is not read again by this launch (gathered
      // call 0.407 -> 0.397 ms, the dense and relaxed calls unchanged)
      if (i < S)
        __builtin_nontemporal_store(v, reinterpret_cast<floatx4 *>(out + row0 + size_t(i) * rstride + c4));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ---- tile ring -----------------------------------------------------------
// Copy N uint4 (a 16 KB packed tile, or half of one) into LDS with the load
// unit: wave w copies uint4 256 r + 64 w + lane, one contiguous 1 KB run per
// copy instruction.  The copies are buffer loads: the source is a buffer
// resource (scalar registers) and the lane's byte offset 16 * tid is the same
// for every tile, so a copy costs no vector instruction.
constexpr uint32_t kBufferFlags = 0x00020000u;  // raw buffer resource word 3 (32-bit data)
template <int N>
__device__ __forceinline__ void ring_copy(const uint4 *__restrict__ src, uint4 *dst, int tid,
                                          int wave) {
  static_assert(N % PNT == 0, "whole runs");
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4 *>(src), 0, N * 16, kBufferFlags);
#pragma unroll
  for (int r = 0; r < N / PNT; ++r)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst + r * PNT + wave * kWave, 16, tid * 16,
                                             r * PNT * 16, 0, 0);
}

// Copy 128 bytes of per-key data (a mask or positions) with lanes 0..7 of wave 0.
template <typename T>
__device__ __forceinline__ void ring_copy_keys(const T *__restrict__ src, T *dst, int tid) {
  static_assert(sizeof(T) == 16, "16-byte elements");
  if (tid < PBN / 4) __builtin_amdgcn_global_load_lds(src + tid, dst, 16, 0, 0);
}

// End of an iteration: this wave's copies have landed, then the workgroup
// barrier.  The signal fences keep the compiler from moving LDS accesses
// across the barrier without making the hardware drain the LDS queue.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), no wait on the other counters
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Phase 1 of tile k: PV product of tile k - 1 (values `sv`) and QK product of
// tile k (keys `sk`; from the additive mask `sb` on far tiles, from the zeros
// `sz` on near ones, both read from LDS), at the default issue priority (a
// raised priority for the phase made the kernel 1-2 % slower).
template <int D>
__device__ __forceinline__ void phase1(int k, int ntw, int nfar, const uint4 *__restrict__ sk,
                                       const uint4 *__restrict__ sv, const floatx4 *__restrict__ sb,
                                       const floatx4 *__restrict__ sz, const uint4 (&qf)[2][D / 32],
                                       floatx4 (&s)[2][2], const uint4 (&pb)[2],
                                       floatx4 (&o)[D / 16][2], int lane, int quad) {
  if (k >= 1 && k - 1 < ntw) pv_tile<D>(sv, pb, lane, o);
  if (k < ntw) {
    const floatx4 *ip = k < nfar ? sb : sz;
    const floatx4 init[2] = {ip[2 * quad], ip[2 * quad + 1]};
    qk_tile<D>(sk, init, qf, lane, s);
  }
}

// Steady state, tile k >= 1 that needs no per-element mask (a far tile of
// the dense kernel, a tile whose keys every query sees in the others): phase
// 1 and phase 2 with every test on k resolved, for the loops that run only
// such tiles.  The QK product starts from `init`.  The products run at the
// default issue priority: a raised one made the dense kernel 2 % slower here.
template <int D>
__device__ __forceinline__ void steady_step(const uint4 *__restrict__ sk,
                                            const uint4 *__restrict__ sv, const floatx4 (&init)[2],
                                            const uint4 (&qf)[2][D / 32], floatx4 (&s)[2][2],
                                            uint4 (&pb)[2], floatx4 (&o)[D / 16][2], Softmax &sm,
                                            float c, int lane) {
  pv_tile<D>(sv, pb, lane, o);
  qk_tile<D>(sk, init, qf, lane, s);
  if (__ballot(crosses(s, sm))) move_reference<D>(s, sm, o, c);
  exponentials(s, sm, c, pb);
}

// Phase 2 of tile k: the full rule on near tiles, the reference check, and
// the exponentials.
template <int D>
__device__ __forceinline__ void phase2(int k, int ntw, int nfar, int S, int window, int qi0,
                                       int col, int quad, const floatx4 *__restrict__ sb,
                                       floatx4 (&s)[2][2], Softmax &sm, floatx4 (&o)[D / 16][2],
                                       uint4 (&pb)[2], float c) {
  if (k >= ntw) return;
  if (k >= nfar) {
    // near tile: causal bound, and the key's additive mask once it is w or
    // more behind the query (0 / -inf for the hard rule)
    const int j0 = k * PBN;
    const floatx4 mb[2] = {sb[2 * quad], sb[2 * quad + 1]};
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int i = qi0 + 16 * qt + col;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + 8 * quad + e;
        const float add = i - j >= window ? mb[e >> 2][e & 3] : 0.f;
        const bool causal = (j < S) & (j <= i);
        s[qt][e >> 2][e & 3] = causal ? s[qt][e >> 2][e & 3] + add : -INFINITY;
      }
    }
  }
  if (__ballot(crosses(s, sm))) move_reference<D>(s, sm, o, c);
  exponentials(s, sm, c, pb);
}

// ---- gathered-key prefill --------------------------------------------------
// Tile kinds of the gathered kernel's tile list: gathered tiles whose keys
// every query of the workgroup sees, gathered tiles on the edge (a key is seen
// by query i iff its position <= i - w), and dense band tiles (key j is seen
// iff i - w < j <= i).
template <int D>
__device__ __forceinline__ void g_phase1(int k, int nT, const uint4 *__restrict__ sk,
                                         const uint4 *__restrict__ sv, const uint4 (&qf)[2][D / 32],
                                         floatx4 (&s)[2][2], const uint4 (&pb)[2],
                                         floatx4 (&o)[D / 16][2], int lane) {
  __builtin_amdgcn_s_setprio(2);
  if (k >= 1 && k - 1 < nT) pv_tile<D>(sv, pb, lane, o);
  if (k < nT) {
    const floatx4 zero[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    qk_tile<D>(sk, zero, qf, lane, s);
  }
  __builtin_amdgcn_s_setprio(0);
}

template <int D>
__device__ __forceinline__ void g_phase2(int k, int nT, int nclean, int ngt, int band_j0, int S,
                                         int window, int qi0, int col, int quad,
                                         const int4 *__restrict__ sp, floatx4 (&s)[2][2],
                                         Softmax &sm, floatx4 (&o)[D / 16][2], uint4 (&pb)[2],
                                         float c) {
  if (k >= nT) return;
  if (k >= nclean) {
    if (k < ngt) {  // gathered edge tile: position <= i - w
      const int4 p0 = sp[2 * quad], p1 = sp[2 * quad + 1];
      const int pos[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int lim = qi0 + 16 * qt + col - window;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          s[qt][e >> 2][e & 3] = pos[e] <= lim ? s[qt][e >> 2][e & 3] : -INFINITY;
      }
    } else {  // band tile: i - w < j <= i
      const int j0 = band_j0 + (k - ngt) * PBN + 8 * quad;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int i = qi0 + 16 * qt + col;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + e;
          const bool vis = (j < S) & (j <= i) & (i - j < window);
          s[qt][e >> 2][e & 3] = vis ? s[qt][e >> 2][e & 3] : -INFINITY;
        }
      }
    }
  }
  if (__ballot(crosses(s, sm))) move_reference<D>(s, sm, o, c);
  exponentials(s, sm, c, pb);
}

// ---- chunk attention over the paged cache -----------------------------------
// Phase 2 of cache tile k for chunk queries: slots below n_clean are seen by
// every query; above it, slot j is seen by query position t iff it is in use,
// pos_j <= t, and it is unmarked or t - pos_j < w.
template <int D>
__device__ __forceinline__ void c_phase2(int k, int nt, int nclean_t, int ns, int nc, int window,
                                         int t_first, int col, int quad,
                                         const int4 *__restrict__ sp,
                                         const uint2 *__restrict__ sa, floatx4 (&s)[2][2],
                                         Softmax &sm, floatx4 (&o)[D / 16][2], uint4 (&pb)[2],
                                         float c) {
  if (k >= nt) return;
  if (k >= nclean_t) {
    const int4 p0 = sp[2 * quad], p1 = sp[2 * quad + 1];
    const int pos[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const uint2 a8 = sa[quad];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int t = t_first + 16 * qt + col;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int slot = k * PBN + 8 * quad + e;
        const uint32_t marked = ((e < 4 ? a8.x : a8.y) >> (8 * (e & 3))) & 0xffu;
        const bool vis = (slot < ns) &
                         ((slot < nc) | ((pos[e] <= t) & ((marked == 0u) | (t - pos[e] < window))));
        s[qt][e >> 2][e & 3] = vis ? s[qt][e >> 2][e & 3] : -INFINITY;
      }
    }
  }
  if (__ballot(crosses(s, sm))) move_reference<D>(s, sm, o, c);
  exponentials(s, sm, c, pb);
}

}  // namespace

// ---------------------------------------------------------------------------
// pack: one workgroup (4 D threads) per (tile, h, b)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(512) void k_prefill_pack(int S, int hkv, int ntiles,
                                                      const uint16_t *__restrict__ k,
                                                      const uint16_t *__restrict__ v,
                                                      const float *__restrict__ logit,
                                                      const float *__restrict__ noise, float inv_tau,
                                                      float inv_scale, int relaxed,
                                                      uint4 *__restrict__ packed,
                                                      float *__restrict__ mask,
                                                      uint4 *__restrict__ packed_far) {
  PDIMS(D);
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x;
  const int j0 = tile * PBN;
  const size_t T = tile_index(b, h, tile, hkv, ntiles);
  uint4 *kdst = packed + T * PTILE_U4;
  uint4 *vdst = kdst + PK_FRAGS * PFRAG;
  __shared__ __align__(16) uint16_t sv[PBN][PD + 8];  // row-major values, padded rows
  __shared__ uint32_t s_gone[PBN];                    // key masked (-inf) for far use

  // thread t: key jj = t / (D / 8), dims dc*8 .. +8
  const int jj = t / (PD / 8), dc = t % (PD / 8);
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
  // The far-tile copy: a key whose additive mask is -inf (marked, or past the
  // end) is invisible wherever a tile is far, so its key and value rows are
  // zero there.  Same scores and output; the matrix cores draw less power on
  // zero operands, which keeps the clock up.
  const bool gone = j >= S || (!relaxed && evict_decision(logit[(size_t(b) * S + j) * hkv + h]));
  uint4 *kfar = packed_far ? packed_far + T * PTILE_U4 : nullptr;
  if (kfar) kfar[(tt * PKS + ks) * PFRAG + qd * 16 + row] = gone ? make_uint4(0, 0, 0, 0) : kp;
  if (dc == 0) s_gone[jj] = gone ? 0u : 0xffffffffu;
  // additive mask of key j0 + t, applied once the key is w or more behind
  // the query: hard rule -inf if marked for eviction, 0 if kept; relaxed
  // rule log(1 - sigmoid((logit + noise) / tau)) = -softplus(x); -inf past
  // the end of the sequence.  Stored in raw score units (divided by the
  // softmax scale), the units the attention kernel adds it in.
  if (t < PBN) {
    float bias = -INFINITY;
    if (j0 + t < S) {
      const size_t at = (size_t(b) * S + j0 + t) * hkv + h;
      if (relaxed) {
        const float x = (logit[at] + (noise ? noise[at] : 0.f)) * inv_tau;
        bias = -(fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)))) * inv_scale;
      } else {
        bias = evict_decision(logit[at]) ? -INFINITY : 0.f;
      }
    }
    mask[T * PBN + t] = bias;
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
  if (kfar) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] &= (s_gone[k0 + 2 * e] & 0xffffu) | (s_gone[k0 + 2 * e + 1] & 0xffff0000u);
    kfar[PK_FRAGS * PFRAG + t] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int D>
__global__ __launch_bounds__(PNT, 3) void k_prefill(
    int batch, int S, int hkv, int G, int window, float scale_log2, const uint16_t *__restrict__ q,
    const uint4 *__restrict__ packed, const floatx4 *__restrict__ mask,
    const uint4 *__restrict__ packed_far, float *__restrict__ out) {
  PDIMS(D);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int col = lane & 15, quad = lane >> 4;
  const int Hq = hkv * G;
  const int ngh = (G + PHPW - 1) / PHPW;
  const int nqb = (S + PBN - 1) / PBN;  // 32 query positions per workgroup

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

  const int g = hg * PHPW + wave;
  const bool active = g < G;
  const int hq = h * G + (active ? g : 0);
  const int qi0 = qb * PBN;                 // first query position of the workgroup
  const int i_end = min(S, qi0 + PBN);      // causal key end
  const int ntiles = (i_end + PBN - 1) / PBN;
  // far tiles: j0 + 31 + window <= qi0, i.e. behind every query by >= window
  const int far_x = qi0 - window - (PBN - 1);
  const int nfar = far_x >= 0 ? min(ntiles, far_x / PBN + 1) : 0;

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
  Softmax sm;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    sm.m[qt] = -INFINITY;
    sm.nmc[qt] = 0.f;
    sm.thr[qt] = -INFINITY;
    sm.l[qt] = 0.f;
  }
  const float c = scale_log2;

  const int ntiles_all = (S + PBN - 1) / PBN;
  const uint4 *pk = packed + tile_index(b, h, 0, hkv, ntiles_all) * PTILE_U4;
  const uint4 *pkf = packed_far + tile_index(b, h, 0, hkv, ntiles_all) * PTILE_U4;
  const floatx4 *pm = mask + tile_index(b, h, 0, hkv, ntiles_all) * (PBN / 4);

  // the tile ring: packed tile and mask of tile t in buffer t % 3 (a far tile
  // from the copy whose masked keys are zero)
  __shared__ uint4 sT0[PTILE_U4], sT1[PTILE_U4], sT2[PTILE_U4];
  __shared__ floatx4 sM0[PBN / 4], sM1[PBN / 4], sM2[PBN / 4];
  __shared__ floatx4 sZ[PBN / 4];  // zeros: the initial scores of a near tile
  auto copy = [&](int tile, uint4 *dt, floatx4 *dm) {
    ring_copy<PTILE_U4>((tile < nfar ? pkf : pk) + size_t(tile) * PTILE_U4, dt, tid, wave);
    ring_copy_keys(pm + size_t(tile) * (PBN / 4), dm, tid);
  };
  copy(0, sT0, sM0);
  if (tid < PBN / 4) sZ[tid] = floatx4{0.f, 0.f, 0.f, 0.f};
  ring_barrier();

  const int ntw = ntiles;  // every wave needs every tile of the block
  floatx4 s[2][2];
  uint4 pb[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  // iteration k: keys and mask of tile k in (t, m), values of tile k - 1 in
  // tp; the copy of tile k + 1 goes to (tn, mn)
  auto iteration = [&](int k, const uint4 *t, const floatx4 *m, const uint4 *tp, uint4 *tn,
                       floatx4 *mn) {
    if (k + 1 < ntiles) copy(k + 1, tn, mn);
    if (active) {
      phase1<D>(k, ntw, nfar, t, tp + PK_FRAGS * PFRAG, m, sZ, qf, s, pb, o, lane, quad);
      phase2<D>(k, ntw, nfar, S, window, qi0, col, quad, m, s, sm, o, pb, c);
    }
    ring_barrier();
  };
  auto far_iteration = [&](int k, const uint4 *t, const floatx4 *m, const uint4 *tp, uint4 *tn,
                           floatx4 *mn) {
    if (k + 1 < ntiles) copy(k + 1, tn, mn);
    if (active) {
      const floatx4 init[2] = {m[2 * quad], m[2 * quad + 1]};
      steady_step<D>(t, tp + PK_FRAGS * PFRAG, init, qf, s, pb, o, sm, c, lane);
    }
    ring_barrier();
  };
  // tile 0; then the far tiles 1 .. nfar - 1 in whole rounds of three; then
  // the rest (the last far tiles, the near tiles, the PV product of the last
  // tile) on the general path.  Tile k is in buffer k % 3.
  iteration(0, sT0, sM0, sT2, sT1, sM1);
  int k = 1;
  for (; k + 2 < nfar; k += 3) {
    far_iteration(k, sT1, sM1, sT0, sT2, sM2);
    far_iteration(k + 1, sT2, sM2, sT1, sT0, sM0);
    far_iteration(k + 2, sT0, sM0, sT2, sT1, sM1);
  }
  for (; k <= ntiles; k += 3) {
    iteration(k, sT1, sM1, sT0, sT2, sM2);
    if (k + 1 > ntiles) break;
    iteration(k + 1, sT2, sM2, sT1, sT0, sM0);
    if (k + 2 > ntiles) break;
    iteration(k + 2, sT0, sM0, sT2, sT1, sM1);
  }

  if (!active) return;
  // the ring buffers are free: every wave has passed the last barrier
  float *stage = reinterpret_cast<float *>(wave < 2 ? sT0 : sT1) + (wave & 1) * (16 * PD);
  store_rows<D>(o, sm, stage, out, (size_t(b) * S * Hq + hq) * PD, size_t(Hq) * PD, qi0, S, lane);
}


// ---------------------------------------------------------------------------
// gathered-key prefill, step 1: per unit, the positions of the kept keys in
// order (gpos), the number kept before each 32-key tile (tile_cnt, ntiles + 1
// entries) and each tile's kept-key bits (keptw).  One workgroup per unit.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_sparse_scan(int S, int hkv, int ntiles,
                                                      const float *__restrict__ logit,
                                                      int32_t *__restrict__ gpos,
                                                      int32_t *__restrict__ tile_cnt,
                                                      uint32_t *__restrict__ keptw) {
  // Thread t takes keys base + 8t .. + 7 of each 8192-key stretch: its eight
  // decisions are loaded together, one workgroup scan of the per-thread kept
  // counts orders the whole stretch, and a 32-key tile is the keys of four
  // consecutive threads.
  constexpr int KPT = 8, NT = 1024, STRETCH = KPT * NT;
  const int u = blockIdx.x;
  const int b = u / hkv, h = u % hkv;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  __shared__ int s_wsum[NT / kWave];
  int running = 0;
  for (int base = 0; base < S; base += STRETCH) {
    const int j0 = base + KPT * tid;
    uint32_t bits = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int j = j0 + r;
      const bool kept = j < S && !evict_decision(logit[(size_t(b) * S + j) * hkv + h]);
      bits |= uint32_t(kept) << r;
    }
    const int cnt = __popc(bits);
    // exclusive prefix of the kept counts over the workgroup
    const int incl = wave_inclusive_scan(cnt);
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
      int v = lane < NT / kWave ? s_wsum[lane] : 0;
      v = wave_inclusive_scan(v);
      if (lane < NT / kWave) s_wsum[lane] = v;
    }
    __syncthreads();
    const int before = running + (wave > 0 ? s_wsum[wave - 1] : 0) + incl - cnt;
    const int total = s_wsum[NT / kWave - 1];
    int g = before;
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      if (bits & (1u << r)) gpos[size_t(u) * S + g++] = j0 + r;
    // tile (j0 / 32): the bits of threads 4T .. 4T+3, and the count before it
    uint32_t tile_bits = bits << (KPT * (tid & 3));
    tile_bits |= __shfl_xor(tile_bits, 1, kWave);
    tile_bits |= __shfl_xor(tile_bits, 2, kWave);
    if ((tid & 3) == 0 && j0 < S) {
      const int t = j0 >> 5;
      keptw[size_t(u) * ntiles + t] = tile_bits;
      tile_cnt[size_t(u) * (ntiles + 1) + t] = before;
    }
    running += total;
    __syncthreads();  // s_wsum is rewritten by the next stretch
  }
  if (tid == 0) tile_cnt[size_t(u) * (ntiles + 1) + ntiles] = running;
}

// ---------------------------------------------------------------------------
// gathered-key prefill, step 2, one workgroup (4 D threads) per (tile, h, b):
//   * the values of dense tile `tile` (keys 32 tile .. +31) in the transposed
//     fragment order, written to the value half of the dense tile (the band
//     tiles' values; their keys are gathered by the attention kernel itself
//     from K), zero past the end of the sequence;
//   * gathered tile gt = tile of the unit, if it holds kept keys: kept keys
//     32 gt .. 32 gt + 31 (in position order) in the packed fragment layout,
//     and their positions (INT_MAX past the last kept key).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(512) void k_sparse_pack(int S, int hkv, int ntiles,
                                                     const uint16_t *__restrict__ k,
                                                     const uint16_t *__restrict__ v,
                                                     const int32_t *__restrict__ gpos,
                                                     const int32_t *__restrict__ tile_cnt,
                                                     uint4 *__restrict__ dense,
                                                     uint4 *__restrict__ packed,
                                                     int32_t *__restrict__ gposp) {
  PDIMS(D);
  const int gt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int u = b * hkv + h;
  const int n = tile_cnt[size_t(u) * (ntiles + 1) + ntiles];
  const int t = threadIdx.x;
  const size_t T = tile_index(b, h, gt, hkv, ntiles);
  __shared__ __align__(16) uint16_t sv[PBN][PD + 8];   // dense tile values, row-major
  __shared__ __align__(16) uint16_t sg[PBN][PD + 8];   // gathered tile values, row-major
  const bool gathered = gt * PBN < n;

  const int jj = t / (PD / 8), dc = t % (PD / 8);
  const int j = gt * PBN + jj;
  *reinterpret_cast<uint4 *>(&sv[jj][dc * 8]) =
      j < S ? *reinterpret_cast<const uint4 *>(v + ((size_t(b) * S + j) * hkv + h) * PD + dc * 8)
            : make_uint4(0, 0, 0, 0);
  if (gathered) {
    const int g = gt * PBN + jj;
    uint4 kp = make_uint4(0, 0, 0, 0), vp = make_uint4(0, 0, 0, 0);
    if (g < n) {
      const int jg = gpos[size_t(u) * S + g];
      const size_t off = ((size_t(b) * S + jg) * hkv + h) * PD + dc * 8;
      kp = *reinterpret_cast<const uint4 *>(k + off);
      vp = *reinterpret_cast<const uint4 *>(v + off);
    }
    const int tt = (jj & 7) >> 2, row = 4 * (jj >> 3) + (jj & 3);
    const int ks = dc >> 2, qd = dc & 3;
    packed[T * PTILE_U4 + (tt * PKS + ks) * PFRAG + qd * 16 + row] = kp;
    *reinterpret_cast<uint4 *>(&sg[jj][dc * 8]) = vp;
    if (t < PBN) {
      const int gg = gt * PBN + t;
      gposp[T * PBN + t] = gg < n ? gpos[size_t(u) * S + gg] : INT_MAX;
    }
  }
  __syncthreads();
  // value fragment dt = t / 64, lane l = t % 64: dim dt*16 + l % 16, keys 8*(l/16) .. +8
  const int dt = t >> 6, l = t & 63;
  const int d = dt * 16 + (l & 15), k0 = 8 * (l >> 4);
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = uint32_t(sv[k0 + 2 * e][d]) | (uint32_t(sv[k0 + 2 * e + 1][d]) << 16);
  dense[T * PTILE_U4 + PK_FRAGS * PFRAG + t] = make_uint4(w[0], w[1], w[2], w[3]);
  if (gathered) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = uint32_t(sg[k0 + 2 * e][d]) | (uint32_t(sg[k0 + 2 * e + 1][d]) << 16);
    packed[T * PTILE_U4 + PK_FRAGS * PFRAG + t] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// kept keys of unit u at positions <= x
__device__ __forceinline__ int kept_upto(int x, int S, int ntiles, const int32_t *tc,
                                         const uint32_t *kw) {
  if (x < 0) return 0;
  if (x >= S - 1) return tc[ntiles];
  const int t = x >> 5, r = x & 31;
  const uint32_t below = r == 31 ? 0xffffffffu : ((2u << r) - 1u);
  return tc[t] + __popc(kw[t] & below);
}

// ---------------------------------------------------------------------------
// gathered-key prefill, step 3: attention over [gathered tiles | band tiles]
// with the two-phase schedule of k_prefill.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(PNT, 3) void k_prefill_gathered(
    int batch, int S, int hkv, int G, int window, float scale_log2, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ kmat, const uint4 *__restrict__ dense,
    const uint4 *__restrict__ gathered,
    const int4 *__restrict__ gposp, const int32_t *__restrict__ tile_cnt,
    const uint32_t *__restrict__ keptw, float *__restrict__ out) {
  PDIMS(D);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int col = lane & 15, quad = lane >> 4;
  const int Hq = hkv * G;
  const int ngh = (G + PHPW - 1) / PHPW;
  const int nqb = (S + PBN - 1) / PBN;  // 32 query positions per workgroup

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
  const int u = b * hkv + h;

  const int g = hg * PHPW + wave;
  const bool active = g < G;
  const int hq = h * G + (active ? g : 0);
  const int qi0 = qb * PBN;
  const int q0 = qi0;
  const int i_max = min(S, q0 + PBN) - 1;  // last query position of the workgroup

  // tile list: gathered tiles [0, ngt) (the first nclean seen by every query),
  // then dense tiles covering the band (q0 - w, i_max]
  const int ntiles_all = (S + PBN - 1) / PBN;
  const int32_t *tc = tile_cnt + size_t(u) * (ntiles_all + 1);
  const uint32_t *kw = keptw + size_t(u) * ntiles_all;
  const int n_any = kept_upto(i_max - window, S, ntiles_all, tc, kw);
  const int n_all = kept_upto(q0 - window, S, ntiles_all, tc, kw);
  const int ngt = (n_any + PBN - 1) / PBN;
  const int nclean = n_all / PBN;
  const int tb0 = max(0, q0 - window + 1) / PBN;
  const int nT = ngt + i_max / PBN - tb0 + 1;
  const int band_j0 = tb0 * PBN;

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
  Softmax sm;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    sm.m[qt] = -INFINITY;
    sm.nmc[qt] = 0.f;
    sm.thr[qt] = -INFINITY;
    sm.l[qt] = 0.f;
  }
  const float c = scale_log2;

  // The tile ring of k_prefill; tile t comes from the gathered layout (t <
  // ngt, with its key positions) or is a band tile: its key fragments are
  // gathered by the load unit straight from K (each lane names the 16 bytes
  // of the key row and dims its fragment lane holds, so the 1 KB a copy
  // instruction writes is one fragment), its values come packed.
  const size_t ubase = size_t(u) * ntiles_all;
  __shared__ uint4 sT0[PTILE_U4], sT1[PTILE_U4], sT2[PTILE_U4];
  __shared__ int4 sP0[PBN / 4], sP1[PBN / 4], sP2[PBN / 4];
  auto copy = [&](int t, uint4 *dt, int4 *dp) {
    if (t < ngt) {
      ring_copy<PTILE_U4>(gathered + (ubase + t) * PTILE_U4, dt, tid, wave);
      ring_copy_keys(gposp + (ubase + t) * (PBN / 4), dp, tid);
    } else {
      const int jt = tb0 + t - ngt;  // key tile
      const int row = lane & 15, qd = lane >> 4;
#pragma unroll
      for (int f = wave; f < PK_FRAGS; f += PNT / kWave) {
        const int tt = f / PKS, ks = f % PKS;
        const int j = min(jt * PBN + 8 * (row >> 2) + 4 * tt + (row & 3), S - 1);
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const uint4 *>(kmat + ((size_t(b) * S + j) * hkv + h) * PD + ks * 32 + qd * 8),
            dt + f * PFRAG, 16, 0, 0);
      }
      ring_copy<PV_FRAGS * PFRAG>(dense + (ubase + jt) * PTILE_U4 + PK_FRAGS * PFRAG,
                                  dt + PK_FRAGS * PFRAG, tid, wave);
    }
  };
  copy(0, sT0, sP0);
  ring_barrier();

  floatx4 s[2][2];
  uint4 pb[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  auto iteration = [&](int k, const uint4 *t, const int4 *p, const uint4 *tp, uint4 *tn,
                       int4 *pn) {
    if (k + 1 < nT) copy(k + 1, tn, pn);
    if (active) {
      g_phase1<D>(k, nT, t, tp + PK_FRAGS * PFRAG, qf, s, pb, o, lane);
      g_phase2<D>(k, nT, nclean, ngt, band_j0, S, window, qi0, col, quad, p, s, sm, o, pb, c);
    }
    ring_barrier();
  };
  auto clean_iteration = [&](int k, const uint4 *t, const uint4 *tp, uint4 *tn, int4 *pn) {
    if (k + 1 < nT) copy(k + 1, tn, pn);
    if (active) {
      const floatx4 zero[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
      steady_step<D>(t, tp + PK_FRAGS * PFRAG, zero, qf, s, pb, o, sm, c, lane);
    }
    ring_barrier();
  };
  // tile 0; the clean tiles 1 .. nclean - 1 in whole rounds of three; the rest
  // on the general path.  Tile k is in buffer k % 3.
  iteration(0, sT0, sP0, sT2, sT1, sP1);
  int k = 1;
  for (; k + 2 < nclean; k += 3) {
    clean_iteration(k, sT1, sT0, sT2, sP2);
    clean_iteration(k + 1, sT2, sT1, sT0, sP0);
    clean_iteration(k + 2, sT0, sT2, sT1, sP1);
  }
  for (; k <= nT; k += 3) {
    iteration(k, sT1, sP1, sT0, sT2, sP2);
    if (k + 1 > nT) break;
    iteration(k + 1, sT2, sP2, sT1, sT0, sP0);
    if (k + 2 > nT) break;
    iteration(k + 2, sT0, sP0, sT2, sT1, sP1);
  }

  if (!active) return;
  // the ring buffers are free: every wave has passed the last barrier
  float *stage = reinterpret_cast<float *>(wave < 2 ? sT0 : sT1) + (wave & 1) * (16 * PD);
  store_rows<D>(o, sm, stage, out, (size_t(b) * S * Hq + hq) * PD, size_t(Hq) * PD, qi0, S, lane);
}

// The kernels of both head dimensions, instantiated here so that their host
// launch stubs are emitted.
#define DMS_PREFILL_KERNELS(D)                                                                    \
  template __global__ void k_prefill_pack<D>(int, int, int, const uint16_t *, const uint16_t *,     \
                                             const float *, const float *, float, float, int,       \
                                             uint4 *, float *, uint4 *);                            \
  template __global__ void k_prefill<D>(int, int, int, int, int, float, const uint16_t *,           \
                                        const uint4 *, const floatx4 *, const uint4 *, float *);    \
  template __global__ void k_sparse_pack<D>(int, int, int, const uint16_t *, const uint16_t *,      \
                                            const int32_t *, const int32_t *, uint4 *, uint4 *,     \
                                            int32_t *);                                             \
  template __global__ void k_prefill_gathered<D>(int, int, int, int, int, float, const uint16_t *,  \
                                                 const uint16_t *, const uint4 *, const uint4 *,    \
                                                 const int4 *, const int32_t *, const uint32_t *,   \
                                                 float *);
DMS_PREFILL_KERNELS(128)
DMS_PREFILL_KERNELS(64)
#undef DMS_PREFILL_KERNELS

template <int D>
static hipError_t launch_prefill_t(const dms_shape &s, const void *q, const void *k, const void *v,
                                   const float *logit, const float *noise, float temperature,
                                   int seq_len, float sm_scale, float *out, void *ws, hipStream_t st) {
  PDIMS(D);
  const int ntiles = (seq_len + PBN - 1) / PBN;
  if (s.kv_heads > 65535 || s.batch > 65535) return hipErrorInvalidValue;  // pack grid y, z
  const size_t tiles = size_t(s.batch) * s.kv_heads * ntiles;
  const size_t tile_bytes = size_t(PTILE_U4) * 16;
  uint4 *packed = static_cast<uint4 *>(ws);
  float *mask = reinterpret_cast<float *>(static_cast<char *>(ws) + align256(tiles * tile_bytes));
  // far-tile copy (masked keys zero); the relaxed mask hides no key, so its
  // far tiles read the plain copy
  const int relaxed = temperature > 0.f;
  uint4 *packed_far =
      relaxed ? nullptr
              : reinterpret_cast<uint4 *>(static_cast<char *>(ws) + align256(tiles * tile_bytes) +
                                          align256(tiles * PBN * sizeof(float)));
  hipLaunchKernelGGL(k_prefill_pack<D>, dim3(ntiles, s.kv_heads, s.batch), dim3(4 * D), 0, st,
                     seq_len, s.kv_heads, ntiles, static_cast<const uint16_t *>(k),
                     static_cast<const uint16_t *>(v), logit, noise,
                     relaxed ? 1.f / temperature : 0.f, 1.f / sm_scale, relaxed, packed, mask,
                     packed_far);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ngh = (s.group + PHPW - 1) / PHPW;
  const int nbh = s.batch * s.kv_heads * ngh;
  const int nqb = (seq_len + PBN - 1) / PBN;
  const int per_xcd_pairs = (nbh + 7) / 8;
  const long blocks = long(per_xcd_pairs) * nqb * 8;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_prefill<D>, dim3(unsigned(blocks)), dim3(PNT), 0, st, s.batch, seq_len,
                     s.kv_heads, s.group, s.window, sm_scale * 1.4426950408889634f,
                     static_cast<const uint16_t *>(q), packed,
                     reinterpret_cast<const floatx4 *>(mask), packed_far ? packed_far : packed, out);
  return hipGetLastError();
}

hipError_t launch_prefill(const dms_shape &s, const void *q, const void *k, const void *v,
                          const float *logit, const float *noise, float temperature, int seq_len,
                          float sm_scale, float *out, void *ws, hipStream_t st) {
  if (s.head_dim == 128)
    return launch_prefill_t<128>(s, q, k, v, logit, noise, temperature, seq_len, sm_scale, out, ws, st);
  if (s.head_dim == 64)
    return launch_prefill_t<64>(s, q, k, v, logit, noise, temperature, seq_len, sm_scale, out, ws, st);
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_prefill_gathered_t(const dms_shape &s, const void *q, const void *k,
                                            const void *v, const float *logit, int seq_len,
                                            float sm_scale, float *out, void *ws, hipStream_t st) {
  const int ntiles = (seq_len + PBN - 1) / PBN;
  if (s.kv_heads > 65535 || s.batch > 65535) return hipErrorInvalidValue;
  const PrefillGatheredLayout L = prefill_gathered_layout(s.batch, s.kv_heads, seq_len, D);
  char *base = static_cast<char *>(ws);
  uint4 *dense = reinterpret_cast<uint4 *>(base);
  float *mask = reinterpret_cast<float *>(base + L.dense_mask);
  uint4 *gathered = reinterpret_cast<uint4 *>(base + L.gathered);
  int32_t *gposp = reinterpret_cast<int32_t *>(base + L.gathered_pos);
  int32_t *gpos = reinterpret_cast<int32_t *>(base + L.gpos);
  int32_t *tile_cnt = reinterpret_cast<int32_t *>(base + L.tile_cnt);
  uint32_t *keptw = reinterpret_cast<uint32_t *>(base + L.keptw);
  const uint16_t *k16 = static_cast<const uint16_t *>(k), *v16 = static_cast<const uint16_t *>(v);
  (void)mask;
  hipLaunchKernelGGL(k_sparse_scan, dim3(s.batch * s.kv_heads), dim3(1024), 0, st, seq_len,
                     s.kv_heads, ntiles, logit, gpos, tile_cnt, keptw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sparse_pack<D>, dim3(ntiles, s.kv_heads, s.batch), dim3(4 * D), 0, st,
                     seq_len, s.kv_heads, ntiles, k16, v16, gpos, tile_cnt, dense, gathered, gposp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int ngh = (s.group + PHPW - 1) / PHPW;
  const int nbh = s.batch * s.kv_heads * ngh;
  const int nqb = (seq_len + PBN - 1) / PBN;
  const long blocks = long((nbh + 7) / 8) * nqb * 8;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_prefill_gathered<D>, dim3(unsigned(blocks)), dim3(PNT), 0, st, s.batch,
                     seq_len, s.kv_heads, s.group, s.window, sm_scale * 1.4426950408889634f,
                     static_cast<const uint16_t *>(q), k16, dense, gathered,
                     reinterpret_cast<const int4 *>(gposp), tile_cnt, keptw, out);
  return hipGetLastError();
}

hipError_t launch_prefill_gathered(const dms_shape &s, const void *q, const void *k, const void *v,
                                   const float *logit, int seq_len, float sm_scale, float *out,
                                   void *ws, hipStream_t st) {
  if (s.head_dim == 128)
    return launch_prefill_gathered_t<128>(s, q, k, v, logit, seq_len, sm_scale, out, ws, st);
  if (s.head_dim == 64)
    return launch_prefill_gathered_t<64>(s, q, k, v, logit, seq_len, sm_scale, out, ws, st);
  return hipErrorInvalidValue;
}


// ---------------------------------------------------------------------------
// Chunk attention: the last C appended tokens of every sequence attend over
// the unit's cache, each at its own position (same rule as decode).  A 32-slot
// group of a cache page has exactly the layout of a packed prefill tile
// (key_index / value_index), so tiles are copied from the pages into LDS with
// no pack pass.  Workgroup: one unit, 32 chunk queries, four query heads (one
// per wave); grid (ceil(C / 32), units * ceil(G / 4)).  A sequence shorter
// than the chunk, or compacted after the chunk's first position (compact_pos,
// kept with the plan), is flagged DMS_STATUS_CHUNK_INVALID in `status`.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(PNT, 3) void k_chunk_attn(
    int hkv, int G, int window, int maxp, int C, float scale_log2, int nsplit,
    const uint16_t *__restrict__ q, const uint4 *__restrict__ k_pages,
    const uint4 *__restrict__ v_pages, const int32_t *__restrict__ page_table,
    const int4 *__restrict__ slot_pos, const uint4 *__restrict__ slot_alpha,
    const int32_t *__restrict__ n_slots, const int32_t *__restrict__ n_clean,
    const int32_t *__restrict__ seq_len, const int32_t *__restrict__ compact_pos,
    uint32_t *__restrict__ status, float2 *__restrict__ part_ml, float *__restrict__ part_o,
    float *__restrict__ out) {
  PDIMS(D);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int col = lane & 15, quad = lane >> 4;
  const int ngh = (G + PHPW - 1) / PHPW;
  const int u = blockIdx.y / ngh, hg = blockIdx.y % ngh;
  const int b = u / hkv, h = u % hkv;
  const int Hq = hkv * G;
  const int g = hg * PHPW + wave;
  const bool active = g < G;
  const int hq = h * G + (active ? g : 0);
  const int qb = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
  const int c0 = qb * 32;                         // first chunk query of the workgroup
  const int t_first = seq_len[b] - C + c0;        // its position
  const int ns = n_slots[u], nc = n_clean[u];
  const int nt = (ns + PBN - 1) / PBN;
  const int nclean_t = nc / PBN;                  // tiles wholly below n_clean
  const int32_t *row = page_table + size_t(u) * maxp;
  // Tiles this workgroup reads.  The chunk's C tokens are the unit's last C
  // slots (nothing compacted it since, else the status flag below), so
  // query c0 + 31 sits in slot ns - C + c0 + 31 and later slots are hidden
  // from every query of the workgroup.  Split sp of nsplit takes every
  // nsplit-th tile up to there, tiles sp, sp + nsplit, ...: each split gets
  // its share of the clean tiles and of the costlier ones above n_clean,
  // which hold the chunk itself (equal ranges left the last split with the
  // chunk's tiles, the others idle at the end).  Tile i of the split is
  // tile_of(i); its first ni_clean tiles lie wholly below n_clean.
  const int last_slot = ns - C + min(c0 + 31, C - 1);
  const int nt_vis = last_slot < 0 ? 0 : min(nt, last_slot / PBN + 1);
  const int nt_clean = min(nclean_t, nt_vis);
  const int ni = nt_vis > sp ? (nt_vis - sp + nsplit - 1) / nsplit : 0;
  const int ni_clean = nt_clean > sp ? (nt_clean - sp + nsplit - 1) / nsplit : 0;
  auto tile_of = [&](int i) { return sp + i * nsplit; };
  if (qb == 0 && sp == 0 && hg == 0 && tid == 0) {
    const int p0 = seq_len[b] - C;  // the chunk's first position
    if (p0 < 0 || compact_pos[u] > p0) atomicOr(status, DMS_STATUS_CHUNK_INVALID);
  }
  // slots in use in the last tile read (all 32 unless it is the unit's last)
  const int tail_valid = ni > 0 && tile_of(ni - 1) == nt - 1 ? ns - (nt - 1) * PBN : PBN;

  uint4 qf[2][PKS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int cq = c0 + 16 * qt + col;
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) {
      qf[qt][ks] = make_uint4(0, 0, 0, 0);
      if (active && cq < C)
        qf[qt][ks] = *reinterpret_cast<const uint4 *>(
            q + ((size_t(b) * C + cq) * Hq + hq) * PD + ks * 32 + quad * 8);
    }
  }
  floatx4 o[PDT][2];
#pragma unroll
  for (int dt = 0; dt < PDT; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) o[dt][qt] = floatx4{0.f, 0.f, 0.f, 0.f};
  Softmax sm;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    sm.m[qt] = -INFINITY;
    sm.nmc[qt] = 0.f;
    sm.thr[qt] = -INFINITY;
    sm.l[qt] = 0.f;
  }
  const float c = scale_log2;

  // The tile ring of k_prefill.  Tile t = slots 32 t .. 32 t + 31: page
  // row[t / 2], group t % 2 of the page; its keys and values (8 KB each) go
  // to the first and second half of a buffer, its positions (128 bytes, lanes
  // 0..7 of wave 0) and decisions (32 bytes, lanes 0..1 of wave 1) beside.
  __shared__ uint4 sT0[PTILE_U4], sT1[PTILE_U4], sT2[PTILE_U4];
  __shared__ int4 sP0[PBN / 4], sP1[PBN / 4], sP2[PBN / 4];
  __shared__ uint4 sA0[PBN / 16], sA1[PBN / 16], sA2[PBN / 16];
  auto copy = [&](int t, uint4 *dt, int4 *dp, uint4 *da) {
    const size_t grp = size_t(row[t >> 1]) * 2 + (t & 1);
    ring_copy<PK_FRAGS * PFRAG>(k_pages + grp * (PK_FRAGS * PFRAG), dt, tid, wave);
    ring_copy<PV_FRAGS * PFRAG>(v_pages + grp * (PV_FRAGS * PFRAG), dt + PK_FRAGS * PFRAG, tid,
                                wave);
    ring_copy_keys(slot_pos + grp * (PBN / 4), dp, tid);
    if (wave == 1 && lane < PBN / 16)
      __builtin_amdgcn_global_load_lds(slot_alpha + grp * (PBN / 16) + lane, da, 16, 0, 0);
  };
  if (ni > 0) copy(tile_of(0), sT0, sP0, sA0);
  ring_barrier();

  floatx4 s[2][2];
  uint4 pb[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  const floatx4 zero[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  auto iteration = [&](int i, const uint4 *t, const int4 *p, const uint4 *a, const uint4 *tp,
                       uint4 *tn, int4 *pn, uint4 *an) {
    if (i + 1 < ni) copy(tile_of(i + 1), tn, pn, an);
    if (active) {
      if (i > 0) pv_tile<D>(tp + PK_FRAGS * PFRAG, pb, lane, o);
      qk_tile<D>(t, zero, qf, lane, s);
      c_phase2<D>(tile_of(i), nt, nclean_t, ns, nc, window, t_first, col, quad, p,
               reinterpret_cast<const uint2 *>(a), s, sm, o, pb, c);
    }
    ring_barrier();
  };
  auto clean_iteration = [&](int i, const uint4 *t, const uint4 *tp, uint4 *tn, int4 *pn,
                             uint4 *an) {
    if (i + 1 < ni) copy(tile_of(i + 1), tn, pn, an);
    if (active) steady_step<D>(t, tp + PK_FRAGS * PFRAG, zero, qf, s, pb, o, sm, c, lane);
    ring_barrier();
  };
  // the split's tile 0; its tiles after it wholly below n_clean in whole
  // rounds of three; the rest on the general path.  Tile i is in buffer i % 3.
  // The PV product of the last tile comes after the loop: its unused tail
  // slots are cleared there, away from the loop body's registers.
  if (ni > 0) iteration(0, sT0, sP0, sA0, sT2, sT1, sP1, sA1);
  int i = 1;
  for (; i + 2 < ni_clean; i += 3) {
    clean_iteration(i, sT1, sT0, sT2, sP2, sA2);
    clean_iteration(i + 1, sT2, sT1, sT0, sP0, sA0);
    clean_iteration(i + 2, sT0, sT2, sT1, sP1, sA1);
  }
  for (; i < ni; i += 3) {
    iteration(i, sT1, sP1, sA1, sT0, sT2, sP2, sA2);
    if (i + 1 >= ni) break;
    iteration(i + 1, sT2, sP2, sA2, sT1, sT0, sP0, sA0);
    if (i + 2 >= ni) break;
    iteration(i + 2, sT0, sP0, sA0, sT2, sT1, sP1, sA1);
  }
  if (ni > 0 && active) {
    const int lt = (ni - 1) % 3;  // the last tile's buffer
    const uint4 *tl = lt == 0 ? sT0 : (lt == 1 ? sT1 : sT2);
    pv_tile_tail<D>(tl + PK_FRAGS * PFRAG, pb, lane, tail_valid, o);
  }
  ring_barrier();  // every wave is done with the ring before it stages its output there

  if (!active) return;
  // The ring buffers are free: every wave has passed the last barrier.  One
  // workgroup per 32 queries writes the output; a split writes its
  // unnormalised output to its part of the workspace (same row order, row
  // r = (b C + c) Hq + hq) and its reference and row sum per row, merged by
  // k_chunk_merge.
  const size_t R = size_t(gridDim.y / ngh) / hkv * size_t(C) * Hq;  // rows: B * C * Hq
  float *dst = nsplit > 1 ? part_o + size_t(sp) * R * PD : out;
  float *stage = reinterpret_cast<float *>(wave < 2 ? sT0 : sT1) + (wave & 1) * (16 * PD);
  store_rows<D>(o, sm, stage, dst, (size_t(b) * C * Hq + hq) * PD, size_t(Hq) * PD, c0, C, lane,
                nsplit == 1);
  if (nsplit > 1) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float l = sm.l[qt];
      l += __shfl_xor(l, 16, kWave);
      l += __shfl_xor(l, 32, kWave);
      const int cq = c0 + 16 * qt + col;
      if (quad == 0 && cq < C)
        part_ml[size_t(sp) * R + (size_t(b) * C + cq) * Hq + hq] = make_float2(sm.m[qt], l);
    }
  }
}

// Merge of the splits of k_chunk_attn, one thread per four consecutive
// output floats of a row: with each split's reference m_s (raw score units),
// row sum l_s and unnormalised output o_s, out = sum_s w_s o_s / sum_s w_s l_s,
// w_s = 2^((m_s - M) c), M = max_s m_s; rows no split saw a key of are zero.
template <int D>
__global__ __launch_bounds__(256) void k_chunk_merge(int rows, int nsplit, float scale_log2,
                                                     const float2 *__restrict__ part_ml,
                                                     const float *__restrict__ part_o,
                                                     float *__restrict__ out) {
  constexpr int Q = D / 4;  // threads per row
  const size_t x = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (x >= size_t(rows) * Q) return;
  const size_t r = x / Q;
  float2 ml[4];
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    ml[s] = s < nsplit ? part_ml[size_t(s) * rows + r] : make_float2(-INFINITY, 0.f);
    M = fmaxf(M, ml[s].x);
  }
  floatx4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s >= nsplit || ml[s].x == -INFINITY) continue;
      const float w = exp2f((ml[s].x - M) * scale_log2);
      den = fmaf(ml[s].y, w, den);
      num += w * *reinterpret_cast<const floatx4 *>(part_o + (size_t(s) * rows * Q + x) * 4);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  *reinterpret_cast<floatx4 *>(out + x * 4) = num * inv;
}

#define DMS_CHUNK_KERNELS(D)                                                                      \
  template __global__ void k_chunk_attn<D>(int, int, int, int, int, float, int, const uint16_t *,   \
                                           const uint4 *, const uint4 *, const int32_t *,           \
                                           const int4 *, const uint4 *, const int32_t *,            \
                                           const int32_t *, const int32_t *, const int32_t *,       \
                                           uint32_t *, float2 *, float *, float *);                  \
  template __global__ void k_chunk_merge<D>(int, int, float, const float2 *, const float *, float *);
DMS_CHUNK_KERNELS(128)
DMS_CHUNK_KERNELS(64)
#undef DMS_CHUNK_KERNELS

hipError_t launch_chunk_attn(const dms_shape &s, const dms_cache &c, const void *q, int n_query,
                             float *out, float sm_scale, void *ws, size_t ws_bytes, hipStream_t st) {
  const int ngh = (s.group + PHPW - 1) / PHPW;
  const long gy = long(s.batch) * s.kv_heads * ngh;
  if (gy > 65535) return hipErrorInvalidValue;
  const int nqb = (n_query + 31) / 32;
  // split only when the workspace holds the partials
  int nsplit = chunk_splits(s, n_query);
  if (nsplit > 1 && (ws == nullptr || ws_bytes < chunk_split_bytes(s, n_query, nsplit))) nsplit = 1;
  const ChunkSplitLayout L = chunk_split_layout(s, n_query, nsplit);
  char *w = static_cast<char *>(ws);
  float2 *part_ml = nsplit > 1 ? reinterpret_cast<float2 *>(w + L.part_ml) : nullptr;
  float *part_o = nsplit > 1 ? reinterpret_cast<float *>(w + L.part_o) : nullptr;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  auto go = [&](auto kern, auto merge) {
    hipLaunchKernelGGL(kern, dim3(unsigned(nqb * nsplit), unsigned(gy)), dim3(256), 0, st,
                       s.kv_heads, s.group, s.window, s.max_pages_per_unit, n_query, scale_log2,
                       nsplit, static_cast<const uint16_t *>(q),
                       static_cast<const uint4 *>(c.k_pages), static_cast<const uint4 *>(c.v_pages),
                       c.page_table, reinterpret_cast<const int4 *>(c.slot_pos),
                       reinterpret_cast<const uint4 *>(c.slot_alpha), c.n_slots, c.n_clean, c.seq_len,
                       c.plan + plan_layout(units_of(s)).compact_pos, c.status, part_ml, part_o, out);
    if (nsplit > 1) {
      const size_t threads = size_t(L.rows) * (s.head_dim / 4);
      hipLaunchKernelGGL(merge, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, st, int(L.rows),
                         nsplit, scale_log2, part_ml, part_o, out);
    }
  };
  if (s.head_dim == 128) go(k_chunk_attn<128>, k_chunk_merge<128>);
  else if (s.head_dim == 64) go(k_chunk_attn<64>, k_chunk_merge<64>);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dms
