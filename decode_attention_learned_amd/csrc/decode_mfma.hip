// Split-K decode attention for bfloat16 caches on the gfx950 matrix cores.
//
// Same result as the generic kernel (see decode_kernels.hip for the method
// and its sources); this file only changes how the two contractions of a
// chunk are carried out.  Per KV head the G query heads share every key and
// value row, so per 32-slot group of a page the work is two small dense
// products:
//   S^T [32 slots x 16] = K [32 x D] . Q^T [D x 16]     (G heads, zero padded)
//   O^T [D x 16]       += V^T [D x 32] . P^T [32 x 16]
// each on v_mfma_f32_16x16x32_bf16 with float32 accumulation.  Every K/V byte
// is loaded from HBM once, straight into the MFMA operand registers, and
// serves all G heads of the group.
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 used below (lane l, q = l / 16):
//   A: row l % 16, eight consecutive k values chosen by q
//   B: column l % 16, the same eight k values
//   C: column l % 16, rows 4q .. 4q + 3
// The two 16-slot tiles of a group take their rows from the slot permutation
//   tile 0 row 4a + r -> slot 8a + r,   tile 1 row 4a + r -> slot 8a + 4 + r,
// so that after the QK products lane l holds the scores of head l % 16 for the
// eight consecutive slots 8q .. 8q + 7.  Those are exactly the eight k values
// it must supply to the PV product.  The page layout (key_index, value_index)
// stores every operand fragment as one contiguous 1 KB block, so each operand
// is one fully coalesced 16-byte-per-lane load.  No data moves between lanes
// except the two shuffles of the row max.
//
// Called through dms_decode_attn_fill, the kernel also takes the step's new
// token (reserved, not yet written): the unit's last chunk stages its key and
// value in LDS, adds it to the final combine as one more softmax term, and
// writes it to its slot.
#include "decode_common.h"

namespace dms {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

#ifndef DMS_DECODE_WAVES
#define DMS_DECODE_WAVES 8
#endif
constexpr int kMfmaWaves = DMS_DECODE_WAVES;  // waves per decode workgroup
constexpr int kMfmaThreads = kMfmaWaves * 64;
constexpr int kGroup = 32;  // slots per group (half a page)
constexpr int kMaxChunkPages = 1024;  // page ids staged in LDS per chunk
constexpr int kCombineCols = 8;       // output columns combined across waves per round

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// K/V bytes are read exactly once per call: nontemporal loads keep them from
// displacing reusable lines (page table, plan, partials) in the caches.
__device__ __forceinline__ uint4 ld16_stream(const uint16_t *p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ floatx4 mfma_bf16(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{lo, hi}, bf16x2v));
}

// acc + lo + hi of a packed bf16 pair, in one v_dot2c_f32_bf16
__device__ __forceinline__ float add_pair(uint32_t pair, float acc) {
  const bf16x2v one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pair), one, acc, false);
}

// Several queries per sequence (a chunk of C tokens just appended, at
// positions seq_len - C .. seq_len - 1): one launch serves queries c0 ..
// c0 + nq - 1 of the chunk, and the 16 B-operand columns hold (query, head)
// pairs col = (c - c0) * G + g, nq * G <= 16.  Decode is nq = C = 1.
// `chunk_status` (chunk queries only, else null): the first launch of a chunk
// flags DMS_STATUS_CHUNK_INVALID for a sequence shorter than the chunk or
// compacted after the chunk's first position.
template <int D>
__global__ __launch_bounds__(kMfmaThreads, 4) void k_decode_mfma(
    int units, int hkv, int G, int window, int maxp, float scale_log2, int nq, int c0, int C,
    const uint16_t *__restrict__ q, uint16_t *k_pages, uint16_t *v_pages,
    const int32_t *__restrict__ page_table, int32_t *slot_pos, uint8_t *slot_alpha,
    const int32_t *__restrict__ n_slots, const int32_t *__restrict__ n_clean_arr,
    const int32_t *__restrict__ seq_len, int32_t *__restrict__ plan,
    const int32_t *__restrict__ append_base, const uint16_t *__restrict__ k_new,
    const uint16_t *__restrict__ v_new, const float *__restrict__ logit_new,
    uint32_t *__restrict__ chunk_status, float2 *__restrict__ part_ml, float *__restrict__ part_o,
    float *__restrict__ out) {
  constexpr int KSTEPS = D / 32;  // QK products per 16-slot tile
  constexpr int DTILES = D / 16;  // PV products per group
  const PlanLayout L = plan_layout(units);
  const int c = blockIdx.x;
  ChunkInfo ci;
  if (!locate_chunk(c, hkv, plan, n_slots, n_clean_arr, seq_len, L, ci)) return;
  const int u = ci.unit, b = ci.b, h = ci.h;
  const int s_begin = ci.s_begin, t = ci.t, nclean = ci.nclean;
  const int32_t *row = page_table + size_t(u) * maxp;
  const int tid = threadIdx.x;
  if (chunk_status != nullptr && c0 == 0 && c == ci.first && tid == 0) {
    const int p0 = t - (C - 1);  // the chunk's first position
    if (p0 < 0 || plan[L.compact_pos + u] > p0) atomicOr(chunk_status, DMS_STATUS_CHUNK_INVALID);
  }

  // The step's token (decode with fill): its slot, reserved by the
  // allocation launch (n_new = 1), is the unit's newest and lies in the
  // unit's last chunk.  That chunk streams the slots before it; the token's
  // key and value are staged in LDS here by the load unit (no registers, no
  // wait), enter the combine below as one more softmax term, and are written
  // to the token's slot after the stream.
  __shared__ __align__(16) uint16_t s_tok[2 * D];  // key, then value
  __shared__ float s_tm[16];                       // the token's score per column (log2 units)
  const int tok_slot = k_new != nullptr && c == ci.first + ci.nch - 1 ? append_base[u] : -1;
  const bool own_tok = tok_slot >= 0;  // a refused unit has no token
  const size_t tok = size_t(b) * hkv + h;  // [B][1][Hkv]
  // The last wave handles the token: with a group count that is not a
  // multiple of the wave count it has one group less than the first waves,
  // so its token work after the stream overlaps their last group.
  constexpr int kTokWave = kMfmaWaves - 1;
  if (own_tok && tid >= kTokWave * kWave && tid < kTokWave * kWave + D / 8) {
    const int piece = tid - kTokWave * kWave;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4 *>(k_new + tok * D) + piece,
                                     reinterpret_cast<uint4 *>(s_tok), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4 *>(v_new + tok * D) + piece,
                                     reinterpret_cast<uint4 *>(s_tok + D), 16, 0, 0);
  }
  const int s_end = own_tok ? tok_slot : ci.s_end;  // the token's slot is not streamed
  const int lim = min(nclean, s_end);  // slots below lim need no liveness test

  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int col = lane & 15;  // (query, head) column in B and C operands, row index in A
  const int quad = lane >> 4;
  const int ncol = nq * G;
  const int cq = col < ncol ? col / G : 0;
  // query positions: this column's, and the first and last of the launch
  const int t_first = t - (C - 1) + c0;
  const int t_last = t_first + nq - 1;
  const int t_col = t_first + cq;

  // page ids of this chunk are staged in LDS, a segment of at most
  // kMaxChunkPages pages at a time (chunks start on a page boundary)
  __shared__ int s_pages[kMaxChunkPages];
  const int p_first = s_begin / kPage;
  const int npages = (s_end - s_begin + kPage - 1) / kPage;

  // Q^T operand: column `col`, dims ks*32 + quad*8 .. +8; columns >= nq * G are zero
  uint4 qb[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) qb[ks] = make_uint4(0, 0, 0, 0);
  if (col < ncol) {
    const int g = col - cq * G;
    const uint16_t *qp =
        q + ((size_t(b) * C + c0 + cq) * hkv * G + size_t(h) * G + g) * D + quad * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qb[ks] = ld16(qp + ks * 32);
  }

  floatx4 o[DTILES];
#pragma unroll
  for (int i = 0; i < DTILES; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  // m_run: the column's reference (-inf until a live slot is seen); m_thr =
  // m_run + kLazy; m_sub: what the exponent subtracts (0 while m_run = -inf)
  float m_run = -INFINITY, l_run = 0.f, m_thr = -INFINITY, m_sub = 0.f;
  constexpr float kLazy = 8.0f;

  const int ngroups = (s_end - s_begin + kGroup - 1) / kGroup;

  // operand registers of one group.  At D = 128 latency is hidden by
  // occupancy (4 waves per SIMD at this register count) rather than by a
  // second register set; D = 64 keeps two groups in flight (below).
  struct Regs {
    uint4 k0[KSTEPS], k1[KSTEPS], v[DTILES];
    int page;
  };
  // Every fragment is a contiguous 1 KB block of the group: lane l reads the
  // 16 bytes at l*8 elements (page layout: key_index / value_index).
  auto load_group = [&](Regs &r, int gi, int seg0) {
    const int pi = (gi * kGroup) / kPage - seg0;
    r.page = __builtin_amdgcn_readfirstlane(s_pages[pi]);
    const size_t base = size_t(r.page) * kPage * D + size_t((gi * kGroup) % kPage) * D + lane * 8;
    const uint16_t *kp = k_pages + base;
    const uint16_t *vp = v_pages + base;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      r.k0[ks] = ld16_stream(kp + ks * 512);
      r.k1[ks] = ld16_stream(kp + (KSTEPS + ks) * 512);
    }
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) r.v[dt] = ld16_stream(vp + dt * 512);
  };

  auto process = [&](Regs &r, int gi) {
    const int gs = s_begin + gi * kGroup;
    const int poff = gs % kPage;
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      s0 = mfma_bf16(r.k0[ks], qb[ks], s0);
      s1 = mfma_bf16(r.k1[ks], qb[ks], s1);
    }
    // scores of head `col` for slots gs + 8*quad + e, in log2 units
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] *= scale_log2;

    if (gs + kGroup > lim) {  // wave-uniform: tail of the chunk or not yet compacted
      // the lane's eight slots: decisions (8 bytes) and positions (2 x 16 bytes),
      // always inside the page, then a branch-free liveness test
      const size_t mb = size_t(r.page) * kPage + poff + quad * 8;
      const uint2 a8 = *reinterpret_cast<const uint2 *>(slot_alpha + mb);
      const int4 p0 = *reinterpret_cast<const int4 *>(slot_pos + mb);
      const int4 p1 = *reinterpret_cast<const int4 *>(slot_pos + mb + 4);
      const int pos[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      uint32_t keep[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int slot = gs + quad * 8 + e;
        const uint32_t marked = ((e < 4 ? a8.x : a8.y) >> (8 * (e & 3))) & 0xffu;
        // live for this column's query; live for at least one query of the launch
        const bool live = (slot < s_end) & ((slot < nclean) | ((pos[e] <= t_col) &
                                            ((marked == 0u) | ((t_col - pos[e]) < window))));
        const bool any = (slot < s_end) & ((slot < nclean) | ((pos[e] <= t_last) &
                                           ((marked == 0u) | ((t_first - pos[e]) < window))));
        sv[e] = live ? sv[e] : -INFINITY;
        keep[e >> 1] |= any ? (0xffffu << (16 * (e & 1))) : 0u;
      }
      // slots dead for every query of the launch, or unused, must not reach
      // the PV product even as 0 * NaN (the mask depends on the slot only,
      // as the value operand row does)
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        r.v[dt].x &= keep[0];
        r.v[dt].y &= keep[1];
        r.v[dt].z &= keep[2];
        r.v[dt].w &= keep[3];
      }
    }

    // Lazy reference: a column's reference m_run moves only when one of its
    // scores exceeds it by more than kLazy (log2 units), so every p <= 2^kLazy;
    // the result is independent of the reference.  The common path is a
    // per-lane compare; the cross-lane maximum and the rescale run only when
    // some score crosses the threshold.
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
    if (__ballot(mx > m_thr)) {
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const bool move = mx > m_thr;  // uniform over the four lanes of a column
      const float corr = move ? (m_run == -INFINITY ? 0.f : exp2f(m_run - mx)) : 1.f;
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) o[dt] *= corr;
      m_run = move ? mx : m_run;
      m_thr = move ? mx + kLazy : m_thr;
      m_sub = m_run == -INFINITY ? 0.f : m_run;
    }
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = exp2f(sv[e] - m_sub);
    const uint4 pb = make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]),
                                pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7]));
    // the row sum adds the bf16-rounded weights that enter the PV product, so
    // numerator and denominator use the same weights
    l_run = add_pair(pb.x, l_run);
    l_run = add_pair(pb.y, l_run);
    l_run = add_pair(pb.z, l_run);
    l_run = add_pair(pb.w, l_run);
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) o[dt] = mfma_bf16(r.v[dt], pb, o[dt]);
  };

  for (int seg0 = 0; seg0 < npages; seg0 += kMaxChunkPages) {
    const int segp = min(kMaxChunkPages, npages - seg0);
    __syncthreads();  // every wave is done with the previous segment
    for (int i = tid; i < segp; i += kMfmaThreads) s_pages[i] = row[p_first + seg0 + i];
    __syncthreads();
    const int g_end = min(ngroups, (seg0 + segp) * (kPage / kGroup));
    if constexpr (D == 64) {
      // At D = 64 a group is 8 KB per wave and two fit the register budget:
      // a wave requests its next group before it computes the current one,
      // halving the dependent round trips of a chunk (short chunks of small
      // heads are latency bound: Llama-1B-shaped step 22.2-23.4 -> 21.4-22.5
      // us, identical outputs).  At D = 128 a second set would cost occupancy.
      for (int gi = seg0 * (kPage / kGroup) + wave; gi < g_end; gi += 2 * kMfmaWaves) {
        Regs r0, r1;
        const bool two = gi + kMfmaWaves < g_end;  // wave-uniform
        load_group(r0, gi, seg0);
        if (two) load_group(r1, gi + kMfmaWaves, seg0);
        process(r0, gi);
        if (two) process(r1, gi + kMfmaWaves);
      }
    } else {
      for (int gi = seg0 * (kPage / kGroup) + wave; gi < g_end; gi += kMfmaWaves) {
        Regs r;
        load_group(r, gi, seg0);
        process(r, gi);
      }
    }
  }
  // The token, by the last wave after its stream (the staging copies issued
  // before it have long landed): its score q . k_new per column (this lane's
  // 32 dims, then the four quads; log2 units) for the combine, and its key,
  // value, position and decision to its slot.  (Ahead of the stream, the wait
  // for the staging copies delays the start of a wave and costs more than
  // the launch it saves; inside the group loop the compiler spills.)
  if (own_tok && wave == kTokWave) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the staging copies have landed
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const uint4 kf = *reinterpret_cast<const uint4 *>(s_tok + ks * 32 + quad * 8);
      const uint32_t qa[4] = {qb[ks].x, qb[ks].y, qb[ks].z, qb[ks].w};
      const uint32_t ka[4] = {kf.x, kf.y, kf.z, kf.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(__uint_as_float(qa[e] << 16), __uint_as_float(ka[e] << 16), acc);
        acc = fmaf(__uint_as_float(qa[e] & 0xffff0000u), __uint_as_float(ka[e] & 0xffff0000u), acc);
      }
    }
    acc += __shfl_xor(acc, 16, kWave);
    acc += __shfl_xor(acc, 32, kWave);
    if (quad == 0) s_tm[col] = acc * scale_log2;
    const int page = row[tok_slot / kPage], off = tok_slot % kPage;
    if (lane < D / 8)
      *reinterpret_cast<uint4 *>(k_pages + size_t(page) * kPage * D + key_index(off, lane * 8, D)) =
          *reinterpret_cast<const uint4 *>(s_tok + lane * 8);
#pragma unroll
    for (int e = 0; e < D / kWave; ++e)
      v_pages[size_t(page) * kPage * D + value_index(off, lane + kWave * e, D)] =
          s_tok[D + lane + kWave * e];
    if (lane == 0) {
      slot_pos[size_t(page) * kPage + off] = t;
      // the decision: sigmoid(logit) > 1/2  <=>  logit > 0 (NaN keeps)
      slot_alpha[size_t(page) * kPage + off] = evict_decision(logit_new[tok]) ? 1 : 0;
    }
  }
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  __shared__ float s_m[kMfmaWaves][16], s_l[kMfmaWaves][16];
  extern __shared__ __align__(16) float s_o[];
  const int ostride = D + 4;
  if (quad == 0) {
    s_m[wave][col] = m_run;
    s_l[wave][col] = l_run;
  }
  // output of column x / D: query c0 + col / G, head h * G + col % G
  const OutMap om{((size_t(b) * C + c0) * hkv * G + size_t(h) * G) * D, size_t(hkv) * G * D, G, D};
  const int rcols = min(ncol, kCombineCols);
  for (int r0 = 0; r0 < ncol; r0 += rcols) {
    if (r0 > 0) __syncthreads();  // every thread is done reading the previous columns
    if (col >= r0 && col < min(ncol, r0 + rcols)) {
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt)
        *reinterpret_cast<floatx4 *>(&s_o[(wave * rcols + col - r0) * ostride + dt * 16 + quad * 4]) = o[dt];
    }
    __syncthreads();
    const int xend = min(ncol, r0 + rcols) * D;
    for (int x = r0 * D + tid; x < xend; x += kMfmaThreads) {
      const int g = x / D, d = x % D;
      float M = s_m[0][g];
#pragma unroll
      for (int w = 1; w < kMfmaWaves; ++w) M = fmaxf(M, s_m[w][g]);
      if (own_tok) M = fmaxf(M, s_tm[g]);
      float Ls = 0.f, O = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kMfmaWaves; ++w) {
          const float mw = s_m[w][g];
          if (mw == -INFINITY) continue;
          const float f = exp2f(mw - M);
          Ls = fmaf(s_l[w][g], f, Ls);
          O = fmaf(s_o[(w * rcols + g - r0) * ostride + d], f, O);
        }
        if (own_tok) {  // the token: weight 2^(score - M), value v_new
          const float f = exp2f(s_tm[g] - M);
          Ls += f;
          O = fmaf(__uint_as_float(uint32_t(s_tok[D + d]) << 16), f, O);
        }
      }
      if (ci.nch == 1) {
        out[om.at(x)] = Ls > 0.f ? O / Ls : 0.f;
      } else {
        publish(part_o + size_t(c) * ncol * D + x, O);
        if (d == 0) {
          publish(reinterpret_cast<float *>(part_ml + size_t(c) * ncol + g), M);
          publish(reinterpret_cast<float *>(part_ml + size_t(c) * ncol + g) + 1, Ls);
        }
      }
    }
  }
  if (ci.nch > 1 && fused_merge(units))  // else merged by k_merge_partials
    count_and_merge(ci, ncol, D, plan + L.merge_count, part_ml, part_o, out, om);
}

bool launch_decode_mfma_part(const dms_shape &s, const dms_cache &c, const void *q, float *out,
                             float scale_log2, const DecodeWorkspace &w, char *ws, hipStream_t st,
                             int nq, int c0, int C, const DecodeFill *fill, bool chunk) {
  auto args = [&](auto kern) {
    const int rcols = nq * s.group < kCombineCols ? nq * s.group : kCombineCols;
    const size_t lds = size_t(kMfmaWaves) * rcols * (s.head_dim + 4) * sizeof(float);
    if (lds > 48 * 1024)  // gfx950 workgroups may use up to 160 KB of LDS
      (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    hipLaunchKernelGGL(kern, dim3(w.max_chunks), dim3(kMfmaThreads), lds, st, units_of(s), s.kv_heads,
                       s.group, s.window,
                       s.max_pages_per_unit, scale_log2, nq, c0, C, static_cast<const uint16_t *>(q),
                       static_cast<uint16_t *>(c.k_pages), static_cast<uint16_t *>(c.v_pages),
                       c.page_table, c.slot_pos, c.slot_alpha, c.n_slots, c.n_clean, c.seq_len,
                       c.plan, c.append_base,
                       fill ? static_cast<const uint16_t *>(fill->k_new) : nullptr,
                       fill ? static_cast<const uint16_t *>(fill->v_new) : nullptr,
                       fill ? fill->logit : nullptr, chunk ? c.status : nullptr,
                       reinterpret_cast<float2 *>(ws + w.part_ml),
                       reinterpret_cast<float *>(ws + w.part_o), out);
  };
  if (s.head_dim == 128) args(k_decode_mfma<128>);
  else if (s.head_dim == 64) args(k_decode_mfma<64>);
  else return false;
  return launch_merge(s, c, w, ws, out, nq * s.group, c0, C, st) == hipSuccess;
}


// A library built with DMS_DECODE_BF16_GENERIC (a test build, checked against
// this one) serves one-query decode of bf16 caches with the vector kernel.
bool launch_decode_mfma(const dms_shape &s, const dms_cache &c, const void *q, float *out,
                        float scale_log2, const DecodeWorkspace &w, char *ws, hipStream_t st,
                        int n_query, const DecodeFill *fill, bool chunk) {
  if (s.kv_dtype != DMS_KV_BF16 || s.group > 16) return false;
#ifdef DMS_DECODE_BF16_GENERIC
  if (!chunk) return false;
#endif
  // queries per launch: as many as fit the 16 operand columns
  const int per = 16 / s.group;
  for (int c0 = 0; c0 < n_query; c0 += per) {
    const int nq = n_query - c0 < per ? n_query - c0 : per;
    if (!launch_decode_mfma_part(s, c, q, out, scale_log2, w, ws, st, nq, c0, n_query,
                                 chunk ? nullptr : fill, chunk))
      return false;
  }
  return true;
}

}  // namespace dms
