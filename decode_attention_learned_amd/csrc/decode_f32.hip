// Split-K decode attention for float32 caches on the gfx950 matrix cores.
//
// Same result as the generic kernel (decode_kernels.hip holds the method and
// its sources); this file carries out the two contractions of a chunk on
// v_mfma_f32_16x16x4_f32, float32 operands and accumulation.  Per 32-slot
// group of a page, for the G query heads of the unit (or the heads of up to
// 16 / G queries of a chunk; zero-padded to 16 columns):
//   S^T [32 slots x 16] = K [32 x D] . Q^T [D x 16]
//   O^T [D x 16]       += V^T [D x 32] . P^T [32 x 16]
// Every K/V byte is loaded from HBM once, straight into operand registers,
// and serves every column.
//
// Operand layouts of v_mfma_f32_16x16x4_f32 (lane l, quad = l / 16): A holds
// element (l % 16, quad), B element (quad, l % 16), the result rows
// 4 quad .. 4 quad + 3 of column l % 16.
//   Product tile T of a group is its slots 16 T .. 16 T + 15 in order, so
//       lane (quad, col) ends the QK product with the scores of column col
//       for slots 16 T + 4 quad .. + 3 of both tiles, and PV k-step e of lane
//       group quad takes slot 16 (e >> 2) + 4 quad + (e & 3): the B operand is
//       the lane's own weight.  No data moves between lanes except the two
//       shuffles of the row maximum.
//   Loads are whole lines.  The page layout keeps 8 consecutive dims of a
//       key, and 8 consecutive slots of a value dim, as 32-byte runs; lane
//       groups 0 and 1 take the two 16-byte halves of the same runs, groups 2
//       and 3 those of the next ones.  Keys: the QK reduction index is
//       permuted, lane (quad, r) holding for m = 0 .. D/16 - 1 dims
//       8 f + 4 (quad & 1) .. + 4 with f = (quad >> 1) D/16 + m, k-step (m, i)
//       taking its dim i; a load instruction reads the runs of 8 layout rows
//       of both layout tiles (key_index: slot 8a + 4t + j sits in tile t, row
//       4a + j).  Values: the A operand of k-steps 4T .. 4T + 3 is half
//       (quad & 1) of the run of slots 8 (2T + (quad >> 1)) .. + 8 for dim
//       dt * 16 + l % 16 (value_index); a load instruction reads 1 KB in one
//       block.
// The softmax is the bf16 kernel's: float32 exp2 form with a lazy reference,
// and the row sums add the same weights that enter the PV product.
#include "decode_common.h"

namespace dms {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kF32Waves = 4;  // waves per workgroup: two workgroups per CU
constexpr int kF32Threads = kF32Waves * kWave;
constexpr int kF32Group = 32;             // slots per group (half a page)
constexpr int kF32ChunkPages = 1024;      // page ids staged in LDS per segment
constexpr float kF32Lazy = 8.0f;          // reference slack, log2 units

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// K/V bytes are read once per call: nontemporal loads keep them from
// displacing reusable lines in the caches.  Every load instruction reads
// whole lines (the operand orders described above).  Measured at B = 64, 8 KV
// heads, 4112 slots per unit, per call: 319-333 us; with value loads of half
// runs 334-336 us; with key loads of half runs too 387 us (351 us with plain
// key loads).
__device__ __forceinline__ floatx4 ld4_stream(const float *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(p));
}

}  // namespace

// Several queries per sequence, as in the bf16 kernel: a chunk of C tokens
// just appended, at positions seq_len - C .. seq_len - 1; one launch serves
// queries c0 .. c0 + nq - 1 of the chunk, and the 16 operand columns hold
// (query, head) pairs col = (c - c0) * G + g, nq * G <= 16.  Decode is
// nq = C = 1.  `chunk_status` (chunk queries only, else null): the first
// launch of a chunk flags DMS_STATUS_CHUNK_INVALID for a sequence shorter
// than the chunk or compacted after the chunk's first position.
template <int D>
__global__ __launch_bounds__(kF32Threads, 2) void k_decode_f32(
    int units, int hkv, int G, int window, int maxp, float scale_log2, int nq, int c0, int C,
    const float *__restrict__ q, const float *__restrict__ k_pages,
    const float *__restrict__ v_pages, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ slot_pos, const uint8_t *__restrict__ slot_alpha,
    const int32_t *__restrict__ n_slots, const int32_t *__restrict__ n_clean_arr,
    const int32_t *__restrict__ seq_len, int32_t *__restrict__ plan,
    uint32_t *__restrict__ chunk_status, float2 *__restrict__ part_ml,
    float *__restrict__ part_o, float *__restrict__ out) {
  constexpr int NH = D / 16;    // 4-float half runs per lane and tile
  constexpr int KS = D / 32;    // key fragments per tile in the page layout
  constexpr int DT = D / 16;    // PV products per k-step
  const PlanLayout L = plan_layout(units);
  const int c = blockIdx.x;
  ChunkInfo ci;
  if (!locate_chunk(c, hkv, plan, n_slots, n_clean_arr, seq_len, L, ci)) return;
  const int u = ci.unit, b = ci.b, h = ci.h;
  const int s_begin = ci.s_begin, s_end = ci.s_end, nclean = ci.nclean;
  const int tid = threadIdx.x;
  if (chunk_status != nullptr && c0 == 0 && c == ci.first && tid == 0) {
    const int p0 = ci.t - (C - 1);  // the chunk's first position
    if (p0 < 0 || plan[L.compact_pos + u] > p0) atomicOr(chunk_status, DMS_STATUS_CHUNK_INVALID);
  }
  const int32_t *row = page_table + size_t(u) * maxp;
  const int lim = min(nclean, s_end);  // slots below lim need no liveness test
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int col = lane & 15;  // (query, head) column in B and results, slot row or dim in A
  const int quad = lane >> 4;
  const int ncol = nq * G;
  const int cq = col < ncol ? col / G : 0;
  // query positions: this column's, and the first and last of the launch
  const int t_first = ci.t - (C - 1) + c0;
  const int t_last = t_first + nq - 1;
  const int t_col = t_first + cq;

  __shared__ int s_pages[kF32ChunkPages];
  const int p_first = s_begin / kPage;
  const int npages = (s_end - s_begin + kPage - 1) / kPage;

  // Q^T operand: column col, the lane's dims (as for its keys); zero for
  // columns >= nq * G
  floatx4 qv[NH];
#pragma unroll
  for (int m = 0; m < NH; ++m) qv[m] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (col < ncol) {
    const int g = col - cq * G;
    const float *qp = q + ((size_t(b) * C + c0 + cq) * hkv * G + size_t(h) * G + g) * D + 4 * (quad & 1);
#pragma unroll
    for (int m = 0; m < NH; ++m)
      qv[m] = *reinterpret_cast<const floatx4 *>(qp + 8 * ((quad >> 1) * NH + m));
  }

  floatx4 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  // m_run: the column's reference (-inf until a live slot is seen); m_thr =
  // m_run + kF32Lazy; m_sub: what the exponent subtracts (0 while m_run = -inf)
  float m_run = -INFINITY, l_run = 0.f, m_thr = -INFINITY, m_sub = 0.f;
  const int ngroups = (s_end - s_begin + kF32Group - 1) / kF32Group;

  // operand registers of one group
  struct Regs {
    floatx4 k[2][NH];        // product tile, the lane's m-th 4 dims of its row col
    floatx4 v[DT][2];        // dim dt * 16 + col, slots 16 T + 4 quad .. + 4
    int page;
  };
  auto load_group = [&](Regs &r, int gi, int seg0) {
    const int pi = (gi * kF32Group) / kPage - seg0;
    r.page = __builtin_amdgcn_readfirstlane(s_pages[pi]);
    const size_t base = size_t(r.page) * kPage * D + size_t((gi * kF32Group) % kPage) * D;
    // keys: row col of product tile T is slot 16 T + col of the group, which
    // the page layout keeps in tile (col >> 2) & 1 at row 4 (2 T + (col >> 3))
    // + (col & 3); the 16 rows of a product tile are two runs of 8 layout rows
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const int lt = (col >> 2) & 1, lrow = 4 * (2 * T + (col >> 3)) + (col & 3);
#pragma unroll
      for (int m = 0; m < NH; ++m) {
        // key_index of (that slot, dims 8 f + 4 (quad & 1) .. + 4)
        const int f = (quad >> 1) * NH + m;
        r.k[T][m] = ld4_stream(k_pages + base + (((lt * KS + (f >> 2)) * 4 + (f & 3)) * 16 + lrow) * 8 +
                               4 * (quad & 1));
      }
    }
    // values: slots 16 T + 4 quad .. + 4 of dim dt * 16 + col, half (quad & 1)
    // of the run of slots 8 (2 T + (quad >> 1)) .. + 8 (value_index); lane
    // groups 0 and 1 read the two halves of the same runs
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int T = 0; T < 2; ++T)
        r.v[dt][T] = ld4_stream(v_pages + base + ((dt * 4 + 2 * T + (quad >> 1)) * 16 + col) * 8 +
                                4 * (quad & 1));
  };

  auto process = [&](Regs &r, int gi) {
    const int gs = s_begin + gi * kF32Group;
    const int poff = gs % kPage;
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NH; ++m) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        s0 = mfma4(r.k[0][m][x], qv[m][x], s0);
        s1 = mfma4(r.k[1][m][x], qv[m][x], s1);
      }
    }
    // scores of column col for slots gs + 16 (e >> 2) + 4 quad + (e & 3), in log2 units
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] *= scale_log2;

    if (gs + kF32Group > lim) {  // wave-uniform: tail of the chunk or not yet compacted
      // the lane's eight slots (4 quad .. + 4 and 16 + 4 quad .. + 4 of the
      // group): decisions (2 x 4 bytes) and positions (2 x 16 bytes), always
      // inside the page, then a branch-free liveness test
      const size_t mb = size_t(r.page) * kPage + poff + quad * 4;
      const uint32_t a4[2] = {*reinterpret_cast<const uint32_t *>(slot_alpha + mb),
                              *reinterpret_cast<const uint32_t *>(slot_alpha + mb + 16)};
      const int4 p0 = *reinterpret_cast<const int4 *>(slot_pos + mb);
      const int4 p1 = *reinterpret_cast<const int4 *>(slot_pos + mb + 16);
      const int pos[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int slot = gs + 16 * (e >> 2) + quad * 4 + (e & 3);
        const uint32_t marked = (a4[e >> 2] >> (8 * (e & 3))) & 0xffu;
        // live for this column's query; live for at least one query of the launch
        const bool live = (slot < s_end) & ((slot < nclean) | ((pos[e] <= t_col) &
                                            ((marked == 0u) | ((t_col - pos[e]) < window))));
        const bool any = (slot < s_end) & ((slot < nclean) | ((pos[e] <= t_last) &
                                           ((marked == 0u) | ((t_first - pos[e]) < window))));
        sv[e] = live ? sv[e] : -INFINITY;
        // a slot hidden from every query of the launch, or unused, must not
        // reach the PV product even as 0 * NaN (a recycled page may hold NaN
        // there; the value row serves every column)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) r.v[dt][e >> 2][e & 3] = any ? r.v[dt][e >> 2][e & 3] : 0.f;
      }
    }

    // Lazy reference: a column's reference m_run moves only when one of its
    // scores exceeds it by more than kF32Lazy (log2 units), so every p <=
    // 2^kF32Lazy; the result is independent of the reference.
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
      for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
      m_run = move ? mx : m_run;
      m_thr = move ? mx + kF32Lazy : m_thr;
      m_sub = m_run == -INFINITY ? 0.f : m_run;
    }
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(sv[e] - m_sub);
      l_run += p[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = mfma4(r.v[dt][e >> 2][e & 3], p[e], o[dt]);
  };

  for (int seg0 = 0; seg0 < npages; seg0 += kF32ChunkPages) {
    const int segp = min(kF32ChunkPages, npages - seg0);
    __syncthreads();  // every wave is done with the previous segment
    for (int i = tid; i < segp; i += kF32Threads) s_pages[i] = row[p_first + seg0 + i];
    __syncthreads();
    const int g_end = min(ngroups, (seg0 + segp) * (kPage / kF32Group));
    for (int gi = seg0 * (kPage / kF32Group) + wave; gi < g_end; gi += kF32Waves) {
      Regs r;
      load_group(r, gi, seg0);
      process(r, gi);
    }
  }

  // combine the waves: per column the row sum over the lane's quads, then
  // the log-sum-exp rule over the waves in LDS
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  constexpr int OS = D + 4;  // row stride of the staged outputs
  __shared__ float s_m[kF32Waves][16], s_l[kF32Waves][16];
  __shared__ __align__(16) float s_o[kF32Waves * 16 * OS];
  if (quad == 0) {
    s_m[wave][col] = m_run;
    s_l[wave][col] = l_run;
  }
  if (col < ncol) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<floatx4 *>(&s_o[(wave * 16 + col) * OS + dt * 16 + quad * 4]) = o[dt];
  }
  __syncthreads();
  // output of column x / D: query c0 + col / G, head h * G + col % G
  const OutMap om{((size_t(b) * C + c0) * hkv * G + size_t(h) * G) * D, size_t(hkv) * G * D, G, D};
  for (int x = tid; x < ncol * D; x += kF32Threads) {
    const int g = x / D, d = x % D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < kF32Waves; ++w) M = fmaxf(M, s_m[w][g]);
    float Ls = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kF32Waves; ++w) {
        const float mw = s_m[w][g];
        if (mw == -INFINITY) continue;
        const float f = exp2f(mw - M);
        Ls = fmaf(s_l[w][g], f, Ls);
        O = fmaf(s_o[(w * 16 + g) * OS + d], f, O);
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
  if (ci.nch > 1 && fused_merge(units))  // else merged by k_merge_partials
    count_and_merge(ci, ncol, D, plan + L.merge_count, part_ml, part_o, out, om);
}

bool launch_decode_f32(const dms_shape &s, const dms_cache &c, const void *q, float *out,
                       float scale_log2, const DecodeWorkspace &w, char *ws, hipStream_t st, int nq,
                       int c0, int C, uint32_t *chunk_status) {
  if (s.kv_dtype != DMS_KV_F32 || nq < 1 || nq * s.group > 16) return false;
  auto run = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(w.max_chunks), dim3(kF32Threads), 0, st, units_of(s), s.kv_heads,
                       s.group, s.window, s.max_pages_per_unit, scale_log2, nq, c0, C,
                       static_cast<const float *>(q), static_cast<const float *>(c.k_pages),
                       static_cast<const float *>(c.v_pages), c.page_table, c.slot_pos, c.slot_alpha,
                       c.n_slots, c.n_clean, c.seq_len, c.plan, chunk_status,
                       reinterpret_cast<float2 *>(ws + w.part_ml),
                       reinterpret_cast<float *>(ws + w.part_o), out);
  };
  if (s.head_dim == 128) run(k_decode_f32<128>);
  else if (s.head_dim == 64) run(k_decode_f32<64>);
  else return false;
  return true;
}

}  // namespace dms
