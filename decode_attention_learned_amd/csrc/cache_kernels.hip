// Cache management kernels: reset, decide + append, compaction.
//
// Method: atlas.scime.ai summary of "Inference-Time Hyper-Scaling with KV
// Cache Compression", section "Approach" (per-head binary eviction decision,
// eviction executed after a delay window) and its table "Measured effects
// reported in the paper" (16-token window).  The decision here is the
// inference form of the Gumbel-sigmoid gate: alpha = logit > 0.
//
// Layout: one page = 64 slots of one unit, 64*D key elements in k_pages and
// 64*D value elements in v_pages, ordered by key_index / value_index
// (dms_internal.h) so that the decode kernel reads whole operand fragments.
#include <type_traits>

#include "dms_internal.h"

namespace dms {

// ---------------------------------------------------------------------------
// block-wide inclusive scan over NT threads (NT a multiple of 64, <= 4096)
// ---------------------------------------------------------------------------
template <int NT>
__device__ int block_inclusive_scan(int x, int *s_tmp, int &total) {
  const int w = threadIdx.x / kWave, l = lane_id();
  constexpr int NW = NT / kWave;
  int incl = wave_inclusive_scan(x);
  if (l == kWave - 1) s_tmp[w] = incl;
  __syncthreads();
  if (w == 0) {
    int v = (l < NW) ? s_tmp[l] : 0;
    int vs = wave_inclusive_scan(v);
    if (l < NW) s_tmp[l] = vs;
  }
  __syncthreads();
  const int off = (w > 0) ? s_tmp[w - 1] : 0;
  total = s_tmp[NW - 1];
  __syncthreads();
  return incl + off;
}

// ---------------------------------------------------------------------------
// reset
// ---------------------------------------------------------------------------
__global__ void k_reset(int units, int maxp, int num_pages, int batch, int32_t *page_table,
                        int32_t *free_list, int32_t *free_top, int32_t *n_slots,
                        int32_t *n_clean, int32_t *append_base, int32_t *seq_len,
                        uint32_t *status, int32_t *page_ref, int32_t *plan) {
  int32_t *compact_pos = plan + plan_layout(units).compact_pos;
  const long i0 = long(blockIdx.x) * blockDim.x + threadIdx.x;
  const long stride = long(gridDim.x) * blockDim.x;
  for (long x = i0; x < long(units) * maxp; x += stride) page_table[x] = -1;
  for (long x = i0; x < num_pages; x += stride) free_list[x] = int32_t(x);
  if (page_ref)
    for (long x = i0; x < num_pages; x += stride) page_ref[x] = 0;
  for (long x = i0; x < units; x += stride) {
    n_slots[x] = 0;
    n_clean[x] = 0;
    append_base[x] = -1;
    compact_pos[x] = -1;
  }
  for (long x = i0; x < batch; x += stride) seq_len[x] = 0;
  if (i0 == 0) {
    *free_top = num_pages;
    *status = 0u;
  }
}

// standalone planner (after reset and compaction)
__global__ __launch_bounds__(kPlanThreads) void k_plan(int units, const int32_t *n_slots,
                                                       int32_t *plan) {
  build_plan(units, [=](int u) { return n_slots[u]; }, plan);
}

hipError_t launch_plan(const dms_shape &s, const dms_cache &c, hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), 0, st, units_of(s), c.n_slots, c.plan);
  return hipGetLastError();
}

hipError_t launch_reset(const dms_shape &s, const dms_cache &c, hipStream_t st) {
  const int units = units_of(s);
  const long work = std::max(long(units) * s.max_pages_per_unit, long(s.num_pages));
  const int blocks = int(std::min<long>((work + 255) / 256, 4096));
  hipLaunchKernelGGL(k_reset, dim3(std::max(blocks, 1)), dim3(256), 0, st, units,
                     s.max_pages_per_unit, s.num_pages, s.batch, c.page_table, c.free_list,
                     c.free_top, c.n_slots, c.n_clean, c.append_base, c.seq_len, c.status,
                     c.page_ref, c.plan);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_plan(s, c, st);
}

// ---------------------------------------------------------------------------
// append, part 1: page allocation and metadata commit (one workgroup)
//
// Units are served in index order.  Unit u needs
//   need_u = ceil((n_slots_u + n_new) / 64) - ceil(n_slots_u / 64)
// new pages; with P_u the inclusive prefix sum of the needs and F the free
// count, a unit with need_u > 0 is served iff P_u <= F and takes the free
// stack entries [F - P_u, F - P_u + need_u).  Since P is non-decreasing the
// refused units are a suffix of the units that needed pages, and the pages
// handed out are distinct.  The result is deterministic.
// ---------------------------------------------------------------------------
constexpr int kAllocThreads = 1024;
// up to this many units the planner reads the new counts from LDS, not back
// from global memory
constexpr int kAllocLdsUnits = 4096;

__global__ __launch_bounds__(kAllocThreads) void k_append_alloc(
    int units, int batch, int maxp, int n_new, int32_t *page_table, int32_t *n_slots,
    int32_t *append_base, int32_t *seq_len, const int32_t *free_list, int32_t *free_top,
    uint32_t *status, int32_t *plan) {
  static_assert(kAllocThreads == kPlanThreads, "the planner runs in this workgroup");
  __shared__ int s_tmp[kAllocThreads / kWave];
  __shared__ int s_taken;
  __shared__ uint32_t s_flags;
  __shared__ int32_t s_ns[kAllocLdsUnits];
  if (threadIdx.x == 0) {
    s_taken = 0;
    s_flags = 0u;
  }
  // the free count, the first kAllocThreads counts and sequence lengths are
  // requested together
  const int F = *free_top;
  const int ns_first = int(threadIdx.x) < units ? n_slots[threadIdx.x] : 0;
  const int len_first = int(threadIdx.x) < batch ? seq_len[threadIdx.x] : 0;
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < units; base += kAllocThreads) {
    const int u = base + threadIdx.x;
    int ns = 0, have = 0, need = 0;
    bool row_ok = true;
    if (u < units) {
      ns = base == 0 ? ns_first : n_slots[u];
      have = (ns + kPage - 1) / kPage;
      const int want = (ns + n_new + kPage - 1) / kPage;
      row_ok = want <= maxp;
      need = row_ok ? want - have : 0;
    }
    int total = 0;
    const int incl = block_inclusive_scan<kAllocThreads>(need, s_tmp, total) + carry;
    if (u < units) {
      const bool ok = row_ok && (need == 0 || incl <= F);
      if (ok) {
        for (int i = 0; i < need; ++i)
          page_table[size_t(u) * maxp + have + i] = free_list[F - incl + i];
        append_base[u] = ns;
        n_slots[u] = ns + n_new;
        if (need > 0) atomicMax(&s_taken, incl);
      } else {
        append_base[u] = -1;
        atomicOr(&s_flags, row_ok ? DMS_STATUS_POOL_EXHAUSTED : DMS_STATUS_ROW_OVERFLOW);
      }
      if (u < kAllocLdsUnits) s_ns[u] = ok ? ns + n_new : ns;
    }
    carry += total;
  }
  for (int b = threadIdx.x; b < batch; b += kAllocThreads)
    seq_len[b] = (b < kAllocThreads ? len_first : seq_len[b]) + n_new;
  __syncthreads();
  if (threadIdx.x == 0) {
    *free_top = F - s_taken;
    if (s_flags) atomicOr(status, s_flags);
  }
  // n_slots changed: rebuild the decode split plan (each thread re-reads only
  // the entries it wrote above; from LDS when they all fit there)
  if (units <= kAllocLdsUnits)
    build_plan(units, [&](int u) { return s_ns[u]; }, plan);
  else
    build_plan(units, [=](int u) { return n_slots[u]; }, plan);
}

// ---------------------------------------------------------------------------
// append, part 2: decisions and the K/V bytes.  Grid (units, ceil(n_new/64)).
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void k_append_write(
    int hkv, int D, int n_new, int maxp, const E *__restrict__ k_new,
    const E *__restrict__ v_new, const float *__restrict__ logit,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ append_base,
    const int32_t *__restrict__ seq_len, E *__restrict__ k_pages, E *__restrict__ v_pages,
    int32_t *__restrict__ slot_pos, uint8_t *__restrict__ slot_alpha) {
  const int u = blockIdx.x;
  const int b = u / hkv, h = u % hkv;
  const int base = append_base[u];
  if (base < 0) return;  // refused by the allocator
  const int i0 = blockIdx.y * kPage;
  const int nt = min(kPage, n_new - i0);
  const int pos0 = seq_len[b] - n_new;  // seq_len was advanced by k_append_alloc

  extern __shared__ __align__(16) unsigned char smem[];
  int *s_page = reinterpret_cast<int *>(smem);
  int *s_off = s_page + kPage;
  E *s_v = reinterpret_cast<E *>(s_off + kPage);  // [64][D + 1]

  const int tid = threadIdx.x;
  if (tid < nt) {
    const int slot = base + i0 + tid;
    const int page = page_table[size_t(u) * maxp + slot / kPage];
    const int off = slot % kPage;
    s_page[tid] = page;
    s_off[tid] = off;
    const size_t tok = (size_t(b) * n_new + i0 + tid) * hkv + h;
    slot_pos[size_t(page) * kPage + off] = pos0 + i0 + tid;
    // the decision: sigmoid(logit) > 1/2  <=>  logit > 0 (NaN keeps)
    slot_alpha[size_t(page) * kPage + off] = evict_decision(logit[tok]) ? 1 : 0;
  }
  __syncthreads();

  // keys: 16-byte pieces (8 or 4 consecutive dims are contiguous in a page)
  constexpr int CE = 16 / int(sizeof(E));  // elements per 16-byte piece
  const int cpr = D / CE;
  for (int x = tid; x < nt * cpr; x += blockDim.x) {
    const int i = x / cpr, c = x % cpr;
    const size_t tok = (size_t(b) * n_new + i0 + i) * hkv + h;
    const uint4 *src = reinterpret_cast<const uint4 *>(k_new + tok * D + c * CE);
    uint4 *dst = reinterpret_cast<uint4 *>(k_pages + size_t(s_page[i]) * kPage * D +
                                           key_index(s_off[i], c * CE, D));
    *dst = *src;
  }
  // values: through LDS, then stored with consecutive threads on consecutive slots
  for (int x = tid; x < nt * D; x += blockDim.x) {
    const int i = x / D, d = x % D;
    const size_t tok = (size_t(b) * n_new + i0 + i) * hkv + h;
    s_v[i * (D + 1) + d] = v_new[tok * D + d];
  }
  __syncthreads();
  for (int x = tid; x < nt * D; x += blockDim.x) {
    const int d = x / nt, i = x % nt;
    v_pages[size_t(s_page[i]) * kPage * D + value_index(s_off[i], d, D)] = s_v[i * (D + 1) + d];
  }
}

hipError_t launch_append_alloc(const dms_shape &s, const dms_cache &c, int n_new, hipStream_t st) {
  hipLaunchKernelGGL(k_append_alloc, dim3(1), dim3(kAllocThreads), 0, st, units_of(s), s.batch,
                     s.max_pages_per_unit, n_new, c.page_table, c.n_slots, c.append_base,
                     c.seq_len, c.free_list, c.free_top, c.status, c.plan);
  return hipGetLastError();
}

hipError_t launch_append(const dms_shape &s, const dms_cache &c, const void *k_new,
                         const void *v_new, const float *logit, int n_new, hipStream_t st) {
  const hipError_t e = launch_append_alloc(s, c, n_new, st);
  return e != hipSuccess ? e : launch_append_write(s, c, k_new, v_new, logit, n_new, st);
}

hipError_t launch_append_write(const dms_shape &s, const dms_cache &c, const void *k_new,
                               const void *v_new, const float *logit, int n_new, hipStream_t st) {
  const int units = units_of(s);
  const dim3 grid(units, (n_new + kPage - 1) / kPage);
  const int D = s.head_dim;
  if (s.kv_dtype == DMS_KV_BF16) {
    const size_t lds = 2 * kPage * sizeof(int) + size_t(kPage) * (D + 1) * sizeof(uint16_t);
    hipLaunchKernelGGL(k_append_write<uint16_t>, grid, dim3(256), lds, st, s.kv_heads, D, n_new,
                       s.max_pages_per_unit, static_cast<const uint16_t *>(k_new),
                       static_cast<const uint16_t *>(v_new), logit, c.page_table,
                       c.append_base, c.seq_len, static_cast<uint16_t *>(c.k_pages),
                       static_cast<uint16_t *>(c.v_pages), c.slot_pos, c.slot_alpha);
  } else {
    const size_t lds = 2 * kPage * sizeof(int) + size_t(kPage) * (D + 1) * sizeof(uint32_t);
    hipLaunchKernelGGL(k_append_write<uint32_t>, grid, dim3(256), lds, st, s.kv_heads, D, n_new,
                       s.max_pages_per_unit, static_cast<const uint32_t *>(k_new),
                       static_cast<const uint32_t *>(v_new), logit, c.page_table,
                       c.append_base, c.seq_len, static_cast<uint32_t *>(c.k_pages),
                       static_cast<uint32_t *>(c.v_pages), c.slot_pos, c.slot_alpha);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// compaction: one workgroup (4 waves) per unit
//
// The region [n_clean, n_slots) is walked one source page at a time.  For
// each page, wave 0 marks the live slots (unmarked, or marked and younger
// than the window), ranks them with a ballot and mbcnt, and publishes each
// slot's destination.  Then every thread loads its share of the live rows
// and columns into registers, the workgroup synchronises, and the data is
// stored at the destinations.  Destinations never exceed sources and every
// read of a page happens before any write of that page, so the move is safe
// in place.  Pages left empty at the tail go back on the free stack.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(256) void k_compact(
    int hkv, int window, int maxp, int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_len, int32_t *__restrict__ n_slots,
    int32_t *__restrict__ n_clean, E *__restrict__ k_pages, E *__restrict__ v_pages,
    int32_t *__restrict__ slot_pos, uint8_t *__restrict__ slot_alpha,
    int32_t *__restrict__ free_list, int32_t *__restrict__ free_top,
    int32_t *__restrict__ compact_pos) {
  constexpr int CE = 16 / int(sizeof(E));           // elements per 16-byte piece
  constexpr int CPR = D / CE;                       // key pieces per slot
  constexpr int SPC = CE;                           // slots per 16-byte value piece
  constexpr int KCH = kPage * CPR / 256;            // key chunks per thread
  constexpr int VCH = D * (kPage / SPC) / 256;      // value chunks per thread
  static_assert(KCH >= 1 && VCH >= 1, "tile too small for 256 threads");

  const int u = blockIdx.x;
  const int b = u / hkv;
  const int lo = n_clean[u];
  const int hi = n_slots[u];
  const int t = seq_len[b] - 1;
  if (threadIdx.x == 0) compact_pos[u] = t;
  if (lo >= hi) return;
  const int thr = t - window;  // a marked slot with pos <= thr is dead
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = lane_id();
  const int32_t *row = page_table + size_t(u) * maxp;

  __shared__ int s_dst[kPage];
  int wp = lo;             // next destination slot (wave 0)
  int clean = lo;          // end of the unmarked prefix (wave 0)
  bool clean_done = false; // a marked survivor has been seen (wave 0)

  for (int P = lo / kPage; P * kPage < hi; ++P) {
    const int page = row[P];
    if (wave == 0) {
      const int s = P * kPage + lane;
      const bool inr = s >= lo && s < hi;
      int pos = 0;
      bool alpha = false;
      if (inr) {
        pos = slot_pos[size_t(page) * kPage + lane];
        alpha = slot_alpha[size_t(page) * kPage + lane] != 0;
      }
      const bool live = inr && (!alpha || pos > thr);
      const uint64_t mask = __ballot(live);
      const int cnt = __popcll(mask);
      s_dst[lane] = live ? wp + lanes_below(mask) : -1;
      if (!clean_done) {
        const uint64_t marked = __ballot(live && alpha);
        if (marked) {
          const int first = __ffsll((unsigned long long)marked) - 1;
          clean += __popcll(mask & ((uint64_t(1) << first) - 1));
          clean_done = true;
        } else {
          clean += cnt;
        }
      }
      wp += cnt;
    }
    __syncthreads();

    // load everything that moves
    uint4 kv[KCH];
    uint4 vv[VCH];
    int32_t mpos = 0;
    uint8_t malpha = 0;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int x = tid + r * 256;
      const int j = x / CPR, c = x % CPR;
      const int d = s_dst[j];
      if (d >= 0 && d != P * kPage + j)
        kv[r] = *reinterpret_cast<const uint4 *>(k_pages + size_t(page) * kPage * D + key_index(j, c * CE, D));
    }
#pragma unroll
    for (int r = 0; r < VCH; ++r) {
      const int x = tid + r * 256;
      const int d = x / (kPage / SPC), jc = x % (kPage / SPC);
      vv[r] = *reinterpret_cast<const uint4 *>(v_pages + size_t(page) * kPage * D + value_index(jc * SPC, d, D));
    }
    if (tid < kPage && s_dst[tid] >= 0) {
      mpos = slot_pos[size_t(page) * kPage + tid];
      malpha = slot_alpha[size_t(page) * kPage + tid];
    }
    __syncthreads();

    // store at the destinations
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int x = tid + r * 256;
      const int j = x / CPR, c = x % CPR;
      const int d = s_dst[j];
      if (d >= 0 && d != P * kPage + j) {
        const int dpage = row[d / kPage];
        *reinterpret_cast<uint4 *>(k_pages + size_t(dpage) * kPage * D + key_index(d % kPage, c * CE, D)) = kv[r];
      }
    }
#pragma unroll
    for (int r = 0; r < VCH; ++r) {
      const int x = tid + r * 256;
      const int d = x / (kPage / SPC), jc = x % (kPage / SPC);
      const E *el = reinterpret_cast<const E *>(&vv[r]);
#pragma unroll
      for (int e = 0; e < SPC; ++e) {
        const int j = jc * SPC + e;
        const int dst = s_dst[j];
        if (dst >= 0 && dst != P * kPage + j) {
          const int dpage = row[dst / kPage];
          v_pages[size_t(dpage) * kPage * D + value_index(dst % kPage, d, D)] = el[e];
        }
      }
    }
    if (tid < kPage) {
      const int dst = s_dst[tid];
      if (dst >= 0 && dst != P * kPage + tid) {
        const int dpage = row[dst / kPage];
        slot_pos[size_t(dpage) * kPage + dst % kPage] = mpos;
        slot_alpha[size_t(dpage) * kPage + dst % kPage] = malpha;
      }
    }
    __syncthreads();
  }

  if (tid == 0) {
    const int pages_before = (hi + kPage - 1) / kPage;
    const int pages_after = (wp + kPage - 1) / kPage;
    const int freed = pages_before - pages_after;
    if (freed > 0) {
      const int at = atomicAdd(free_top, freed);
      for (int i = 0; i < freed; ++i) {
        free_list[at + i] = page_table[size_t(u) * maxp + pages_after + i];
        page_table[size_t(u) * maxp + pages_after + i] = -1;
      }
    }
    n_slots[u] = wp;
    n_clean[u] = clean;
  }
}

template <typename E, int D>
static void launch_compact_t(const dms_shape &s, const dms_cache &c, hipStream_t st) {
  hipLaunchKernelGGL((k_compact<E, D>), dim3(units_of(s)), dim3(256), 0, st, s.kv_heads,
                     s.window, s.max_pages_per_unit, c.page_table, c.seq_len, c.n_slots,
                     c.n_clean, static_cast<E *>(c.k_pages), static_cast<E *>(c.v_pages),
                     c.slot_pos, c.slot_alpha, c.free_list, c.free_top,
                     c.plan + plan_layout(units_of(s)).compact_pos);
}

hipError_t launch_compact(const dms_shape &s, const dms_cache &c, hipStream_t st) {
  const bool bf = s.kv_dtype == DMS_KV_BF16;
  if (bf && s.head_dim == 64) launch_compact_t<uint16_t, 64>(s, c, st);
  else if (bf && s.head_dim == 128) launch_compact_t<uint16_t, 128>(s, c, st);
  else if (!bf && s.head_dim == 64) launch_compact_t<uint32_t, 64>(s, c, st);
  else launch_compact_t<uint32_t, 128>(s, c, st);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_plan(s, c, st);
}

// ---------------------------------------------------------------------------
// export: one workgroup (4 waves) per unit copies the retained set R(t),
// t = seq_len[b] - 1 (or, with all_slots, every slot in use), in slot order,
// which is position order: positions, decisions, and keys and values as
// plain [D] rows, undoing the fragment order of the pages.  For each page,
// wave 0 ranks the selected slots with a ballot and mbcnt; then every thread
// copies its share of their elements.  Only the first max_out are written;
// count_out gets the full count.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(256) void k_export(
    int hkv, int window, int maxp, int all_slots, int max_out,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_len,
    const int32_t *__restrict__ n_slots, const int32_t *__restrict__ n_clean,
    const E *__restrict__ k_pages, const E *__restrict__ v_pages,
    const int32_t *__restrict__ slot_pos, const uint8_t *__restrict__ slot_alpha,
    int32_t *__restrict__ count_out, int32_t *__restrict__ pos_out,
    uint8_t *__restrict__ alpha_out, E *__restrict__ k_out, E *__restrict__ v_out) {
  const int u = blockIdx.x;
  const int b = u / hkv;
  const int hi = n_slots[u], nc = n_clean[u];
  const int t = seq_len[b] - 1;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int32_t *row = page_table + size_t(u) * maxp;
  __shared__ int s_dst[kPage];
  int cnt = 0;  // selected slots so far (wave 0)
  for (int P = 0; P * kPage < hi; ++P) {
    const int page = row[P];
    if (wave == 0) {
      const int slot = P * kPage + lane;
      bool sel = slot < hi;
      if (sel && !all_slots && slot >= nc) {
        const size_t m = size_t(page) * kPage + lane;
        sel = slot_alpha[m] == 0 || (t - slot_pos[m]) < window;
      }
      const uint64_t mask = __ballot(sel);
      s_dst[lane] = sel ? cnt + lanes_below(mask) : -1;
      cnt += __popcll(mask);
    }
    __syncthreads();
    if (tid < kPage) {
      const int dst = s_dst[tid];
      if (dst >= 0 && dst < max_out) {
        const size_t o = size_t(u) * max_out + dst;
        if (pos_out) pos_out[o] = slot_pos[size_t(page) * kPage + tid];
        if (alpha_out) alpha_out[o] = slot_alpha[size_t(page) * kPage + tid];
      }
    }
    for (int x = tid; x < kPage * D; x += 256) {
      const int j = x / D, d = x % D;
      const int dst = s_dst[j];
      if (dst >= 0 && dst < max_out) {
        const size_t o = (size_t(u) * max_out + dst) * D + d;
        if (k_out) k_out[o] = k_pages[size_t(page) * kPage * D + key_index(j, d, D)];
        if (v_out) v_out[o] = v_pages[size_t(page) * kPage * D + value_index(j, d, D)];
      }
    }
    __syncthreads();  // s_dst is rewritten for the next page
  }
  if (tid == 0) count_out[u] = cnt;
}

hipError_t launch_export(const dms_shape &s, const dms_cache &c, int all_slots, int max_out,
                         int32_t *count_out, int32_t *pos_out, uint8_t *alpha_out, void *k_out,
                         void *v_out, hipStream_t st) {
  auto go = [&](auto kern, auto *kp, auto *vp) {
    using E = std::remove_const_t<std::remove_pointer_t<decltype(kp)>>;
    hipLaunchKernelGGL(kern, dim3(units_of(s)), dim3(256), 0, st, s.kv_heads, s.window,
                       s.max_pages_per_unit, all_slots, max_out, c.page_table, c.seq_len,
                       c.n_slots, c.n_clean, kp, vp, c.slot_pos, c.slot_alpha, count_out, pos_out,
                       alpha_out, static_cast<E *>(k_out), static_cast<E *>(v_out));
  };
  const bool bf = s.kv_dtype == DMS_KV_BF16;
  const uint16_t *k16 = static_cast<const uint16_t *>(c.k_pages), *v16 = static_cast<const uint16_t *>(c.v_pages);
  const uint32_t *k32 = static_cast<const uint32_t *>(c.k_pages), *v32 = static_cast<const uint32_t *>(c.v_pages);
  if (bf && s.head_dim == 64) go(k_export<uint16_t, 64>, k16, v16);
  else if (bf) go(k_export<uint16_t, 128>, k16, v16);
  else if (s.head_dim == 64) go(k_export<uint32_t, 64>, k32, v32);
  else go(k_export<uint32_t, 128>, k32, v32);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// prefix sharing, part 1 (one workgroup): for receiver unit du = d * hkv + h
// and source unit su = src * hkv + h, the source's full clean pages
// [0, P), P = n_clean / 64, are entered in the receiver's row and their
// page_ref counts raised; the T = ceil(n_slots / 64) - P remaining pages are
// taken from the free stack in unit order (prefix sums, as in append).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAllocThreads) void k_share_alloc(
    int hkv, int maxp, int src, int dst_first, int n_dst, int units, int32_t *page_table,
    int32_t *n_slots, int32_t *n_clean, int32_t *append_base, int32_t *seq_len,
    const int32_t *free_list, int32_t *free_top, int32_t *page_ref, uint32_t *status,
    int32_t *plan) {
  __shared__ int s_tmp[kAllocThreads / kWave];
  __shared__ int s_taken;
  __shared__ uint32_t s_flags;
  if (threadIdx.x == 0) {
    s_taken = 0;
    s_flags = 0u;
  }
  const int F = *free_top;
  const int n = n_dst * hkv;
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < n; base += kAllocThreads) {
    const int x = base + threadIdx.x;
    int need = 0, du = 0, su = 0, P = 0;
    bool empty = true;
    if (x < n) {
      const int d = dst_first + x / hkv, h = x % hkv;
      du = d * hkv + h;
      su = src * hkv + h;
      empty = n_slots[du] == 0;
      P = n_clean[su] / kPage;
      need = empty ? (n_slots[su] + kPage - 1) / kPage - P : 0;
    }
    int total = 0;
    const int incl = block_inclusive_scan<kAllocThreads>(need, s_tmp, total) + carry;
    if (x < n) {
      const bool ok = empty && (need == 0 || incl <= F);
      if (ok) {
        const int32_t *srow = page_table + size_t(su) * maxp;
        int32_t *drow = page_table + size_t(du) * maxp;
        for (int i = 0; i < P; ++i) {
          drow[i] = srow[i];
          atomicAdd(&page_ref[srow[i]], 1);
        }
        for (int i = 0; i < need; ++i) drow[P + i] = free_list[F - incl + i];
        n_slots[du] = n_slots[su];
        n_clean[du] = n_clean[su];
        append_base[du] = -1;
        plan[plan_layout(units).compact_pos + du] = plan[plan_layout(units).compact_pos + su];
        if (x % hkv == 0) seq_len[dst_first + x / hkv] = seq_len[src];
        if (need > 0) atomicMax(&s_taken, incl);
      } else {
        atomicOr(&s_flags, empty ? DMS_STATUS_POOL_EXHAUSTED : DMS_STATUS_NOT_EMPTY);
      }
    }
    carry += total;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    *free_top = F - s_taken;
    if (s_flags) atomicOr(status, s_flags);
  }
  __syncthreads();
  // every unit's n_slots is read back by the planner: make this workgroup's
  // writes visible to all of its threads first
  __threadfence_block();
  build_plan(units, [=](int u) { return n_slots[u]; }, plan);
}

// prefix sharing, part 2: copy the source's page P + i into the receiver's
// page P + i (keys, values, positions, decisions), one workgroup per
// (page, receiver unit); pages the receiver did not get are skipped.
template <typename E, int D>
__global__ __launch_bounds__(256) void k_share_copy(int hkv, int maxp, int src, int dst_first,
                                                    const int32_t *__restrict__ page_table,
                                                    const int32_t *__restrict__ n_slots,
                                                    const int32_t *__restrict__ n_clean,
                                                    E *__restrict__ k_pages, E *__restrict__ v_pages,
                                                    int32_t *__restrict__ slot_pos,
                                                    uint8_t *__restrict__ slot_alpha) {
  const int i = blockIdx.x, x = blockIdx.y;
  const int du = (dst_first + x / hkv) * hkv + x % hkv;
  const int su = src * hkv + x % hkv;
  const int P = n_clean[su] / kPage;
  const int T = (n_slots[su] + kPage - 1) / kPage - P;
  if (i >= T || P + i >= maxp) return;
  const int dp = page_table[size_t(du) * maxp + P + i];
  const int sp = page_table[size_t(su) * maxp + P + i];
  if (dp < 0 || dp == sp) return;
  constexpr int U4 = kPage * D * int(sizeof(E)) / 16;  // uint4 per page of keys (or values)
  const uint4 *ks = reinterpret_cast<const uint4 *>(k_pages + size_t(sp) * kPage * D);
  const uint4 *vs = reinterpret_cast<const uint4 *>(v_pages + size_t(sp) * kPage * D);
  uint4 *kd = reinterpret_cast<uint4 *>(k_pages + size_t(dp) * kPage * D);
  uint4 *vd = reinterpret_cast<uint4 *>(v_pages + size_t(dp) * kPage * D);
  for (int e = threadIdx.x; e < U4; e += blockDim.x) {
    kd[e] = ks[e];
    vd[e] = vs[e];
  }
  if (threadIdx.x < kPage) {
    slot_pos[size_t(dp) * kPage + threadIdx.x] = slot_pos[size_t(sp) * kPage + threadIdx.x];
    slot_alpha[size_t(dp) * kPage + threadIdx.x] = slot_alpha[size_t(sp) * kPage + threadIdx.x];
  }
}

hipError_t launch_share(const dms_shape &s, const dms_cache &c, int src, int dst_first, int n_dst,
                        hipStream_t st) {
  hipLaunchKernelGGL(k_share_alloc, dim3(1), dim3(kAllocThreads), 0, st, s.kv_heads,
                     s.max_pages_per_unit, src, dst_first, n_dst, units_of(s), c.page_table,
                     c.n_slots, c.n_clean, c.append_base, c.seq_len, c.free_list, c.free_top,
                     c.page_ref, c.status, c.plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(s.max_pages_per_unit, n_dst * s.kv_heads);
  auto copy = [&](auto kern, auto *kp, auto *vp) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, s.kv_heads, s.max_pages_per_unit, src,
                       dst_first, c.page_table, c.n_slots, c.n_clean, kp, vp, c.slot_pos,
                       c.slot_alpha);
  };
  const bool bf = s.kv_dtype == DMS_KV_BF16;
  if (s.head_dim == 128) {
    if (bf) copy(k_share_copy<uint16_t, 128>, static_cast<uint16_t *>(c.k_pages), static_cast<uint16_t *>(c.v_pages));
    else copy(k_share_copy<uint32_t, 128>, static_cast<uint32_t *>(c.k_pages), static_cast<uint32_t *>(c.v_pages));
  } else {
    if (bf) copy(k_share_copy<uint16_t, 64>, static_cast<uint16_t *>(c.k_pages), static_cast<uint16_t *>(c.v_pages));
    else copy(k_share_copy<uint32_t, 64>, static_cast<uint32_t *>(c.k_pages), static_cast<uint32_t *>(c.v_pages));
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// release (one workgroup): every page of the released units goes back on the
// free stack unless another holder remains.  With r = page_ref before the
// decrement, the holder that sees r <= 0 is the last one and frees the page.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAllocThreads) void k_release(int hkv, int maxp, int first, int nseq,
                                                         int units, int32_t *page_table,
                                                         int32_t *n_slots, int32_t *n_clean,
                                                         int32_t *append_base, int32_t *seq_len,
                                                         int32_t *free_list, int32_t *free_top,
                                                         int32_t *page_ref, int32_t *plan) {
  const int n = nseq * hkv;
  for (int x = threadIdx.x; x < n; x += kAllocThreads) {
    const int u = first * hkv + x;
    int32_t *row = page_table + size_t(u) * maxp;
    const int np = (n_slots[u] + kPage - 1) / kPage;
    for (int i = 0; i < np; ++i) {
      const int pg = row[i];
      if (atomicAdd(&page_ref[pg], -1) <= 0) {
        page_ref[pg] = 0;
        free_list[atomicAdd(free_top, 1)] = pg;
      }
    }
    for (int i = 0; i < maxp; ++i) row[i] = -1;
    n_slots[u] = 0;
    n_clean[u] = 0;
    append_base[u] = -1;
    plan[plan_layout(units).compact_pos + u] = -1;
  }
  for (int b = threadIdx.x; b < nseq; b += kAllocThreads) seq_len[first + b] = 0;
  __syncthreads();
  build_plan(units, [=](int u) { return n_slots[u]; }, plan);
}

hipError_t launch_release(const dms_shape &s, const dms_cache &c, int first, int n, hipStream_t st) {
  hipLaunchKernelGGL(k_release, dim3(1), dim3(kAllocThreads), 0, st, s.kv_heads,
                     s.max_pages_per_unit, first, n, units_of(s), c.page_table, c.n_slots,
                     c.n_clean, c.append_base, c.seq_len, c.free_list, c.free_top, c.page_ref,
                     c.plan);
  return hipGetLastError();
}

}  // namespace dms
