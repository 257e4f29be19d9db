/*
 * dms.h - C ABI of libdms.so: Dynamic Memory Sparsification (DMS) attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (atlas.scime.ai summary of "Inference-Time Hyper-Scaling with KV
 * Cache Compression", arXiv 2506.05345, section "Approach"): every KV head
 * makes a binary keep/evict decision for each token; a token marked for
 * eviction is removed only after a delay window (16 tokens: same page, table
 * "Measured effects reported in the paper"); attention reads only what is
 * retained.  Decode cost is the KV bytes read per step (zhaoyang97 Paper-Notes
 * page, motivation section: decode is bandwidth bound and reads the whole
 * cache every step).
 *
 * Conventions shared by every call
 *   - All pointers are device pointers unless stated otherwise.  The library
 *     allocates no memory and keeps no pointer after a call returns: every
 *     buffer belongs to the caller.  Its one piece of global state is the
 *     static device scratch array of dms_decode_attn_noalloc (one per GPU,
 *     resident until the process ends); no other call touches it.
 *   - Calls enqueue kernels on `stream` (a hipStream_t; NULL = the default
 *     stream) and return without synchronising.  Calls on one cache must be
 *     ordered on one stream; calls on disjoint state may run on any streams.
 *   - Return value: DMS_OK (0) or a negative DMS_E* code, decided on the host
 *     before anything is enqueued (DMS_EHIP: a launch failed).
 *   - Errors found on the device (pool exhausted, page-table row full) do not
 *     stop the call: the affected unit's write is skipped and a bit is OR-ed
 *     into the sticky word cache->status, which the caller reads after a
 *     synchronisation and clears with dms_reset or by writing 0.
 *
 * Notation: B sequences, Hkv KV heads, G query heads per KV head (query head
 * hq reads KV head hq / G), D head dimension, P = 64 slots per page, w the
 * delay window.  A "unit" is one (sequence b, KV head h) pair, u = b*Hkv + h.
 */
#ifndef DMS_H
#define DMS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DMS_ABI_VERSION 5
#define DMS_PAGE_SIZE 64

/* host-side return codes */
#define DMS_OK 0
#define DMS_EINVAL (-1)       /* null pointer, negative size, window < 1, ... */
#define DMS_EUNSUPPORTED (-2) /* head_dim, group, dtype or page size not built */
#define DMS_EWORKSPACE (-3)   /* decode workspace smaller than dms_decode_workspace_bytes */
#define DMS_EHIP (-4)         /* a HIP launch returned an error */
#define DMS_ESCRATCH (-5)     /* the shape needs more than DMS_NOALLOC_SCRATCH_BYTES of scratch */

/* size of the static per-GPU scratch array of dms_decode_attn_noalloc */
#define DMS_NOALLOC_SCRATCH_BYTES (16u << 20)

/* device-side sticky status bits (cache->status) */
#define DMS_STATUS_POOL_EXHAUSTED 1u /* free pages ran out; that unit's tokens were dropped */
#define DMS_STATUS_ROW_OVERFLOW 2u   /* a unit needed more than max_pages_per_unit pages */
#define DMS_STATUS_NOT_EMPTY 4u      /* dms_share_prefix target unit held tokens; left as it was */
#define DMS_STATUS_CHUNK_INVALID 8u  /* dms_decode_attn_multi: a sequence held fewer tokens than the
                                        chunk, or was compacted after the chunk's first position;
                                        that sequence's outputs are unspecified */

/* key/value element types */
#define DMS_KV_F32 0
#define DMS_KV_BF16 1

typedef struct dms_shape {
  int32_t batch;              /* B >= 1 */
  int32_t kv_heads;           /* Hkv >= 1 */
  int32_t group;              /* G in [1, 16] */
  int32_t head_dim;           /* D in {64, 128} */
  int32_t page_size;          /* must be DMS_PAGE_SIZE */
  int32_t window;             /* w >= 1 (16 on the pages; 1 = evict at once) */
  int32_t max_pages_per_unit; /* columns of the page table */
  int32_t num_pages;          /* pages in the shared pool */
  int32_t kv_dtype;           /* DMS_KV_F32 or DMS_KV_BF16 */
} dms_shape;

/*
 * The paged cache.  Every field is a caller-owned device buffer.
 *   k_pages     [num_pages][P*D]  keys, in the order of the decode kernel's
 *   v_pages     [num_pages][P*D]  matrix-core operand fragments (below)
 *   page_table  [units][max_pages_per_unit] int32, -1 = no page
 *   slot_pos    [num_pages][P] int32  sequence position held by each slot
 *   slot_alpha  [num_pages][P] uint8  1 = marked for eviction
 *   n_slots     [units] int32  slots in use; slot s lives in page s / P
 *   n_clean     [units] int32  slots [0, n_clean) hold unmarked tokens only
 *   append_base [units] int32  first slot of the last append, -1 if refused
 *   seq_len     [B] int32      tokens appended so far (next position)
 *   free_list   [num_pages] int32, free_top [1] int32: stack of free pages
 *   status      [1] uint32     sticky DMS_STATUS_* bits
 *   plan        [dms_plan_words(shape)] int32, opaque: the decode split plan,
 *               rebuilt on the device by every call that changes n_slots,
 *               and per unit the position of its last compaction
 *   page_ref    [num_pages] int32: holders of a page beyond the first (pages
 *               shared by dms_share_prefix); may be NULL when no prefix is
 *               ever shared
 * A unit's slots hold its retained tokens in ascending position order,
 * followed by tokens appended since its last compaction; a slot is dead when
 * its token is marked and w or more positions old, and dead slots are skipped
 * by attention until dms_compact removes them.
 *
 * Element order inside a page (E = kv_dtype element; slot j in 0..63, dim d
 * in 0..D-1).  A page is two groups of 32 slots, g = j / 32, js = j % 32, each
 * holding 32*D keys then (in v_pages) 32*D values:
 *   key (j, d)   at g*32*D + (((t*(D/32) + d/32)*4 + (d/8)%4)*16 + r)*8 + d%8,
 *                t = (js%8)/4, r = 4*(js/8) + js%4
 *   value (j, d) at g*32*D + (((d/16)*4 + js/8)*16 + d%16)*8 + js%8
 * so that each 16-slot x 32-dim key fragment and each 16-dim x 32-slot value
 * fragment of a bf16 matrix product is one contiguous 1 KB block, and eight
 * consecutive dims of a key, or eight consecutive slots of a value dim, are
 * contiguous.  dms_export_retained reads a cache back in plain row order.
 */
typedef struct dms_cache {
  void *k_pages;
  void *v_pages;
  int32_t *page_table;
  int32_t *slot_pos;
  uint8_t *slot_alpha;
  int32_t *n_slots;
  int32_t *n_clean;
  int32_t *append_base;
  int32_t *seq_len;
  int32_t *free_list;
  int32_t *free_top;
  uint32_t *status;
  int32_t *plan;
  int32_t *page_ref;
} dms_cache;

/* ABI version (DMS_ABI_VERSION).  Never fails. */
int dms_version(void);

/* Static text for a DMS_* return code.  Never fails. */
const char *dms_strerror(int code);

/* Host-only check of a shape: DMS_OK, DMS_EINVAL or DMS_EUNSUPPORTED. */
int dms_check_shape(const dms_shape *shape);

/* int32 words of cache->plan for this shape; 0 if the shape is invalid. */
size_t dms_plan_words(const dms_shape *shape);

/*
 * Read a cache back: for every unit, its retained set R(t) at t = seq_len[b] - 1
 * (the slots alive at t: below n_clean, unmarked, or marked and t - pos < w;
 * atlas.scime.ai summary, "Approach": eviction carried out after the delay
 * window), or with all_slots = 1 every slot in use, dead ones included.  In
 * slot order, which is ascending position order.
 *   all_slots     0 or 1
 *   max_per_unit  >= 0: rows per unit in the outputs below
 *   count_out     [units] int32: the number of entries (all of them, also
 *                 beyond max_per_unit); required
 *   pos_out       [units][max_per_unit] int32 positions, or NULL
 *   alpha_out     [units][max_per_unit] uint8 decisions (1 = marked), or NULL
 *   k_out, v_out  [units][max_per_unit][D] in kv_dtype, plain rows, or NULL
 * Only the first min(count, max_per_unit) rows of a unit are written; the
 * rest of the outputs is left as it was.  Must not run between
 * dms_append_reserve and dms_decode_attn_fill.  Host errors: DMS_EINVAL for
 * a null count_out, a negative max_per_unit or all_slots not 0 or 1.
 */
int dms_export_retained(const dms_shape *shape, const dms_cache *cache, int32_t all_slots,
                        int32_t max_per_unit, int32_t *count_out, int32_t *pos_out,
                        uint8_t *alpha_out, void *k_out, void *v_out, hipStream_t stream);

/*
 * Empty every unit: page_table = -1, free_list = 0..num_pages-1,
 * free_top = num_pages, n_slots = n_clean = seq_len = 0, append_base = -1,
 * status = 0, page_ref = 0 (if given), plan rebuilt.  Must run once on fresh buffers before any
 * other call.
 */
int dms_reset(const dms_shape *shape, const dms_cache *cache, hipStream_t stream);

/*
 * Decide and append n_new tokens to every unit.
 * Decision (atlas.scime.ai summary, "Approach"; zhaoyang97 notes, key design
 * item 2): the inference form of the Gumbel-sigmoid gate, alpha = logit > 0
 * compared in float32 (NaN and +-0 keep).  Append (notes, motivation: the
 * cache grows by one entry per token and head): token i of sequence b gets
 * position seq_len[b] + i and the next free slot of its unit.
 *   k_new, v_new  [B][n_new][Hkv][D] in kv_dtype (no conversion is done)
 *   logit         [B][n_new][Hkv] float32
 *   n_new         >= 0 (0 is a no-op)
 * Pages come from the free stack; units are served in index order and a
 * unit whose pages do not fit is refused whole: its tokens are dropped,
 * append_base[u] = -1 and DMS_STATUS_POOL_EXHAUSTED (or _ROW_OVERFLOW) is
 * set.  seq_len advances for every sequence either way.
 */
int dms_append(const dms_shape *shape, const dms_cache *cache, const void *k_new,
               const void *v_new, const float *logit, int32_t n_new, hipStream_t stream);

/*
 * Reclaim evicted slots (atlas.scime.ai summary, "Approach": the eviction is
 * carried out once the delay window has passed).  For each unit, with
 * t = seq_len[b] - 1, the slots in [n_clean, n_slots) whose token is marked
 * and t - pos >= w are removed; the survivors move down in order (stable
 * stream compaction), whole pages left empty go back on the free stack and
 * n_slots / n_clean are updated and the decode plan is rebuilt.  Attention
 * results do not depend on when or whether this runs; memory use and bytes
 * read do.  The position t is recorded per unit (see dms_decode_attn_multi).
 */
int dms_compact(const dms_shape *shape, const dms_cache *cache, hipStream_t stream);

/*
 * Bytes of decode workspace for this shape.  0 if the shape is invalid.
 * The workspace needs no initialisation and holds nothing between calls.
 */
size_t dms_decode_workspace_bytes(const dms_shape *shape);

/*
 * Decode attention over the retained entries (atlas.scime.ai summary,
 * "Approach"; zhaoyang97 notes, motivation: one query per step reads the
 * cache).  For query head hq = h*G + g of sequence b, with t = seq_len[b]-1:
 *   out = sum_j softmax_j(sm_scale * <q, k_j>) v_j over the slots j of unit
 *   (b, h) that are alive at t (unmarked, or marked and t - pos < w).
 *   q    [B][Hq][D] in kv_dtype, Hq = Hkv*G
 *   out  [B][Hq][D] float32
 * The caller appends token t before this call, so each query sees its own
 * token.  A unit with no slots gives zeros.  Both products run on the matrix
 * cores: bf16 caches in bf16 with float32 accumulation, float32 caches in
 * float32 throughout.  The work of each unit is split
 * into chunks of whole pages following cache->plan (sized on the device from
 * the live lengths: one chunk per unit when the units are many and of even
 * length), and the chunk partials of a split unit are merged with the
 * log-sum-exp rule: with fewer than 512 units by a second kernel launch on
 * the stream, else by the unit's last chunk inside the decode launch.
 * The call uses per-unit counters inside cache->plan and leaves them zero;
 * two decode calls on one cache must not run concurrently.
 */
int dms_decode_attn(const dms_shape *shape, const dms_cache *cache, const void *q, float *out,
                    float sm_scale, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dms_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc.  Same
 * result and same kernels as dms_decode_attn (identical outputs), but the
 * split-K partials live in the library's own static device array of
 * DMS_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held from the first use until
 * the process ends, instead of a caller's workspace.  The call allocates
 * nothing.  Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents (nothing in it needs to start at zero): two calls that
 * overlap in time on one GPU (on different streams) race and give undefined
 * outputs.  Arguments and host errors as for dms_decode_attn without the
 * workspace, plus DMS_ESCRATCH when dms_decode_workspace_bytes(shape) exceeds
 * DMS_NOALLOC_SCRATCH_BYTES (with D = 128: more than 2016 units at G = 16,
 * more than 8066 at G = 4),
 * and DMS_EHIP if the array's device address cannot be obtained.
 */
int dms_decode_attn_noalloc(const dms_shape *shape, const dms_cache *cache, const void *q,
                            float *out, float sm_scale, hipStream_t stream);

/*
 * One decode step in two calls, for callers that attend right after
 * appending one token per sequence: together equivalent to
 * dms_append(n_new = 1) followed by dms_decode_attn, with one launch less.
 * The cache state afterwards is the same, byte for byte (page ids aside,
 * which depend on the free stack's order).  The outputs agree to rounding:
 * on bf16 caches the decode launch takes the new token as one more softmax
 * term, its weight kept in float32 where the cached tokens' weights are
 * rounded to bf16 for the matrix cores; other caches give identical outputs.
 *
 * dms_append_reserve: the slot, page and count part of dms_append(n_new = 1)
 * (positions seq_len[b], pages from the free stack in unit order, refusal
 * and status flags as there; decode plan rebuilt).  The reserved slots hold
 * no token yet: the next call on the cache (same stream) must be
 * dms_decode_attn_fill, and no other call may come in between.
 *
 * dms_decode_attn_fill: attends as dms_decode_attn, the new token included
 * (atlas.scime.ai summary, "Approach": a query always sees its own token),
 * and writes the token reserved in every unit that was not refused into its
 * slot, with the decision alpha = logit > 0 as dms_append.
 *   k_new, v_new  [B][1][Hkv][D] in kv_dtype;  logit [B][1][Hkv] float32
 *   q, out, sm_scale, workspace as for dms_decode_attn
 * Host errors as for dms_decode_attn, plus DMS_EINVAL for a null k_new,
 * v_new or logit, or a k_new or v_new that is not 16-byte aligned.
 */
int dms_append_reserve(const dms_shape *shape, const dms_cache *cache, hipStream_t stream);
int dms_decode_attn_fill(const dms_shape *shape, const dms_cache *cache, const void *k_new,
                         const void *v_new, const float *logit, const void *q, float *out,
                         float sm_scale, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Share a sequence's prompt with other sequences (several reasoning threads
 * from one prompt; zhaoyang97 Paper-Notes, framework section: many parallel
 * generations, and the same cache budget spent on more of them).  For every
 * KV head, sequences dst_first .. dst_first + n_dst - 1 receive the state of
 * sequence src_seq: its full pages below n_clean (tokens that stay retained
 * for good, which no later call writes) are shared, not copied, and their
 * page_ref counts go up by one per receiver; the rest of its slots are
 * copied into pages taken from the free stack.  n_slots, n_clean and seq_len
 * are copied; the receivers then append and compact independently.
 * Receivers must be empty (n_slots == 0); a non-empty one is left unchanged
 * with DMS_STATUS_NOT_EMPTY set, one that cannot get its pages with
 * DMS_STATUS_POOL_EXHAUSTED (deterministic order as for dms_append).
 * cache->page_ref is required.  Host errors: DMS_EINVAL for a null
 * page_ref, a source inside the receiver range or indices out of range.
 */
int dms_share_prefix(const dms_shape *shape, const dms_cache *cache, int32_t src_seq,
                     int32_t dst_first, int32_t n_dst, hipStream_t stream);

/*
 * Empty sequences first .. first + n - 1: each page of their units goes back
 * on the free stack unless another holder remains (page_ref > 0, then
 * decremented).  n_slots = n_clean = seq_len = 0, append_base = -1,
 * page_table rows = -1, plan rebuilt.  cache->page_ref is required.
 */
int dms_release(const dms_shape *shape, const dms_cache *cache, int32_t first, int32_t n,
                hipStream_t stream);

/* Bytes of workspace for dms_decode_attn_multi (partials for 16 columns). */
size_t dms_decode_multi_workspace_bytes(const dms_shape *shape);

/*
 * Bytes of workspace with which dms_decode_attn_multi splits a chunk of
 * n_query >= 32 queries on a bf16 cache over the chip: when the tiled
 * kernel's workgroups (one per 32 queries and sequence, KV head and group
 * of 4 query heads) are fewer than one resident round (768), each takes a
 * part of its keys and a merge launch combines the parts, which needs
 * splits x B x n_query x Hq x (D + 2) floats.  At least
 * dms_decode_multi_workspace_bytes(shape); equal to it where no split
 * applies.  0 if the arguments are invalid.
 */
size_t dms_decode_multi_split_workspace_bytes(const dms_shape *shape, int32_t n_query);

/*
 * Attention of the last n_query tokens of every sequence (a chunk appended
 * with dms_append(n_new = n_query)) over the cache: query c of sequence b
 * sits at position t_c = seq_len[b] - n_query + c and attends over the slots
 * j with pos_j <= t_c and (alpha_j == 0 or t_c - pos_j < w), the same rule as
 * dms_decode_attn at each t_c (atlas.scime.ai summary, "Approach": eviction
 * carried out after the delay window; the earlier queries of the chunk do
 * not see its later tokens).  Call it after appending the chunk and before
 * any dms_compact: a compaction at the chunk's last position would drop
 * slots that earlier queries of the chunk still see.  The kernels check this
 * per sequence: one that holds fewer than n_query tokens, or whose units were
 * compacted after the chunk's first position, gets unspecified outputs and
 * sets DMS_STATUS_CHUNK_INVALID in cache->status.
 *   q    [B][n_query][Hq][D] in kv_dtype,   out [B][n_query][Hq][D] float32
 * n_query >= 1.  bf16 caches: chunks of 32 queries or more run a tiled kernel
 * that reads the cache once per 32 queries, each group of 32 up to its last
 * query's slot (split over the chip, then merged, when the workspace is at
 * least dms_decode_multi_split_workspace_bytes(shape, n_query)); shorter
 * ones run the split-K decode kernel in launches of 16 / G queries.  float32
 * caches: chunks of 32 queries or more run a tiled kernel on the float32
 * matrix instruction (one pass over the cache per 32 queries), shorter ones
 * the float32 split-K decode kernel in launches of 16 / G queries.  Workspace:
 * at least dms_decode_multi_workspace_bytes.  Errors as for dms_decode_attn.
 */
int dms_decode_attn_multi(const dms_shape *shape, const dms_cache *cache, const void *q,
                          int32_t n_query, float *out, float sm_scale, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of prefill workspace for `seq_len` tokens of this shape.  bf16:
 * keys and values re-laid out per 32-key tile for the matrix cores, one float
 * per key (its decision as an additive mask), and the re-laid keys and values
 * again with every key masked out under the hard rule zeroed (read where all
 * of a tile's keys are at least w behind every query).  float32: 256 (its
 * kernel uses none).  0 if the arguments are invalid.
 */
size_t dms_prefill_workspace_bytes(const dms_shape *shape, int32_t seq_len);

/*
 * Masked prefill attention over a whole prompt, no cache (the same rule
 * applied to every query row; atlas.scime.ai summary, "Approach" and
 * "Measured effects" for the 16-token window).  Row i of query head hq
 * attends to key j of KV head hq/G iff
 *   j <= i  and  not (alpha_j and i >= j + w),   alpha_j = logit_j > 0.
 *   q      [B][S][Hq][D]  kv_dtype
 *   k, v   [B][S][Hkv][D] kv_dtype
 *   logit  [B][S][Hkv]    float32
 *   out    [B][S][Hq][D]  float32
 *   workspace  at least dms_prefill_workspace_bytes(shape, S) bytes, 16-byte
 *              aligned, no initialisation needed, nothing kept after the call
 * Only batch, kv_heads, group, head_dim (64 or 128), window and kv_dtype of
 * `shape` are read.  bf16 inputs run on the matrix cores (group <= 16);
 * float32 inputs run a kernel of their own on the float32 matrix
 * instruction (float32 operands, any group), the same kernel for all three
 * prefill calls, skipping tiles no query of a block sees.  The cache is
 * filled separately with dms_append.
 */
int dms_prefill_attn(const dms_shape *shape, const void *q, const void *k, const void *v,
                     const float *logit, int32_t seq_len, float sm_scale, float *out,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Prefill attention with the relaxed (training-form) decision: the binary
 * decision of atlas.scime.ai's summary ("Approach": learned per head, relaxed
 * with a Gumbel-sigmoid while retrofitting) replaced by
 *   a~_j = sigmoid((logit_j + noise_j) / temperature),
 * key j keeping the weight factor (1 - a~_j) for queries at least w positions
 * after it and its full weight inside the window, i.e. scores
 *   sm_scale <q_i, k_j> + (i - j >= w ? log(1 - a~_j) : 0),   j <= i.
 * The pages give neither the noise law nor the temperature; both are inputs.
 * noise: [B][S][Hkv] float32 (e.g. logistic draws for a Gumbel-sigmoid), or
 * NULL for none.  temperature > 0 and finite, else DMS_EINVAL.  logit and
 * noise must be finite.  Other arguments, the workspace
 * (dms_prefill_workspace_bytes) and errors as for dms_prefill_attn.  As the
 * temperature goes to 0 without noise the result tends to dms_prefill_attn's.
 */
int dms_prefill_attn_relaxed(const dms_shape *shape, const void *q, const void *k, const void *v,
                             const float *logit, const float *noise, float temperature,
                             int32_t seq_len, float sm_scale, float *out, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of workspace for dms_prefill_attn_gathered: the dense prefill
 * workspace, the same layout again for the gathered kept keys, and per
 * (sequence, KV head) the kept positions and per-tile counts (float32: 256,
 * unused).  0 if the arguments are invalid.
 */
size_t dms_prefill_gathered_workspace_bytes(const dms_shape *shape, int32_t seq_len);

/*
 * Masked prefill attention, same result as dms_prefill_attn, computed over
 * the keys each query can see rather than over the whole causal triangle.
 * With the rule of atlas.scime.ai's summary ("Approach"; 16-token window in
 * "Measured effects"), the keys visible to query i are exactly
 *   the kept keys (alpha_j = 0) with j <= i - w,   and
 *   every key with i - w < j <= i,
 * two disjoint sets.  The kept keys of each (sequence, KV head) are gathered
 * once in position order; each block of queries then attends to a prefix of
 * the gathered keys plus the dense band of its last w positions, in one
 * softmax.  At an eviction rate p the work is about (1 - p) of the dense
 * kernel's plus the band.  Arguments, layouts and errors as for
 * dms_prefill_attn; the workspace must hold
 * dms_prefill_gathered_workspace_bytes(shape, S) bytes.
 */
int dms_prefill_attn_gathered(const dms_shape *shape, const void *q, const void *k, const void *v,
                              const float *logit, int32_t seq_len, float sm_scale, float *out,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DMS_H */
