// libdms C ABI: host-side argument checks and dispatch.  Nothing here
// allocates, synchronises or keeps state between calls.
#include <stdint.h>

#include "dms_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_cache(const dms_shape *s, const dms_cache *c) {
  if (!c) return DMS_EINVAL;
  if (!c->k_pages || !c->v_pages || !c->page_table || !c->slot_pos || !c->slot_alpha ||
      !c->n_slots || !c->n_clean || !c->append_base || !c->seq_len || !c->free_list ||
      !c->free_top || !c->status || !c->plan)
    return DMS_EINVAL;
  if (!aligned16(c->k_pages) || !aligned16(c->v_pages) || !aligned16(c->slot_pos) ||
      !aligned16(c->slot_alpha))
    return DMS_EINVAL;
  (void)s;
  return DMS_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? DMS_OK : DMS_EHIP; }

}  // namespace

extern "C" {

int dms_version(void) { return DMS_ABI_VERSION; }

const char *dms_strerror(int code) {
  switch (code) {
    case DMS_OK: return "ok";
    case DMS_EINVAL: return "invalid argument";
    case DMS_EUNSUPPORTED: return "unsupported shape or dtype";
    case DMS_EWORKSPACE: return "decode workspace too small";
    case DMS_EHIP: return "HIP launch failed";
    case DMS_ESCRATCH: return "shape needs more decode scratch than the library's static buffer holds";
    default: return "unknown error code";
  }
}

int dms_check_shape(const dms_shape *s) {
  if (!s) return DMS_EINVAL;
  if (s->batch < 1 || s->kv_heads < 1 || s->group < 1 || s->window < 1) return DMS_EINVAL;
  if (s->max_pages_per_unit < 1 || s->num_pages < 1) return DMS_EINVAL;
  if (int64_t(s->batch) * s->kv_heads > (int64_t(1) << 24)) return DMS_EINVAL;
  if (int64_t(s->max_pages_per_unit) * DMS_PAGE_SIZE > (int64_t(1) << 30)) return DMS_EINVAL;
  if (s->page_size != DMS_PAGE_SIZE) return DMS_EUNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return DMS_EUNSUPPORTED;
  if (s->group > 16) return DMS_EUNSUPPORTED;
  if (s->kv_dtype != DMS_KV_F32 && s->kv_dtype != DMS_KV_BF16) return DMS_EUNSUPPORTED;
  return DMS_OK;
}

int dms_reset(const dms_shape *shape, const dms_cache *cache, hipStream_t stream) {
  int rc = dms_check_shape(shape);
  if (rc) return rc;
  if ((rc = check_cache(shape, cache))) return rc;
  return from_hip(dms::launch_reset(*shape, *cache, stream));
}

int dms_append(const dms_shape *shape, const dms_cache *cache, const void *k_new,
               const void *v_new, const float *logit, int32_t n_new, hipStream_t stream) {
  int rc = dms_check_shape(shape);
  if (rc) return rc;
  if ((rc = check_cache(shape, cache))) return rc;
  if (n_new < 0) return DMS_EINVAL;
  if (n_new == 0) return DMS_OK;
  if (!k_new || !v_new || !logit) return DMS_EINVAL;
  if (!aligned16(k_new)) return DMS_EINVAL;
  if (int64_t(n_new) > int64_t(shape->max_pages_per_unit) * DMS_PAGE_SIZE) return DMS_EINVAL;
  if (int64_t(n_new) > int64_t(65535) * DMS_PAGE_SIZE) return DMS_EINVAL;  // grid.y limit
  return from_hip(dms::launch_append(*shape, *cache, k_new, v_new, logit, n_new, stream));
}

int dms_compact(const dms_shape *shape, const dms_cache *cache, hipStream_t stream) {
  int rc = dms_check_shape(shape);
  if (rc) return rc;
  if ((rc = check_cache(shape, cache))) return rc;
  return from_hip(dms::launch_compact(*shape, *cache, stream));
}

int dms_export_retained(const dms_shape *shape, const dms_cache *cache, int32_t all_slots,
                        int32_t max_per_unit, int32_t *count_out, int32_t *pos_out,
                        uint8_t *alpha_out, void *k_out, void *v_out, hipStream_t stream) {
  int rc = dms_check_shape(shape);
  if (rc) return rc;
  if ((rc = check_cache(shape, cache))) return rc;
  if (!count_out || max_per_unit < 0 || (all_slots != 0 && all_slots != 1)) return DMS_EINVAL;
  return from_hip(dms::launch_export(*shape, *cache, all_slots, max_per_unit, count_out, pos_out,
                                     alpha_out, k_out, v_out, stream));
}

size_t dms_plan_words(const dms_shape *shape) {
  if (dms_check_shape(shape) != DMS_OK) return 0;
  return dms::plan_layout(dms::units_of(*shape)).words;
}

size_t dms_decode_workspace_bytes(const dms_shape *shape) {
  if (dms_check_shape(shape) != DMS_OK) return 0;
  return dms::decode_workspace_layout(dms::units_of(*shape), shape->group, shape->head_dim).bytes;
}

int dms_decode_attn(const dms_shape *shape, const dms_cache *cache, const void *q, float *out,
                    float sm_scale, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = dms_check_shape(shape);
  if (rc) return rc;
  if ((rc = check_cache(shape, cache))) return rc;
  if (!q || !out || !workspace) return DMS_EINVAL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return DMS_EINVAL;
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return DMS_EINVAL;
  if (workspace_bytes < dms_decode_workspace_bytes(shape)) return DMS_EWORKSPACE;
  return from_hip(dms::launch_decode(*shape, *cache, q, out, sm_scale, workspace, stream));
}

int dms_decode_attn_noalloc(const dms_shape *shape, const dms_cache *cache, const void *q,
                            float *out, float sm_scale, hipStream_t stream) {
  int rc = dms_check_shape(shape);
  if (rc) return rc;
  if ((rc = check_cache(shape, cache))) return rc;
  if (!q || !out) return DMS_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return DMS_EINVAL;
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return DMS_EINVAL;
  if (dms_decode_workspace_bytes(shape) > DMS_NOALLOC_SCRATCH_BYTES) return DMS_ESCRATCH;
  void *ws = nullptr;
  if (dms::scratch_address(stream, &ws) != hipSuccess) return DMS_EHIP;
  return from_hip(dms::launch_decode(*shape, *cache, q, out, sm_scale, ws, stream));
}

int dms_append_reserve(const dms_shape *shape, const dms_cache *cache, hipStream_t stream) {
  int rc = dms_check_shape(shape);
  if (rc) return rc;
  if ((rc = check_cache(shape, cache))) return rc;
  return from_hip(dms::launch_append_alloc(*shape, *cache, 1, stream));
}

int dms_decode_attn_fill(const dms_shape *shape, const dms_cache *cache, const void *k_new,
                         const void *v_new, const float *logit, const void *q, float *out,
                         float sm_scale, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  int rc = dms_check_shape(shape);
  if (rc) return rc;
  if ((rc = check_cache(shape, cache))) return rc;
  if (!k_new || !v_new || !logit || !q || !out || !workspace) return DMS_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(out) ||
      !aligned16(workspace))
    return DMS_EINVAL;
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return DMS_EINVAL;
  if (workspace_bytes < dms_decode_workspace_bytes(shape)) return DMS_EWORKSPACE;
  const dms::DecodeFill fill{k_new, v_new, logit};
  return from_hip(dms::launch_decode(*shape, *cache, q, out, sm_scale, workspace, stream, &fill));
}

int dms_share_prefix(const dms_shape *shape, const dms_cache *cache, int32_t src_seq,
                     int32_t dst_first, int32_t n_dst, hipStream_t stream) {
  int rc = dms_check_shape(shape);
  if (rc) return rc;
  if ((rc = check_cache(shape, cache))) return rc;
  if (!cache->page_ref) return DMS_EINVAL;
  const int64_t B = shape->batch;
  if (src_seq < 0 || src_seq >= B || dst_first < 0 || n_dst < 1 || int64_t(dst_first) + n_dst > B)
    return DMS_EINVAL;
  if (src_seq >= dst_first && src_seq < dst_first + n_dst) return DMS_EINVAL;
  if (int64_t(n_dst) * shape->kv_heads > 65535) return DMS_EINVAL;  // copy grid y
  return from_hip(dms::launch_share(*shape, *cache, src_seq, dst_first, n_dst, stream));
}

int dms_release(const dms_shape *shape, const dms_cache *cache, int32_t first, int32_t n,
                hipStream_t stream) {
  int rc = dms_check_shape(shape);
  if (rc) return rc;
  if ((rc = check_cache(shape, cache))) return rc;
  if (!cache->page_ref) return DMS_EINVAL;
  if (first < 0 || n < 0 || int64_t(first) + n > shape->batch) return DMS_EINVAL;
  if (n == 0) return DMS_OK;
  return from_hip(dms::launch_release(*shape, *cache, first, n, stream));
}

size_t dms_decode_multi_workspace_bytes(const dms_shape *shape) {
  if (dms_check_shape(shape) != DMS_OK) return 0;
  return dms::decode_workspace_layout(dms::units_of(*shape), 16, shape->head_dim).bytes;
}

size_t dms_decode_multi_split_workspace_bytes(const dms_shape *shape, int32_t n_query) {
  const size_t base = dms_decode_multi_workspace_bytes(shape);
  if (base == 0 || n_query < 1) return 0;
  if (shape->kv_dtype != DMS_KV_BF16 || n_query < 32) return base;
  const size_t split = dms::chunk_split_bytes(*shape, n_query, dms::chunk_splits(*shape, n_query));
  return split > base ? split : base;
}

int dms_decode_attn_multi(const dms_shape *shape, const dms_cache *cache, const void *q,
                          int32_t n_query, float *out, float sm_scale, void *workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  int rc = dms_check_shape(shape);
  if (rc) return rc;
  if ((rc = check_cache(shape, cache))) return rc;
  if (n_query < 1) return DMS_EINVAL;
  if (!q || !out || !workspace) return DMS_EINVAL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return DMS_EINVAL;
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return DMS_EINVAL;
  if (workspace_bytes < dms_decode_multi_workspace_bytes(shape)) return DMS_EWORKSPACE;
  return from_hip(dms::launch_decode_multi(*shape, *cache, q, n_query, out, sm_scale, workspace,
                                           workspace_bytes, stream));
}

static int check_prefill_shape(const dms_shape *shape, int32_t seq_len) {
  if (!shape) return DMS_EINVAL;
  if (shape->batch < 1 || shape->kv_heads < 1 || shape->group < 1 || shape->window < 1)
    return DMS_EINVAL;
  if (seq_len < 0) return DMS_EINVAL;
  if (shape->head_dim != 128 && shape->head_dim != 64) return DMS_EUNSUPPORTED;
  if (shape->kv_dtype == DMS_KV_F32) return DMS_OK;  // the float32 kernel: any group
  if (shape->kv_dtype != DMS_KV_BF16 || shape->group > 16) return DMS_EUNSUPPORTED;
  return DMS_OK;
}

// float32 prefill uses no workspace; this many bytes are still asked for, so
// that 0 keeps meaning invalid arguments
constexpr size_t kPrefillF32Workspace = 256;

size_t dms_prefill_workspace_bytes(const dms_shape *shape, int32_t seq_len) {
  if (check_prefill_shape(shape, seq_len) != DMS_OK) return 0;
  if (shape->kv_dtype == DMS_KV_F32) return kPrefillF32Workspace;
  return dms::prefill_workspace_bytes(shape->batch, shape->kv_heads, seq_len, shape->head_dim);
}

int dms_prefill_attn(const dms_shape *shape, const void *q, const void *k, const void *v,
                     const float *logit, int32_t seq_len, float sm_scale, float *out,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_prefill_shape(shape, seq_len);
  if (rc) return rc;
  if (seq_len == 0) return DMS_OK;
  if (!q || !k || !v || !logit || !out || !workspace) return DMS_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace))
    return DMS_EINVAL;
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return DMS_EINVAL;
  if (workspace_bytes < dms_prefill_workspace_bytes(shape, seq_len)) return DMS_EWORKSPACE;
  if (shape->kv_dtype == DMS_KV_F32)
    return from_hip(dms::launch_prefill_f32(*shape, q, k, v, logit, nullptr, 0.f, seq_len, sm_scale,
                                            out, stream));
  return from_hip(dms::launch_prefill(*shape, q, k, v, logit, nullptr, 0.f, seq_len, sm_scale, out,
                                      workspace, stream));
}

int dms_prefill_attn_relaxed(const dms_shape *shape, const void *q, const void *k, const void *v,
                             const float *logit, const float *noise, float temperature,
                             int32_t seq_len, float sm_scale, float *out, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  int rc = check_prefill_shape(shape, seq_len);
  if (rc) return rc;
  if (!(temperature > 0.0f) || temperature == INFINITY) return DMS_EINVAL;
  if (seq_len == 0) return DMS_OK;
  if (!q || !k || !v || !logit || !out || !workspace) return DMS_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace))
    return DMS_EINVAL;
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return DMS_EINVAL;
  if (workspace_bytes < dms_prefill_workspace_bytes(shape, seq_len)) return DMS_EWORKSPACE;
  if (shape->kv_dtype == DMS_KV_F32)
    return from_hip(dms::launch_prefill_f32(*shape, q, k, v, logit, noise, temperature, seq_len,
                                            sm_scale, out, stream));
  return from_hip(dms::launch_prefill(*shape, q, k, v, logit, noise, temperature, seq_len, sm_scale,
                                      out, workspace, stream));
}

size_t dms_prefill_gathered_workspace_bytes(const dms_shape *shape, int32_t seq_len) {
  if (check_prefill_shape(shape, seq_len) != DMS_OK) return 0;
  if (shape->kv_dtype == DMS_KV_F32) return kPrefillF32Workspace;
  return dms::prefill_gathered_layout(shape->batch, shape->kv_heads, seq_len, shape->head_dim).total;
}

int dms_prefill_attn_gathered(const dms_shape *shape, const void *q, const void *k, const void *v,
                              const float *logit, int32_t seq_len, float sm_scale, float *out,
                              void *workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_prefill_shape(shape, seq_len);
  if (rc) return rc;
  if (seq_len == 0) return DMS_OK;
  if (!q || !k || !v || !logit || !out || !workspace) return DMS_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace))
    return DMS_EINVAL;
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return DMS_EINVAL;
  if (workspace_bytes < dms_prefill_gathered_workspace_bytes(shape, seq_len)) return DMS_EWORKSPACE;
  // float32: the float32 kernel, which skips the tiles no query of a block sees
  if (shape->kv_dtype == DMS_KV_F32)
    return from_hip(dms::launch_prefill_f32(*shape, q, k, v, logit, nullptr, 0.f, seq_len, sm_scale,
                                            out, stream));
  return from_hip(
      dms::launch_prefill_gathered(*shape, q, k, v, logit, seq_len, sm_scale, out, workspace, stream));
}

}  // extern "C"
