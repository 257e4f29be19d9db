"""ctypes binding of libdms.so: the C ABI declared in include/dms.h, name for name.

Argument marshalling only: every computation happens in the HIP kernels.
:func:`load` raises if the library has not been built; there is no fallback.

Two builds of the same sources exist: ``libdms.so`` (the product) and
``libdms_generic.so``, a test build whose one-query decode of bf16 caches runs
the vector kernel instead of the matrix-core one, so tests can check the two
against each other.  :func:`variant` switches the calls of this module to it
for the duration of a ``with`` block.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdms.so")
VARIANT_PATHS = {"": LIB_PATH, "generic": os.path.join(_HERE, "libdms_generic.so")}

DMS_PAGE_SIZE = 64
DMS_OK = 0
DMS_EINVAL = -1
DMS_EUNSUPPORTED = -2
DMS_EWORKSPACE = -3
DMS_EHIP = -4
DMS_ESCRATCH = -5
DMS_NOALLOC_SCRATCH_BYTES = 16 << 20
DMS_STATUS_POOL_EXHAUSTED = 1
DMS_STATUS_ROW_OVERFLOW = 2
DMS_STATUS_NOT_EMPTY = 4
DMS_STATUS_CHUNK_INVALID = 8
DMS_KV_F32 = 0
DMS_KV_BF16 = 1

# every symbol include/dms.h declares
EXPORTS = (
    "dms_version",
    "dms_strerror",
    "dms_check_shape",
    "dms_plan_words",
    "dms_export_retained",
    "dms_reset",
    "dms_append",
    "dms_compact",
    "dms_share_prefix",
    "dms_release",
    "dms_decode_workspace_bytes",
    "dms_decode_attn",
    "dms_decode_attn_noalloc",
    "dms_append_reserve",
    "dms_decode_attn_fill",
    "dms_decode_multi_workspace_bytes",
    "dms_decode_multi_split_workspace_bytes",
    "dms_decode_attn_multi",
    "dms_prefill_workspace_bytes",
    "dms_prefill_attn",
    "dms_prefill_attn_relaxed",
    "dms_prefill_gathered_workspace_bytes",
    "dms_prefill_attn_gathered",
)


class DmsShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("max_pages_per_unit", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
    ]


class DmsCacheStruct(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("slot_pos", ctypes.c_void_p),
        ("slot_alpha", ctypes.c_void_p),
        ("n_slots", ctypes.c_void_p),
        ("n_clean", ctypes.c_void_p),
        ("append_base", ctypes.c_void_p),
        ("seq_len", ctypes.c_void_p),
        ("free_list", ctypes.c_void_p),
        ("free_top", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("plan", ctypes.c_void_p),
        ("page_ref", ctypes.c_void_p),
    ]


class DmsError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {code} ({strerror(code)})")


_libs: dict = {}
_active = ""


@contextlib.contextmanager
def variant(name: str):
    """Route this module's calls to the build `name` ("" = the product library)."""
    global _active
    if name not in VARIANT_PATHS:
        raise ValueError(f"unknown library build {name!r}")
    prev, _active = _active, name
    try:
        load()
        yield
    finally:
        _active = prev


def load() -> ctypes.CDLL:
    """Load the active build once; raise if it is missing (build it with __graft_entry__.build())."""
    if _active in _libs:
        return _libs[_active]
    path = VARIANT_PATHS[_active]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first "
                           "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    SP = ctypes.POINTER(DmsShape)
    CP = ctypes.POINTER(DmsCacheStruct)
    sig = {
        "dms_version": ([], ctypes.c_int),
        "dms_strerror": ([ctypes.c_int], ctypes.c_char_p),
        "dms_check_shape": ([SP], ctypes.c_int),
        "dms_plan_words": ([SP], ctypes.c_size_t),
        "dms_export_retained": ([SP, CP, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P],
                                ctypes.c_int),
        "dms_reset": ([SP, CP, P], ctypes.c_int),
        "dms_append": ([SP, CP, P, P, P, ctypes.c_int32, P], ctypes.c_int),
        "dms_compact": ([SP, CP, P], ctypes.c_int),
        "dms_share_prefix": ([SP, CP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P], ctypes.c_int),
        "dms_release": ([SP, CP, ctypes.c_int32, ctypes.c_int32, P], ctypes.c_int),
        "dms_decode_workspace_bytes": ([SP], ctypes.c_size_t),
        "dms_decode_attn": ([SP, CP, P, P, ctypes.c_float, P, ctypes.c_size_t, P], ctypes.c_int),
        "dms_decode_attn_noalloc": ([SP, CP, P, P, ctypes.c_float, P], ctypes.c_int),
        "dms_append_reserve": ([SP, CP, P], ctypes.c_int),
        "dms_decode_attn_fill": ([SP, CP, P, P, P, P, P, ctypes.c_float, P, ctypes.c_size_t, P],
                                 ctypes.c_int),
        "dms_decode_multi_workspace_bytes": ([SP], ctypes.c_size_t),
        "dms_decode_multi_split_workspace_bytes": ([SP, ctypes.c_int32], ctypes.c_size_t),
        "dms_decode_attn_multi": ([SP, CP, P, ctypes.c_int32, P, ctypes.c_float, P, ctypes.c_size_t, P],
                                  ctypes.c_int),
        "dms_prefill_workspace_bytes": ([SP, ctypes.c_int32], ctypes.c_size_t),
        "dms_prefill_attn": ([SP, P, P, P, P, ctypes.c_int32, ctypes.c_float, P, P, ctypes.c_size_t, P],
                             ctypes.c_int),
        "dms_prefill_attn_relaxed": ([SP, P, P, P, P, P, ctypes.c_float, ctypes.c_int32, ctypes.c_float, P,
                                      P, ctypes.c_size_t, P], ctypes.c_int),
        "dms_prefill_gathered_workspace_bytes": ([SP, ctypes.c_int32], ctypes.c_size_t),
        "dms_prefill_attn_gathered": ([SP, P, P, P, P, ctypes.c_int32, ctypes.c_float, P, P,
                                       ctypes.c_size_t, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _libs[_active] = lib
    return lib


def strerror(code: int) -> str:
    return load().dms_strerror(code).decode()


def check(fn: str, code: int) -> None:
    if code != DMS_OK:
        raise DmsError(fn, code)


def _p(t) -> int | None:
    """Device pointer of a tensor (None for None)."""
    return None if t is None else t.data_ptr()


def version() -> int:
    return load().dms_version()


def check_shape(shape: DmsShape) -> int:
    return load().dms_check_shape(ctypes.byref(shape))


def plan_words(shape: DmsShape) -> int:
    return load().dms_plan_words(ctypes.byref(shape))


def decode_workspace_bytes(shape: DmsShape) -> int:
    return load().dms_decode_workspace_bytes(ctypes.byref(shape))


def dms_reset(shape, cache, stream) -> int:
    return load().dms_reset(ctypes.byref(shape), ctypes.byref(cache), stream)


def dms_append(shape, cache, k_new, v_new, logit, n_new, stream) -> int:
    return load().dms_append(ctypes.byref(shape), ctypes.byref(cache), _p(k_new), _p(v_new),
                             _p(logit), int(n_new), stream)


def dms_export_retained(shape, cache, all_slots, max_per_unit, count_out, pos_out, alpha_out,
                        k_out, v_out, stream) -> int:
    return load().dms_export_retained(ctypes.byref(shape), ctypes.byref(cache), int(all_slots),
                                      int(max_per_unit), _p(count_out), _p(pos_out), _p(alpha_out),
                                      _p(k_out), _p(v_out), stream)


def dms_compact(shape, cache, stream) -> int:
    return load().dms_compact(ctypes.byref(shape), ctypes.byref(cache), stream)


def dms_decode_attn(shape, cache, q, out, sm_scale, workspace, workspace_bytes, stream) -> int:
    return load().dms_decode_attn(ctypes.byref(shape), ctypes.byref(cache), _p(q), _p(out),
                                  float(sm_scale), _p(workspace), int(workspace_bytes), stream)


def dms_decode_attn_noalloc(shape, cache, q, out, sm_scale, stream) -> int:
    return load().dms_decode_attn_noalloc(ctypes.byref(shape), ctypes.byref(cache), _p(q), _p(out),
                                          float(sm_scale), stream)


def dms_append_reserve(shape, cache, stream) -> int:
    return load().dms_append_reserve(ctypes.byref(shape), ctypes.byref(cache), stream)


def dms_decode_attn_fill(shape, cache, k_new, v_new, logit, q, out, sm_scale, workspace,
                         workspace_bytes, stream) -> int:
    return load().dms_decode_attn_fill(ctypes.byref(shape), ctypes.byref(cache), _p(k_new),
                                       _p(v_new), _p(logit), _p(q), _p(out), float(sm_scale),
                                       _p(workspace), int(workspace_bytes), stream)


def prefill_workspace_bytes(shape: DmsShape, seq_len: int) -> int:
    return load().dms_prefill_workspace_bytes(ctypes.byref(shape), int(seq_len))


def dms_prefill_attn(shape, q, k, v, logit, seq_len, sm_scale, out, workspace, workspace_bytes,
                     stream) -> int:
    return load().dms_prefill_attn(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(logit),
                                   int(seq_len), float(sm_scale), _p(out), _p(workspace),
                                   int(workspace_bytes), stream)


def prefill_gathered_workspace_bytes(shape: DmsShape, seq_len: int) -> int:
    return load().dms_prefill_gathered_workspace_bytes(ctypes.byref(shape), int(seq_len))


def dms_prefill_attn_gathered(shape, q, k, v, logit, seq_len, sm_scale, out, workspace,
                              workspace_bytes, stream) -> int:
    return load().dms_prefill_attn_gathered(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(logit),
                                            int(seq_len), float(sm_scale), _p(out), _p(workspace),
                                            int(workspace_bytes), stream)


def dms_prefill_attn_relaxed(shape, q, k, v, logit, noise, temperature, seq_len, sm_scale, out,
                             workspace, workspace_bytes, stream) -> int:
    return load().dms_prefill_attn_relaxed(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(logit),
                                           _p(noise), float(temperature),
                                           int(seq_len), float(sm_scale), _p(out), _p(workspace),
                                           int(workspace_bytes), stream)


def decode_multi_workspace_bytes(shape: DmsShape) -> int:
    return load().dms_decode_multi_workspace_bytes(ctypes.byref(shape))


def decode_multi_split_workspace_bytes(shape: DmsShape, n_query: int) -> int:
    return load().dms_decode_multi_split_workspace_bytes(ctypes.byref(shape), int(n_query))


def dms_decode_attn_multi(shape, cache, q, n_query, out, sm_scale, workspace, workspace_bytes,
                          stream) -> int:
    return load().dms_decode_attn_multi(ctypes.byref(shape), ctypes.byref(cache), _p(q), int(n_query),
                                        _p(out), float(sm_scale), _p(workspace), int(workspace_bytes),
                                        stream)


def dms_share_prefix(shape, cache, src_seq, dst_first, n_dst, stream) -> int:
    return load().dms_share_prefix(ctypes.byref(shape), ctypes.byref(cache), int(src_seq), int(dst_first),
                                   int(n_dst), stream)


def dms_release(shape, cache, first, n, stream) -> int:
    return load().dms_release(ctypes.byref(shape), ctypes.byref(cache), int(first), int(n), stream)
