"""Torch-side ownership of a DMS paged cache and thin calls into libdms.

PyTorch only allocates device memory and supplies the stream; every step
(reset, decide + append, compaction, decode, prefill) runs in the library's
HIP kernels.  Shapes and layouts are those of include/dms.h.
"""

from __future__ import annotations

import math

import torch

from . import lib

PAGE = lib.DMS_PAGE_SIZE
_DTYPES = {torch.float32: lib.DMS_KV_F32, torch.bfloat16: lib.DMS_KV_BF16}


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


class DmsCache:
    """A paged DMS cache for `batch` sequences x `kv_heads` KV heads.

    Buffers (all on `device`): see the dms_cache struct in include/dms.h.
    """

    def __init__(self, batch: int, kv_heads: int, group: int, head_dim: int,
                 dtype: torch.dtype = torch.bfloat16, num_pages: int | None = None,
                 max_pages_per_unit: int = 64, window: int = 16, device="cuda:0"):
        lib.load()
        self.device = torch.device(device)
        if dtype not in _DTYPES:
            raise TypeError(f"unsupported KV dtype {dtype}")
        self.dtype = dtype
        self.batch, self.kv_heads, self.group, self.head_dim = batch, kv_heads, group, head_dim
        self.window = window
        self.units = batch * kv_heads
        self.max_pages_per_unit = max_pages_per_unit
        self.num_pages = num_pages if num_pages is not None else self.units * max_pages_per_unit
        self.shape = lib.DmsShape(batch, kv_heads, group, head_dim, PAGE, window,
                                  max_pages_per_unit, self.num_pages, _DTYPES[dtype])
        rc = lib.check_shape(self.shape)
        lib.check("dms_check_shape", rc)
        dev = self.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.k_pages = torch.zeros((self.num_pages, PAGE, head_dim), dtype=dtype, device=dev)
        self.v_pages = torch.zeros((self.num_pages, PAGE, head_dim), dtype=dtype, device=dev)
        self.page_table = torch.empty((self.units, max_pages_per_unit), **i32)
        self.slot_pos = torch.zeros((self.num_pages, PAGE), **i32)
        self.slot_alpha = torch.zeros((self.num_pages, PAGE), dtype=torch.uint8, device=dev)
        self.n_slots = torch.empty((self.units,), **i32)
        self.n_clean = torch.empty((self.units,), **i32)
        self.append_base = torch.empty((self.units,), **i32)
        self.seq_len = torch.empty((batch,), **i32)
        self.free_list = torch.empty((self.num_pages,), **i32)
        self.free_top = torch.empty((1,), **i32)
        self.status = torch.empty((1,), **i32)
        self.plan = torch.empty((lib.plan_words(self.shape),), **i32)
        self.page_ref = torch.empty((self.num_pages,), **i32)
        self._bind()
        self.workspace_bytes = lib.decode_workspace_bytes(self.shape)
        self.workspace = torch.empty((self.workspace_bytes,), dtype=torch.uint8, device=dev)
        self.reset()

    # The cache state: every buffer the library reads or writes, in the order of
    # the dms_cache struct.  The library keeps nothing else, so these tensors
    # are the whole state (a checkpoint is a copy of them).
    STATE = ("k_pages", "v_pages", "page_table", "slot_pos", "slot_alpha", "n_slots", "n_clean",
             "append_base", "seq_len", "free_list", "free_top", "status", "plan", "page_ref")

    def _bind(self) -> None:
        """(Re)build the dms_cache struct from the state tensors' addresses."""
        self.cache = lib.DmsCacheStruct(*[getattr(self, n).data_ptr() for n in self.STATE])

    def state_dict(self) -> dict:
        """Copies of the state tensors (for torch.save)."""
        return {n: getattr(self, n).clone() for n in self.STATE}

    def load_state_dict(self, state: dict) -> None:
        """Overwrite the state with a checkpoint of a cache of the same shape."""
        for n in self.STATE:
            dst = getattr(self, n)
            src = state[n]
            if src.shape != dst.shape or src.dtype != dst.dtype:
                raise ValueError(f"checkpoint field {n}: {tuple(src.shape)} {src.dtype}, "
                                 f"cache holds {tuple(dst.shape)} {dst.dtype}")
            dst.copy_(src)

    # -- calls -------------------------------------------------------------
    def reset(self) -> None:
        lib.check("dms_reset", lib.dms_reset(self.shape, self.cache, _stream()))

    def append(self, k: torch.Tensor, v: torch.Tensor, logit: torch.Tensor) -> None:
        """k, v [B, n, Hkv, D] (cache dtype), logit [B, n, Hkv] float32."""
        n = k.shape[1]
        kshape = (self.batch, n, self.kv_heads, self.head_dim)
        _need(k, "k", self.dtype, kshape, self.device)
        _need(v, "v", self.dtype, kshape, self.device)
        _need(logit, "logit", torch.float32, kshape[:3], self.device)
        lib.check("dms_append", lib.dms_append(self.shape, self.cache, k, v, logit, n, _stream()))

    def compact(self) -> None:
        lib.check("dms_compact", lib.dms_compact(self.shape, self.cache, _stream()))

    def decode(self, q: torch.Tensor, out: torch.Tensor | None = None,
               sm_scale: float | None = None) -> torch.Tensor:
        """q [B, Hq, D] (cache dtype) -> out [B, Hq, D] float32."""
        qshape = (self.batch, self.kv_heads * self.group, self.head_dim)
        _need(q, "q", self.dtype, qshape, self.device)
        if out is None:
            out = torch.empty(qshape, dtype=torch.float32, device=self.device)
        _need(out, "out", torch.float32, qshape, self.device)
        scale = 1.0 / math.sqrt(self.head_dim) if sm_scale is None else sm_scale
        lib.check("dms_decode_attn", lib.dms_decode_attn(
            self.shape, self.cache, q, out, scale, self.workspace, self.workspace_bytes, _stream()))
        return out

    def step(self, k: torch.Tensor, v: torch.Tensor, logit: torch.Tensor, q: torch.Tensor,
             out: torch.Tensor | None = None, sm_scale: float | None = None) -> torch.Tensor:
        """One decode step: append one token per sequence (k, v [B, 1, Hkv, D],
        logit [B, 1, Hkv]) and attend its query q [B, Hq, D] -> out [B, Hq, D]
        float32.  Equivalent to append() then decode(), with one launch less
        (dms_append_reserve + dms_decode_attn_fill): the same cache state, and
        outputs equal to rounding (the new token's weight stays float32)."""
        kshape = (self.batch, 1, self.kv_heads, self.head_dim)
        _need(k, "k", self.dtype, kshape, self.device)
        _need(v, "v", self.dtype, kshape, self.device)
        _need(logit, "logit", torch.float32, kshape[:3], self.device)
        qshape = (self.batch, self.kv_heads * self.group, self.head_dim)
        _need(q, "q", self.dtype, qshape, self.device)
        if out is None:
            out = torch.empty(qshape, dtype=torch.float32, device=self.device)
        _need(out, "out", torch.float32, qshape, self.device)
        scale = 1.0 / math.sqrt(self.head_dim) if sm_scale is None else sm_scale
        self.reserve()
        self.fill_and_decode(k, v, logit, q, out, scale)
        return out

    def reserve(self) -> None:
        """First half of step(): slots, pages and counts for one token per sequence."""
        lib.check("dms_append_reserve", lib.dms_append_reserve(self.shape, self.cache, _stream()))

    def fill_and_decode(self, k: torch.Tensor, v: torch.Tensor, logit: torch.Tensor,
                        q: torch.Tensor, out: torch.Tensor, sm_scale: float) -> torch.Tensor:
        """Second half of step() (argument checks are step()'s): attend with the
        reserved token included, and write it to its slot."""
        lib.check("dms_decode_attn_fill", lib.dms_decode_attn_fill(
            self.shape, self.cache, k, v, logit, q, out, sm_scale, self.workspace,
            self.workspace_bytes, _stream()))
        return out

    def share_prefix(self, src_seq: int, dst_first: int, n_dst: int) -> None:
        """Sequences dst_first .. dst_first + n_dst - 1 (empty) take over the state
        of sequence src_seq, sharing its clean full pages (dms_share_prefix)."""
        lib.check("dms_share_prefix", lib.dms_share_prefix(self.shape, self.cache, src_seq, dst_first,
                                                           n_dst, _stream()))

    def release(self, first: int, n: int = 1) -> None:
        """Empty sequences first .. first + n - 1 and return their pages (dms_release)."""
        lib.check("dms_release", lib.dms_release(self.shape, self.cache, first, n, _stream()))

    def decode_chunk(self, q: torch.Tensor, out: torch.Tensor | None = None,
                     sm_scale: float | None = None) -> torch.Tensor:
        """q [B, C, Hq, D] (bf16): queries of the last C appended tokens of every
        sequence -> out [B, C, Hq, D] float32.  Call before compacting."""
        if q.dim() != 4 or q.shape[0] != self.batch:
            raise ValueError("q must be [B, C, Hq, D]")
        n_query = q.shape[1]
        qshape = (self.batch, n_query, self.kv_heads * self.group, self.head_dim)
        _need(q, "q", self.dtype, qshape, self.device)
        if out is None:
            out = torch.empty(qshape, dtype=torch.float32, device=self.device)
        _need(out, "out", torch.float32, qshape, self.device)
        # the workspace that lets long chunks split their tiles over the chip
        need = lib.decode_multi_split_workspace_bytes(self.shape, n_query)
        if getattr(self, "_multi_ws", None) is None or self._multi_ws.numel() < need:
            self._multi_ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=self.device)
        scale = 1.0 / math.sqrt(self.head_dim) if sm_scale is None else sm_scale
        lib.check("dms_decode_attn_multi", lib.dms_decode_attn_multi(
            self.shape, self.cache, q, n_query, out, scale, self._multi_ws, self._multi_ws.numel(), _stream()))
        return out

    # -- inspection (host copies; for tests and reports) -------------------
    def status_word(self) -> int:
        return int(self.status.item())

    def pages_in_use(self) -> int:
        return self.num_pages - int(self.free_top.item())

    def export(self, all_slots: bool = False, max_per_unit: int | None = None, kv: bool = True):
        """dms_export_retained: (count [units], pos [units, m], alpha [units, m],
        k [units, m, D], v [units, m, D]) as device tensors, m = max_per_unit (default:
        the longest unit).  The retained set R(t) of every unit at its last position,
        or with `all_slots` every slot in use; rows past a unit's count are zero.
        k and v are None when `kv` is false."""
        if max_per_unit is None:
            max_per_unit = int(self.n_slots.max().item()) if self.units else 0
        dev = self.device
        m = max(int(max_per_unit), 0)
        count = torch.empty((self.units,), dtype=torch.int32, device=dev)
        pos = torch.zeros((self.units, m), dtype=torch.int32, device=dev)
        alpha = torch.zeros((self.units, m), dtype=torch.uint8, device=dev)
        k = v = None
        if kv:
            k = torch.zeros((self.units, m, self.head_dim), dtype=self.dtype, device=dev)
            v = torch.zeros_like(k)
        lib.check("dms_export_retained", lib.dms_export_retained(
            self.shape, self.cache, 1 if all_slots else 0, m, count, pos, alpha, k, v, _stream()))
        return count, pos, alpha, k, v

    def slots(self, unit: int):
        """(pos, alpha) of every slot of `unit`, in slot order, as CPU tensors."""
        n = int(self.n_slots[unit].item())
        pages = self.page_table[unit, : (n + PAGE - 1) // PAGE].long()
        pos = self.slot_pos[pages].reshape(-1)[:n].cpu()
        alpha = self.slot_alpha[pages].reshape(-1)[:n].cpu()
        return pos, alpha

    def slot_kv(self, units=None):
        """{unit: (k [n, D], v [n, D])} of every slot of each unit in `units` (default:
        all), in slot order, as CPU tensors, read back through dms_export_retained."""
        count, _, _, k, v = self.export(all_slots=True)
        count = count.cpu()
        units = range(self.units) if units is None else units
        return {u: (k[u, :int(count[u])].cpu(), v[u, :int(count[u])].cpu()) for u in units}


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, logit: torch.Tensor,
            window: int = 16, sm_scale: float | None = None,
            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
            method: str = "dense", noise: torch.Tensor | None = None,
            temperature: float = 1.0) -> torch.Tensor:
    """Masked DMS prefill: q [B, S, Hq, D], k, v [B, S, Hkv, D] (bf16, or float32 for the
    float32 kernel), logit [B, S, Hkv] f32.

    method "dense" runs dms_prefill_attn (every causal tile, masked), "gathered"
    runs dms_prefill_attn_gathered (gathered kept keys plus the window band),
    "relaxed" runs dms_prefill_attn_relaxed (keep factor 1 - sigmoid((logit +
    noise) / temperature) outside the window; noise [B, S, Hkv] f32 or None).
    `workspace` (uint8, at least the method's workspace size) is allocated when
    not given."""
    if method not in ("dense", "gathered", "relaxed"):
        raise ValueError(f"unknown prefill method {method!r}")
    lib.load()
    b, s, hq, d = q.shape
    hkv = k.shape[2]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    dev = q.device
    _need(k, "k", q.dtype, (b, s, hkv, d), dev)
    _need(v, "v", q.dtype, (b, s, hkv, d), dev)
    _need(logit, "logit", torch.float32, (b, s, hkv), dev)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if out is None:
        out = torch.empty((b, s, hq, d), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (b, s, hq, d), dev)
    shape = lib.DmsShape(b, hkv, hq // hkv, d, PAGE, window, 1, 1, _DTYPES.get(q.dtype, -1))
    scale = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    gathered = method == "gathered"
    need = (lib.prefill_gathered_workspace_bytes if gathered else lib.prefill_workspace_bytes)(shape, s)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    if method == "relaxed":
        if noise is not None:
            _need(noise, "noise", torch.float32, (b, s, hkv), dev)
        lib.check("dms_prefill_attn_relaxed", lib.dms_prefill_attn_relaxed(
            shape, q, k, v, logit, noise, temperature, s, scale, out, workspace, workspace.numel(),
            _stream()))
        return out
    call = lib.dms_prefill_attn_gathered if gathered else lib.dms_prefill_attn
    name = "dms_prefill_attn_gathered" if gathered else "dms_prefill_attn"
    lib.check(name, call(shape, q, k, v, logit, s, scale, out, workspace, workspace.numel(), _stream()))
    return out
