"""Helpers shared by the GPU parity tests: an oracle-side mirror of a cache and
exports of the GPU cache state.  The mirror is built only from oracle/ code
and the seeded inputs; nothing on the oracle side is read from the GPU path.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import dms_oracle as orc

PAGE = 64
BF16_TOL = dict(rtol=2e-2, atol=2e-2)   # |o - o_ref| <= 2e-2 + 2e-2 |o_ref|
F32_ATOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class HostModel:
    """One :class:`oracle.dms_oracle.UnitCache` per (sequence, KV head) unit,
    fed with exactly the tensors the GPU receives, on the same compaction
    schedule."""

    def __init__(self, batch, kv_heads, group, head_dim, window):
        self.batch, self.kv_heads, self.group, self.head_dim = batch, kv_heads, group, head_dim
        self.window = window
        self.units = [orc.UnitCache(window, head_dim, dtype=np.float32)
                      for _ in range(batch * kv_heads)]

    def append(self, k, v, logit, refused=()):
        """k, v [B, n, Hkv, D], logit [B, n, Hkv] (CPU tensors)."""
        alpha = orc.eviction_decisions(logit.numpy())
        kf = k.float().numpy()
        vf = v.float().numpy()
        n = k.shape[1]
        for b in range(self.batch):
            for h in range(self.kv_heads):
                u = b * self.kv_heads + h
                if u in refused:
                    self.units[u].skip(n)
                else:
                    self.units[u].append(alpha[b, :, h], kf[b, :, h, :], vf[b, :, h, :])

    def compact(self):
        for uc in self.units:
            uc.compact()

    def decode(self, q, scale, units=None):
        """q [B, Hq, D] CPU tensor -> {unit: [G, D] float64}."""
        qf = q.double().numpy()
        g = self.group
        out = {}
        for u in (range(len(self.units)) if units is None else units):
            b, h = divmod(u, self.kv_heads)
            if self.units[u].n_slots == 0 or not self.units[u].live().any():
                out[u] = np.zeros((g, self.head_dim))
            else:
                out[u] = self.units[u].attend(qf[b, h * g:(h + 1) * g], scale)
        return out


def export_meta(cache):
    """Host copies of the cache metadata."""
    return dict(
        n_slots=cache.n_slots.cpu().numpy(),
        n_clean=cache.n_clean.cpu().numpy(),
        seq_len=cache.seq_len.cpu().numpy(),
        page_table=cache.page_table.cpu().numpy(),
        slot_pos=cache.slot_pos.cpu().numpy(),
        slot_alpha=cache.slot_alpha.cpu().numpy(),
        free_list=cache.free_list.cpu().numpy(),
        free_top=int(cache.free_top.item()),
        status=int(cache.status.item()),
    )


def unit_slots(meta, u):
    n = int(meta["n_slots"][u])
    pages = meta["page_table"][u, : (n + PAGE - 1) // PAGE]
    pos = meta["slot_pos"][pages].reshape(-1)[:n]
    alpha = meta["slot_alpha"][pages].reshape(-1)[:n]
    return pos, alpha


def check_slots_exact(cache, model, meta=None):
    """GPU slot order and decisions equal the mirror's, unit by unit (bit-exact)."""
    meta = export_meta(cache) if meta is None else meta
    for u, uc in enumerate(model.units):
        pos, alpha = unit_slots(meta, u)
        assert pos.tolist() == uc.pos.tolist(), f"unit {u}: slot positions differ"
        assert (alpha != 0).tolist() == uc.alpha.tolist(), f"unit {u}: decisions differ"
    return meta


def check_live_sets(cache, model, meta=None):
    """The set the GPU attends over (slots alive at t) equals R(t) of the oracle."""
    meta = export_meta(cache) if meta is None else meta
    for u, uc in enumerate(model.units):
        b = u // model.kv_heads
        t = int(meta["seq_len"][b]) - 1
        pos, alpha = unit_slots(meta, u)
        live = (alpha == 0) | ((t - pos) < model.window)
        assert pos[live].tolist() == uc.pos[uc.live(t)].tolist(), f"unit {u}: live sets differ"
    return meta


def check_pages(cache, meta=None):
    """Page conservation: every page is free or owned by exactly one unit."""
    meta = export_meta(cache) if meta is None else meta
    num_pages = cache.num_pages
    owned = []
    for u in range(cache.units):
        n = int(meta["n_slots"][u])
        npg = (n + PAGE - 1) // PAGE
        row = meta["page_table"][u]
        assert np.all(row[:npg] >= 0), f"unit {u}: missing page"
        assert np.all(row[npg:] == -1), f"unit {u}: stale page-table entries"
        owned.extend(row[:npg].tolist())
    free = meta["free_list"][: meta["free_top"]].tolist()
    assert meta["free_top"] + len(owned) == num_pages
    assert sorted(owned + free) == list(range(num_pages))
    return meta


def gpu_kv(cache, units=None):
    """{unit: (k [n, D], v [n, D])} float32 CPU arrays of the units' slots in slot
    order, read back through dms_export_retained (all slots)."""
    return {u: (k.float().numpy(), v.float().numpy())
            for u, (k, v) in cache.slot_kv(units).items()}


def check_kv_exact(cache, model, units):
    units = list(units)
    kv = gpu_kv(cache, units)
    for u in units:
        k, v = kv[u]
        uc = model.units[u]
        assert np.array_equal(k, uc.k), f"unit {u}: key bytes differ"
        assert np.array_equal(v, uc.v), f"unit {u}: value bytes differ"


def compare_outputs(out_gpu, ref, kv_heads, group, dtype, what=""):
    """out_gpu [B, Hq, D] CPU float32; ref {unit: [G, D]}.  Returns max abs error."""
    o = out_gpu.double().numpy()
    worst = 0.0
    for u, r in ref.items():
        b, h = divmod(u, kv_heads)
        got = o[b, h * group:(h + 1) * group]
        err = np.abs(got - r)
        worst = max(worst, float(err.max()))
        if dtype == torch.float32:
            assert err.max() <= F32_ATOL, f"{what} unit {u}: max abs err {err.max():.3g} > {F32_ATOL}"
        else:
            bound = BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(r)
            assert np.all(err <= bound), f"{what} unit {u}: err {err.max():.3g} beyond 2e-2 abs/rel"
    return worst


def scale_of(d):
    return 1.0 / math.sqrt(d)


def decode_build(kernel):
    """Context that routes library calls to the build running `kernel` for one-query
    bf16 decode: "mfma" (the product library) or "generic" (the test build)."""
    from decode_attention_learned_amd import lib

    return lib.variant("" if kernel == "mfma" else "generic")


def check_accounting(cache):
    """Every page is on the free stack or in some unit's row; page_ref = holders - 1."""
    torch.cuda.synchronize()
    n = cache.n_slots.cpu().long()
    rows = cache.page_table.cpu()
    holders = torch.zeros(cache.num_pages, dtype=torch.long)
    for u in range(cache.units):
        np_ = (int(n[u]) + 63) // 64
        for pg in rows[u, :np_].tolist():
            assert pg >= 0
            holders[pg] += 1
    top = int(cache.free_top.item())
    free = cache.free_list[:top].cpu().long()
    assert len(set(free.tolist())) == top, "a page is on the free stack twice"
    assert torch.all(holders[free] == 0), "a held page is on the free stack"
    assert top + int((holders > 0).sum()) == cache.num_pages, "pages lost"
    ref = cache.page_ref.cpu().long()
    held = holders > 0
    assert torch.equal(ref[held], holders[held] - 1)
    assert torch.all(ref[~held] == 0)
