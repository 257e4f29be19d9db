"""Freed-page poisoning: pages on the free stack are filled with bf16 NaN keys
and values (and nonsense positions and decisions) after every call that frees
pages.  Whatever a recycled page still holds beyond a unit's slots in use, no
kernel may let it reach an output: append, decode (both step paths), chunk
queries (the split-K kernel for short chunks, the tiled kernel for long
ones), compaction, release and prompt sharing must give the oracle's outputs,
all finite, with exact page accounting.
"""

import copy
import math

import numpy as np
import pytest
import torch

import workloads as wl
from decode_attention_learned_amd import DmsCache
from harness import BF16_TOL, HostModel, check_pages, check_slots_exact, compare_outputs, say
from oracle import dms_oracle as orc

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def poison_free_pages(cache):
    """NaN keys and values, position -123456789 and decision 0xff in every free page."""
    torch.cuda.synchronize()
    top = int(cache.free_top.item())
    ids = cache.free_list[:top].long()
    if ids.numel():
        cache.k_pages.view(torch.int16)[ids] = NAN_BF16
        cache.v_pages.view(torch.int16)[ids] = NAN_BF16
        cache.slot_pos[ids] = -123456789
        cache.slot_alpha[ids] = 0xFF
    torch.cuda.synchronize()
    return top


def _check(out, ref, hkv, g, what):
    assert torch.isfinite(out).all(), f"{what}: non-finite output"
    compare_outputs(out.cpu(), ref, hkv, g, torch.bfloat16, what=what)


def test_poisoned_free_pages_never_reach_outputs(gpu):
    b, hkv, g, d = 3, 2, 4, 128
    w = wl.Workload(name="poison", kind="decode", batch=b, kv_heads=hkv, group=g, head_dim=d,
                    dtype="bf16", context=333, evict_rate=0.8, seed=9501, steps=0,
                    prompt_chunk=333, compact_every=16)
    rates = wl.unit_eviction_rates(w)
    maxp = 24
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, num_pages=b * hkv * maxp, max_pages_per_unit=maxp,
                     device=gpu)
    model = HostModel(b, hkv, g, d, w.window)
    scale = 1.0 / math.sqrt(d)
    poison_free_pages(cache)                         # the whole pool, before the first append
    k, v, logit = wl.prompt_chunk_inputs(w, 0, w.context, rates=rates)
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    model.append(k, v, logit)
    cache.compact()
    model.compact()
    poison_free_pages(cache)
    check_pages(cache, check_slots_exact(cache, model))

    # decode steps, alternating the two step paths, compaction every 5 steps
    for step in range(23):
        q, k, v, logit = wl.decode_step_inputs(w, step, rates=rates)
        model.append(k, v, logit)
        if step % 2:
            out = cache.step(k.to(gpu), v.to(gpu), logit.to(gpu), q.to(gpu))
        else:
            cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
            out = cache.decode(q.to(gpu))
        _check(out, model.decode(q, scale), hkv, g, f"step {step}")
        if step % 5 == 4:
            cache.compact()
            model.compact()
            poison_free_pages(cache)
    check_pages(cache, check_slots_exact(cache, model))

    # chunk queries: 5 tokens (split-K kernel), then 40 (tiled kernel), compacting after each
    wc = wl.Workload(name="poison_chunk", kind="prefill", batch=b, kv_heads=hkv, group=g,
                     head_dim=d, dtype="bf16", context=45, evict_rate=0.8, seed=9502)
    qc, kc, vc, lc = wl.prefill_inputs(wc)
    alpha_c = orc.eviction_decisions(lc.numpy())
    t0 = 0
    for n in (5, 40):
        sl = slice(t0, t0 + n)
        base = [uc.length for uc in model.units]
        cache.append(kc[:, sl].contiguous().to(gpu), vc[:, sl].contiguous().to(gpu),
                     lc[:, sl].contiguous().to(gpu))
        out = cache.decode_chunk(qc[:, sl].contiguous().to(gpu))
        torch.cuda.synchronize()
        assert cache.status_word() == 0
        assert torch.isfinite(out).all(), f"chunk of {n}: non-finite output"
        model.append(kc[:, sl], vc[:, sl], lc[:, sl])
        o = out.cpu().double().numpy()
        for u, uc in enumerate(model.units):
            bi, h = divmod(u, hkv)
            for c in range(n):
                # query c of the chunk: the decode rule at its own position over
                # the unit's slots (retained before the chunk, then the chunk)
                t = base[u] + c
                vis = (uc.pos <= t) & (~uc.alpha | (t - uc.pos < w.window))
                ref = orc.softmax_attention(qc[bi, t0 + c, h * g:(h + 1) * g].float().numpy(),
                                            uc.k[vis], uc.v[vis], scale)
                got = o[bi, c, h * g:(h + 1) * g]
                assert np.all(np.abs(got - ref) <= BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref)), \
                    f"chunk of {n}, query {c}, unit {u}"
        cache.compact()
        model.compact()
        poison_free_pages(cache)
        t0 += n
    check_pages(cache, check_slots_exact(cache, model))

    # release sequence 1, poison its pages, share sequence 0's prompt with it
    cache.release(1, 1)
    poison_free_pages(cache)
    cache.share_prefix(0, 1, 1)
    torch.cuda.synchronize()
    for h in range(hkv):   # the receiver's units now hold what the source's hold
        model.units[1 * hkv + h] = copy.deepcopy(model.units[0 * hkv + h])
    for step in range(23, 30):
        q, k, v, logit = wl.decode_step_inputs(w, step, rates=rates)
        model.append(k, v, logit)
        out = cache.step(k.to(gpu), v.to(gpu), logit.to(gpu), q.to(gpu))
        _check(out, model.decode(q, scale), hkv, g, f"after sharing, step {step}")
        if step % 3 == 2:
            cache.compact()
            model.compact()
            poison_free_pages(cache)
    torch.cuda.synchronize()
    assert cache.status_word() == 0
    check_slots_exact(cache, model)
    say("poisoned free pages: every output finite and equal to the oracle")
