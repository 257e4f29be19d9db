"""The two-call decode step (dms_append_reserve + dms_decode_attn_fill: the
decode launch takes the step's token as one more softmax term and writes it
to its page) against dms_append + dms_decode_attn on a twin cache, and against
the oracle: the same cache state (slot positions and decisions, K/V bytes,
counts, status; page ids may differ, as compaction returns pages from
concurrent workgroups); outputs bit-identical where the token is written by
the append's kernel ahead of the decode (float32 caches, and bf16 with the
generic kernel forced) and within 2e-3 on the bf16 matrix-core kernel, which
takes the token itself (its weight is not rounded to bf16 there), with one
chunk per unit and with split chunks, across page crossings, compactions and
refused units."""

import numpy as np
import pytest
import torch

import workloads as wl
from decode_attention_learned_amd import DmsCache, lib
from harness import (HostModel, check_pages, compare_outputs, decode_build, export_meta, gpu_kv, say,
                     scale_of, unit_slots)
from oracle import dms_oracle as orc

pytestmark = pytest.mark.gpu


def _workload(b, hkv, g, d, dtype, context, rate, seed):
    return wl.Workload(name="step_case", kind="decode", batch=b, kv_heads=hkv, group=g, head_dim=d,
                       dtype=dtype, context=context, evict_rate=rate, seed=seed, steps=0,
                       prompt_chunk=context, compact_every=16)


def _twins(w, dev, num_pages=None, max_pages=None):
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    max_pages = max_pages or (w.context + 200) // 64 + 3
    num_pages = num_pages or w.units * max_pages
    a, b = (DmsCache(w.batch, w.kv_heads, w.group, w.head_dim, tdt, num_pages=num_pages,
                     max_pages_per_unit=max_pages, window=w.window, device=dev) for _ in range(2))
    rates = wl.unit_eviction_rates(w)
    k, v, logit = wl.prompt_chunk_inputs(w, 0, w.context, rates=rates)
    for c in (a, b):
        c.append(k.to(dev), v.to(dev), logit.to(dev))
        c.compact()
    return a, b, rates


def _same_state(a, b, units):
    ma, mb = export_meta(a), export_meta(b)
    # page ids may differ: compaction returns emptied pages to the free stack
    # from concurrent workgroups, so the two caches' stacks need not agree
    for key in ("n_slots", "n_clean", "seq_len"):
        assert np.array_equal(ma[key], mb[key]), key
    assert ma["free_top"] == mb["free_top"] and ma["status"] == mb["status"]
    units = list(units)
    kva, kvb = gpu_kv(a, units), gpu_kv(b, units)
    for u in units:
        pa, aa = unit_slots(ma, u)
        pb, ab = unit_slots(mb, u)
        assert np.array_equal(pa, pb) and np.array_equal(aa, ab), f"unit {u}: slots differ"
        (ka, va), (kb, vb) = kva[u], kvb[u]
        assert np.array_equal(ka, kb) and np.array_equal(va, vb), f"unit {u}: K/V differ"
    check_pages(b, mb)


def _agree(oa, ob, exact, what):
    if exact:
        assert torch.equal(oa, ob), f"{what}: outputs differ"
    else:
        err = (oa - ob).abs().max().item()
        assert torch.allclose(oa, ob, atol=2e-3, rtol=2e-3), f"{what}: max difference {err:.3g}"


def _run(w, dev, steps, every, rates, a, b, check_every=5, exact=False, model=None):
    for step in range(steps):
        q, k, v, logit = wl.decode_step_inputs(w, step, rates=rates)
        if model is not None:
            model.append(k, v, logit)
        q, k, v, logit = q.to(dev), k.to(dev), v.to(dev), logit.to(dev)
        a.append(k, v, logit)
        oa = a.decode(q)
        ob = b.step(k, v, logit, q)
        _agree(oa, ob, exact, f"step {step}")
        if model is not None:
            compare_outputs(ob.cpu(), model.decode(q.cpu(), scale_of(w.head_dim)), w.kv_heads,
                            w.group, a.dtype, what=f"step {step} (fill path vs oracle)")
        if every and (step + 1) % every == 0:
            a.compact()
            b.compact()
            if model is not None:
                model.compact()
        if step % check_every == check_every - 1:
            _same_state(a, b, range(w.units))
    torch.cuda.synchronize()
    _same_state(a, b, range(w.units))


@pytest.mark.parametrize("kernel", ["mfma", "generic"])
@pytest.mark.parametrize("dims", [(3, 2, 5, 128), (2, 3, 4, 64), (1, 1, 16, 128)])
def test_step_matches_append_then_decode_bf16(gpu, kernel, dims):
    with decode_build(kernel):
        _step_bf16(gpu, kernel, dims)


def _step_bf16(gpu, kernel, dims):
    b, hkv, g, d = dims
    w = _workload(b, hkv, g, d, "bf16", 123, 0.6, 8100 + d + g)
    say(f"step vs append+decode, bf16 {kernel} B={b} Hkv={hkv} G={g} D={d}")
    a, bb, rates = _twins(w, gpu)
    model = HostModel(b, hkv, g, d, w.window)
    k, v, logit = wl.prompt_chunk_inputs(w, 0, w.context, rates=rates)
    model.append(k, v, logit)
    model.compact()
    _run(w, gpu, 150, 7, rates, a, bb, exact=kernel == "generic", model=model)
    assert bb.status_word() == 0


def test_step_matches_append_then_decode_f32(gpu):
    w = _workload(1, 2, 2, 64, "f32", 200, 0.5, 8201)
    a, b, rates = _twins(w, gpu)
    _run(w, gpu, 80, 16, rates, a, b, exact=True)


def test_step_one_chunk_per_unit(gpu):
    """512 units of even length: the plan gives each unit one chunk (the headline
    plan).  Every step's fill-path output is checked against the oracle."""
    w = _workload(64, 8, 4, 128, "bf16", 300, 0.875, 8301)
    a, b, rates = _twins(w, gpu)
    plan = b.plan.cpu()
    assert int(plan[0]) == w.units, "expected one chunk per unit"
    model = HostModel(w.batch, w.kv_heads, w.group, w.head_dim, w.window)
    k, v, logit = wl.prompt_chunk_inputs(w, 0, w.context, rates=rates)
    model.append(k, v, logit)
    model.compact()
    _run(w, gpu, 40, 16, rates, a, b, check_every=20, model=model)


def test_step_with_refused_units(gpu):
    """A pool too small for the next page of every unit: the same units are
    refused (no token written, status set) on both paths."""
    w = _workload(1, 4, 2, 64, "bf16", 127, 0.0, 8401)
    a, b, rates = _twins(w, gpu, num_pages=10, max_pages=4)   # 8 pages in use, 2 free
    for step in range(3):
        q, k, v, logit = wl.decode_step_inputs(w, step, rates=rates)
        q, k, v, logit = q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu)
        a.append(k, v, logit)
        oa = a.decode(q)
        ob = b.step(k, v, logit, q)
        _agree(oa, ob, False, f"step {step}")
    torch.cuda.synchronize()
    assert b.status_word() & lib.DMS_STATUS_POOL_EXHAUSTED
    assert b.append_base.cpu().tolist() == a.append_base.cpu().tolist()
    _same_state(a, b, range(w.units))


def test_step_full_size_qwen3_8b_cr8(gpu):
    """The headline shape, as bench.py runs it (dms_append_reserve +
    dms_decode_attn_fill, compaction every 16 steps): twin caches, and sampled
    units against the oracle at steps 0, 7, 15, 16 (right after a compaction)
    and 19."""
    w = wl.get("qwen3_8b_cr8")
    say("step vs append+decode at full size (building two 32768-token caches)")
    tdt = torch.bfloat16
    caches = []
    rates = wl.unit_eviction_rates(w)
    sample = list(range(0, w.units, 37)) + [w.units - 1]
    mirror = {u: orc.UnitCache(w.window, w.head_dim, dtype=np.float32) for u in sample}

    def feed(k, v, logit):
        alpha = orc.eviction_decisions(logit.cpu().numpy())
        for u, uc in mirror.items():
            bi, h = divmod(u, w.kv_heads)
            uc.append(alpha[bi, :, h], k[bi, :, h].float().cpu().numpy(),
                      v[bi, :, h].float().cpu().numpy())

    for ci_ in range(2):
        c = DmsCache(w.batch, w.kv_heads, w.group, w.head_dim, tdt, num_pages=w.units * 140,
                     max_pages_per_unit=140, window=w.window, device=gpu)
        for ci, start in enumerate(range(0, w.context, w.prompt_chunk)):
            n = min(w.prompt_chunk, w.context - start)
            k, v, logit = wl.prompt_chunk_inputs(w, ci, n, device=gpu, rates=rates)
            c.append(k, v, logit)
            c.compact()
            if ci_ == 0:
                feed(k, v, logit)
                for uc in mirror.values():
                    uc.compact()
        caches.append(c)
    a, b = caches
    scale = scale_of(w.head_dim)
    worst = 0.0
    for step in range(20):
        q, k, v, logit = wl.decode_step_inputs(w, step, device=gpu, rates=rates)
        feed(k, v, logit)
        a.append(k, v, logit)
        oa = a.decode(q)
        ob = b.step(k, v, logit, q)
        _agree(oa, ob, False, f"step {step}")
        if step in (0, 7, 15, 16, 19):
            ref = {u: uc.attend(q[u // w.kv_heads, (u % w.kv_heads) * w.group:
                                  (u % w.kv_heads + 1) * w.group].double().cpu().numpy(), scale)
                   for u, uc in mirror.items()}
            worst = max(worst, compare_outputs(ob.cpu(), ref, w.kv_heads, w.group, tdt,
                                               what=f"step {step} (fill path vs oracle)"))
        if (step + 1) % 16 == 0:
            a.compact()
            b.compact()
            for uc in mirror.values():
                uc.compact()
    torch.cuda.synchronize()
    say(f"full-size fill path vs oracle: max abs err {worst:.2e} over {len(sample)} units")
    assert b.status_word() == 0
    _same_state(a, b, range(0, w.units, 61))


def test_repeated_fill_leaves_the_step_state(gpu):
    """bench.py times the decode launch by repeating dms_decode_attn_fill after
    one reserve: a repeated fill serves the same reserved token again (the same
    slots streamed, the token's slot rewritten with the same bytes), so the
    cache ends as after the one step and every repeat gives the same output."""
    w = _workload(4, 8, 4, 128, "bf16", 300, 0.875, 8601)
    a, b, rates = _twins(w, gpu)
    scale = scale_of(w.head_dim)
    for step in range(3):
        q, k, v, logit = wl.decode_step_inputs(w, step, rates=rates)
        q, k, v, logit = q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu)
        oa = a.step(k, v, logit, q)
        b.reserve()
        outs = [b.fill_and_decode(k, v, logit, q, torch.empty_like(oa), scale) for _ in range(4)]
        for i, ob in enumerate(outs):
            assert torch.equal(oa, ob), f"step {step}, fill {i}: outputs differ"
        _same_state(a, b, range(w.units))
        assert torch.equal(a.append_base.cpu(), b.append_base.cpu())
    assert b.status_word() == 0
