"""GPU parity of the decode path (decide + append, compaction, split-K decode)
against the float64 oracle, through the C ABI.

Bit-exact: slot order, decisions, retained sets, compacted K/V bytes, page
accounting.  Within tolerance: attention outputs (1e-5 max-abs for float32
caches; |o - o_ref| <= 2e-2 + 2e-2 |o_ref| for bfloat16).
"""

import math

import numpy as np
import pytest
import torch

import workloads as wl
from decode_attention_learned_amd import DmsCache, lib
from harness import (F32_ATOL, HostModel, check_kv_exact, check_live_sets, check_pages,
                     check_slots_exact, compare_outputs, decode_build, export_meta, say, scale_of)
from oracle import dms_oracle as orc

pytestmark = pytest.mark.gpu


def _dtype(w):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def run_decode(w, dev, *, steps=None, compact_every="default", check_steps=None,
               max_pages=None, num_pages=None, gen_device="cpu", kv_units=None, window=None,
               prompt_chunk=None):
    """Build the prompt, then decode `steps` steps, checking against the oracle mirror.

    Returns (cache, model, list of GPU outputs checked)."""
    window = w.window if window is None else window
    steps = w.steps if steps is None else steps
    every = w.compact_every if compact_every == "default" else compact_every
    chunk = w.prompt_chunk if prompt_chunk is None else prompt_chunk
    need = (w.context + steps) // 64 + 3
    max_pages = need if max_pages is None else max_pages
    cache = DmsCache(w.batch, w.kv_heads, w.group, w.head_dim, _dtype(w),
                     num_pages=num_pages or w.units * max_pages, max_pages_per_unit=max_pages,
                     window=window, device=dev)
    model = HostModel(w.batch, w.kv_heads, w.group, w.head_dim, window)
    rates = wl.unit_eviction_rates(w)
    for ci, start in enumerate(range(0, w.context, chunk)):
        n = min(chunk, w.context - start)
        k, v, logit = wl.prompt_chunk_inputs(w, ci, n, device=gen_device, rates=rates)
        cache.append(k.to(dev), v.to(dev), logit.to(dev))
        model.append(k.cpu(), v.cpu(), logit.cpu())
        if every is not None:
            cache.compact()
            model.compact()
    torch.cuda.synchronize()
    meta = check_slots_exact(cache, model)
    check_pages(cache, meta)
    if kv_units:
        check_kv_exact(cache, model, kv_units)
    scale = scale_of(w.head_dim)
    outs = []
    for step in range(steps):
        q, k, v, logit = wl.decode_step_inputs(w, step, device=gen_device, rates=rates)
        cache.append(k.to(dev), v.to(dev), logit.to(dev))
        model.append(k.cpu(), v.cpu(), logit.cpu())
        out = cache.decode(q.to(dev))
        if check_steps is None or step in check_steps:
            ref = model.decode(q.cpu(), scale)
            compare_outputs(out.cpu(), ref, w.kv_heads, w.group, _dtype(w), what=f"step {step}")
            check_live_sets(cache, model)
            outs.append(out.clone())
        if every is not None and (step + 1) % every == 0:
            cache.compact()
            model.compact()
            meta = check_slots_exact(cache, model)
            check_pages(cache, meta)
    assert cache.status_word() == 0
    return cache, model, outs


def small(name, **kw):
    base = wl.get(name)
    d = dict(base.__dict__)
    d.update(kw)
    d.pop("extra", None)
    return wl.Workload(**d)


# ---------------------------------------------------------------- tiny float32 workload, every step
def test_tiny_f32_every_step(gpu):
    w = wl.get("tiny_f32")
    say("tiny_f32: 512-token prompt + 64 steps, fp32, G=2, D=64")
    cache, model, _ = run_decode(w, gpu, kv_units=range(w.units))
    check_kv_exact(cache, model, range(w.units))


def test_tiny_f32_first_token_is_exact(gpu):
    w = small("tiny_f32", context=0, steps=1)
    q, k, v, logit = wl.decode_step_inputs(w, 0)
    cache = DmsCache(1, 2, 2, 64, torch.float32, max_pages_per_unit=2, device=gpu)
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    out = cache.decode(q.to(gpu)).cpu()
    for h in range(2):
        for g in range(2):
            assert torch.equal(out[0, h * 2 + g], v[0, 0, h])


# ---------------------------------------------------------------- bf16 shapes, both decode kernels
@pytest.mark.parametrize("kernel", ["mfma", "generic"])
@pytest.mark.parametrize("dims", [(3, 2, 5, 128), (2, 3, 4, 64), (1, 1, 16, 128), (2, 1, 1, 64)])
def test_bf16_small_every_step(gpu, kernel, dims):
    b, hkv, g, d = dims
    w = small("qwen3_8b_cr8", batch=b, kv_heads=hkv, group=g, head_dim=d, context=301,
              steps=40, evict_rate=0.6, compact_every=7, prompt_chunk=100, seed=77 + d + g)
    say(f"bf16 {kernel} B={b} Hkv={hkv} G={g} D={d}")
    with decode_build(kernel):
        cache, model, _ = run_decode(w, gpu, kv_units=range(w.units))
        check_kv_exact(cache, model, range(w.units))


@pytest.mark.parametrize("every", [1, 16, None])
def test_compaction_schedule_does_not_change_results(gpu, every):
    w = small("llama1b_cr4", batch=2, context=700, steps=40, prompt_chunk=350, seed=2101)
    say(f"compaction every {every}")
    run_decode(w, gpu, compact_every=every)


@pytest.mark.parametrize("rate", [0.0, 1.0])
def test_all_keep_and_all_evict(gpu, rate):
    w = small("llama1b_cr4", batch=2, kv_heads=2, context=200, steps=20, evict_rate=rate,
              prompt_chunk=200, seed=2202)
    cache, model, _ = run_decode(w, gpu)
    meta = export_meta(cache)
    n = meta["n_slots"]
    if rate == 0.0:
        assert np.all(n == 220)          # nothing leaves
    else:
        assert np.all(n <= 16 + 16)      # at most the window plus uncompacted tail


def test_all_keep_matches_dense_causal_sdpa(gpu):
    """Nothing marked: GPU decode equals dense causal attention (torch SDPA on CPU, float64)."""
    b, hkv, g, d, s = 2, 2, 4, 128, 150
    w = small("llama1b_cr4", batch=b, kv_heads=hkv, group=g, head_dim=d, context=s - 1, steps=1,
              evict_rate=0.0, prompt_chunk=200, seed=2303)
    cache, _, outs = run_decode(w, gpu)
    rates = wl.unit_eviction_rates(w)
    kp, vp, _ = wl.prompt_chunk_inputs(w, 0, s - 1, rates=rates)
    q, kd, vd, _ = wl.decode_step_inputs(w, 0, rates=rates)
    keys = torch.cat([kp, kd], 1).double()       # [B, S, Hkv, D]
    vals = torch.cat([vp, vd], 1).double()
    for bi in range(b):
        kk = keys[bi].permute(1, 0, 2).repeat_interleave(g, 0)   # [Hq, S, D]
        vv = vals[bi].permute(1, 0, 2).repeat_interleave(g, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[bi].double()[:, None, :], kk, vv, scale=1 / math.sqrt(d))[:, 0]
        got = outs[0][bi].cpu().double()
        assert torch.allclose(got, ref, rtol=2e-2, atol=2e-2)


def test_window_one_sees_only_unmarked_and_itself(gpu):
    w = small("llama1b_cr4", batch=2, kv_heads=2, context=130, steps=10, evict_rate=0.7,
              prompt_chunk=130, seed=2404)
    run_decode(w, gpu, window=1)


def test_window_larger_than_history(gpu):
    w = small("llama1b_cr4", batch=1, kv_heads=2, context=20, steps=10, evict_rate=0.9,
              prompt_chunk=20, seed=2505)
    run_decode(w, gpu, window=64)


def test_determinism_bitwise(gpu):
    w = small("qwen3_8b_cr8", batch=4, context=1500, steps=3, prompt_chunk=500, seed=3303)
    _, _, a = run_decode(w, gpu)
    _, _, b = run_decode(w, gpu)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_empty_unit_gives_zeros(gpu):
    cache = DmsCache(2, 2, 2, 64, torch.bfloat16, max_pages_per_unit=2, device=gpu)
    q = torch.randn((2, 4, 64), device=gpu).to(torch.bfloat16)
    out = cache.decode(q)
    assert torch.count_nonzero(out) == 0


# ---------------------------------------------------------------- device-detected errors
def test_pool_exhaustion_then_recovery(gpu):
    """A pool too small for every unit: units past the first that does not fit are refused
    whole (status bit set, tokens dropped); after compaction frees pages, appends resume."""
    b, hkv, g, d, win = 1, 4, 2, 64, 16
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, num_pages=6, max_pages_per_unit=4, window=win,
                     device=gpu)
    model = HostModel(b, hkv, g, d, win)
    w = small("llama1b_cr4", batch=b, kv_heads=hkv, group=g, head_dim=d, evict_rate=1.0, seed=2606)
    rates = wl.unit_eviction_rates(w)
    # 100 tokens need 2 pages per unit: units 0..2 fit in 6 pages, unit 3 is refused
    k, v, logit = wl.prompt_chunk_inputs(w, 0, 100, rates=rates)
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    model.append(k, v, logit, refused={3})
    torch.cuda.synchronize()
    assert cache.status_word() & lib.DMS_STATUS_POOL_EXHAUSTED
    assert int(cache.append_base[3].item()) == -1
    meta = check_slots_exact(cache, model)
    check_pages(cache, meta)
    # everything is marked: compaction keeps the last 16 of each unit and frees a page each
    cache.compact()
    model.compact()
    meta = check_slots_exact(cache, model)
    check_pages(cache, meta)
    assert meta["free_top"] == 3
    cache.status.zero_()
    q, k, v, logit = wl.decode_step_inputs(w, 0, rates=rates)
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    model.append(k, v, logit)
    out = cache.decode(q.to(gpu))
    torch.cuda.synchronize()
    assert cache.status_word() == 0
    check_slots_exact(cache, model)
    compare_outputs(out.cpu(), model.decode(q, scale_of(d)), hkv, g, torch.bfloat16)


def test_row_overflow_sets_status(gpu):
    cache = DmsCache(1, 2, 1, 64, torch.bfloat16, num_pages=64, max_pages_per_unit=2, device=gpu)
    w = small("llama1b_cr4", batch=1, kv_heads=2, group=1, evict_rate=0.0, seed=2707)
    # a single append longer than a row is refused on the host
    k, v, logit = wl.prompt_chunk_inputs(w, 0, 129)
    with pytest.raises(lib.DmsError):
        cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    # 100 tokens fit in 2 pages; 100 more would need 4: refused on the device
    k, v, logit = wl.prompt_chunk_inputs(w, 1, 100)
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    torch.cuda.synchronize()
    assert cache.status_word() == 0
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    torch.cuda.synchronize()
    assert cache.status_word() & lib.DMS_STATUS_ROW_OVERFLOW
    assert cache.n_slots.cpu().tolist() == [100, 100]
    assert cache.seq_len.cpu().tolist() == [200]
    assert cache.append_base.cpu().tolist() == [-1, -1]
    check_pages(cache)


# ---------------------------------------------------------------- full-size workloads
def test_llama1b_cr4_full(gpu):
    """Llama-3.2-1B shape, B=16, 4096 context, 256 steps: every step checked."""
    w = wl.get("llama1b_cr4")
    say("llama1b_cr4 full size")
    cache, model, _ = run_decode(w, gpu, gen_device=gpu, check_steps=set(range(0, 256, 3)) | {255},
                                 kv_units=range(0, w.units, 17))


def test_qwen3_8b_cr8_full_sampled(gpu):
    """Qwen3-8B shape, B=64, 32768 context at CR 8: every unit at sampled steps."""
    w = wl.get("qwen3_8b_cr8")
    say("qwen3_8b_cr8 full size: building 32768-token context")
    cache, model, _ = run_decode(w, gpu, steps=17, check_steps={0, 16}, gen_device=gpu,
                                 max_pages=140, kv_units=range(0, w.units, 97))
    meta = export_meta(cache)
    cr = (w.context + 17) * w.units / meta["n_slots"].sum()
    say(f"realised compression ratio {cr:.2f}")
    assert 7.0 < cr < 9.0


def test_qwen3_8b_cr8_f32_full_sampled(gpu):
    """The same shape with float32 keys and values (the float32 matrix-core decode
    kernel at the size the bench times): every unit at sampled steps."""
    w = wl.get("qwen3_8b_cr8_f32")
    say("qwen3_8b_cr8_f32 full size: building 32768-token context")
    cache, _, _ = run_decode(w, gpu, steps=17, check_steps={0, 16}, gen_device=gpu,
                             max_pages=140, kv_units=range(0, w.units, 97))
    assert cache.k_pages.dtype == torch.float32


def test_qwen32b_width_ragged_full_sampled(gpu):
    """Qwen2.5-32B heads (G=5), per-unit Beta(7,1) rates: ragged lengths, every unit."""
    w = wl.get("qwen32b_width")
    say("qwen32b_width full size (ragged)")
    cache, _, _ = run_decode(w, gpu, steps=2, gen_device=gpu, max_pages=516,
                             num_pages=w.units * 140)
    n = cache.n_slots.cpu().numpy()
    say(f"retained per unit: min {n.min()} max {n.max()} mean {n.mean():.0f}")
    assert n.max() > 4 * n.mean() / 2


def test_qwen3_cr1_control_subset(gpu):
    """CR=1 control (nothing evicted), full shape: retained counts for all units, outputs
    for 2 sequences x 8 KV heads."""
    w = wl.get("qwen3_8b_cr1")
    say("qwen3_8b_cr1 control full size")
    dev = gpu
    max_pages = 32768 // 64 + 2
    cache = DmsCache(w.batch, w.kv_heads, w.group, w.head_dim, torch.bfloat16,
                     num_pages=w.units * max_pages, max_pages_per_unit=max_pages, device=dev)
    keep_units = list(range(16))  # sequences 0 and 1
    keys = {u: [] for u in keep_units}
    vals = {u: [] for u in keep_units}
    for ci in range(w.context // w.prompt_chunk):
        k, v, logit = wl.prompt_chunk_inputs(w, ci, w.prompt_chunk, device=dev)
        cache.append(k, v, logit)
        cache.compact()
        for u in keep_units:
            b, h = divmod(u, w.kv_heads)
            keys[u].append(k[b, :, h].float().cpu().numpy())
            vals[u].append(v[b, :, h].float().cpu().numpy())
    q, k, v, logit = wl.decode_step_inputs(w, 0, device=dev)
    cache.append(k, v, logit)
    out = cache.decode(q).cpu()
    assert np.all(cache.n_slots.cpu().numpy() == w.context + 1)
    scale = scale_of(w.head_dim)
    ref = {}
    for u in keep_units:
        b, h = divmod(u, w.kv_heads)
        kk = np.concatenate(keys[u] + [k[b, :, h].float().cpu().numpy()])
        vv = np.concatenate(vals[u] + [v[b, :, h].float().cpu().numpy()])
        qq = q[b, h * w.group:(h + 1) * w.group].double().cpu().numpy()
        ref[u] = orc.softmax_attention(qq, kk, vv, scale)
    compare_outputs(out, ref, w.kv_heads, w.group, torch.bfloat16)


@pytest.mark.parametrize("kernel", ["mfma", "generic"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_dead_uncompacted_slot_with_dominant_score_is_excluded(gpu, kernel, dtype):
    """A marked token whose key dominates every query must stop counting once it is
    `window` positions old, even while its slot is still in the cache (no compaction).
    If it leaked in, the output would be pulled to its value vector."""
    if dtype == torch.float32 and kernel == "generic":
        pytest.skip("float32 caches run the float32 matrix-core kernel in both builds")
    with decode_build(kernel):
        _dominant_dead_slot(gpu, dtype)


def _dominant_dead_slot(gpu, dtype):
    b, hkv, g, d, win = 2, 2, 3, 128, 16
    gen = torch.Generator().manual_seed(4242)
    n = 150
    q = torch.randn((b, hkv * g, d), generator=gen)
    k = torch.randn((b, n, hkv, d), generator=gen) * 0.1
    v = torch.randn((b, n, hkv, d), generator=gen)
    logit = torch.full((b, n, hkv), -1.0)
    for bi in range(b):
        for h in range(hkv):
            for j in (3, 70, 130):          # dominant, marked tokens
                k[bi, j, h] = q[bi, h * g:(h + 1) * g].mean(0) * 4
                v[bi, j, h] = 4.0
                logit[bi, j, h] = 1.0
    q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    cache = DmsCache(b, hkv, g, d, dtype, max_pages_per_unit=4, window=win, device=gpu)
    model = HostModel(b, hkv, g, d, win)
    for t in range(n):
        cache.append(k[:, t:t + 1].contiguous().to(gpu), v[:, t:t + 1].contiguous().to(gpu),
                     logit[:, t:t + 1].contiguous().to(gpu))
        model.append(k[:, t:t + 1], v[:, t:t + 1], logit[:, t:t + 1])
        if t in (10, 80, 135, 140, 149):
            out = cache.decode(q.to(gpu)).cpu()
            compare_outputs(out, model.decode(q, scale_of(d)), hkv, g, dtype, what=f"t={t}")
    assert np.all(cache.n_slots.cpu().numpy() == n)   # nothing was compacted


# ---------------------------------------------------------------- constant values (pin P8)
@pytest.mark.parametrize("kernel", ["mfma", "generic"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_constant_values_give_the_constant(gpu, kernel, dtype):
    """Every value row of a unit equal to one vector c: whatever the scores and
    the retained set, the output is c (weights sum to one).  The decode kernels
    add into the row sums exactly the weights that multiply the values (the
    matrix-core kernel: the bf16-rounded ones), so the ratio is c up to float32
    rounding: 1e-5 relative."""
    if dtype == torch.float32 and kernel == "generic":
        pytest.skip("float32 caches run the float32 matrix-core kernel in both builds")
    with decode_build(kernel):
        _constant_values(gpu, dtype)


def _constant_values(gpu, dtype):
    b, hkv, g, d = 2, 2, 4, 64
    w = small("llama1b_cr4", batch=b, kv_heads=hkv, group=g, head_dim=d, evict_rate=0.6, seed=2901)
    rates = wl.unit_eviction_rates(w)
    k, _, logit = wl.prompt_chunk_inputs(w, 0, 700, rates=rates)
    c = torch.linspace(-2.0, 2.0, d).to(dtype)
    v = c.expand(b, 700, hkv, d).contiguous()
    cache = DmsCache(b, hkv, g, d, dtype, max_pages_per_unit=14, device=gpu)
    cache.append(k.to(dtype).to(gpu), v.to(gpu), logit.to(gpu))
    cache.compact()
    q = torch.randn((b, hkv * g, d), generator=torch.Generator().manual_seed(5)).to(dtype)
    out = cache.decode(q.to(gpu)).cpu().double()
    ref = c.double().expand_as(out)
    assert torch.max(torch.abs(out - ref) / (1e-3 + ref.abs())).item() <= 1e-5


# ---------------------------------------------------------------- split plan
def _plan(cache):
    """(chunk count, chunk size C, first_chunk [units + 1], chunk_unit [count]) from the
    device plan (layout: 16 header words, first chunk per unit + 1, owning unit per chunk)."""
    p = cache.plan.cpu().numpy()
    units = cache.units
    count, C = int(p[0]), int(p[1])
    first = p[16:16 + units + 1]
    owner = p[16 + units + 1:16 + units + 1 + count]
    return count, C, first, owner


def _check_plan(cache, budget):
    """The plan covers every unit with max(1, ceil(n / C)) chunks, in unit order, within
    `budget` chunks.  Returns (chunk count, C, n_slots)."""
    n = cache.n_slots.cpu().numpy().astype(np.int64)
    count, C, first, owner = _plan(cache)
    assert C % 64 == 0 and C >= 64
    nch = np.where(n > 0, (n + C - 1) // C, 1)
    assert first[0] == 0 and np.array_equal(np.diff(first), nch), "first_chunk is the prefix sum"
    assert first[-1] == count
    assert np.array_equal(owner, np.repeat(np.arange(cache.units), nch)), "chunk -> unit map"
    assert count <= budget, f"{count} chunks over the budget {budget}"
    return count, C, n


def _plan_case(b, hkv, tokens, logit_of_unit, dev, seed, dtype=torch.bfloat16):
    """A cache of b x hkv units (G = 4, D = 128, bf16 unless `dtype`): `tokens` appended
    tokens (unit u's logits all logit_of_unit(u)), a compaction, then one more token,
    kept.  Returns (cache, q, k, v, logits) with the full token history on the host."""
    g = torch.Generator().manual_seed(seed)
    T = tokens + 1
    cache = DmsCache(b, hkv, 4, 128, dtype, max_pages_per_unit=T // 64 + 3, device=dev)
    k = torch.randn(b, T, hkv, 128, generator=g).to(dtype)
    v = torch.randn(b, T, hkv, 128, generator=g).to(dtype)
    q = torch.randn(b, 4 * hkv, 128, generator=g).to(dtype)
    lg = torch.tensor([[logit_of_unit(bi * hkv + h) for h in range(hkv)] for bi in range(b)],
                      dtype=torch.float32)[:, None, :].repeat(1, T, 1)
    lg[:, -1] = -1.0
    cache.append(k[:, :tokens].contiguous().to(dev), v[:, :tokens].contiguous().to(dev),
                 lg[:, :tokens].contiguous().to(dev))
    cache.compact()
    cache.append(k[:, tokens:].contiguous().to(dev), v[:, tokens:].contiguous().to(dev),
                 lg[:, tokens:].contiguous().to(dev))
    torch.cuda.synchronize()
    return cache, q, k, v, lg


def _check_units(out, q, k, v, lg, units, hkv):
    alpha = orc.eviction_decisions(lg.numpy())
    t = k.shape[1] - 1
    for u in units:
        bi, h = divmod(u, hkv)
        ref = orc.decode_output(q[bi, 4 * h:4 * h + 4].float().numpy(), k[bi, :, h].float().numpy(),
                                v[bi, :, h].float().numpy(), alpha[bi, :, h], t, 16, scale_of(128))
        got = out[bi, 4 * h:4 * h + 4].double().numpy()
        if k.dtype == torch.float32:
            assert np.abs(got - ref).max() <= F32_ATOL, f"unit {u}"
        else:
            assert np.all(np.abs(got - ref) <= 2e-2 + 2e-2 * np.abs(ref)), f"unit {u}"


def test_split_plan_even_units_fill_one_round(gpu):
    """512 units of equal length: one chunk per unit (no merge); 128 units of equal
    length (6000 slots): split to at most one round of 512 workgroups, chunks of at
    least 2048 slots.  Outputs against the oracle on sampled units."""
    cache, q, k, v, lg = _plan_case(64, 8, 300, lambda u: -1.0, gpu, 91)
    count, _, _ = _check_plan(cache, 512)
    assert count == 512
    _check_units(cache.decode(q.to(gpu)).cpu(), q, k, v, lg, range(0, 512, 37), 8)
    cache, q, k, v, lg = _plan_case(16, 8, 6000, lambda u: -1.0, gpu, 92)
    count, _, _ = _check_plan(cache, 512)
    assert 128 < count <= 512
    _check_units(cache.decode(q.to(gpu)).cpu(), q, k, v, lg, range(0, 128, 11), 8)


def test_split_plan_ragged_units_take_up_to_three_rounds(gpu):
    """Ragged lengths (a quarter of the units keep everything, the rest only the window):
    more than one round's worth of chunks, at most three; outputs against the oracle."""
    cache, q, k, v, lg = _plan_case(32, 8, 3000, lambda u: -1.0 if u % 4 == 0 else 1.0, gpu, 93)
    count, _, n = _check_plan(cache, 3 * 512)
    assert n.max() > 2 * n.mean()
    assert count > 512
    _check_units(cache.decode(q.to(gpu)).cpu(), q, k, v, lg, list(range(0, 256, 9)) + [1, 4], 8)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_split_plan_ragged_800_units(gpu, dtype):
    """100 sequences x 8 KV heads with ragged lengths (a quarter of the units keep
    everything): the plan takes more chunks than units (about 1200 for 800),
    which the plan buffer and the decode grid must hold, and split units merge
    inside the decode launch (the fused merge of 512 units or more).  Plan on
    the host, then outputs of every sampled unit against the oracle, and the
    merge counters left at zero for the next call; bf16 and float32 caches
    (each dtype's matrix-core kernel)."""
    cache, q, k, v, lg = _plan_case(100, 8, 3000, lambda u: -1.0 if u % 4 == 0 else 1.0, gpu, 94, dtype)
    cap = lib.plan_words(cache.shape) - 16 - (cache.units + 1) - 2 * cache.units
    count, _, n = _check_plan(cache, cap)
    assert n.max() > 2 * n.mean()
    assert count > cache.units, f"expected more chunks than units, got {count}"
    for _ in range(2):   # a second call reuses the counters the first left behind
        out = cache.decode(q.to(gpu)).cpu()
        torch.cuda.synchronize()
        _check_units(out, q, k, v, lg, list(range(0, 800, 23)) + [4, 799], 8)
    p = cache.plan.cpu().numpy()
    merge = p[16 + cache.units + 1 + cap: 16 + cache.units + 1 + cap + cache.units]
    assert np.all(merge == 0), "merge counters not reset"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_chunk_longer_than_the_staged_page_ids(gpu, dtype):
    """One unit of 70,000 retained slots among 1536 units, all others evicting
    every token: the lengths are ragged and the units as many as the ragged
    budget (3 x 512 chunks), so every unit is one chunk and the long one spans
    1095 pages, more than the 1024 page ids each matrix-core decode kernel (bf16
    and float32) stages in LDS at a time: it walks that chunk in two segments.  The long unit's
    queries are zero, so every weight is exactly 1 and its output is the mean
    of its 70,001 values to float32 rounding (pinned to 1e-4 against the
    oracle); other units are checked at the bf16 tolerance (either dtype)."""
    b, hkv, g, d = 192, 8, 2, 64
    n_long, chunk = 70000, 4096
    maxp = n_long // 64 + 4
    cache = DmsCache(b, hkv, g, d, dtype, num_pages=b * hkv * 72 + maxp, max_pages_per_unit=maxp,
                     device=gpu)
    gen = torch.Generator(device=gpu).manual_seed(7301)
    k0, v0 = [], []                 # unit 0 (sequence 0, KV head 0): every token
    tail_k, tail_v = None, None     # the last chunk, for the other units
    for start in range(0, n_long, chunk):
        n = min(chunk, n_long - start)
        k = torch.randn((b, n, hkv, d), generator=gen, device=gpu).to(dtype)
        v = torch.randn((b, n, hkv, d), generator=gen, device=gpu).to(dtype)
        logit = torch.ones((b, n, hkv), device=gpu)
        logit[0, :, 0] = -1.0
        cache.append(k, v, logit)
        cache.compact()
        k0.append(k[0, :, 0].float().cpu().numpy())
        v0.append(v[0, :, 0].float().cpu().numpy())
        tail_k, tail_v = k[:, -32:].float().cpu().numpy(), v[:, -32:].float().cpu().numpy()
    q = torch.randn((b, hkv * g, d), generator=gen, device=gpu).to(dtype)
    q[0, :g] = 0
    k = torch.randn((b, 1, hkv, d), generator=gen, device=gpu).to(dtype)
    v = torch.randn((b, 1, hkv, d), generator=gen, device=gpu).to(dtype)
    logit = torch.ones((b, 1, hkv), device=gpu)
    logit[0, :, 0] = -1.0
    cache.append(k, v, logit)
    out = cache.decode(q).cpu()
    torch.cuda.synchronize()
    assert cache.status_word() == 0
    n_slots = cache.n_slots.cpu().numpy()
    assert n_slots[0] == n_long + 1 and n_slots[1:].max() <= 16 + chunk
    plan = cache.plan.cpu().numpy()
    assert plan[0] == b * hkv, "expected one chunk per unit"
    assert plan[1] > 1024 * 64, "expected a chunk of more than 1024 pages"
    scale = 1.0 / math.sqrt(d)
    # unit 0: all 70,001 keys seen, zero queries -> the plain mean of the values
    kk = np.concatenate(k0 + [k[0, :, 0].float().cpu().numpy()])
    vv = np.concatenate(v0 + [v[0, :, 0].float().cpu().numpy()])
    ref0 = orc.decode_output(np.zeros((g, d)), kk, vv, np.zeros(n_long + 1, dtype=np.int8), n_long, 16, scale)
    err0 = float(np.abs(out[0, :g].double().numpy() - ref0).max())
    assert err0 <= 1e-4, f"long unit: max err {err0:.3g}"
    # other units: every token marked, so the last 16 (the window) are seen
    ref = {}
    t = n_long
    for u in (1, 7, 8, 777, b * hkv - 1):
        bi, h = divmod(u, hkv)
        kk = np.zeros((t + 1, d))
        vv = np.zeros((t + 1, d))
        kk[t - 32:t] = tail_k[bi, :, h]
        vv[t - 32:t] = tail_v[bi, :, h]
        kk[t] = k[bi, 0, h].float().cpu().numpy()
        vv[t] = v[bi, 0, h].float().cpu().numpy()
        ref[u] = orc.decode_output(q[bi, h * g:(h + 1) * g].float().cpu().numpy(), kk, vv,
                                   np.ones(t + 1, dtype=np.int8), t, 16, scale)
    worst = compare_outputs(out, ref, hkv, g, dtype, what="short units beside a long one")
    say(f"1095-page chunk: long unit max err {err0:.2e}; short units {worst:.2e}")
