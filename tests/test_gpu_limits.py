"""Caches at the size limits of their addressing, through the C ABI.

A pool of 270,000 pages of 64 slots x 128 dims holds 4.4 GB of bf16 keys and
as much of values: a page id above 262,143 starts beyond element 2^31 and
byte 2^32 of its pool.
The allocator hands out the top of the free stack first, so every page these
tests touch lies there.  Each call that addresses pages (append, the decode
step with its token, compaction, chunk queries, prefix sharing, export) must
give the oracle's results: a byte offset computed in 32 bits would wrap and
read or write another page.
"""

import math

import numpy as np
import pytest
import torch

import workloads as wl
from decode_attention_learned_amd import DmsCache
from harness import BF16_TOL, HostModel, check_kv_exact, check_slots_exact, compare_outputs, say
from oracle import dms_oracle as orc

pytestmark = pytest.mark.gpu

PAGES = 270_000      # > 2^31 / (64 * 128) = 262,144


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pages_beyond_two_to_the_31_elements(gpu, dtype):
    b, hkv, g, d, prompt, steps = 2, 2, 4, 128, 700, 40
    w = wl.Workload(name="limits_case", kind="decode", batch=b, kv_heads=hkv, group=g, head_dim=d,
                    dtype="f32" if dtype == torch.float32 else "bf16", context=prompt, evict_rate=0.6,
                    seed=7100, steps=steps, prompt_chunk=prompt)
    say(f"limits case: {PAGES} pages of {dtype}, pool of "
        f"{PAGES * 64 * d * (2 if dtype == torch.bfloat16 else 4) / 2**30:.1f} GiB per K and V")
    maxp = (prompt + steps) // 64 + 3
    cache = DmsCache(b, hkv, g, d, dtype, num_pages=PAGES, max_pages_per_unit=maxp, device=gpu)
    model = HostModel(b, hkv, g, d, w.window)
    rates = wl.unit_eviction_rates(w)
    k, v, logit = wl.prompt_chunk_inputs(w, 0, prompt, rates=rates)
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    model.append(k, v, logit)
    cache.compact()
    model.compact()
    pt = cache.page_table.cpu()
    used = pt[pt >= 0]
    assert int(used.min()) > 262_143, "the pages in use must lie beyond element 2^31"
    scale = 1.0 / math.sqrt(d)
    for step in range(steps):
        q, k, v, logit = wl.decode_step_inputs(w, step, rates=rates)
        if step % 2:
            out = cache.step(k.to(gpu), v.to(gpu), logit.to(gpu), q.to(gpu))
        else:
            cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
            out = cache.decode(q.to(gpu))
        model.append(k, v, logit)
        if step in (0, 17, steps - 1):
            compare_outputs(out.cpu(), model.decode(q, scale), hkv, g, dtype, what=f"step {step}")
        if step == 20:
            cache.compact()
            model.compact()
    meta = check_slots_exact(cache, model)
    check_kv_exact(cache, model, range(b * hkv))
    assert cache.status_word() == 0
    assert meta is not None


def test_chunk_queries_and_sharing_beyond_two_to_the_31_elements(gpu):
    """Chunk queries (the tiled kernel, 64 queries) and a shared prompt on pages
    beyond element 2^31, against the oracle."""
    b, hkv, g, d, prompt, n = 2, 2, 4, 128, 600, 64
    total = prompt + n
    w = wl.Workload(name="limits_chunk", kind="prefill", batch=b, kv_heads=hkv, group=g, head_dim=d,
                    dtype="bf16", context=total, evict_rate=0.6, seed=7200)
    q, k, v, logit = wl.prefill_inputs(w)
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, num_pages=PAGES,
                     max_pages_per_unit=total // 64 + 2, device=gpu)
    cache.append(k[:, :prompt].contiguous().to(gpu), v[:, :prompt].contiguous().to(gpu),
                 logit[:, :prompt].contiguous().to(gpu))
    cache.compact()
    pt = cache.page_table.cpu()
    assert int(pt[pt >= 0].min()) > 262_143
    sl = slice(prompt, total)
    cache.append(k[:, sl].contiguous().to(gpu), v[:, sl].contiguous().to(gpu),
                 logit[:, sl].contiguous().to(gpu))
    out = cache.decode_chunk(q[:, sl].contiguous().to(gpu)).cpu().double().numpy()
    assert cache.status_word() == 0
    alpha = orc.eviction_decisions(logit.numpy())
    for bi in range(b):
        for h in range(hkv):
            for c in (0, 31, 32, 63):
                t = prompt + c
                ref = orc.decode_output(q[bi, t, h * g:(h + 1) * g].float().numpy(),
                                        k[bi, :, h].float().numpy(), v[bi, :, h].float().numpy(),
                                        alpha[bi, :, h], t, 16, 1.0 / math.sqrt(d))
                got = out[bi, c, h * g:(h + 1) * g]
                assert np.all(np.abs(got - ref) <= BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref))
    # sequence 1 takes over sequence 0's prompt (shared clean pages): decoding the
    # same query gives sequence 0's output bit for bit
    cache.compact()
    cache.release(1)
    cache.share_prefix(0, 1, 1)
    qq = q[:, total - 1].contiguous()
    qq[1] = qq[0]
    o = cache.decode(qq.to(gpu)).cpu()
    assert torch.equal(o[0], o[1])
    assert cache.status_word() == 0
