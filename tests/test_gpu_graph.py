"""The calls under HIP graph capture, through the C ABI.

No call allocates, synchronises or clears memory with a memset, so a decode
step (dms_append_reserve + dms_decode_attn_fill, with a dms_compact every few
steps) and a prefill call can be captured once and replayed.  Each test runs
a captured cache beside an eager twin fed the same inputs: every replay's
output must equal the eager call's bitwise (same kernels, same data), with
eager work and synchronisations between the replays, and the two caches
must end with the same retained sets, K/V bytes and page counts.
"""

import dataclasses
import math

import pytest
import torch

import workloads as wl
from decode_attention_learned_amd import DmsCache, lib, prefill
from decode_attention_learned_amd.cache import PAGE, _DTYPES
from harness import say

pytestmark = pytest.mark.gpu


def _content(cache):
    count, pos, alpha, k, v = cache.export(all_slots=True)
    return [count.cpu(), pos.cpu(), alpha.cpu(), k.cpu(), v.cpu(), cache.seq_len.cpu(),
            cache.n_slots.cpu(), cache.n_clean.cpu()]


@pytest.mark.parametrize("name,batch", [("llama1b_cr4", 4), ("qwen3_8b_cr8", 2), ("qwen3_8b_cr8_f32", 2)])
def test_decode_step_graph_replays_match_eager(gpu, name, batch):
    w = dataclasses.replace(wl.get(name), batch=batch, context=1500, prompt_chunk=1500, replicas=1)
    say(f"graph case: {name} B={batch} context {w.context}")
    steps, every = 24, 4
    maxp = (w.context + steps) // 64 + 3
    dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    caches = [DmsCache(w.batch, w.kv_heads, w.group, w.head_dim, dtype,
                       max_pages_per_unit=maxp, window=w.window, device=gpu) for _ in range(2)]
    k, v, logit = (t.to(gpu) for t in wl.prompt_chunk_inputs(w, 0, w.context))
    for c in caches:
        c.append(k, v, logit)
        c.compact()
    scale = 1.0 / math.sqrt(w.head_dim)
    # static inputs and outputs of the captured step
    q0, k0, v0, l0 = (t.to(gpu) for t in wl.decode_step_inputs(w, 0))
    sq, sk, sv, sl = q0.clone(), k0.clone(), v0.clone(), l0.clone()
    sout = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=gpu)
    eout = torch.empty_like(sout)
    g_cap, eager = caches

    def step(cache, q, kk, vv, ll, out):
        cache.reserve()
        cache.fill_and_decode(kk, vv, ll, q, out, scale)

    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g_step, g_compact = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step, stream=stream):
        step(g_cap, sq, sk, sv, sl, sout)
    with torch.cuda.graph(g_compact, stream=stream):
        g_cap.compact()
    torch.cuda.synchronize()
    # capture launched nothing: the captured cache still equals its twin
    for a, b in zip(_content(g_cap), _content(eager)):
        assert torch.equal(a, b)
    for i in range(steps):
        q, kk, vv, ll = (t.to(gpu) for t in wl.decode_step_inputs(w, i))
        for dst, src in zip((sq, sk, sv, sl), (q, kk, vv, ll)):
            dst.copy_(src)
        g_step.replay()
        step(eager, q, kk, vv, ll, eout)
        if (i + 1) % every == 0:
            g_compact.replay()
            eager.compact()
        torch.cuda.synchronize()
        assert torch.equal(sout, eout), f"replay {i}: output differs from the eager step"
        assert torch.isfinite(sout).all()
    assert g_cap.status_word() == 0 and eager.status_word() == 0
    for a, b in zip(_content(g_cap), _content(eager)):
        assert torch.equal(a, b)
    assert g_cap.pages_in_use() == eager.pages_in_use()


@pytest.mark.parametrize("method", ["dense", "gathered"])
def test_prefill_graph_replays_match_eager(gpu, method):
    w = dataclasses.replace(wl.get("prefill_8k"), batch=2, context=1000, seed=6300)
    say(f"graph case: prefill {method} S={w.context}")
    q, k, v, logit = (t.to(gpu) for t in wl.prefill_inputs(w))
    sq, sk, sv, sl = q.clone(), k.clone(), v.clone(), logit.clone()
    shape = lib.DmsShape(w.batch, w.kv_heads, w.group, w.head_dim, PAGE, w.window, 1, 1,
                         _DTYPES[torch.bfloat16])
    need = (lib.prefill_gathered_workspace_bytes if method == "gathered"
            else lib.prefill_workspace_bytes)(shape, w.context)
    ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=gpu)
    out = torch.empty(tuple(q.shape), dtype=torch.float32, device=gpu)
    prefill(sq, sk, sv, sl, window=w.window, out=out, workspace=ws, method=method)  # warm
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        prefill(sq, sk, sv, sl, window=w.window, out=out, workspace=ws, method=method)
    torch.cuda.synchronize()
    for r in range(4):
        # new inputs each replay: a rescaled query and logits shifted across the threshold
        sq.copy_(q * (1 + r))
        sl.copy_(logit + 0.5 * r)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref = prefill(sq, sk, sv, sl, window=w.window, method=method)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r}: graph output differs from the eager call"
