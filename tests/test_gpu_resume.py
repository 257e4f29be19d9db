"""Checkpoint/resume and guard canaries for the cache calls, through the C ABI.

Checkpoint: the library keeps no state of its own, so the cache tensors are the
whole state.  A cache saved after k steps (torch.save of CPU copies, loaded
back with weights_only=True) and restored into a fresh DmsCache must continue
with outputs bitwise equal to the cache that was never interrupted, and with
the same retained sets, K/V bytes and page counts.  Page ids may differ: pages
freed by a compaction go back to the free stack in whatever order the
workgroups finish.

Canaries: every caller-owned buffer (the cache state, the outputs, the
workspaces) is a view into a larger allocation whose head and tail are filled
with a byte pattern.  After a run of every call that writes, each pattern must
be intact: no kernel writes outside the rows its arguments give it.
"""

import dataclasses
import io
import math

import pytest
import torch

import workloads as wl
from decode_attention_learned_amd import DmsCache, lib, prefill
from decode_attention_learned_amd.cache import PAGE, _DTYPES, _stream
from harness import say

pytestmark = pytest.mark.gpu

BASE = dataclasses.replace(wl.get("llama1b_cr4"), name="resume_case", batch=3, kv_heads=2, group=4,
                           head_dim=128, context=700, steps=48, prompt_chunk=700, replicas=1,
                           seed=6100)


def _cache(gpu, w, maxp=24):
    return DmsCache(w.batch, w.kv_heads, w.group, w.head_dim, torch.bfloat16,
                    max_pages_per_unit=maxp, window=w.window, device=gpu)


def _prompt(cache, w, gpu):
    k, v, logit = wl.prompt_chunk_inputs(w, 0, w.context)
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    cache.compact()


def _step(cache, w, step, gpu):
    """Decode step `step`: the one-launch form on even steps, append + decode on odd."""
    q, k, v, logit = (t.to(gpu) for t in wl.decode_step_inputs(w, step))
    if step % 2 == 0:
        out = cache.step(k, v, logit, q)
    else:
        cache.append(k, v, logit)
        out = cache.decode(q)
    if (step + 1) % w.compact_every == 0:
        cache.compact()
    return out


def _chunk(cache, w, n, gpu):
    """Append a chunk of n tokens and attend its queries."""
    g = torch.Generator().manual_seed(w.seed + 77)
    kshape = (w.batch, n, w.kv_heads, w.head_dim)
    k = torch.randn(kshape, generator=g).to(torch.bfloat16).to(gpu)
    v = torch.randn(kshape, generator=g).to(torch.bfloat16).to(gpu)
    logit = (torch.randn(kshape[:3], generator=g) * 2).to(gpu)
    q = torch.randn((w.batch, n, w.q_heads, w.head_dim), generator=g).to(torch.bfloat16).to(gpu)
    cache.append(k, v, logit)
    return cache.decode_chunk(q)


def _content(cache):
    count, pos, alpha, k, v = cache.export(all_slots=True)
    return (count.cpu(), pos.cpu(), alpha.cpu(), k.cpu(), v.cpu(), cache.seq_len.cpu(),
            cache.n_slots.cpu(), cache.n_clean.cpu(), cache.pages_in_use())


def _same_content(a, b):
    for x, y in zip(a[:-1], b[:-1]):
        assert torch.equal(x, y)
    assert a[-1] == b[-1]


@pytest.mark.parametrize("at_step", [0, 21])
def test_resume_from_checkpoint_is_bitwise_equal(gpu, at_step):
    w = BASE
    say(f"resume case: checkpoint after step {at_step}")
    a = _cache(gpu, w)
    _prompt(a, w, gpu)
    for step in range(at_step):
        _step(a, w, step, gpu)
    torch.cuda.synchronize()
    buf = io.BytesIO()
    torch.save({n: t.cpu() for n, t in a.state_dict().items()}, buf)
    buf.seek(0)
    saved = torch.load(buf, weights_only=True)

    b = _cache(gpu, w)
    b.load_state_dict({n: t.to(gpu) for n, t in saved.items()})
    _same_content(_content(a), _content(b))
    for step in range(at_step, w.steps):
        oa = _step(a, w, step, gpu)
        ob = _step(b, w, step, gpu)
        assert torch.equal(oa, ob), f"step {step}: resumed output differs"
    ca = _chunk(a, w, 40, gpu)
    cb = _chunk(b, w, 40, gpu)
    assert torch.equal(ca, cb), "chunk queries differ after resume"
    a.compact()
    b.compact()
    assert a.status_word() == 0 and b.status_word() == 0
    _same_content(_content(a), _content(b))


def test_checkpoint_of_another_shape_is_refused(gpu):
    a = _cache(gpu, BASE)
    other = _cache(gpu, dataclasses.replace(BASE, batch=2))
    with pytest.raises(ValueError, match="checkpoint field"):
        a.load_state_dict(other.state_dict())


# -- canaries --------------------------------------------------------------------------------
PAD = 4096          # bytes of pattern on each side (keeps every view 256-byte aligned)
PATTERN = 0xA5


class Guarded:
    """Views into pattern-filled allocations; check() asserts every pattern intact."""

    def __init__(self, gpu):
        self.gpu = gpu
        self.raws = []

    def like(self, t: torch.Tensor) -> torch.Tensor:
        nbytes = t.numel() * t.element_size()
        raw = torch.full((PAD + nbytes + PAD,), PATTERN, dtype=torch.uint8, device=self.gpu)
        view = raw[PAD:PAD + nbytes].view(t.dtype).view(t.shape)
        view.copy_(t)
        self.raws.append((raw, nbytes, tuple(t.shape)))
        return view

    def new(self, shape, dtype, fill=0):
        return self.like(torch.full(shape, fill, dtype=dtype, device=self.gpu))

    def check(self):
        torch.cuda.synchronize()
        for raw, nbytes, shape in self.raws:
            head = raw[:PAD]
            tail = raw[PAD + nbytes:]
            bad_h = int((head != PATTERN).sum())
            bad_t = int((tail != PATTERN).sum())
            assert bad_h == 0 and bad_t == 0, \
                f"buffer of shape {shape}: {bad_h} head and {bad_t} tail pattern bytes overwritten"


def test_no_call_writes_outside_its_buffers(gpu):
    w = BASE
    say("canary case: every writing call over guarded buffers")
    gd = Guarded(gpu)
    cache = _cache(gpu, w, maxp=28)
    for n in DmsCache.STATE:
        setattr(cache, n, gd.like(getattr(cache, n)))
    cache._bind()
    cache.workspace = gd.like(cache.workspace)
    cache.reset()
    _prompt(cache, w, gpu)
    out = gd.new((w.batch, w.q_heads, w.head_dim), torch.float32)
    for step in range(20):
        q, k, v, logit = (t.to(gpu) for t in wl.decode_step_inputs(w, step))
        if step % 2:
            cache.step(k, v, logit, q, out=out)
        else:
            cache.append(k, v, logit)
            cache.decode(q, out=out)
        if step == 15:
            cache.compact()
    # chunk queries: a grid this small splits its tiles over the chip (partials in _multi_ws)
    n = 64
    cache._multi_ws = gd.new((max(lib.decode_multi_split_workspace_bytes(cache.shape, n), 1),),
                             torch.uint8)
    chunk_out = gd.new((w.batch, n, w.q_heads, w.head_dim), torch.float32)
    g = torch.Generator().manual_seed(5)
    kshape = (w.batch, n, w.kv_heads, w.head_dim)
    cache.append(torch.randn(kshape, generator=g).to(torch.bfloat16).to(gpu),
                 torch.randn(kshape, generator=g).to(torch.bfloat16).to(gpu),
                 torch.randn(kshape[:3], generator=g).to(gpu))
    q = torch.randn((w.batch, n, w.q_heads, w.head_dim), generator=g).to(torch.bfloat16).to(gpu)
    cache.decode_chunk(q, out=chunk_out)
    cache.compact()
    # prompt sharing, release, the no-alloc decode
    cache.release(1, 2)
    cache.share_prefix(0, 1, 2)
    q1 = wl.decode_step_inputs(w, 99)[0].to(gpu)
    cache.decode(q1, out=out)
    rc = lib.dms_decode_attn_noalloc(cache.shape, cache.cache, q1, out,
                                     1.0 / math.sqrt(w.head_dim), _stream())
    lib.check("dms_decode_attn_noalloc", rc)
    # export into guarded rows
    m = int(cache.n_slots.max().item())
    units = cache.units
    count = gd.new((units,), torch.int32)
    pos = gd.new((units, m), torch.int32)
    alpha = gd.new((units, m), torch.uint8)
    ek = gd.new((units, m, w.head_dim), torch.bfloat16)
    ev = gd.new((units, m, w.head_dim), torch.bfloat16)
    lib.check("dms_export_retained", lib.dms_export_retained(
        cache.shape, cache.cache, 1, m, count, pos, alpha, ek, ev, _stream()))
    assert cache.status_word() == 0
    gd.check()


@pytest.mark.parametrize("method", ["dense", "gathered", "relaxed"])
def test_prefill_writes_only_its_output(gpu, method):
    w = dataclasses.replace(wl.get("prefill_8k"), batch=2, kv_heads=2, context=333, seed=6200)
    say(f"canary case: prefill {method} S={w.context}")
    q, k, v, logit = (t.to(gpu) for t in wl.prefill_inputs(w))
    gd = Guarded(gpu)
    shape = lib.DmsShape(w.batch, w.kv_heads, w.group, w.head_dim, PAGE, w.window, 1, 1,
                         _DTYPES[torch.bfloat16])
    if method == "gathered":
        nbytes = lib.prefill_gathered_workspace_bytes(shape, w.context)
    else:
        nbytes = lib.prefill_workspace_bytes(shape, w.context)
    ws = gd.new((max(nbytes, 1),), torch.uint8)
    out = gd.new(tuple(q.shape), torch.float32)
    noise = torch.zeros_like(logit) if method == "relaxed" else None
    prefill(q, k, v, logit, window=w.window, out=out, workspace=ws, method=method, noise=noise)
    gd.check()
