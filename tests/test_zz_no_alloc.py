"""dms_decode_attn_noalloc (the decode call whose split-K partials live in the
library's static per-GPU scratch array instead of a caller's workspace)
against dms_decode_attn and the oracle, through the C ABI: two calls in a
row, the second on a smaller cache, both with split units (so the partials
and the merge use the scratch array), then again after a call on the first
cache; plus the host-side size limit."""

import math

import numpy as np
import pytest
import torch

from decode_attention_learned_amd import DmsCache, lib
from harness import compare_outputs, say
from oracle import dms_oracle as orc


def _case(dev, b, hkv, g, d, tokens, seed):
    """A bf16 cache with `tokens` tokens per unit (rate 0.6), compacted, plus one kept token."""
    gen = torch.Generator().manual_seed(seed)
    T = tokens + 1
    k = torch.randn(b, T, hkv, d, generator=gen).to(torch.bfloat16)
    v = torch.randn(b, T, hkv, d, generator=gen).to(torch.bfloat16)
    q = torch.randn(b, hkv * g, d, generator=gen).to(torch.bfloat16)
    lg = torch.randn(b, T, hkv, generator=gen) + 0.25
    lg[:, -1] = -1.0
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, max_pages_per_unit=T // 64 + 3, device=dev)
    cache.append(k[:, :tokens].contiguous().to(dev), v[:, :tokens].contiguous().to(dev),
                 lg[:, :tokens].contiguous().to(dev))
    cache.compact()
    cache.append(k[:, tokens:].contiguous().to(dev), v[:, tokens:].contiguous().to(dev),
                 lg[:, tokens:].contiguous().to(dev))
    torch.cuda.synchronize()
    return cache, q, k, v, lg


def _noalloc(cache, q, stream=None):
    """One call on `stream` (torch's current stream when None; the default
    stream is the null stream, whose device is the current one; a stream of
    its own makes the library take the device from the stream)."""
    out = torch.full((cache.batch, cache.kv_heads * cache.group, cache.head_dim), float("nan"),
                     device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream()
    if stream is not None:
        s.wait_stream(torch.cuda.current_stream())
    rc = lib.dms_decode_attn_noalloc(cache.shape, cache.cache, q, out, 1.0 / math.sqrt(cache.head_dim),
                                     s.cuda_stream)
    lib.check("dms_decode_attn_noalloc", rc)
    if stream is not None:
        torch.cuda.current_stream().wait_stream(s)
    return out


def _oracle(q, k, v, lg, hkv, g, d):
    alpha = orc.eviction_decisions(lg.numpy())
    t = k.shape[1] - 1
    ref = {}
    for u in range(k.shape[0] * hkv):
        bi, h = divmod(u, hkv)
        ref[u] = orc.decode_output(q[bi, h * g:(h + 1) * g].float().numpy(), k[bi, :, h].float().numpy(),
                                   v[bi, :, h].float().numpy(), alpha[bi, :, h], t, 16, 1 / math.sqrt(d))
    return ref


@pytest.mark.gpu
def test_noalloc_decode_equals_decode_twice_then_smaller(gpu):
    # 64 units, then 8, each long enough (about 4800 and 2400 retained slots) that the
    # plan splits even lengths (chunks of at least 2048 slots)
    cases = [(8, 8, 4, 128, 12000, 9701), (2, 4, 5, 64, 6000, 9702)]
    built = [_case(gpu, *c) for c in cases]
    for (cache, q, k, v, lg), (b, hkv, g, d, _, _) in zip(built + built[:1], cases + cases[:1]):
        assert int(cache.plan[0].item()) > cache.units, "expected split units (merge path)"
        qd = q.to(gpu)
        ref_out = cache.decode(qd)
        out = _noalloc(cache, qd)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "dms_decode_attn_noalloc differs from dms_decode_attn"
        worst = compare_outputs(out.cpu(), _oracle(q, k, v, lg, hkv, g, d), hkv, g, torch.bfloat16,
                                what=f"noalloc B={b} Hkv={hkv}")
        say(f"noalloc B={b} Hkv={hkv} G={g} D={d}: identical to dms_decode_attn, "
            f"max err vs oracle {worst:.2e}")
        assert cache.status_word() == 0


@pytest.mark.gpu
def test_noalloc_on_a_stream_of_its_own(gpu):
    """The same call issued on a non-default stream gives the same outputs."""
    cache, q, k, v, lg = _case(gpu, 4, 8, 4, 128, 2000, 9703)
    qd = q.to(gpu)
    ref_out = cache.decode(qd)
    side = torch.cuda.Stream(device=gpu)
    out = _noalloc(cache, qd, stream=side)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "dms_decode_attn_noalloc on a side stream differs"
    assert cache.status_word() == 0


def test_noalloc_rejects_shapes_beyond_the_scratch_size():
    """Host-side: a shape whose partials exceed the static array is refused
    before anything is enqueued (no GPU needed)."""
    import ctypes
    L = lib.load()
    full = lib.DmsCacheStruct(*([0x1000] * 14))
    fake = ctypes.c_void_p(0x1000)
    fits = lib.DmsShape(1, 2016, 16, 128, 64, 16, 8, 64, lib.DMS_KV_BF16)
    over = lib.DmsShape(1, 2017, 16, 128, 64, 16, 8, 64, lib.DMS_KV_BF16)
    assert lib.decode_workspace_bytes(fits) <= lib.DMS_NOALLOC_SCRATCH_BYTES < lib.decode_workspace_bytes(over)
    assert L.dms_decode_attn_noalloc(ctypes.byref(over), ctypes.byref(full), fake, fake, 0.1, None) \
        == lib.DMS_ESCRATCH
    assert L.dms_decode_attn_noalloc(ctypes.byref(fits), ctypes.byref(full), None, fake, 0.1, None) \
        == lib.DMS_EINVAL
    assert L.dms_decode_attn_noalloc(ctypes.byref(fits), ctypes.byref(full), fake, fake, 0.0, None) \
        == lib.DMS_EINVAL
    assert "scratch" in lib.strerror(lib.DMS_ESCRATCH)
