"""GPU parity of chunk queries (dms_decode_attn_multi) against the float64 oracle.

A chunk of C tokens is appended to a cache that already holds a compacted
prompt; query c of the chunk (position t0 + c) must equal the oracle's decode
step at t0 + c over the whole token history, i.e. it sees the chunk's earlier
tokens, not its later ones, and marked keys still inside their window.
Tolerance |o - o_ref| <= 2e-2 + 2e-2 |o_ref| (bf16 inputs, fp32 accumulation).
"""

import math

import numpy as np
import pytest
import torch

import workloads as wl
from decode_attention_learned_amd import DmsCache
from harness import BF16_TOL, say
from oracle import dms_oracle as orc

pytestmark = pytest.mark.gpu


def _tokens(b, hkv, g, d, total, rate, seed):
    w = wl.Workload(name="chunk_case", kind="prefill", batch=b, kv_heads=hkv, group=g, head_dim=d,
                    dtype="bf16", context=total, evict_rate=rate, seed=seed)
    return wl.prefill_inputs(w)          # q [B, T, Hq, D], k, v [B, T, Hkv, D], logit [B, T, Hkv]


def _run(gpu, b, hkv, g, d, prompt, chunks, rate, seed, window=16, compact_between=False, pages=None):
    total = prompt + sum(chunks)
    q, k, v, logit = _tokens(b, hkv, g, d, total, rate, seed)
    maxp = pages or (total + 63) // 64 + 1
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, max_pages_per_unit=maxp, window=window, device=gpu)
    if prompt:
        cache.append(k[:, :prompt].contiguous().to(gpu), v[:, :prompt].contiguous().to(gpu),
                     logit[:, :prompt].contiguous().to(gpu))
        cache.compact()
    alpha = orc.eviction_decisions(logit.numpy())           # [B, T, Hkv]
    scale = 1.0 / math.sqrt(d)
    t0 = prompt
    worst = 0.0
    for n in chunks:
        sl = slice(t0, t0 + n)
        cache.append(k[:, sl].contiguous().to(gpu), v[:, sl].contiguous().to(gpu),
                     logit[:, sl].contiguous().to(gpu))
        out = cache.decode_chunk(q[:, sl].contiguous().to(gpu)).cpu().double().numpy()
        assert cache.status_word() == 0
        for bi in range(b):
            for h in range(hkv):
                kh = k[bi, :, h].float().numpy()
                vh = v[bi, :, h].float().numpy()
                for c in range(n):
                    t = t0 + c
                    ref = orc.decode_output(q[bi, t, h * g:(h + 1) * g].float().numpy(), kh, vh,
                                            alpha[bi, :, h], t, window, scale)
                    got = out[bi, c, h * g:(h + 1) * g]
                    err = np.abs(got - ref)
                    worst = max(worst, float(err.max()))
                    assert np.all(err <= BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref)), \
                        f"chunk at {t0}, query {c}, seq {bi}, head {h}: max err {err.max():.3g}"
        if compact_between:
            cache.compact()
        t0 += n
    return worst


@pytest.mark.parametrize("chunk", [1, 2, 3, 4, 7, 16, 33])
def test_chunk_queries(gpu, chunk):
    worst = _run(gpu, 2, 2, 4, 128, 300, [chunk], 0.6, 6100 + chunk)
    say(f"chunk {chunk}: max err {worst:.2e}")


@pytest.mark.parametrize("g,d", [(1, 128), (5, 128), (8, 64), (16, 64)])
def test_chunk_group_sizes(gpu, g, d):
    """16 / G queries per launch: one (G=16), two (G=8, C=3), several (G=1, C=20)."""
    _run(gpu, 1, 2, g, d, 200, [20 if g == 1 else 3], 0.75, 6200 + g)


def test_chunks_in_sequence_with_compaction(gpu):
    """Several chunks, compacting after each (never before its queries)."""
    _run(gpu, 2, 2, 4, 128, 130, [5, 16, 1, 40], 0.8, 6301, compact_between=True)


def test_chunk_on_empty_cache(gpu):
    """A first chunk of 40 tokens with no prompt: the chunk's own keys only,
    the earliest queries seeing a single key."""
    _run(gpu, 2, 2, 4, 128, 0, [40], 0.5, 6401)


@pytest.mark.parametrize("window", [1, 16, 40])
def test_chunk_windows(gpu, window):
    """Marked keys leaving the window inside the chunk: query c sees a marked
    key j iff t0 + c - j < w, so successive queries of one chunk differ."""
    _run(gpu, 1, 2, 4, 128, 100, [24], 0.9, 6500 + window, window=window)


def test_chunk_split_k(gpu):
    """Long retained lists (8192-token prompt, nothing marked): the split-K
    plan cuts every unit into several chunks and the merge runs per query."""
    _run(gpu, 2, 2, 4, 128, 8192, [6], 0.0, 6601)


def test_single_query_chunk_equals_decode(gpu):
    """C = 1 through the chunk entry point equals dms_decode_attn bit for bit
    (same kernel, one column group)."""
    b, hkv, g, d = 2, 2, 4, 128
    q, k, v, logit = _tokens(b, hkv, g, d, 301, 0.6, 6701)
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, max_pages_per_unit=8, device=gpu)
    cache.append(k[:, :300].contiguous().to(gpu), v[:, :300].contiguous().to(gpu),
                 logit[:, :300].contiguous().to(gpu))
    cache.compact()
    cache.append(k[:, 300:].contiguous().to(gpu), v[:, 300:].contiguous().to(gpu),
                 logit[:, 300:].contiguous().to(gpu))
    a = cache.decode(q[:, 300].contiguous().to(gpu))
    m = cache.decode_chunk(q[:, 300:].contiguous().to(gpu))
    assert torch.equal(a, m[:, 0])


@pytest.mark.parametrize("chunk", [32, 64, 129])
def test_long_chunks_tiled_kernel(gpu, chunk):
    """Chunks of 32 queries or more run the tiled chunk kernel (32 queries per
    workgroup, cache tiles straight from the pages): ragged query blocks."""
    worst = _run(gpu, 2, 2, 4, 128, 1000, [chunk], 0.75, 6800 + chunk)
    say(f"tiled chunk {chunk}: max err {worst:.2e}")


def test_long_chunk_after_steps_with_dead_tail(gpu):
    """A chunk on a cache whose tail holds dead, not yet compacted slots and a
    clean prefix that is not a whole number of tiles."""
    _run(gpu, 2, 2, 4, 128, 517, [7, 9, 48], 0.9, 6901)


def test_long_chunk_group_five(gpu):
    """G = 5: the second head group of a workgroup has one active wave."""
    _run(gpu, 1, 2, 5, 128, 300, [40], 0.7, 7001)


def test_prefill_sized_chunk(gpu):
    """A 512-token chunk into a 2048-token cache (chunked prefill)."""
    worst = _run(gpu, 1, 2, 4, 128, 2048, [512], 0.875, 7101)
    say(f"512-token chunk: max err {worst:.2e}")
