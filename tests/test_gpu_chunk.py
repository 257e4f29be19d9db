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


@pytest.mark.parametrize("chunk", [4, 40])
def test_compaction_between_append_and_chunk_queries_is_flagged(gpu, chunk):
    """A compaction after the chunk was appended may have dropped keys that its
    earlier queries still see (and moves chunk tokens into the clean prefix):
    both chunk kernels (split-K for 4 queries, tiled for 40) flag
    DMS_STATUS_CHUNK_INVALID; the same chunk queried before compacting is not
    flagged, and neither is the next chunk after the compaction."""
    from decode_attention_learned_amd import lib
    b, hkv, g, d = 2, 2, 4, 128
    q, k, v, logit = _tokens(b, hkv, g, d, 200 + 2 * chunk, 0.8, 7201 + chunk)
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, max_pages_per_unit=8, device=gpu)
    cache.append(k[:, :200].contiguous().to(gpu), v[:, :200].contiguous().to(gpu),
                 logit[:, :200].contiguous().to(gpu))
    cache.compact()
    sl = slice(200, 200 + chunk)
    cache.append(k[:, sl].contiguous().to(gpu), v[:, sl].contiguous().to(gpu),
                 logit[:, sl].contiguous().to(gpu))
    cache.decode_chunk(q[:, sl].contiguous().to(gpu))
    torch.cuda.synchronize()
    assert cache.status_word() == 0
    cache.compact()
    cache.decode_chunk(q[:, sl].contiguous().to(gpu))
    torch.cuda.synchronize()
    assert cache.status_word() == lib.DMS_STATUS_CHUNK_INVALID
    cache.status.zero_()
    sl = slice(200 + chunk, 200 + 2 * chunk)
    cache.append(k[:, sl].contiguous().to(gpu), v[:, sl].contiguous().to(gpu),
                 logit[:, sl].contiguous().to(gpu))
    cache.decode_chunk(q[:, sl].contiguous().to(gpu))
    torch.cuda.synchronize()
    assert cache.status_word() == 0


@pytest.mark.parametrize("chunk", [5, 33])
def test_chunk_longer_than_the_sequence_is_flagged(gpu, chunk):
    from decode_attention_learned_amd import lib
    b, hkv, g, d = 1, 2, 4, 128
    q, k, v, logit = _tokens(b, hkv, g, d, chunk, 0.5, 7301 + chunk)
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, max_pages_per_unit=4, device=gpu)
    cache.append(k[:, :3].contiguous().to(gpu), v[:, :3].contiguous().to(gpu),
                 logit[:, :3].contiguous().to(gpu))
    cache.decode_chunk(q.contiguous().to(gpu))
    torch.cuda.synchronize()
    assert cache.status_word() == lib.DMS_STATUS_CHUNK_INVALID


@pytest.mark.parametrize("chunk", [32, 70])
def test_long_chunks_tiled_kernel_head_dim_64(gpu, chunk):
    """The tiled chunk kernel at head_dim 64 (Llama-3.2-1B heads)."""
    worst = _run(gpu, 2, 2, 4, 64, 700, [chunk], 0.75, 7400 + chunk)
    say(f"tiled chunk D=64 {chunk}: max err {worst:.2e}")


@pytest.mark.parametrize("chunks,d,g", [([1, 3], 64, 2), ([40], 64, 2), ([5, 17], 128, 2),
                                         ([7, 13], 128, 5), ([4, 9], 64, 16), ([31], 128, 4)])
def test_chunk_queries_float32_cache(gpu, chunks, d, g):
    """float32 caches: chunks shorter than 32 queries through the float32 split-K
    decode kernel, in launches of 16 / G queries (G = 5 leaves a partial last
    launch, G = 16 one query per launch), against the oracle at the float32
    tolerance (1e-5 max abs), with compaction between chunks."""
    from harness import F32_ATOL
    b, hkv, prompt, window = 1, 2, 300, 16
    total = prompt + sum(chunks)
    w = wl.Workload(name="chunk_f32", kind="prefill", batch=b, kv_heads=hkv, group=g, head_dim=d,
                    dtype="f32", context=total, evict_rate=0.5, seed=7500 + d + len(chunks))
    q, k, v, logit = wl.prefill_inputs(w)
    cache = DmsCache(b, hkv, g, d, torch.float32, max_pages_per_unit=(total + 63) // 64 + 1,
                     window=window, device=gpu)
    cache.append(k[:, :prompt].contiguous().to(gpu), v[:, :prompt].contiguous().to(gpu),
                 logit[:, :prompt].contiguous().to(gpu))
    cache.compact()
    alpha = orc.eviction_decisions(logit.numpy())
    scale = 1.0 / math.sqrt(d)
    t0, worst = prompt, 0.0
    for n in chunks:
        sl = slice(t0, t0 + n)
        cache.append(k[:, sl].contiguous().to(gpu), v[:, sl].contiguous().to(gpu),
                     logit[:, sl].contiguous().to(gpu))
        out = cache.decode_chunk(q[:, sl].contiguous().to(gpu)).cpu().double().numpy()
        assert cache.status_word() == 0
        for h in range(hkv):
            for c in range(n):
                ref = orc.decode_output(q[0, t0 + c, h * g:(h + 1) * g].double().numpy(),
                                        k[0, :, h].double().numpy(), v[0, :, h].double().numpy(),
                                        alpha[0, :, h], t0 + c, window, scale)
                err = np.abs(out[0, c, h * g:(h + 1) * g] - ref).max()
                worst = max(worst, float(err))
                assert err <= F32_ATOL, f"chunk at {t0}, query {c}, head {h}: {err:.3g}"
        cache.compact()
        t0 += n
    say(f"float32 chunk queries {chunks} D={d} G={g}: max abs err {worst:.2e}")


def test_float32_chunk_compacted_after_append_is_flagged(gpu):
    from decode_attention_learned_amd import lib
    w = wl.Workload(name="chunk_f32_flag", kind="prefill", batch=1, kv_heads=2, group=2, head_dim=64,
                    dtype="f32", context=120, evict_rate=0.8, seed=7601)
    q, k, v, logit = wl.prefill_inputs(w)
    cache = DmsCache(1, 2, 2, 64, torch.float32, max_pages_per_unit=4, device=gpu)
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    cache.compact()
    cache.decode_chunk(q[:, 112:].contiguous().to(gpu))
    torch.cuda.synchronize()
    assert cache.status_word() == lib.DMS_STATUS_CHUNK_INVALID


@pytest.mark.parametrize("zero_q", [True, False])
def test_chunk_split_and_one_pass_agree(gpu, zero_q):
    """Split-K of the tiled chunk kernel against its one-pass form and the
    oracle: one sequence, 8 KV heads x G=4, D=128, a compacted 2000-token
    prompt, then a 256-token chunk.  8 x 8 = 64 tiled workgroups, so the
    library splits each four ways when the workspace allows (DmsCache sizes
    it so) and runs one pass with the minimal workspace.
    With zero queries every score is 0 and every weight exactly 1 in both
    paths, so each output is the mean of the visible values to float32
    rounding: both forms and the oracle agree to 1e-5, and a tile missed or
    read twice by a split would show.  With random queries the weights enter
    the PV product in bf16 (2^-9 relative), rounded against different
    references in the two forms, so they agree to a few 1e-3 and each meets
    the bf16 tolerance against the oracle."""
    from decode_attention_learned_amd import lib
    b, hkv, g, d, prompt, n = 1, 8, 4, 128, 2000, 256
    q, k, v, logit = _tokens(b, hkv, g, d, prompt + n, 0.75, 6301)
    if zero_q:
        q = torch.zeros_like(q)
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, max_pages_per_unit=(prompt + n) // 64 + 2, device=gpu)
    cache.append(k[:, :prompt].contiguous().to(gpu), v[:, :prompt].contiguous().to(gpu),
                 logit[:, :prompt].contiguous().to(gpu))
    cache.compact()
    sl = slice(prompt, prompt + n)
    cache.append(k[:, sl].contiguous().to(gpu), v[:, sl].contiguous().to(gpu), logit[:, sl].contiguous().to(gpu))
    qc = q[:, sl].contiguous().to(gpu)
    assert lib.decode_multi_split_workspace_bytes(cache.shape, n) > lib.decode_multi_workspace_bytes(cache.shape)
    split = cache.decode_chunk(qc)
    one = torch.empty_like(split)
    small = torch.empty((lib.decode_multi_workspace_bytes(cache.shape),), dtype=torch.uint8, device=gpu)
    lib.check("dms_decode_attn_multi", lib.dms_decode_attn_multi(
        cache.shape, cache.cache, qc, n, one, 1.0 / math.sqrt(d), small, small.numel(),
        torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert cache.status_word() == 0
    gap = float((split - one).abs().max())
    assert gap <= (1e-5 if zero_q else 4e-3), f"split and one-pass outputs differ by {gap:.3g}"
    alpha = orc.eviction_decisions(logit.numpy())
    worst = 0.0
    for h in range(hkv):
        kh, vh = k[0, :, h].float().numpy(), v[0, :, h].float().numpy()
        for c in (0, 1, 31, 32, 100, 255):
            t = prompt + c
            ref = orc.decode_output(q[0, t, h * g:(h + 1) * g].float().numpy(), kh, vh, alpha[0, :, h], t,
                                    16, 1.0 / math.sqrt(d))
            for got_t in (split, one):
                got = got_t[0, c, h * g:(h + 1) * g].cpu().double().numpy()
                err = np.abs(got - ref)
                worst = max(worst, float(err.max()))
                bound = 1e-5 if zero_q else BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref)
                assert np.all(err <= bound), (h, c, float(err.max()))
    say(f"chunk split vs one pass (zero q {zero_q}): max gap {gap:.2e}; vs oracle {worst:.2e}")


@pytest.mark.parametrize("chunks,d,g", [([32, 70], 128, 5), ([100], 64, 16), ([40, 33], 64, 2)])
def test_chunk_queries_float32_tiled(gpu, chunks, d, g):
    """float32 caches, chunks of 32 queries or more: the tiled kernel on the
    float32 matrix instruction, every query against the oracle at the float32
    tolerance (1e-5 max abs), with compaction between chunks.  Every page
    starts as NaN, so the slots past n_slots of a unit's last page are NaN
    and must not reach any output."""
    from harness import F32_ATOL
    b, hkv, prompt, window = 2, 2, 500, 16
    total = prompt + sum(chunks)
    w = wl.Workload(name="chunk_f32_tiled", kind="prefill", batch=b, kv_heads=hkv, group=g, head_dim=d,
                    dtype="f32", context=total, evict_rate=0.6, seed=7700 + d + g)
    q, k, v, logit = wl.prefill_inputs(w)
    cache = DmsCache(b, hkv, g, d, torch.float32, max_pages_per_unit=(total + 63) // 64 + 1,
                     window=window, device=gpu)
    cache.k_pages.fill_(float("nan"))
    cache.v_pages.fill_(float("nan"))
    cache.append(k[:, :prompt].contiguous().to(gpu), v[:, :prompt].contiguous().to(gpu),
                 logit[:, :prompt].contiguous().to(gpu))
    cache.compact()
    alpha = orc.eviction_decisions(logit.numpy())
    scale = 1.0 / math.sqrt(d)
    t0, worst = prompt, 0.0
    for n in chunks:
        sl = slice(t0, t0 + n)
        cache.append(k[:, sl].contiguous().to(gpu), v[:, sl].contiguous().to(gpu),
                     logit[:, sl].contiguous().to(gpu))
        out = cache.decode_chunk(q[:, sl].contiguous().to(gpu)).cpu().double().numpy()
        assert cache.status_word() == 0
        assert np.isfinite(out).all()
        for bi in range(b):
            for h in range(hkv):
                kh, vh = k[bi, :, h].double().numpy(), v[bi, :, h].double().numpy()
                for c in range(n):
                    ref = orc.decode_output(q[bi, t0 + c, h * g:(h + 1) * g].double().numpy(), kh, vh,
                                            alpha[bi, :, h], t0 + c, window, scale)
                    err = np.abs(out[bi, c, h * g:(h + 1) * g] - ref).max()
                    worst = max(worst, float(err))
                    assert err <= F32_ATOL, f"chunk at {t0}, seq {bi}, query {c}, head {h}: {err:.3g}"
        cache.compact()
        t0 += n
    say(f"float32 tiled chunk queries {chunks} D={d} G={g}: max abs err {worst:.2e}")


def test_float32_long_chunk_compacted_after_append_is_flagged(gpu):
    """The tiled float32 kernel flags a chunk compacted after its append, as the
    vector path does."""
    from decode_attention_learned_amd import lib
    w = wl.Workload(name="chunk_f32_flag_long", kind="prefill", batch=1, kv_heads=2, group=2, head_dim=64,
                    dtype="f32", context=200, evict_rate=0.8, seed=7602)
    q, k, v, logit = wl.prefill_inputs(w)
    cache = DmsCache(1, 2, 2, 64, torch.float32, max_pages_per_unit=5, device=gpu)
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    cache.compact()
    cache.decode_chunk(q[:, 150:].contiguous().to(gpu))
    torch.cuda.synchronize()
    assert cache.status_word() == lib.DMS_STATUS_CHUNK_INVALID
