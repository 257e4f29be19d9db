"""Seeded random sequences of cache operations against the oracle, through the C ABI.

Each case draws a shape (sequences, KV heads, group, head dim, dtype), a
window and an eviction rate, then a random sequence of appends of random
lengths, one-launch decode steps (dms_append_reserve + dms_decode_attn_fill),
decodes, compactions and chunk queries (a chunk appended and queried at
once).  After every call that attends, the outputs must meet the oracle at
the dtype's tolerance (decode and steps against the oracle's incremental
cache, chunk queries against decode_output at each query's position over the
whole token history); at the end slot order, decisions and page accounting
must match bit for bit and the status word must be clear.
"""

import math

import numpy as np
import pytest
import torch
from scipy.stats import norm

from decode_attention_learned_amd import DmsCache
from harness import BF16_TOL, F32_ATOL, HostModel, check_pages, check_slots_exact, compare_outputs, say
from oracle import dms_oracle as orc

pytestmark = pytest.mark.gpu


def _logits(gen, shape, rate):
    if rate <= 0.0:
        return torch.full(shape, -1.0)
    if rate >= 1.0:
        return torch.full(shape, 1.0)
    return torch.randn(shape, generator=gen) + float(norm.ppf(rate))


@pytest.mark.parametrize("seed", range(24))
def test_random_operation_sequences(gpu, seed):
    rng = np.random.default_rng(9000 + seed)
    gen = torch.Generator().manual_seed(9000 + seed)
    dtype = torch.float32 if seed % 3 == 0 else torch.bfloat16
    b, hkv = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 4, 5, 8, 16]))
    d = int(rng.choice([64, 128]))
    window = int(rng.choice([1, 4, 16, 40]))
    rate = float(rng.choice([0.0, 0.3, 0.75, 0.95, 1.0]))
    hq = hkv * g
    say(f"random ops seed {seed}: B={b} Hkv={hkv} G={g} D={d} {dtype} w={window} rate={rate}")
    cache = DmsCache(b, hkv, g, d, dtype, max_pages_per_unit=2000 // 64 + 4, window=window, device=gpu)
    model = HostModel(b, hkv, g, d, window)
    scale = 1.0 / math.sqrt(d)
    hist_k, hist_v, hist_a = [], [], []      # full token history on the host

    def tokens(n):
        k = torch.randn((b, n, hkv, d), generator=gen).to(dtype)
        v = torch.randn((b, n, hkv, d), generator=gen).to(dtype)
        return k, v, _logits(gen, (b, n, hkv), rate)

    def record(k, v, logit):
        model.append(k, v, logit)
        hist_k.append(k.double())
        hist_v.append(v.double())
        hist_a.append(orc.eviction_decisions(logit.numpy()))

    def query():
        return torch.randn((b, hq, d), generator=gen).to(dtype)

    total = 0
    kinds = ["append", "step", "decode", "compact", "chunk"]
    for op in range(28):
        kind = "append" if op == 0 else str(rng.choice(kinds, p=[0.25, 0.25, 0.15, 0.15, 0.2]))
        if kind in ("append", "chunk") and total > 1700:
            kind = "compact"
        if kind == "append":
            n = int(rng.integers(1, 150))
            k, v, logit = tokens(n)
            cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
            record(k, v, logit)
            total += n
        elif kind == "step":
            k, v, logit = tokens(1)
            q = query()
            out = cache.step(k.to(gpu), v.to(gpu), logit.to(gpu), q.to(gpu)).cpu()
            record(k, v, logit)
            total += 1
            compare_outputs(out, model.decode(q, scale), hkv, g, dtype, what=f"op {op} step")
        elif kind == "decode":
            q = query()
            out = cache.decode(q.to(gpu)).cpu()
            compare_outputs(out, model.decode(q, scale), hkv, g, dtype, what=f"op {op} decode")
        elif kind == "compact":
            cache.compact()
            model.compact()
        else:
            n = int(rng.integers(1, 90))
            k, v, logit = tokens(n)
            q = torch.randn((b, n, hq, d), generator=gen).to(dtype)
            cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
            record(k, v, logit)
            total += n
            out = cache.decode_chunk(q.to(gpu)).cpu().double().numpy()
            K, V = torch.cat(hist_k, 1).numpy(), torch.cat(hist_v, 1).numpy()
            A = np.concatenate(hist_a, axis=1)
            t0 = total - n
            for bi in range(b):
                for h in range(hkv):
                    for c in range(n):
                        ref = orc.decode_output(q[bi, c, h * g:(h + 1) * g].double().numpy(), K[bi, :, h],
                                                V[bi, :, h], A[bi, :, h], t0 + c, window, scale)
                        got = out[bi, c, h * g:(h + 1) * g]
                        err = np.abs(got - ref)
                        if dtype == torch.float32:
                            assert err.max() <= F32_ATOL, f"op {op} chunk query {c}: {err.max():.3g}"
                        else:
                            bound = BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref)
                            assert np.all(err <= bound), f"op {op} chunk query {c}: {err.max():.3g}"
        assert cache.status_word() == 0, f"op {op} ({kind}): status {cache.status_word()}"
    meta = check_slots_exact(cache, model)
    check_pages(cache, meta)
