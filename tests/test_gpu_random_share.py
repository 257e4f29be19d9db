"""Seeded random sequences of cache operations with prompt sharing and release,
against the oracle, through the C ABI.

As the random operation test, with two more calls: dms_release empties a
random sequence (its pages return or lose a holder) and dms_share_prefix
gives an empty sequence the state of another (their clean pages shared).
Each sequence keeps its own token history, so after sharing and release the
sequences hold different lengths and every chunk query has its own positions
per sequence.  After every call that attends, the outputs meet the oracle at
the dtype's tolerance; at the end slot order and decisions match bit for bit
and every page is free or held with page_ref = holders - 1.
"""

import copy
import math

import numpy as np
import pytest
import torch
from scipy.stats import norm

from decode_attention_learned_amd import DmsCache
from harness import BF16_TOL, F32_ATOL, HostModel, check_accounting, check_slots_exact, compare_outputs, say
from oracle import dms_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(16))
def test_random_sequences_with_sharing_and_release(gpu, seed):
    rng = np.random.default_rng(9800 + seed)
    gen = torch.Generator().manual_seed(9800 + seed)
    dtype = torch.float32 if seed % 4 == 0 else torch.bfloat16
    b, hkv = int(rng.integers(2, 5)), int(rng.integers(1, 3))
    g = int(rng.choice([1, 4, 5, 16]))
    d = int(rng.choice([64, 128]))
    window = int(rng.choice([1, 16, 40]))
    rate = float(rng.choice([0.0, 0.5, 0.9]))
    hq = hkv * g
    say(f"random share seed {seed}: B={b} Hkv={hkv} G={g} D={d} {dtype} w={window} rate={rate}")
    cache = DmsCache(b, hkv, g, d, dtype, max_pages_per_unit=1800 // 64 + 4, window=window, device=gpu)
    model = HostModel(b, hkv, g, d, window)
    scale = 1.0 / math.sqrt(d)
    hist = [[] for _ in range(b)]    # per sequence: (k [n, Hkv, D], v, alpha [n, Hkv]) float64 / bool

    def tokens(n):
        k = torch.randn((b, n, hkv, d), generator=gen).to(dtype)
        v = torch.randn((b, n, hkv, d), generator=gen).to(dtype)
        if rate == 0.0:
            logit = torch.full((b, n, hkv), -1.0)
        else:
            logit = torch.randn((b, n, hkv), generator=gen) + float(norm.ppf(rate))
        return k, v, logit

    def record(k, v, logit):
        model.append(k, v, logit)
        a = orc.eviction_decisions(logit.numpy())
        for bi in range(b):
            hist[bi].append((k[bi].double().numpy(), v[bi].double().numpy(), a[bi]))

    def length(bi):
        return sum(x[0].shape[0] for x in hist[bi])

    kinds = ["append", "step", "decode", "compact", "chunk", "release", "share"]
    done = {k: 0 for k in kinds}
    for op in range(30):
        kind = "append" if op == 0 else str(rng.choice(kinds, p=[0.2, 0.2, 0.1, 0.15, 0.15, 0.1, 0.1]))
        if kind in ("append", "chunk") and max(length(bi) for bi in range(b)) > 1500:
            kind = "compact"
        if kind == "append":
            n = int(rng.integers(1, 130))
            k, v, logit = tokens(n)
            cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
            record(k, v, logit)
        elif kind == "step":
            k, v, logit = tokens(1)
            q = torch.randn((b, hq, d), generator=gen).to(dtype)
            out = cache.step(k.to(gpu), v.to(gpu), logit.to(gpu), q.to(gpu)).cpu()
            record(k, v, logit)
            compare_outputs(out, model.decode(q, scale), hkv, g, dtype, what=f"op {op} step")
        elif kind == "decode":
            if min(length(bi) for bi in range(b)) == 0:
                continue       # a sequence with no token has no query position
            q = torch.randn((b, hq, d), generator=gen).to(dtype)
            out = cache.decode(q.to(gpu)).cpu()
            compare_outputs(out, model.decode(q, scale), hkv, g, dtype, what=f"op {op} decode")
        elif kind == "compact":
            cache.compact()
            model.compact()
        elif kind == "release":
            r = int(rng.integers(0, b))
            cache.release(r, 1)
            for h in range(hkv):
                model.units[r * hkv + h] = orc.UnitCache(window, d, dtype=np.float32)
            hist[r] = []
        elif kind == "share":
            empty = [bi for bi in range(b) if length(bi) == 0]
            full = [bi for bi in range(b) if length(bi) > 0]
            if not empty or not full:
                continue
            src, dst = int(rng.choice(full)), int(rng.choice(empty))
            cache.share_prefix(src, dst, 1)
            for h in range(hkv):
                model.units[dst * hkv + h] = copy.deepcopy(model.units[src * hkv + h])
            hist[dst] = list(hist[src])
            check_accounting(cache)
        else:
            n = int(rng.integers(1, 80))
            k, v, logit = tokens(n)
            q = torch.randn((b, n, hq, d), generator=gen).to(dtype)
            t0 = [length(bi) for bi in range(b)]
            cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
            record(k, v, logit)
            out = cache.decode_chunk(q.to(gpu)).cpu().double().numpy()
            for bi in range(b):
                K = np.concatenate([x[0] for x in hist[bi]])
                V = np.concatenate([x[1] for x in hist[bi]])
                A = np.concatenate([x[2] for x in hist[bi]])
                for h in range(hkv):
                    for c in range(n):
                        ref = orc.decode_output(q[bi, c, h * g:(h + 1) * g].double().numpy(), K[:, h],
                                                V[:, h], A[:, h], t0[bi] + c, window, scale)
                        err = np.abs(out[bi, c, h * g:(h + 1) * g] - ref)
                        if dtype == torch.float32:
                            assert err.max() <= F32_ATOL, f"op {op} seq {bi} chunk query {c}: {err.max():.3g}"
                        else:
                            bound = BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref)
                            assert np.all(err <= bound), f"op {op} seq {bi} chunk query {c}: {err.max():.3g}"
        assert cache.status_word() == 0, f"op {op} ({kind}): status {cache.status_word()}"
        done[kind] += 1
    say(f"  calls made: {done}")
    check_slots_exact(cache, model)
    check_accounting(cache)
