"""Seeded random prefill cases against the oracle, through the C ABI.

Each case draws a shape (sequences, KV heads, group, head dim, dtype), a
sequence length (ragged against the 32-token tiles), a window, an eviction
rate and a method (dense, gathered, relaxed with a random temperature and
logistic noise), and compares every output row with the oracle at the
dtype's tolerance.
"""

import math

import numpy as np
import pytest
import torch
from scipy.stats import norm

from decode_attention_learned_amd import prefill
from harness import BF16_TOL, F32_ATOL, say
from oracle import dms_oracle as orc
from oracle import soft_mask as smo

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill_cases(gpu, seed):
    rng = np.random.default_rng(9500 + seed)
    gen = torch.Generator().manual_seed(9500 + seed)
    dtype = torch.float32 if seed % 3 == 0 else torch.bfloat16
    b, hkv = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 4, 5, 8, 16]))
    d = int(rng.choice([64, 128]))
    s = int(rng.integers(1, 600))
    window = int(rng.choice([1, 4, 16, 40]))
    rate = float(rng.choice([0.0, 0.3, 0.75, 0.95, 1.0]))
    method = str(rng.choice(["dense", "gathered", "relaxed"]))
    tau = float(rng.choice([0.3, 1.0, 3.0]))
    say(f"random prefill seed {seed}: B={b} Hkv={hkv} G={g} D={d} S={s} {dtype} w={window} "
        f"rate={rate} {method}")
    q = torch.randn((b, s, hkv * g, d), generator=gen).to(dtype)
    k = torch.randn((b, s, hkv, d), generator=gen).to(dtype)
    v = torch.randn((b, s, hkv, d), generator=gen).to(dtype)
    if rate <= 0.0 or rate >= 1.0:
        logit = torch.full((b, s, hkv), -1.0 if rate <= 0.0 else 1.0)
    else:
        logit = torch.randn((b, s, hkv), generator=gen) + float(norm.ppf(rate))
    u = torch.rand((b, s, hkv), generator=gen, dtype=torch.float64).clamp(1e-12, 1 - 1e-12)
    noise = (torch.log(u) - torch.log1p(-u)).to(torch.float32)
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=window, method=method,
                  noise=noise.to(gpu) if method == "relaxed" else None, temperature=tau).cpu()
    assert torch.isfinite(out).all()
    scale = 1.0 / math.sqrt(d)
    rows = np.arange(s)
    alpha = orc.eviction_decisions(logit.numpy())
    for bi in range(b):
        qn, kn, vn = q[bi].double().numpy(), k[bi].double().numpy(), v[bi].double().numpy()
        if method == "relaxed":
            ref = smo.soft_prefill_rows(qn, kn, vn, logit[bi].numpy(), noise[bi].numpy(), tau, rows,
                                        window, scale)
        else:
            ref = orc.prefill_rows(qn, kn, vn, alpha[bi], rows, window, scale)
        err = np.abs(out[bi].double().numpy() - ref)
        if dtype == torch.float32:
            assert err.max() <= F32_ATOL, f"seq {bi}: max abs err {err.max():.3g}"
        else:
            bound = BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref)
            assert np.all(err <= bound), f"seq {bi}: max err {err.max():.3g}"
