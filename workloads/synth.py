"""Seeded random draws for the named workloads.

Recipe (stated once here, used by tests and the benchmark alike):

* q, k, v entries ~ N(0, 1), drawn in float32 and rounded to bfloat16
  (round-to-nearest-even, torch's ``.to(torch.bfloat16)``) for bf16 workloads;
  the softmax scale 1/sqrt(D) is applied by the kernel, not to the data.
* eviction logits ~ N(mu, 1) in float32, i.i.d. per (sequence, token, KV head);
  mu = Phi^{-1}(rate) so that a fraction `rate` of logits is positive.
  A rate of 0 or 1 gives the constant logit -1 or +1 (nothing / everything marked).
* per-unit rates are either the workload's constant or, for ragged workloads,
  one Beta(a, b) draw per (sequence, KV head) from NumPy's PCG64.
* every tensor comes from its own ``torch.Generator`` whose seed is a fixed
  mix of (workload seed, replica, stream tag, index), so any chunk or step
  can be regenerated alone, in any order, on the CPU or on the GPU.
"""

from __future__ import annotations

from statistics import NormalDist

import numpy as np
import torch

from .configs import Workload

_TAGS = {"prompt": 1, "decode": 2, "prefill": 3, "rates": 4, "noise": 5}


def logit_mean_for_rate(rate: float) -> float | None:
    """mu with P(N(mu, 1) > 0) = rate; None for the constant-logit rates 0 and 1."""
    if rate <= 0.0 or rate >= 1.0:
        return None
    return NormalDist().inv_cdf(rate)


def _seed(w: Workload, replica: int, tag: str, index: int) -> int:
    return (((w.seed * 1_000_003 + replica) * 10_007 + _TAGS[tag]) * 1_000_033 + index) % (2**63 - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _kv_dtype(w: Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def unit_eviction_rates(w: Workload, replica: int = 0) -> np.ndarray:
    """[B, Hkv] float64 fraction of tokens marked for eviction, per unit."""
    if w.beta_rate is not None:
        a, b = w.beta_rate
        rng = np.random.Generator(np.random.PCG64(_seed(w, replica, "rates", 0)))
        return rng.beta(a, b, size=(w.batch, w.kv_heads))
    return np.full((w.batch, w.kv_heads), float(w.evict_rate), dtype=np.float64)


def _logits(w: Workload, rates: np.ndarray, n: int, gen: torch.Generator, device) -> torch.Tensor:
    """[B, n, Hkv] float32 logits with per-unit means from `rates`."""
    mu = np.zeros_like(rates)
    const = np.zeros_like(rates)
    for idx, r in np.ndenumerate(rates):
        m = logit_mean_for_rate(float(r))
        if m is None:
            const[idx] = 1.0 if r >= 1.0 else -1.0
        else:
            mu[idx] = m
    noise = torch.randn((w.batch, n, w.kv_heads), generator=gen, device=device, dtype=torch.float32)
    mu_t = torch.as_tensor(mu, dtype=torch.float32, device=device)[:, None, :]
    c_t = torch.as_tensor(const, dtype=torch.float32, device=device)[:, None, :]
    is_const = c_t != 0
    return torch.where(is_const, c_t.expand_as(noise), noise + mu_t)


def prompt_chunk_inputs(w: Workload, chunk: int, n: int, device="cpu", replica: int = 0,
                        rates: np.ndarray | None = None):
    """Prompt tokens of chunk `chunk` (n tokens per sequence).

    Returns (k, v, logit): k, v [B, n, Hkv, D] in the workload dtype and
    logit [B, n, Hkv] float32.
    """
    if rates is None:
        rates = unit_eviction_rates(w, replica)
    g = _gen(device, _seed(w, replica, "prompt", chunk))
    shape = (w.batch, n, w.kv_heads, w.head_dim)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(_kv_dtype(w))
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(_kv_dtype(w))
    logit = _logits(w, rates, n, g, device)
    return k, v, logit


def decode_step_inputs(w: Workload, step: int, device="cpu", replica: int = 0,
                       rates: np.ndarray | None = None):
    """Inputs of decode step `step`: (q [B, Hq, D], k [B, 1, Hkv, D], v, logit [B, 1, Hkv])."""
    if rates is None:
        rates = unit_eviction_rates(w, replica)
    g = _gen(device, _seed(w, replica, "decode", step))
    q = torch.randn((w.batch, w.q_heads, w.head_dim), generator=g, device=device,
                    dtype=torch.float32).to(_kv_dtype(w))
    shape = (w.batch, 1, w.kv_heads, w.head_dim)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(_kv_dtype(w))
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(_kv_dtype(w))
    logit = _logits(w, rates, 1, g, device)
    return q, k, v, logit


def prefill_inputs(w: Workload, device="cpu", replica: int = 0, seq_len: int | None = None):
    """Prefill inputs: q [B, S, Hq, D], k, v [B, S, Hkv, D] (workload dtype), logit [B, S, Hkv] f32."""
    s = w.context if seq_len is None else int(seq_len)
    rates = unit_eviction_rates(w, replica)
    g = _gen(device, _seed(w, replica, "prefill", 0))
    q = torch.randn((w.batch, s, w.q_heads, w.head_dim), generator=g, device=device,
                    dtype=torch.float32).to(_kv_dtype(w))
    shape = (w.batch, s, w.kv_heads, w.head_dim)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(_kv_dtype(w))
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(_kv_dtype(w))
    logit = _logits(w, rates, s, g, device)
    return q, k, v, logit


def logistic_noise(w: Workload, device="cpu", replica: int = 0, seq_len: int | None = None) -> torch.Tensor:
    """[B, S, Hkv] float32 draws of the standard logistic law (the difference of
    two standard Gumbel draws), by inversion of uniforms: log(u) - log(1 - u)."""
    s = w.context if seq_len is None else int(seq_len)
    g = _gen(device, _seed(w, replica, "noise", 0))
    u = torch.rand((w.batch, s, w.kv_heads), generator=g, device=device, dtype=torch.float64)
    u = u.clamp(1e-12, 1.0 - 1e-12)
    return (torch.log(u) - torch.log1p(-u)).to(torch.float32)
