"""The seeded generator: determinism, shapes and realised eviction rates (checks the data, not a kernel)."""

import math

import numpy as np
import pytest
import torch

import workloads as wl


def test_logit_mean_for_rate():
    assert wl.logit_mean_for_rate(0.5) == pytest.approx(0.0, abs=1e-15)
    assert wl.logit_mean_for_rate(0.875) == pytest.approx(1.1503493803760079, abs=1e-12)
    assert wl.logit_mean_for_rate(0.75) == pytest.approx(0.6744897501960817, abs=1e-12)
    assert wl.logit_mean_for_rate(0.0) is None and wl.logit_mean_for_rate(1.0) is None


def test_chunks_are_reproducible_and_distinct():
    w = wl.get("tiny_f32")
    a = wl.prompt_chunk_inputs(w, 0, 32)
    b = wl.prompt_chunk_inputs(w, 0, 32)
    c = wl.prompt_chunk_inputs(w, 1, 32)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    assert a[0].shape == (1, 32, 2, 64) and a[0].dtype == torch.float32
    assert a[2].shape == (1, 32, 2) and a[2].dtype == torch.float32


def test_bf16_workload_dtypes():
    w = wl.get("llama1b_cr4")
    q, k, v, logit = wl.decode_step_inputs(w, 3)
    assert q.shape == (16, 32, 64) and q.dtype == torch.bfloat16
    assert k.shape == (16, 1, 8, 64) and k.dtype == torch.bfloat16
    assert logit.dtype == torch.float32


@pytest.mark.parametrize("name", ["tiny_f32", "llama1b_cr4", "qwen3_8b_cr8"])
def test_realised_eviction_rate_within_4_sigma(name):
    w = wl.get(name)
    _, _, logit = wl.prompt_chunk_inputs(w, 0, 512 if w.batch < 16 else 256)
    n = logit.numel()
    p = w.evict_rate
    frac = float((logit > 0).float().mean())
    assert abs(frac - p) <= 4 * math.sqrt(p * (1 - p) / n)


def test_constant_rates():
    w = wl.get("qwen3_8b_cr1")
    _, _, logit = wl.prompt_chunk_inputs(w, 0, 8)
    assert bool((logit == -1.0).all())


def test_beta_rates_are_per_unit_and_aggregate_cr_near_8():
    w = wl.get("qwen32b_width")
    rates = wl.unit_eviction_rates(w)
    assert rates.shape == (32, 8)
    assert np.all((rates > 0) & (rates < 1))
    # aggregate compression ratio sum(L) / sum(|R|) at L = 32768, w = 16
    kept = (1 - rates) * (32768 - 16) + 16
    cr = 32768 * rates.size / kept.sum()
    assert 6.0 < cr < 11.0


def test_logistic_noise_law():
    """The noise generator draws the standard logistic law: mean 0, variance
    pi^2 / 3, CDF 1 / (1 + e^-x) at x = 1 (0.7311), within sampling error."""
    import math

    w = wl.Workload(name="noise_case", kind="prefill", batch=4, kv_heads=8, group=4, head_dim=128,
                    dtype="bf16", context=4096, evict_rate=0.5, seed=77)
    n = wl.logistic_noise(w).double()
    assert n.shape == (4, 4096, 8)
    cnt = n.numel()
    assert abs(n.mean().item()) < 5 * math.sqrt(math.pi ** 2 / 3 / cnt)
    assert abs(n.var().item() - math.pi ** 2 / 3) < 0.05
    p1 = (n <= 1.0).double().mean().item()
    assert abs(p1 - 1 / (1 + math.exp(-1))) < 5 * math.sqrt(0.2 / cnt)
    assert torch.equal(wl.logistic_noise(w), n.float())
