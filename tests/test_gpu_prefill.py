"""GPU parity of the masked prefill kernels against the float64 oracle, through the C ABI.

Both entry points are covered: dms_prefill_attn ("dense": every causal tile,
masked) and dms_prefill_attn_gathered ("gathered": kept keys gathered per head
plus the window band).  Tolerance: |o - o_ref| <= 2e-2 + 2e-2 |o_ref|
element-wise (bf16 inputs, fp32 accumulation).
"""

import math

import numpy as np
import pytest
import torch

import workloads as wl
from decode_attention_learned_amd import DmsCache, prefill
from harness import BF16_TOL, HostModel, compare_outputs, say
from oracle import dms_oracle as orc

pytestmark = pytest.mark.gpu


def _inputs(b, s, hkv, g, d=128, rate=0.5, seed=0):
    w = wl.Workload(name="prefill_case", kind="prefill", batch=b, kv_heads=hkv, group=g,
                    head_dim=d, dtype="bf16", context=s, evict_rate=rate, seed=seed)
    return w, wl.prefill_inputs(w)


def _check_rows(out, q, k, v, logit, rows, window, what=""):
    """Compare GPU rows against oracle.prefill_rows for every sequence."""
    b_n, s, hq, d = q.shape
    scale = 1.0 / math.sqrt(d)
    alpha = orc.eviction_decisions(logit.numpy())
    worst = 0.0
    for bi in range(b_n):
        ref = orc.prefill_rows(q[bi].float().numpy(), k[bi].float().numpy(), v[bi].float().numpy(),
                               alpha[bi], rows, window, scale)
        got = out[bi, rows].double().numpy()
        err = np.abs(got - ref)
        worst = max(worst, float(err.max()))
        bound = BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref)
        assert np.all(err <= bound), f"{what} seq {bi}: max err {err.max():.3g}"
    return worst


METHODS = ["dense", "gathered"]


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("b,s,hkv,g", [(2, 200, 2, 4), (1, 97, 1, 1), (1, 130, 2, 2), (1, 150, 1, 5),
                                       (2, 64, 1, 8), (1, 1, 1, 4), (1, 33, 3, 4), (1, 385, 1, 4)])
def test_prefill_small_all_rows(gpu, b, s, hkv, g, method):
    w, (q, k, v, logit) = _inputs(b, s, hkv, g, seed=5100 + s + g)
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method=method).cpu()
    worst = _check_rows(out, q, k, v, logit, np.arange(s), 16,
                        what=f"{method} B={b} S={s} Hkv={hkv} G={g}")
    say(f"prefill {method} B={b} S={s} Hkv={hkv} G={g}: max err {worst:.2e}")


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("window", [1, 3, 16, 40, 100])
def test_prefill_windows(gpu, window, method):
    w, (q, k, v, logit) = _inputs(1, 300, 2, 4, rate=0.7, seed=5200 + window)
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=window, method=method).cpu()
    _check_rows(out, q, k, v, logit, np.arange(300), window, what=f"{method} window {window}")


@pytest.mark.parametrize("rate", [0.0, 0.3, 0.875, 0.97, 1.0])
def test_prefill_gathered_rates(gpu, rate):
    """Gathered kernel over the range of eviction rates: from no key gathered
    away (everything kept) to nothing gathered (only the band), on 3 query
    blocks and 12 key tiles with a ragged end."""
    w, (q, k, v, logit) = _inputs(2, 371, 2, 4, rate=rate, seed=5500 + int(rate * 100))
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method="gathered").cpu()
    worst = _check_rows(out, q, k, v, logit, np.arange(371), 16, what=f"gathered rate {rate}")
    say(f"prefill gathered rate {rate}: max err {worst:.2e}")


def test_prefill_methods_agree(gpu):
    """Dense and gathered kernels on the same inputs: both within tolerance of
    the oracle on every row, and within tolerance of each other."""
    w, (q, k, v, logit) = _inputs(2, 700, 2, 4, rate=0.875, seed=5601)
    qd, kd, vd, ld = q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu)
    dense = prefill(qd, kd, vd, ld, window=16, method="dense").cpu()
    gath = prefill(qd, kd, vd, ld, window=16, method="gathered").cpu()
    _check_rows(gath, q, k, v, logit, np.arange(700), 16, what="gathered")
    assert torch.allclose(dense, gath, rtol=2e-2, atol=2e-2)


@pytest.mark.parametrize("method", METHODS)
def test_prefill_all_keep_is_causal_sdpa(gpu, method):
    """Nothing marked: the kernel is plain causal attention (torch SDPA on CPU, float64)."""
    w, (q, k, v, logit) = _inputs(2, 257, 2, 4, rate=0.0, seed=5301)
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method=method).cpu()
    for bi in range(2):
        qq = q[bi].double().permute(1, 0, 2)
        kk = k[bi].double().permute(1, 0, 2).repeat_interleave(4, 0)
        vv = v[bi].double().permute(1, 0, 2).repeat_interleave(4, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True,
                                                               scale=1 / math.sqrt(128))
        assert torch.allclose(out[bi].double(), ref.permute(1, 0, 2), rtol=2e-2, atol=2e-2)


@pytest.mark.parametrize("method", METHODS)
def test_prefill_all_evict_is_sliding_window_sdpa(gpu, method):
    """Everything marked: attention over the last 16 positions (SDPA with a band mask)."""
    w, (q, k, v, logit) = _inputs(1, 200, 2, 4, rate=1.0, seed=5302)
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method=method).cpu()
    i = torch.arange(200)[:, None]
    j = torch.arange(200)[None, :]
    band = (i - j >= 0) & (i - j < 16)
    qq = q[0].double().permute(1, 0, 2)
    kk = k[0].double().permute(1, 0, 2).repeat_interleave(4, 0)
    vv = v[0].double().permute(1, 0, 2).repeat_interleave(4, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=band,
                                                           scale=1 / math.sqrt(128))
    assert torch.allclose(out[0].double(), ref.permute(1, 0, 2), rtol=2e-2, atol=2e-2)


def test_prefill_matches_decode_path(gpu):
    """Prefill row t and the decode step at t see the same set: both GPU paths agree
    with each other and with the oracle."""
    b, s, hkv, g = 2, 180, 2, 4
    w, (q, k, v, logit) = _inputs(b, s, hkv, g, rate=0.6, seed=5401)
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16).cpu()
    cache = DmsCache(b, hkv, g, 128, torch.bfloat16, max_pages_per_unit=4, device=gpu)
    for t in range(s):
        cache.append(k[:, t:t + 1].contiguous().to(gpu), v[:, t:t + 1].contiguous().to(gpu),
                     logit[:, t:t + 1].contiguous().to(gpu))
        if t in (0, 15, 16, 17, 90, 179):
            dec = cache.decode(q[:, t].contiguous().to(gpu)).cpu()
            assert torch.allclose(dec, out[:, t], rtol=2e-2, atol=2e-2), f"t={t}"
        if t % 32 == 31:
            cache.compact()


@pytest.mark.parametrize("method", METHODS)
def test_prefill_8k_sampled_rows(gpu, method):
    """Masked prefill at full size (B=4, S=8192, 32/8 heads, CR 8): query rows
    [0, 512) and [7680, 8192) of every sequence and head against the oracle."""
    w = wl.get("prefill_8k")
    say(f"prefill_8k {method}: B=4 S=8192 Hq=32 Hkv=8 D=128")
    q, k, v, logit = wl.prefill_inputs(w, device=gpu)
    out = prefill(q, k, v, logit, window=16, method=method)
    rows = np.concatenate([np.arange(0, 512), np.arange(7680, 8192)])
    out_rows = out[:, torch.as_tensor(rows, device=gpu)].cpu()
    qc, kc, vc, lc = q.cpu(), k.cpu(), v.cpu(), logit.cpu()
    scale = 1.0 / math.sqrt(128)
    alpha = orc.eviction_decisions(lc.numpy())
    for bi in range(w.batch):
        ref = orc.prefill_rows(qc[bi].float().numpy(), kc[bi].float().numpy(), vc[bi].float().numpy(),
                               alpha[bi], rows, 16, scale)
        got = out_rows[bi].double().numpy()
        err = np.abs(got - ref)
        bound = BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref)
        assert np.all(err <= bound), f"seq {bi}: max err {err.max():.3g}"
        say(f"  seq {bi}: max err {err.max():.2e}")


# ---------------------------------------------------------------- relaxed mask
def _check_relaxed(out, q, k, v, logit, noise, tau, rows, window, what=""):
    from oracle import soft_mask as smo

    b_n, s, hq, d = q.shape
    worst = 0.0
    for bi in range(b_n):
        ref = smo.soft_prefill_rows(q[bi].float().numpy(), k[bi].float().numpy(), v[bi].float().numpy(),
                                    logit[bi].numpy(), noise[bi].numpy() if noise is not None else 0.0,
                                    tau, rows, window, 1.0 / math.sqrt(d))
        got = out[bi, rows].double().numpy()
        err = np.abs(got - ref)
        worst = max(worst, float(err.max()))
        assert np.all(err <= BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref)), \
            f"{what} seq {bi}: max err {err.max():.3g}"
    return worst


@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0])
@pytest.mark.parametrize("with_noise", [False, True])
def test_prefill_relaxed_all_rows(gpu, tau, with_noise):
    """Relaxed-mask prefill against the float64 relaxed oracle, every row,
    logits with mean 0 so that keep factors spread over (0, 1)."""
    w, (q, k, v, logit) = _inputs(2, 230, 2, 4, rate=0.5, seed=5700 + int(tau * 10))
    noise = wl.logistic_noise(w) if with_noise else None
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method="relaxed",
                  noise=noise.to(gpu) if noise is not None else None, temperature=tau).cpu()
    worst = _check_relaxed(out, q, k, v, logit, noise, tau, np.arange(230), 16,
                           what=f"relaxed tau {tau} noise {with_noise}")
    say(f"prefill relaxed tau={tau} noise={with_noise}: max err {worst:.2e}")


@pytest.mark.parametrize("window", [1, 40])
def test_prefill_relaxed_windows(gpu, window):
    w, (q, k, v, logit) = _inputs(1, 300, 2, 4, rate=0.7, seed=5800 + window)
    noise = wl.logistic_noise(w)
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=window, method="relaxed",
                  noise=noise.to(gpu), temperature=0.5).cpu()
    _check_relaxed(out, q, k, v, logit, noise, 0.5, np.arange(300), window, what=f"relaxed window {window}")


def test_prefill_relaxed_cold_limit_is_hard_rule(gpu):
    """Temperature 1e-4 without noise: the relaxed kernel gives the hard-rule
    result (logits kept at |logit| >= 0.05 so every factor saturates)."""
    w, (q, k, v, logit) = _inputs(2, 200, 2, 4, rate=0.6, seed=5901)
    logit = torch.where(logit.abs() < 0.05, torch.full_like(logit, 0.5), logit)
    qd, kd, vd, ld = q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu)
    relaxed = prefill(qd, kd, vd, ld, window=16, method="relaxed", temperature=1e-4).cpu()
    _check_rows(relaxed, q, k, v, logit, np.arange(200), 16, what="relaxed, cold")


def test_prefill_relaxed_8k_sampled_rows(gpu):
    """Relaxed mask at full size (B=4, S=8192, 32/8 heads), temperature 1 with
    logistic noise: rows [0, 256) and [7936, 8192) against the oracle."""
    w = wl.get("prefill_8k")
    q, k, v, logit = wl.prefill_inputs(w, device=gpu)
    noise = wl.logistic_noise(w, device=gpu)
    out = prefill(q, k, v, logit, window=16, method="relaxed", noise=noise, temperature=1.0)
    rows = np.concatenate([np.arange(0, 256), np.arange(7936, 8192)])
    out_rows = out[:, torch.as_tensor(rows, device=gpu)].cpu()
    full = torch.zeros((w.batch, w.context, w.q_heads, 128), dtype=torch.float32)
    full[:, torch.as_tensor(rows)] = out_rows
    worst = _check_relaxed(full, q.cpu(), k.cpu(), v.cpu(), logit.cpu(), noise.cpu(), 1.0, rows, 16,
                           what="relaxed 8k")
    say(f"prefill relaxed 8k: max err {worst:.2e}")


@pytest.mark.parametrize("method", METHODS + ["relaxed"])
def test_prefill_constant_values(gpu, method):
    """Constant value rows: the output is the constant.  The prefill kernels
    add the same bf16-rounded weights into the row sums as into the PV
    product, so the ratio is exact up to float32 rounding (1e-5 relative)."""
    w, (q, k, v, logit) = _inputs(2, 333, 2, 4, rate=0.8, seed=5951)
    c = torch.linspace(-3.0, 3.0, 128).to(torch.bfloat16)
    v = c.expand_as(v).contiguous()
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method=method,
                  temperature=0.5).cpu().double()
    ref = c.double().expand_as(out)
    assert torch.max(torch.abs(out - ref) / (1e-3 + ref.abs())).item() <= 1e-5


# ---------------------------------------------------------------- head_dim 64 (Llama-3.2-1B heads)
@pytest.mark.parametrize("method", METHODS + ["relaxed"])
@pytest.mark.parametrize("b,s,hkv,g", [(2, 200, 2, 4), (1, 97, 1, 1), (1, 33, 3, 5), (1, 385, 1, 4),
                                       (1, 1, 1, 4)])
def test_prefill_head_dim_64_all_rows(gpu, b, s, hkv, g, method):
    """head_dim 64: every row against the oracle (dense and gathered: the hard
    rule; relaxed: the relaxed oracle at temperature 0.5 with logistic noise)."""
    w, (q, k, v, logit) = _inputs(b, s, hkv, g, d=64, rate=0.7, seed=6100 + s + g)
    if method == "relaxed":
        noise = wl.logistic_noise(w)
        out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method="relaxed",
                      noise=noise.to(gpu), temperature=0.5).cpu()
        worst = _check_relaxed(out, q, k, v, logit, noise, 0.5, np.arange(s), 16,
                               what=f"relaxed D=64 B={b} S={s}")
    else:
        out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method=method).cpu()
        worst = _check_rows(out, q, k, v, logit, np.arange(s), 16,
                            what=f"{method} D=64 B={b} S={s} Hkv={hkv} G={g}")
    say(f"prefill {method} D=64 B={b} S={s} Hkv={hkv} G={g}: max err {worst:.2e}")


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("rate", [0.0, 1.0])
def test_prefill_head_dim_64_special_cases(gpu, method, rate):
    """head_dim 64, nothing marked: causal SDPA; everything marked: band SDPA
    of width 16 (torch on CPU, float64)."""
    w, (q, k, v, logit) = _inputs(1, 150, 2, 4, d=64, rate=rate, seed=6201)
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method=method).cpu()
    i = torch.arange(150)[:, None]
    j = torch.arange(150)[None, :]
    mask = (j <= i) if rate == 0.0 else ((i - j >= 0) & (i - j < 16))
    qq = q[0].double().permute(1, 0, 2)
    kk = k[0].double().permute(1, 0, 2).repeat_interleave(4, 0)
    vv = v[0].double().permute(1, 0, 2).repeat_interleave(4, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=1 / 8.0)
    assert torch.allclose(out[0].double(), ref.permute(1, 0, 2), rtol=2e-2, atol=2e-2)


@pytest.mark.parametrize("method", METHODS + ["relaxed"])
def test_prefill_head_dim_64_constant_values(gpu, method):
    w, (q, k, v, logit) = _inputs(2, 333, 2, 4, d=64, rate=0.8, seed=6301)
    c = torch.linspace(-3.0, 3.0, 64).to(torch.bfloat16)
    v = c.expand_as(v).contiguous()
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method=method,
                  temperature=0.5).cpu().double()
    ref = c.double().expand_as(out)
    assert torch.max(torch.abs(out - ref) / (1e-3 + ref.abs())).item() <= 1e-5


@pytest.mark.parametrize("method", METHODS)
def test_prefill_llama1b_shape_sampled_rows(gpu, method):
    """A Llama-3.2-1B-shaped prompt (32 query / 8 KV heads, head_dim 64, CR 4):
    B=4, S=4096; rows [0, 256) and [3840, 4096) of every head against the oracle."""
    w = wl.Workload(name="prefill_llama", kind="prefill", batch=4, kv_heads=8, group=4, head_dim=64,
                    dtype="bf16", context=4096, evict_rate=0.75, seed=6401)
    q, k, v, logit = wl.prefill_inputs(w, device=gpu)
    out = prefill(q, k, v, logit, window=16, method=method)
    rows = np.concatenate([np.arange(0, 256), np.arange(3840, 4096)])
    out_rows = out[:, torch.as_tensor(rows, device=gpu)].cpu()
    full = torch.zeros((4, 4096, 32, 64), dtype=torch.float32)
    full[:, torch.as_tensor(rows)] = out_rows
    worst = _check_rows(full, q.cpu(), k.cpu(), v.cpu(), logit.cpu(), rows, 16,
                        what=f"llama-shaped {method}")
    say(f"prefill {method} Llama-1B shape, S=4096: max err {worst:.2e}")


# ------------------------------------------------------------- float32 inputs
# Float32 inputs run the float32 matrix-core kernel for all three methods; the
# tolerance is the float32 one, max |o - o_ref| <= 1e-5 (inputs exact in float64).
F32_ATOL = 1e-5


def _inputs_f32(b, s, hkv, g, d, rate=0.5, seed=0):
    w = wl.Workload(name="prefill_f32_case", kind="prefill", batch=b, kv_heads=hkv, group=g,
                    head_dim=d, dtype="f32", context=s, evict_rate=rate, seed=seed)
    return w, wl.prefill_inputs(w)


def _check_rows_f32(out, q, k, v, logit, rows, window, what=""):
    b_n, s, hq, d = q.shape
    alpha = orc.eviction_decisions(logit.numpy())
    worst = 0.0
    for bi in range(b_n):
        ref = orc.prefill_rows(q[bi].numpy(), k[bi].numpy(), v[bi].numpy(), alpha[bi], rows, window,
                               1.0 / math.sqrt(d))
        err = np.abs(out[bi, rows].double().numpy() - ref)
        worst = max(worst, float(err.max()))
        assert err.max() <= F32_ATOL, f"{what} seq {bi}: max err {err.max():.3g}"
    return worst


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("b,s,hkv,g,d", [(2, 200, 2, 4, 128), (1, 97, 1, 1, 64), (1, 150, 1, 5, 128),
                                         (1, 1, 1, 4, 64), (2, 385, 1, 3, 64), (1, 70, 2, 20, 64)])
def test_prefill_f32_all_rows(gpu, b, s, hkv, g, d, method):
    w, (q, k, v, logit) = _inputs_f32(b, s, hkv, g, d, rate=0.6, seed=6400 + s + g + d)
    assert q.dtype == torch.float32
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method=method).cpu()
    worst = _check_rows_f32(out, q, k, v, logit, np.arange(s), 16,
                            what=f"f32 {method} B={b} S={s} Hkv={hkv} G={g} D={d}")
    say(f"prefill f32 {method} B={b} S={s} Hkv={hkv} G={g} D={d}: max err {worst:.2e}")


@pytest.mark.parametrize("window", [1, 40])
@pytest.mark.parametrize("rate", [0.0, 0.9, 1.0])
def test_prefill_f32_windows_and_rates(gpu, window, rate):
    """Windows and eviction rates from nothing marked to everything marked, where
    whole far tiles are skipped (rate 1: only the band is seen)."""
    w, (q, k, v, logit) = _inputs_f32(1, 300, 2, 2, 128, rate=rate, seed=6500 + window)
    qd, kd, vd, ld = q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu)
    dense = prefill(qd, kd, vd, ld, window=window, method="dense").cpu()
    _check_rows_f32(dense, q, k, v, logit, np.arange(300), window, what=f"f32 w={window} rate={rate}")
    gath = prefill(qd, kd, vd, ld, window=window, method="gathered").cpu()
    assert torch.equal(dense, gath), "float32 gathered and dense run the same kernel"


def test_prefill_f32_all_keep_is_causal_sdpa(gpu):
    w, (q, k, v, logit) = _inputs_f32(1, 129, 2, 2, 64, rate=0.0, seed=6601)
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16).cpu()
    qq = q[0].double().permute(1, 0, 2)
    kk = k[0].double().permute(1, 0, 2).repeat_interleave(2, 0)
    vv = v[0].double().permute(1, 0, 2).repeat_interleave(2, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=1 / 8)
    assert (out[0].double() - ref.permute(1, 0, 2)).abs().max() <= F32_ATOL


@pytest.mark.parametrize("tau,with_noise", [(0.5, True), (2.0, False)])
def test_prefill_f32_relaxed(gpu, tau, with_noise):
    from oracle import soft_mask as smo

    w, (q, k, v, logit) = _inputs_f32(2, 170, 2, 4, 128, rate=0.5, seed=6700)
    noise = wl.logistic_noise(w) if with_noise else None
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16, method="relaxed",
                  noise=noise.to(gpu) if noise is not None else None, temperature=tau).cpu()
    for bi in range(2):
        ref = smo.soft_prefill_rows(q[bi].numpy(), k[bi].numpy(), v[bi].numpy(), logit[bi].numpy(),
                                    noise[bi].numpy() if noise is not None else 0.0, tau,
                                    np.arange(170), 16, 1.0 / math.sqrt(128))
        assert np.abs(out[bi].double().numpy() - ref).max() <= F32_ATOL


def test_prefill_f32_matches_f32_decode(gpu):
    """Prefill row t equals the float32 cache's decode at step t (both float32
    paths, both exact-input), including after compactions."""
    b, s, hkv, g, d = 1, 120, 2, 2, 64
    w, (q, k, v, logit) = _inputs_f32(b, s, hkv, g, d, rate=0.7, seed=6801)
    out = prefill(q.to(gpu), k.to(gpu), v.to(gpu), logit.to(gpu), window=16).cpu()
    cache = DmsCache(b, hkv, g, d, torch.float32, max_pages_per_unit=3, device=gpu)
    for t in range(s):
        cache.append(k[:, t:t + 1].contiguous().to(gpu), v[:, t:t + 1].contiguous().to(gpu),
                     logit[:, t:t + 1].contiguous().to(gpu))
        if t in (0, 15, 16, 63, 64, 119):
            dec = cache.decode(q[:, t].contiguous().to(gpu)).cpu()
            assert (dec - out[:, t]).abs().max() <= 2 * F32_ATOL, f"t={t}"
        if t % 32 == 31:
            cache.compact()


def test_prefill_f32_8k_sampled_rows(gpu):
    """The 8K prefill shape (B=4, S=8192, 32/8 heads, D=128, CR 8) with float32
    inputs, in the launch configuration the bench times: rows [0, 256) and
    [7936, 8192) of every sequence and head against the oracle at 1e-5."""
    import dataclasses

    w = dataclasses.replace(wl.get("prefill_8k"), dtype="f32")
    q, k, v, logit = wl.prefill_inputs(w, device=gpu)
    assert q.dtype == torch.float32
    out = prefill(q, k, v, logit, window=16)
    rows = np.concatenate([np.arange(0, 256), np.arange(7936, 8192)])
    out_rows = out[:, torch.as_tensor(rows, device=gpu)].cpu()
    full = torch.zeros((w.batch, w.context, w.q_heads, 128), dtype=torch.float32)
    full[:, torch.as_tensor(rows)] = out_rows
    worst = _check_rows_f32(full, q.cpu(), k.cpu(), v.cpu(), logit.cpu(), rows, 16, what="f32 8k")
    say(f"prefill f32 8k: max err {worst:.2e}")
