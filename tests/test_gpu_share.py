"""GPU tests of prompt sharing (dms_share_prefix) and sequence release (dms_release).

The reference is the same workload without sharing: every sequence appends
the prompt itself.  Sharing must not change any attention output (bit for
bit: the same bytes in the same slot order under the same split plan), and
the page accounting must stay exact: every page is free or held, and a
page's reference count is its holders minus one.
"""

import math

import numpy as np
import pytest
import torch

import workloads as wl
from decode_attention_learned_amd import DmsCache, lib
from harness import BF16_TOL, check_accounting, say
from oracle import dms_oracle as orc

pytestmark = pytest.mark.gpu


def _prompt_and_steps(b, hkv, g, d, prompt, steps, rate, seed):
    """The prompt (one sequence's worth, to be replicated) and per-sequence steps."""
    w = wl.Workload(name="share_case", kind="prefill", batch=1, kv_heads=hkv, group=g, head_dim=d,
                    dtype="bf16", context=prompt, evict_rate=rate, seed=seed)
    _, pk, pv, pl = wl.prefill_inputs(w)
    w2 = wl.Workload(name="share_steps", kind="prefill", batch=b, kv_heads=hkv, group=g, head_dim=d,
                     dtype="bf16", context=steps, evict_rate=rate, seed=seed + 1)
    sq, sk, sv, sl = wl.prefill_inputs(w2)
    return (pk, pv, pl), (sq, sk, sv, sl)


def _run_pair(gpu, b, hkv, g, d, prompt, steps, rate, seed, n_share=None, release=None):
    (pk, pv, pl), (sq, sk, sv, sl) = _prompt_and_steps(b, hkv, g, d, prompt, steps, rate, seed)
    maxp = (prompt + steps) // 64 + 3
    shared = DmsCache(b, hkv, g, d, torch.bfloat16, max_pages_per_unit=maxp, device=gpu)
    plain = DmsCache(b, hkv, g, d, torch.bfloat16, max_pages_per_unit=maxp, device=gpu)
    n_share = b - 1 if n_share is None else n_share
    rep = lambda x: x.expand(b, *x.shape[1:]).contiguous().to(gpu)   # noqa: E731
    plain.append(rep(pk), rep(pv), rep(pl))
    if n_share < b - 1:   # the same sequences hold the prompt in both caches
        plain.release(1 + n_share, b - 1 - n_share)
    plain.compact()
    # the shared cache: the prompt goes into sequence 0 only, then to 1 .. n_share
    one = lambda x: torch.cat([x, torch.zeros((b - 1, *x.shape[1:]), dtype=x.dtype)]).to(gpu)  # noqa: E731
    shared.append(one(pk), one(pv), one(pl))
    # append writes every sequence: empty 1 .. b - 1 again before sharing
    shared.release(1, b - 1)
    shared.compact()
    shared.share_prefix(0, 1, n_share)
    check_accounting(shared)
    assert shared.status_word() == 0
    assert torch.equal(shared.n_slots[: (1 + n_share) * hkv], plain.n_slots[: (1 + n_share) * hkv])
    pages_plain = plain.num_pages - int(plain.free_top.item())
    pages_shared = shared.num_pages - int(shared.free_top.item())
    active = slice(0, 1 + n_share)
    worst = 0.0
    for t in range(steps):
        for c in (plain, shared):
            c.append(sk[:, t:t + 1].contiguous().to(gpu), sv[:, t:t + 1].contiguous().to(gpu),
                     sl[:, t:t + 1].contiguous().to(gpu))
        q = sq[:, t].contiguous().to(gpu)
        a = plain.decode(q)
        s_ = shared.decode(q)
        assert torch.equal(a[active], s_[active]), f"step {t}: sharing changed the output"
        if release is not None and t == steps // 2:
            shared.release(*release)
            plain.release(*release)
            check_accounting(shared)
            lo, cnt = release
            active = [i for i in range(1 + n_share) if not (lo <= i < lo + cnt)]
        if t % 16 == 15:
            plain.compact()
            shared.compact()
            check_accounting(shared)
    assert shared.status_word() == 0
    return pages_plain, pages_shared


def test_shared_prompt_decodes_identically(gpu):
    pp, ps = _run_pair(gpu, 4, 2, 4, 128, 1500, 40, 0.5, 7001)
    say(f"pages held after sharing: {ps} vs {pp} unshared")
    assert ps < pp


def test_share_then_release_some(gpu):
    _run_pair(gpu, 6, 2, 4, 128, 1000, 48, 0.7, 7101, release=(1, 2))


def test_share_with_nothing_clean(gpu):
    """Every prompt token marked (only the window survives): no clean page,
    so everything is copied and nothing shared."""
    _run_pair(gpu, 3, 2, 4, 128, 300, 20, 1.0, 7201)


def test_share_into_part_of_the_batch(gpu):
    _run_pair(gpu, 5, 2, 4, 64, 700, 20, 0.0, 7301, n_share=2)


def test_share_against_oracle(gpu):
    """Receivers of a shared prompt against the float64 oracle over their own
    histories (prompt, then their own tokens)."""
    b, hkv, g, d, prompt, steps = 3, 2, 4, 128, 600, 12
    (pk, pv, pl), (sq, sk, sv, sl) = _prompt_and_steps(b, hkv, g, d, prompt, steps, 0.8, 7401)
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, max_pages_per_unit=(prompt + steps) // 64 + 3, device=gpu)
    pad = lambda x: torch.cat([x, torch.zeros((b - 1, *x.shape[1:]), dtype=x.dtype)]).to(gpu)  # noqa: E731
    cache.append(pad(pk), pad(pv), pad(pl))
    cache.release(1, b - 1)
    cache.compact()
    cache.share_prefix(0, 1, b - 1)
    scale = 1.0 / math.sqrt(d)
    for t in range(steps):
        cache.append(sk[:, t:t + 1].contiguous().to(gpu), sv[:, t:t + 1].contiguous().to(gpu),
                     sl[:, t:t + 1].contiguous().to(gpu))
        out = cache.decode(sq[:, t].contiguous().to(gpu)).cpu().double().numpy()
    for bi in range(b):
        for h in range(hkv):
            kh = torch.cat([pk[0, :, h], sk[bi, :, h]]).float().numpy()
            vh = torch.cat([pv[0, :, h], sv[bi, :, h]]).float().numpy()
            al = orc.eviction_decisions(torch.cat([pl[0, :, h], sl[bi, :, h]]).numpy())
            ref = orc.decode_output(sq[bi, steps - 1, h * g:(h + 1) * g].float().numpy(), kh, vh, al,
                                    prompt + steps - 1, 16, scale)
            err = np.abs(out[bi, h * g:(h + 1) * g] - ref)
            assert np.all(err <= BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref))


def test_share_into_non_empty_sequence_is_refused(gpu):
    b, hkv, g, d = 3, 2, 4, 64
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, max_pages_per_unit=6, device=gpu)
    w = wl.Workload(name="share_case", kind="prefill", batch=b, kv_heads=hkv, group=g, head_dim=d,
                    dtype="bf16", context=200, evict_rate=0.5, seed=7501)
    _, k, v, logit = wl.prefill_inputs(w)
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    cache.compact()
    before = cache.n_slots.clone()
    cache.share_prefix(0, 1, 2)
    assert cache.status_word() & lib.DMS_STATUS_NOT_EMPTY
    assert torch.equal(cache.n_slots, before)
    check_accounting(cache)


def test_release_everything_returns_every_page(gpu):
    b, hkv, g, d = 4, 2, 4, 64
    (pk, pv, pl), _ = _prompt_and_steps(b, hkv, g, d, 900, 1, 0.6, 7601)
    cache = DmsCache(b, hkv, g, d, torch.bfloat16, max_pages_per_unit=20, device=gpu)
    pad = lambda x: torch.cat([x, torch.zeros((b - 1, *x.shape[1:]), dtype=x.dtype)]).to(gpu)  # noqa: E731
    cache.append(pad(pk), pad(pv), pad(pl))
    cache.release(1, b - 1)
    cache.compact()
    cache.share_prefix(0, 1, b - 1)
    check_accounting(cache)
    cache.release(0, b)
    check_accounting(cache)
    assert int(cache.free_top.item()) == cache.num_pages
    assert int(cache.page_ref.abs().sum().item()) == 0
