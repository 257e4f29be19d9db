"""dms_export_retained against the oracle's cache mirror, bit for bit.

The retained set R(t) of every unit (positions, decisions, K and V rows) read
back through the C ABI must equal the live slots of oracle.dms_oracle.UnitCache
after the same appends and compactions; with all_slots the dead slots not yet
compacted come along, in slot order.  Counts also equal the closed form
#{j <= t - w : alpha_j = 0} + min(w, t + 1) (pin P3).
"""

import numpy as np
import pytest
import torch

import workloads as wl
from decode_attention_learned_amd import DmsCache
from harness import HostModel, say
from oracle import dms_oracle as orc

pytestmark = pytest.mark.gpu


def _build(gpu, b, hkv, g, d, dtype, prompt, steps, rate, seed, compact_at=()):
    w = wl.Workload(name="export_case", kind="decode", batch=b, kv_heads=hkv, group=g, head_dim=d,
                    dtype="f32" if dtype == torch.float32 else "bf16", context=prompt,
                    evict_rate=rate, seed=seed, steps=steps, prompt_chunk=prompt, compact_every=16)
    rates = wl.unit_eviction_rates(w)
    cache = DmsCache(b, hkv, g, d, dtype, max_pages_per_unit=(prompt + steps) // 64 + 3,
                     device=gpu)
    model = HostModel(b, hkv, g, d, w.window)
    k, v, logit = wl.prompt_chunk_inputs(w, 0, prompt, rates=rates)
    cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
    model.append(k, v, logit)
    cache.compact()
    model.compact()
    alphas = [orc.eviction_decisions(logit.numpy())]
    for step in range(steps):
        _, k, v, logit = wl.decode_step_inputs(w, step, rates=rates)
        cache.append(k.to(gpu), v.to(gpu), logit.to(gpu))
        model.append(k, v, logit)
        alphas.append(orc.eviction_decisions(logit.numpy()))
        if step in compact_at:
            cache.compact()
            model.compact()
    torch.cuda.synchronize()
    return cache, model, np.concatenate(alphas, axis=1)   # alpha [B, T, Hkv]


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64),
                                     (torch.float32, 128)])
def test_export_matches_oracle_bit_for_bit(gpu, dtype, d):
    b, hkv, g = 2, 3, 2
    cache, model, alpha = _build(gpu, b, hkv, g, d, dtype, 300, 45, 0.7, 9100 + d,
                                 compact_at=(9, 30))
    count, pos, al, k, v = (x.cpu() if x is not None else None for x in cache.export())
    cnt_all, pos_all, al_all, k_all, v_all = (x.cpu() for x in cache.export(all_slots=True))
    w = 16
    for u, uc in enumerate(model.units):
        bi, h = divmod(u, hkv)
        t = uc.length - 1
        live = uc.live(t)
        n = int(live.sum())
        assert int(count[u]) == n == orc.retained_count(alpha[bi, :, h], t, w)
        closed = int(np.sum(~alpha[bi, : max(0, t - w + 1), h])) + min(w, t + 1)
        assert n == closed
        assert pos[u, :n].tolist() == uc.pos[live].tolist()
        assert pos[u, :n].tolist() == orc.retained_positions(alpha[bi, :, h], t, w).tolist()
        assert (al[u, :n].numpy() != 0).tolist() == uc.alpha[live].tolist()
        assert np.array_equal(k[u, :n].float().numpy(), uc.k[live])
        assert np.array_equal(v[u, :n].float().numpy(), uc.v[live])
        # every slot in use, dead ones included
        m = uc.n_slots
        assert int(cnt_all[u]) == m == int(cache.n_slots[u].item())
        assert pos_all[u, :m].tolist() == uc.pos.tolist()
        assert (al_all[u, :m].numpy() != 0).tolist() == uc.alpha.tolist()
        assert np.array_equal(k_all[u, :m].float().numpy(), uc.k)
        assert np.array_equal(v_all[u, :m].float().numpy(), uc.v)
    assert int((cnt_all - count).sum()) > 0, "expected dead slots not yet compacted"


def test_export_truncates_rows_but_counts_all(gpu):
    cache, model, _ = _build(gpu, 1, 2, 1, 64, torch.bfloat16, 200, 10, 0.5, 9201)
    full = cache.export()
    cut = cache.export(max_per_unit=7)
    assert torch.equal(full[0], cut[0])
    assert cut[1].shape == (2, 7)
    assert torch.equal(cut[1], full[1][:, :7])
    assert torch.equal(cut[3], full[3][:, :7])
    none = cache.export(max_per_unit=0, kv=False)
    assert torch.equal(none[0], full[0])


def test_export_of_an_empty_cache(gpu):
    cache = DmsCache(2, 2, 2, 64, torch.bfloat16, max_pages_per_unit=2, device=gpu)
    count, pos, _, _, _ = cache.export(max_per_unit=4)
    assert count.cpu().tolist() == [0, 0, 0, 0]
    assert torch.count_nonzero(pos) == 0
    say("export of an empty cache: counts 0")
