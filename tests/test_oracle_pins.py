"""Pins of the float64 oracle against facts that do not come from the oracle.

Each test names what fixes the expected value: a library routine at a special
case the pages determine, a closed form, a hand-worked fixture, brute force,
or an invariant.  Mutation tests at the end plant mistakes in the oracle (on
the CPU) and check that the pins catch them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import bruteforce as bf
from oracle import dms_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dms_hand_examples.json")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _sdpa(q, k, v, mask, scale):
    """torch SDPA on CPU float64.  q [Hq, S, D], k, v [Hq, S, D], mask [S, S] bool (True = attend)."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q, dtype=torch.float64)[None],
        torch.as_tensor(k, dtype=torch.float64)[None],
        torch.as_tensor(v, dtype=torch.float64)[None],
        attn_mask=torch.as_tensor(mask)[None, None] if mask is not None else None,
        is_causal=mask is None,
        scale=scale,
    )[0].numpy()


def _random_seq(rng, s, hq, hkv, d):
    q = rng.standard_normal((s, hq, d))
    k = rng.standard_normal((s, hkv, d))
    v = rng.standard_normal((s, hkv, d))
    return q, k, v


def _gqa_expand(x, group):
    """[S, Hkv, D] -> [Hq, S, D] with query head hq reading KV head hq // group."""
    t = torch.as_tensor(x).permute(1, 0, 2)
    return t.repeat_interleave(group, dim=0).numpy()


# ---------------------------------------------------------------- decisions
def test_decision_threshold_and_specials():
    logit = np.array([-1.0, -0.0, 0.0, 1e-30, 1e-45, 2.5, np.nan, -np.inf, np.inf], dtype=np.float32)
    alpha = orc.eviction_decisions(logit)
    assert alpha.tolist() == [False, False, False, True, True, True, False, False, True]


def test_window_must_be_positive():
    with pytest.raises(ValueError):
        orc.visibility_mask(np.zeros(4, dtype=bool), 0)
    with pytest.raises(ValueError):
        orc.retained_positions(np.zeros(4, dtype=bool), 3, 0)


# ---------------------------------------------------------------- P1 / P2: library special cases
@pytest.mark.parametrize("group", [1, 2, 5])
def test_all_keep_is_dense_causal_attention(group):
    """Nothing marked: DMS attention is plain causal attention (torch SDPA, float64)."""
    rng = _rng(11 + group)
    s, hkv, d = 48, 2, 8
    q, k, v = _random_seq(rng, s, hkv * group, hkv, d)
    alpha = np.zeros((s, hkv), dtype=bool)
    scale = 1 / math.sqrt(d)
    ours = orc.prefill_attention(q, k, v, alpha, 16, scale)
    ref = _sdpa(q.transpose(1, 0, 2), _gqa_expand(k, group), _gqa_expand(v, group), None, scale)
    np.testing.assert_allclose(ours, ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [1, 3, 16])
def test_all_evict_is_sliding_window_attention(window):
    """Everything marked: each query sees exactly the last `window` tokens (SDPA with a band mask)."""
    rng = _rng(23 + window)
    s, hkv, group, d = 40, 2, 2, 4
    q, k, v = _random_seq(rng, s, hkv * group, hkv, d)
    alpha = np.ones((s, hkv), dtype=bool)
    scale = 1 / math.sqrt(d)
    i = np.arange(s)[:, None]
    j = np.arange(s)[None, :]
    band = (i - j >= 0) & (i - j < window)
    ours = orc.prefill_attention(q, k, v, alpha, window, scale)
    ref = _sdpa(q.transpose(1, 0, 2), _gqa_expand(k, group), _gqa_expand(v, group), band, scale)
    np.testing.assert_allclose(ours, ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_all_evict_sees_exactly_window_keys():
    alpha = np.ones(50, dtype=bool)
    for t in range(50):
        assert orc.retained_positions(alpha, t, 16).tolist() == list(range(max(0, t - 15), t + 1))


# ---------------------------------------------------------------- P3: closed-form retained count
@pytest.mark.parametrize("rate", [0.0, 0.5, 0.875, 1.0])
@pytest.mark.parametrize("window", [1, 2, 16])
def test_retained_count_closed_form(rate, window):
    """|R(t)| = #{j <= t - w : alpha_j = 0} + min(w, t + 1)."""
    rng = _rng(int(rate * 1000) + window)
    alpha = rng.random(200) < rate
    for t in range(200):
        closed = int(np.sum(~alpha[: max(0, t - window + 1)])) + min(window, t + 1)
        assert orc.retained_count(alpha, t, window) == closed


# ---------------------------------------------------------------- hand-worked fixtures
def test_golden_retained_sets():
    g = json.load(open(GOLDEN))["retained_sets"]
    alpha = np.ones(g["n_tokens"], dtype=bool)
    alpha[g["kept_positions"]] = False
    for case in g["cases"]:
        assert orc.retained_positions(alpha, case["t"], g["window"]).tolist() == case["retained"]


def _num(x):
    return math.log(3.0) if x == "ln3" else float(x)


def test_golden_decode_outputs():
    for case in json.load(open(GOLDEN))["decode_outputs"]["cases"]:
        k = np.array([[_num(x)] for x in case["k"]])
        v = np.array([[_num(x)] for x in case["v"]])
        q = np.array(case["q"], dtype=np.float64)
        out = orc.decode_output(q, k, v, np.array(case["alpha"], dtype=bool), case["t"],
                                case["window"], 1.0)
        np.testing.assert_allclose(out, np.array(case["out"]), rtol=0, atol=1e-14, err_msg=case["name"])


# ---------------------------------------------------------------- P4: brute force on tiny inputs
@pytest.mark.parametrize("window,n", [(1, 10), (2, 10), (3, 9), (4, 8)])
def test_oracle_matches_bruteforce_process(window, n):
    """Every decision vector of length n: the oracle's sets and outputs equal the process simulation."""
    rng = _rng(100 * window + n)
    d, group = 2, 3 if window == 3 else 2
    keys = rng.standard_normal((n, d))
    values = rng.standard_normal((n, d))
    qs = rng.standard_normal((n, group, d))
    scale = 0.7
    for bits in bf.all_decision_vectors(n):
        alpha = np.array(bits, dtype=bool)
        seen = bf.run_process(bits, window)
        outs = bf.decode_outputs(qs.tolist(), keys.tolist(), values.tolist(), bits, window, scale)
        for t in range(n):
            assert orc.retained_positions(alpha, t, window).tolist() == seen[t]
            ours = orc.decode_output(qs[t], keys, values, alpha, t, window, scale)
            np.testing.assert_allclose(ours, np.array(outs[t]), rtol=0, atol=1e-12)


def test_bruteforce_dims_one_and_four():
    rng = _rng(7)
    for d in (1, 4):
        n, window = 7, 2
        keys = rng.standard_normal((n, d))
        values = rng.standard_normal((n, d))
        qs = rng.standard_normal((n, 1, d))
        for bits in bf.all_decision_vectors(n):
            outs = bf.decode_outputs(qs.tolist(), keys.tolist(), values.tolist(), bits, window, 0.5)
            for t in range(n):
                ours = orc.decode_output(qs[t], keys, values, np.array(bits, bool), t, window, 0.5)
                np.testing.assert_allclose(ours, np.array(outs[t]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P5: compaction schedule
def test_compaction_schedule_invariance():
    """Every compact/no-compact schedule over 7 steps gives the same visible sets and outputs."""
    rng = _rng(5)
    n, d, window = 7, 3, 2
    keys = rng.standard_normal((n, d))
    values = rng.standard_normal((n, d))
    qs = rng.standard_normal((n, 2, d))
    for bits in bf.all_decision_vectors(n):
        alpha = np.array(bits, dtype=bool)
        ref = [orc.decode_output(qs[t], keys, values, alpha, t, window, 0.9) for t in range(n)]
        for sched in bf.all_decision_vectors(n):
            cache = orc.UnitCache(window, d)
            for t in range(n):
                cache.append(alpha[t:t + 1], keys[t:t + 1], values[t:t + 1])
                live_pos = cache.pos[cache.live()].tolist()
                assert live_pos == orc.retained_positions(alpha, t, window).tolist()
                np.testing.assert_allclose(cache.attend(qs[t], 0.9), ref[t], rtol=0, atol=1e-13)
                if sched[t]:
                    cache.compact()
                    assert cache.pos.tolist() == live_pos


# ---------------------------------------------------------------- P6 .. P9 invariants
def test_decode_equals_prefill_row():
    rng = _rng(9)
    s, hkv, group, d, window = 64, 2, 2, 8, 4
    q, k, v = _random_seq(rng, s, hkv * group, hkv, d)
    alpha = rng.random((s, hkv)) < 0.6
    pre = orc.prefill_attention(q, k, v, alpha, window, 0.3)
    for h in range(hkv):
        cache = orc.UnitCache(window, d)
        for t in range(s):
            cache.append(alpha[t:t + 1, h], k[t:t + 1, h], v[t:t + 1, h])
            out = cache.attend(q[t, h * group:(h + 1) * group], 0.3)
            np.testing.assert_allclose(out, pre[t, h * group:(h + 1) * group], rtol=0, atol=1e-12)
            if t % 5 == 4:
                cache.compact()


def test_first_step_returns_first_value_exactly():
    rng = _rng(3)
    v0 = rng.standard_normal((1, 16))
    out = orc.decode_output(rng.standard_normal((4, 16)), rng.standard_normal((1, 16)), v0,
                            np.array([True]), 0, 16, 0.25)
    assert np.array_equal(out, np.repeat(v0, 4, axis=0))


def test_constant_values_give_constant_output():
    rng = _rng(4)
    n, d = 100, 8
    v = np.full((n, d), 1.375)
    alpha = rng.random(n) < 0.8
    for t in (0, 17, 99):
        out = orc.decode_output(rng.standard_normal((3, d)) * 4, rng.standard_normal((n, d)), v,
                                alpha, t, 16, 1.0)
        np.testing.assert_allclose(out, 1.375, rtol=0, atol=1e-14)


def test_eviction_is_permanent():
    rng = _rng(8)
    alpha = rng.random(300) < 0.9
    for t in range(299):
        now = set(orc.retained_positions(alpha, t, 16).tolist())
        nxt = set(orc.retained_positions(alpha, t + 1, 16).tolist())
        assert nxt <= now | {t + 1}
        assert t + 1 in nxt


def test_equal_scores_average_retained_values():
    """All-zero keys: attention is the plain mean over R(t) (closed form, no softmax needed)."""
    rng = _rng(12)
    n, d = 80, 5
    alpha = rng.random(n) < 0.7
    v = rng.standard_normal((n, d))
    for t in (0, 15, 16, 40, 79):
        r = [j for j in range(t + 1) if not alpha[j] or t - j < 16]
        expect = np.mean(v[r], axis=0)
        out = orc.decode_output(rng.standard_normal((2, d)), np.zeros((n, d)), v, alpha, t, 16, 1.0)
        np.testing.assert_allclose(out, np.vstack([expect, expect]), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- mutation tests
def _pins_pass(monkeypatch, mutated_mask=None, mutated_softmax=None):
    if mutated_mask is not None:
        monkeypatch.setattr(orc, "visibility_mask", mutated_mask)
    if mutated_softmax is not None:
        monkeypatch.setattr(orc, "softmax_attention", mutated_softmax)
    try:
        test_all_evict_is_sliding_window_attention(16)
        test_all_keep_is_dense_causal_attention(2)
        test_golden_decode_outputs()
        test_golden_retained_sets()
    except AssertionError:
        return False
    return True


def test_pins_pass_unmutated(monkeypatch):
    assert _pins_pass(monkeypatch)


def test_pins_catch_window_off_by_one(monkeypatch):
    real = orc.visibility_mask

    def off_by_one(alpha, window, rows=None):
        return real(alpha, window + 1, rows)

    assert not _pins_pass(monkeypatch, mutated_mask=off_by_one)


def test_pins_catch_inverted_decision(monkeypatch):
    real = orc.visibility_mask

    def inverted(alpha, window, rows=None):
        return real(~np.asarray(alpha, dtype=bool), window, rows)

    assert not _pins_pass(monkeypatch, mutated_mask=inverted)


def test_pins_catch_missing_causal_bound(monkeypatch):
    def acausal(alpha, window, rows=None):
        alpha = np.asarray(alpha, dtype=bool)
        s = alpha.shape[0]
        i = (np.arange(s) if rows is None else np.asarray(rows))[:, None]
        j = np.arange(s)[None, :]
        return ~(alpha[None, :] & ((i - j) >= window))

    assert not _pins_pass(monkeypatch, mutated_mask=acausal)


def test_pins_catch_transposed_contraction(monkeypatch):
    def transposed(q, k, v, scale):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        s = scale * (q @ k.T)
        e = np.exp(s - s.max(axis=0, keepdims=True))   # normalised over the wrong axis
        return (e @ v) / e.sum(axis=0, keepdims=True).sum()

    assert not _pins_pass(monkeypatch, mutated_softmax=transposed)


def test_mask_rows_match_full_mask():
    rng = _rng(21)
    alpha = rng.random(90) < 0.6
    full = orc.visibility_mask(alpha, 16)
    rows = np.array([0, 5, 15, 16, 17, 60, 89])
    assert np.array_equal(orc.visibility_mask(alpha, 16, rows), full[rows])


# ---------------------------------------------------------------- is_visible, the rule itself
def _is_visible_pins(fn):
    """Check a visibility predicate fn(i, j, alpha_j, w) against (a) the brute-force
    process simulation (a token enters when produced; a marked token is removed
    once `w` more tokens have been produced) over every decision vector of small
    lengths, and (b) the hand-worked retained sets of the golden fixture."""
    for window, n in ((1, 8), (2, 8), (3, 7), (4, 7)):
        for bits in bf.all_decision_vectors(n):
            seen = bf.run_process(bits, window)
            for i in range(n):
                got = [j for j in range(n) if fn(i, j, bits[j], window)]
                assert got == seen[i], (bits, window, i)
    g = json.load(open(GOLDEN))["retained_sets"]
    alpha = [j not in g["kept_positions"] for j in range(g["n_tokens"])]
    for case in g["cases"]:
        t = case["t"]
        got = [j for j in range(g["n_tokens"]) if fn(t, j, alpha[j], g["window"])]
        assert got == case["retained"], t


def test_is_visible_matches_process_and_hand_worked_sets():
    _is_visible_pins(orc.is_visible)


def test_is_visible_agrees_with_visibility_mask():
    """The scalar rule and the mask builder state the same set (element by element)."""
    rng = _rng(31)
    for window in (1, 2, 16):
        alpha = rng.random(70) < 0.7
        mask = orc.visibility_mask(alpha, window)
        for i in range(70):
            for j in range(70):
                assert mask[i, j] == orc.is_visible(i, j, alpha[j], window)


def test_is_visible_rejects_a_zero_window():
    with pytest.raises(ValueError):
        orc.is_visible(3, 1, True, 0)


@pytest.mark.parametrize("mutation", ["late_by_one", "early_by_one", "acausal", "decision_ignored"])
def test_is_visible_pins_catch_planted_mistakes(mutation):
    """Plausible mistakes in the predicate fail the pins above."""
    def planted(i, j, alpha_j, window):
        if mutation == "late_by_one":
            return (j <= i) and not (bool(alpha_j) and (i - j) > window)
        if mutation == "early_by_one":
            return (j <= i) and not (bool(alpha_j) and (i - j) >= window - 1)
        if mutation == "acausal":
            return not (bool(alpha_j) and (i - j) >= window)
        return j <= i
    with pytest.raises(AssertionError):
        _is_visible_pins(planted)
