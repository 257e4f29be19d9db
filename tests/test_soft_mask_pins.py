"""Pins of the relaxed-mask oracle (oracle/soft_mask.py) against facts that do
not come from it: the hard rule as the zero-temperature limit, dense causal
attention when nothing is marked, and hand-derived closed forms.  Mutation
tests plant mistakes in the oracle on the CPU and check the pins catch them.
"""

import math

import numpy as np
import pytest
import torch

from oracle import dms_oracle as orc
from oracle import soft_mask as sm


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _seq(rng, s, hq, hkv, d):
    return (rng.standard_normal((s, hq, d)), rng.standard_normal((s, hkv, d)),
            rng.standard_normal((s, hkv, d)))


def test_relaxed_decision_values():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4 (closed forms)
    a = sm.relaxed_decision([0.0, math.log(3.0), -math.log(3.0)], [0.0, 0.0, 0.0], 1.0)
    assert np.allclose(a, [0.5, 0.75, 0.25], rtol=0, atol=1e-15)
    # temperature scales the argument: logit 2 ln 3 at tau = 2 is sigmoid(ln 3)
    assert abs(sm.relaxed_decision(2 * math.log(3.0), 0.0, 2.0) - 0.75) < 1e-15
    # noise adds to the logit
    assert abs(sm.relaxed_decision(0.0, math.log(3.0), 1.0) - 0.75) < 1e-15
    # log(1 - a~) at large arguments stays finite and ~ -x
    assert abs(sm.log_keep_factor(800.0, 0.0, 1.0) + 800.0) < 1e-12


@pytest.mark.parametrize("window", [1, 4, 16])
def test_zero_temperature_is_the_hard_rule(window):
    """tau -> 0 without noise: keep factor 0 for logit > 0 and 1 for logit < 0,
    i.e. exactly the hard DMS mask (logits kept away from 0)."""
    rng = _rng(40 + window)
    s, hq, hkv, d = 60, 4, 2, 8
    q, k, v = _seq(rng, s, hq, hkv, d)
    logit = rng.standard_normal((s, hkv))
    logit = np.where(np.abs(logit) < 0.05, 0.5, logit)
    noise = np.zeros_like(logit)
    rows = np.arange(s)
    soft = sm.soft_prefill_rows(q, k, v, logit, noise, 1e-4, rows, window, 0.3)
    hard = orc.prefill_rows(q, k, v, orc.eviction_decisions(logit), rows, window, 0.3)
    assert np.max(np.abs(soft - hard)) < 1e-12


def test_nothing_marked_is_causal_sdpa():
    """Very negative logits: every keep factor is 1 (log factor 0), so the
    relaxed mask is plain causal attention (torch SDPA, CPU float64)."""
    rng = _rng(50)
    s, hq, hkv, d = 40, 4, 2, 8
    q, k, v = _seq(rng, s, hq, hkv, d)
    logit = np.full((s, hkv), -1e4)
    out = sm.soft_prefill_rows(q, k, v, logit, np.zeros_like(logit), 1.0, np.arange(s), 16, 0.25)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q).permute(1, 0, 2)[None],
        torch.as_tensor(k).permute(1, 0, 2).repeat_interleave(2, 0)[None],
        torch.as_tensor(v).permute(1, 0, 2).repeat_interleave(2, 0)[None],
        is_causal=True, scale=0.25)[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


@pytest.mark.parametrize("logit,noise,tau,v0", [
    (0.0, 0.0, 1.0, 3.0),                    # a~ = 1/2: (v0/2 + 0) / (1/2 + 1) = 1 for v0 = 3
    (math.log(3.0), 0.0, 1.0, 5.0),          # a~ = 3/4: (v0/4) / (1/4 + 1) = 1 for v0 = 5
    (0.0, math.log(3.0), 1.0, 5.0),          # same through the noise
    (2 * math.log(3.0), 0.0, 2.0, 5.0),      # same through the temperature
    (-math.log(3.0), 0.0, 1.0, 7.0 / 3.0),   # a~ = 1/4: (3 v0 / 4) / (3/4 + 1) = 1 for v0 = 7/3
])
def test_two_key_closed_form(logit, noise, tau, v0):
    """Query 1 with window 1 sees key 0 outside the window (factor 1 - a~) and
    itself inside it (factor 1); equal scores (zero keys) and v1 = 0 give
    out = (1 - a~) v0 / (2 - a~), worked out by hand to 1 in every case."""
    q = np.ones((2, 1, 1))
    k = np.zeros((2, 1, 1))
    v = np.array([[[v0]], [[0.0]]])
    out = sm.soft_prefill_rows(q, k, v, np.array([[logit], [-5.0]]), np.array([[noise], [0.0]]), tau,
                               [1], 1, 1.0)
    assert abs(out[0, 0, 0] - 1.0) < 1e-14


def test_window_keys_carry_no_factor():
    """Inside the window the factor is 1 whatever the logit: with every key
    marked hard (logit 50) and tau 1, a query of window 16 sees its last 16
    keys with full weight and the older ones with weight e^-50 ~ 0, i.e.
    sliding-window attention to 1e-12 (older factor e^-50 ~ 2e-22)."""
    rng = _rng(60)
    s, hq, hkv, d = 50, 2, 1, 4
    q, k, v = _seq(rng, s, hq, hkv, d)
    logit = np.full((s, hkv), 50.0)
    out = sm.soft_prefill_rows(q, k, v, logit, np.zeros_like(logit), 1.0, np.arange(s), 16, 0.5)
    hard = orc.prefill_rows(q, k, v, np.ones((s, hkv), bool), np.arange(s), 16, 0.5)
    assert np.max(np.abs(out - hard)) < 1e-12


def _pins_pass(monkeypatch, mutated=None):
    if mutated is not None:
        monkeypatch.setattr(sm, "log_keep_factor", mutated)
    try:
        for case in [(0.0, 0.0, 1.0, 3.0), (math.log(3.0), 0.0, 1.0, 5.0), (2 * math.log(3.0), 0.0, 2.0, 5.0)]:
            test_two_key_closed_form(*case)
        test_zero_temperature_is_the_hard_rule(4)
        test_window_keys_carry_no_factor()
    except AssertionError:
        return False
    return True


def test_pins_pass_unmutated(monkeypatch):
    assert _pins_pass(monkeypatch)


def test_pins_catch_wrong_sign(monkeypatch):
    def plus(logit, noise, tau):
        x = (np.asarray(logit, np.float64) + np.asarray(noise, np.float64)) / tau
        return np.logaddexp(0.0, x)
    assert not _pins_pass(monkeypatch, plus)


def test_pins_catch_temperature_ignored(monkeypatch):
    def no_tau(logit, noise, tau):
        return -np.logaddexp(0.0, np.asarray(logit, np.float64) + np.asarray(noise, np.float64))
    assert not _pins_pass(monkeypatch, no_tau)


def test_pins_catch_keep_probability_swapped(monkeypatch):
    def swapped(logit, noise, tau):   # log(a~) instead of log(1 - a~)
        x = (np.asarray(logit, np.float64) + np.asarray(noise, np.float64)) / tau
        return -np.logaddexp(0.0, -x)
    assert not _pins_pass(monkeypatch, swapped)
