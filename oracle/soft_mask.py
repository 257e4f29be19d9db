"""Float64 CPU oracle for the training-form (relaxed) DMS attention mask.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute this module.

What the pages fix, and what is read into them
----------------------------------------------
* atlas.scime.ai summary of "Inference-Time Hyper-Scaling with KV Cache
  Compression", section "Approach": the per-head eviction decision is binary
  at inference and relaxed with a Gumbel-sigmoid while the model is
  retrofitted; eviction takes effect only after the delay window.
* zhaoyang97 Paper-Notes page, key-design section, item 2: the relaxation
  makes the token selection differentiable.

The pages print neither the noise distribution nor the temperature, nor how
the relaxed decision enters attention.  Reading taken (R18):

* relaxed decision  a~_j = sigmoid((logit_j + n_j) / tau), with the noise n_j
  an input (logistic noise, the difference of two Gumbel draws, for a
  Gumbel-sigmoid; zero for the noise-free relaxation) and tau > 0;
* key j keeps the weight factor (1 - a~_j) for every query i with
  i - j >= w (outside the delay window) and its full weight inside it, i.e.
  the additive log-mask  log(1 - a~_j) = -softplus((logit_j + n_j) / tau);
* as tau -> 0 with n = 0 this is the hard rule of ``dms_oracle`` (keep
  factor 1 for logit < 0, 0 for logit > 0).

Parity of this relaxation against the paper's own training code is
unpinned: only the limits and the closed forms tested in
``tests/test_oracle_pins.py`` fix it.
"""

from __future__ import annotations

import numpy as np

__all__ = ["relaxed_decision", "log_keep_factor", "soft_prefill_rows"]


def relaxed_decision(logit, noise, tau: float) -> np.ndarray:
    """a~ = sigmoid((logit + noise) / tau) in float64."""
    x = (np.asarray(logit, dtype=np.float64) + np.asarray(noise, dtype=np.float64)) / float(tau)
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def log_keep_factor(logit, noise, tau: float) -> np.ndarray:
    """log(1 - a~) = -log(1 + e^x), x = (logit + noise) / tau, in float64."""
    x = (np.asarray(logit, dtype=np.float64) + np.asarray(noise, dtype=np.float64)) / float(tau)
    return -np.logaddexp(0.0, x)


def soft_prefill_rows(q, k, v, logit, noise, tau: float, rows, window: int, scale: float) -> np.ndarray:
    """Relaxed-mask prefill attention for selected query rows of one sequence.

    q [S, Hq, D]; k, v [S, Hkv, D]; logit, noise [S, Hkv].  Row i of head hq
    (KV head h = hq // G) attends over keys j <= i with scores
    scale * <q_i, k_j> + (log_keep[j, h] if i - j >= window else 0).
    Returns [len(rows), Hq, D] float64.
    """
    if window < 1:
        raise ValueError("window must be >= 1")
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    log_keep = log_keep_factor(logit, noise, tau)                  # [S, Hkv]
    s_len, hq_n, _ = q.shape
    hkv_n = k.shape[1]
    if hq_n % hkv_n:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq_n // hkv_n
    rows = np.asarray(rows, dtype=np.int64)
    i = rows[:, None]
    j = np.arange(s_len)[None, :]
    causal = j <= i                                                 # [R, S]
    outside = (i - j) >= window
    out = np.empty((rows.shape[0], hq_n, q.shape[2]), dtype=np.float64)
    for h in range(hkv_n):
        bias = np.where(outside, log_keep[None, :, h], 0.0)         # [R, S]
        kh = k[:, h, :].astype(np.float64)
        vh = v[:, h, :].astype(np.float64)
        for g in range(group):
            hq = h * group + g
            qh = q[rows, hq, :].astype(np.float64)
            s = float(scale) * (qh @ kh.T) + bias
            s = np.where(causal, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            out[:, hq, :] = (e @ vh) / e.sum(axis=1, keepdims=True)
    return out
