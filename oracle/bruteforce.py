"""Brute-force DMS enumerator in pure Python floats (no NumPy).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

This is a second, operational statement of the same mechanism, written so
that it shares no formula with :mod:`oracle.dms_oracle`: instead of a
visibility predicate it runs the cache as a process in time, the way the
pages describe it.  Each token enters the cache when it is produced; a token
whose binary decision is "evict" is put on a pending list and physically
removed once the delay window has elapsed (atlas.scime.ai summary of
"Inference-Time Hyper-Scaling with KV Cache Compression", section "Approach";
the 16-token window in its table "Measured effects reported in the paper").
Attention is a double loop with ``math.exp``.

Its purpose is to pin the oracle on tiny inputs: for every decision vector of
length n <= 10 the two must give the same retained sets and outputs.
"""

from __future__ import annotations

import math
from itertools import product


def run_process(alphas, window):
    """Simulate the cache step by step.

    alphas: list of 0/1 decisions, one per token (token t is produced at step t).
    Returns a list whose entry t is the list of positions the query of step t
    reads, in the order they sit in the cache.
    """
    if window < 1:
        raise ValueError("window must be >= 1")
    cache = []            # positions, oldest first
    due = {}              # step -> positions whose removal falls due at that step
    seen = []
    for t, a in enumerate(alphas):
        # removals that fall due before the query of step t reads the cache
        for p in due.pop(t, []):
            cache.remove(p)
        cache.append(t)
        if a:
            # marked now; removed when `window` more tokens have been produced
            due.setdefault(t + window, []).append(t)
        seen.append(list(cache))
    return seen


def attend(q, keys, values, scale):
    """Softmax attention of one query over explicit key/value lists, in floats."""
    scores = []
    for k in keys:
        dot = 0.0
        for a, b in zip(q, k):
            dot += a * b
        scores.append(scale * dot)
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = sum(weights)
    out = [0.0] * len(values[0])
    for w_, v in zip(weights, values):
        for d in range(len(out)):
            out[d] += w_ * v[d]
    return [o / total for o in out]


def decode_outputs(q_steps, keys, values, alphas, window, scale):
    """Outputs of every decode step for one unit.

    q_steps[t][g] is query head g at step t; keys[t], values[t] are token t's
    vectors.  Returns out[t][g] = list of D floats.
    """
    seen = run_process(alphas, window)
    outs = []
    for t, positions in enumerate(seen):
        ks = [keys[p] for p in positions]
        vs = [values[p] for p in positions]
        outs.append([attend(qg, ks, vs, scale) for qg in q_steps[t]])
    return outs


def all_decision_vectors(n):
    """Every 0/1 vector of length n."""
    return [list(bits) for bits in product((0, 1), repeat=n)]
