"""Plain float64 CPU oracle for Dynamic Memory Sparsification (DMS) attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute this module.
The product package (``decode_attention_learned_amd``) never imports it and it
never imports the product package: the two share no code.

What is computed, and where the pages state it
----------------------------------------------
Pages are cited by site and section, as a reader of the pages finds them:

* [scime/Approach]  atlas.scime.ai summary of "Inference-Time Hyper-Scaling with
  KV Cache Compression" (arXiv 2506.05345), section "Approach": each KV head
  makes a learned binary eviction decision per token (Gumbel-sigmoid during
  training), and an eviction is carried out only after a delay window.
* [scime/Effects]   same page, table "Measured effects reported in the paper"
  and "Surprising findings": the delay window is 16 tokens, versus eviction
  at once.
* [chatpaper/Abstract]  chatpaper.ai page, English abstract: DMS postpones
  eviction instead of dropping cached tokens early.
* [notes/Motivation]  zhaoyang97 Paper-Notes page on the same paper, section
  研究背景与动机 (motivation): each decode step reads the whole KV cache, and
  the cache grows linearly with the sequence.
* [notes/DMS-design]  same notes page, section 关键设计 (key design), item 2:
  one decision function per layer and head, relaxed with Gumbel-sigmoid.

Readings taken where the pages are silent (numbered as in the design notes):

* R1  decision: a token is marked for eviction iff its logit is > 0 (the
      sigmoid exceeds 1/2), compared in float32; +-0 and NaN mean keep.
* R2  window: a marked token j is still visible to query i while i - j < w;
      the query token always sees itself.
* R3  the decision of token j is known when j is appended.
* R4  order within a decode step: append token t, then attend with query t.
* R7  grouped-query attention: query head hq reads KV head hq // G.
* R11 the retained set is ordered by ascending position; compaction is stable.
* R12 prompt tokens are decided like generated tokens.
* R14 no attention sinks: nothing is kept except by the rule above.

Every function below is written for clarity, not speed; the only library
primitives used are matrix products, ``max``, ``exp`` and ``sum``.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "eviction_decisions",
    "is_visible",
    "visibility_mask",
    "retained_positions",
    "retained_count",
    "softmax_attention",
    "decode_output",
    "prefill_attention",
    "prefill_rows",
    "UnitCache",
]


# ---------------------------------------------------------------------------
# Step 1: the per-head, per-token binary decision  [scime/Approach], R1
# ---------------------------------------------------------------------------
def eviction_decisions(logit) -> np.ndarray:
    """alpha = 1 (evict after the window) iff sigmoid(logit) > 1/2, i.e. logit > 0.

    The inference form of the Gumbel-sigmoid decision of [scime/Approach] and
    [notes/DMS-design]: with the noise off, the relaxed mask is sigmoid(logit)
    and the binary decision thresholds it at one half.  The compare is done
    in float32, the precision the logits are handed over in (R1).
    """
    return np.asarray(logit, dtype=np.float32) > np.float32(0.0)


# ---------------------------------------------------------------------------
# Steps 2-3: delayed eviction  [scime/Approach], [scime/Effects], R2, R3
# ---------------------------------------------------------------------------
def is_visible(i: int, j: int, alpha_j: bool, window: int) -> bool:
    """May query position i attend to key position j?

    Causal (j <= i), and a token marked for eviction leaves once it is
    `window` positions old: it is seen by queries j .. j + window - 1.
    """
    if window < 1:
        raise ValueError("window must be >= 1")
    return (j <= i) and not (bool(alpha_j) and (i - j) >= window)


def visibility_mask(alpha, window: int, rows=None) -> np.ndarray:
    """Boolean mask M[i, j] = is_visible(i, j, alpha[j], window): [S, S], or
    [len(rows), S] for the query rows given."""
    if window < 1:
        raise ValueError("window must be >= 1")
    alpha = np.asarray(alpha, dtype=bool)
    s = alpha.shape[0]
    i = (np.arange(s) if rows is None else np.asarray(rows, dtype=np.int64))[:, None]
    j = np.arange(s)[None, :]
    return (j <= i) & ~(alpha[None, :] & ((i - j) >= window))


def retained_positions(alpha, t: int, window: int) -> np.ndarray:
    """R(t): the positions j <= t still in the cache after token t is appended,
    ascending (R11).  Row t of :func:`visibility_mask`."""
    if window < 1:
        raise ValueError("window must be >= 1")
    alpha = np.asarray(alpha, dtype=bool)
    j = np.arange(t + 1)
    keep = ~alpha[: t + 1] | ((t - j) < window)
    return j[keep]


def retained_count(alpha, t: int, window: int) -> int:
    """|R(t)|, counted from the set itself (the closed form is a test pin)."""
    return int(retained_positions(alpha, t, window).shape[0])


# ---------------------------------------------------------------------------
# Step 5: attention over the retained entries  [notes/Motivation]
# ---------------------------------------------------------------------------
def softmax_attention(q, k, v, scale: float) -> np.ndarray:
    """softmax(scale * q k^T) v in float64.  q [G, D], k [N, D], v [N, D] -> [G, D].

    The row maximum is subtracted before exp; that changes no value in exact
    arithmetic and keeps exp in range.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        raise ValueError("attention over an empty set")
    s = float(scale) * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return (e @ v) / e.sum(axis=1, keepdims=True)


def decode_output(q, k_hist, v_hist, alpha_hist, t: int, window: int, scale: float) -> np.ndarray:
    """Decode step t of one (sequence, KV head) unit.

    q [G, D] are the G query heads of the group (R7); k_hist / v_hist [>t, D]
    and alpha_hist [>t] hold every token of the unit by position.  The query
    attends over R(t) only (R4: token t was appended first).
    """
    r = retained_positions(alpha_hist, t, window)
    k_hist = np.asarray(k_hist)
    v_hist = np.asarray(v_hist)
    return softmax_attention(q, k_hist[r], v_hist[r], scale)


def prefill_rows(q, k, v, alpha, rows, window: int, scale: float) -> np.ndarray:
    """Masked prefill attention for selected query rows of one sequence.

    q [S, Hq, D]; k, v [S, Hkv, D]; alpha [S, Hkv] bool.  Row i of head hq
    attends over {j : is_visible(i, j, alpha[j, hq // G], window)}, the same
    set as R(i) (R12: prompt tokens follow the decode rule).  Returns
    [len(rows), Hq, D] float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    alpha = np.asarray(alpha, dtype=bool)
    s_len, hq_n, _ = q.shape
    hkv_n = k.shape[1]
    if hq_n % hkv_n:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq_n // hkv_n
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], hq_n, q.shape[2]), dtype=np.float64)
    for h in range(hkv_n):
        mask = visibility_mask(alpha[:, h], window, rows)          # [R, S]
        kh = k[:, h, :].astype(np.float64)
        vh = v[:, h, :].astype(np.float64)
        for g in range(group):
            hq = h * group + g
            qh = q[rows, hq, :].astype(np.float64)                  # [R, D]
            s = float(scale) * (qh @ kh.T)                           # [R, S]
            s = np.where(mask, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)                                        # exp(-inf) = 0
            out[:, hq, :] = (e @ vh) / e.sum(axis=1, keepdims=True)
    return out


def prefill_attention(q, k, v, alpha, window: int, scale: float) -> np.ndarray:
    """All rows of :func:`prefill_rows` for one sequence: [S, Hq, D] float64."""
    return prefill_rows(q, k, v, alpha, np.arange(np.asarray(q).shape[0]), window, scale)


# ---------------------------------------------------------------------------
# Step 4: the cache as a container between compactions
# ---------------------------------------------------------------------------
class UnitCache:
    """What one (sequence, KV head) unit's cache holds, in slot order.

    Tokens are appended at the tail (the cache grows by one entry per token,
    [notes/Motivation]).  A marked token whose window has passed is dead: it
    is skipped by attention at once (the rule of :func:`is_visible`) and its
    slot is given back only by :meth:`compact`, which keeps the survivors in
    order (R11).  After ``compact(t)`` the slots hold exactly R(t).  Between
    compactions they hold R(t_c) followed by the tokens appended since.
    """

    def __init__(self, window: int, head_dim: int, dtype=np.float64):
        if window < 1:
            raise ValueError("window must be >= 1")
        self.window = int(window)
        self._pos = np.zeros((0,), dtype=np.int64)
        self._alpha = np.zeros((0,), dtype=bool)
        self._k = np.zeros((0, head_dim), dtype=dtype)
        self._v = np.zeros((0, head_dim), dtype=dtype)
        self._pending = []   # appended (pos, alpha, k, v) blocks not yet joined
        self.length = 0      # positions consumed by the sequence

    def append(self, alpha, k, v) -> None:
        """Append n tokens at positions length .. length + n - 1."""
        alpha = np.asarray(alpha, dtype=bool).reshape(-1)
        n = alpha.shape[0]
        pos = np.arange(self.length, self.length + n, dtype=np.int64)
        self._pending.append((pos, alpha.copy(),
                              np.array(k, dtype=self._k.dtype).reshape(n, -1),
                              np.array(v, dtype=self._v.dtype).reshape(n, -1)))
        self.length += n

    def _join(self) -> None:
        """Join pending appends onto the slot arrays (storage only, order kept)."""
        if self._pending:
            self._pos = np.concatenate([self._pos] + [p[0] for p in self._pending])
            self._alpha = np.concatenate([self._alpha] + [p[1] for p in self._pending])
            self._k = np.concatenate([self._k] + [p[2] for p in self._pending])
            self._v = np.concatenate([self._v] + [p[3] for p in self._pending])
            self._pending = []

    @property
    def pos(self) -> np.ndarray:
        self._join()
        return self._pos

    @property
    def alpha(self) -> np.ndarray:
        self._join()
        return self._alpha

    @property
    def k(self) -> np.ndarray:
        self._join()
        return self._k

    @property
    def v(self) -> np.ndarray:
        self._join()
        return self._v

    def skip(self, n: int) -> None:
        """Advance the position counter by n tokens that were not stored."""
        self.length += int(n)

    def live(self, t: int | None = None) -> np.ndarray:
        """Boolean per slot: visible to the query at position t (default: last)."""
        if t is None:
            t = self.length - 1
        return ~self.alpha | ((t - self.pos) < self.window)

    def compact(self, t: int | None = None) -> None:
        """Drop dead slots, keeping the order of the survivors."""
        keep = self.live(t)
        self._pos = self._pos[keep]
        self._alpha = self._alpha[keep]
        self._k = self._k[keep]
        self._v = self._v[keep]

    def attend(self, q, scale: float) -> np.ndarray:
        """Decode output for the G queries q [G, D] at position length - 1."""
        keep = self.live()
        return softmax_attention(q, self.k[keep], self.v[keep], scale)

    @property
    def n_slots(self) -> int:
        return int(self.pos.shape[0])
