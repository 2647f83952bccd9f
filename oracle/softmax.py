"""Softmax pieces in fp64: safe softmax, the per-tile online update, merging.

TEST INFRASTRUCTURE (see the package docstring).  Every function here works
on plain NumPy arrays in float64 and follows one passage of the pages:

* safe_softmax          -- "What is FlashAttention?", "Start with a safe
                           softmax": subtract the row maximum, and return all
                           zeros for a row whose every score is masked.
* online_softmax_tiles  -- flash-attn-triton docs, "Tiling softmax is exact
                           algebra", Fig. 3: running max m, running sum l,
                           correction alpha, unnormalised accumulator, one
                           divide after the last tile, L = m + log l.  Fig. 3
                           works in base 2 (exp2 with log2(e) folded into the
                           scores); the same steps are taken here in base 2 and
                           L is returned in natural-log units.
* partial_softmax_state,
  merge_partials        -- "What is FlashAttention?", "What you will build",
                           item 01 ("merging two partial results"): the pages
                           name the merge without printing it; it is the Fig. 3
                           correction applied to two blocks of keys at once.
"""

from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634  # log2(e)
LN2 = 0.6931471805599453    # ln(2)


def safe_softmax(scores: np.ndarray) -> np.ndarray:
    """Row softmax over the last axis with the row maximum subtracted.

    Entries equal to -inf are masked out.  A row whose entries are all -inf
    has no visible key: its weights are all zero and no NaN is produced.
    """
    s = np.asarray(scores, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    live = np.isfinite(m)
    shifted = np.where(live, s - np.where(live, m, 0.0), -np.inf)
    e = np.exp(shifted)
    denom = np.sum(e, axis=-1, keepdims=True)
    return np.where(live, e / np.where(live, denom, 1.0), 0.0)


def partial_softmax_state(scores: np.ndarray, values: np.ndarray):
    """State (m, l, acc) of one block of keys, in natural-log units.

    ``scores``: [R, n] scaled scores (-inf = masked), ``values``: [n, d].
    m is the row maximum, l = sum exp(s - m), acc = exp(s - m) @ values.
    An empty or fully masked block has m = -inf, l = 0, acc = 0.
    """
    s = np.asarray(scores, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    R = s.shape[0]
    if s.shape[1] == 0:
        return (np.full(R, -np.inf), np.zeros(R), np.zeros((R, v.shape[1])))
    m = np.max(s, axis=1)
    live = np.isfinite(m)
    p = np.where(live[:, None], np.exp(s - np.where(live, m, 0.0)[:, None]), 0.0)
    return m, p.sum(axis=1), p @ v


def merge_partials(a, b):
    """Merge two partial states (m, l, acc) over disjoint key sets.

    With m = max(m1, m2) each partial is rescaled by exp(m_k - m); a partial
    with m_k = -inf (no visible key) contributes nothing.
    """
    m1, l1, a1 = a
    m2, l2, a2 = b
    m = np.maximum(m1, m2)
    live = np.isfinite(m)
    mref = np.where(live, m, 0.0)
    c1 = np.where(np.isfinite(m1), np.exp(m1 - mref), 0.0)
    c2 = np.where(np.isfinite(m2), np.exp(m2 - mref), 0.0)
    return m, l1 * c1 + l2 * c2, a1 * c1[:, None] + a2 * c2[:, None]


def finish_state(state):
    """Output and natural-log logsumexp of a complete state: O = acc / l."""
    m, l, acc = state
    live = l > 0
    o = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
    L = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, L


def online_softmax_tiles(scores: np.ndarray, values: np.ndarray, tile: int):
    """The Fig. 3 recurrence over key tiles of width ``tile`` (base 2).

    ``scores``: [R, n] scaled scores, natural units (-inf = masked);
    ``values``: [n, d].  Returns (O, L) with L in natural-log units.
    The scores are moved to base 2 once (qk = s * log2 e), then per tile:
    m_new = max(m, rowmax qk); p = 2^(qk - m_new); alpha = 2^(m - m_new);
    l = l * alpha + rowsum p; acc = acc * alpha + p @ v; m = m_new.
    After the last tile: O = acc / l and L = (m + log2 l) * ln 2.
    Rows that have seen no visible key keep m = -inf; their alpha and p are
    taken as 0 so that no NaN arises (the pages require masked rows handled).
    """
    qk_all = np.asarray(scores, dtype=np.float64) * LOG2E
    v = np.asarray(values, dtype=np.float64)
    R, n = qk_all.shape
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, v.shape[1]))
    for j0 in range(0, n, tile):
        qk = qk_all[:, j0:j0 + tile]
        m_new = np.maximum(m, np.max(qk, axis=1))
        live = np.isfinite(m_new)
        ref = np.where(live, m_new, 0.0)
        p = np.where(live[:, None], np.exp2(qk - ref[:, None]), 0.0)
        alpha = np.where(np.isfinite(m), np.exp2(m - ref), 0.0)
        l = l * alpha + p.sum(axis=1)
        acc = acc * alpha[:, None] + p @ v[j0:j0 + tile]
        m = m_new
    live = l > 0
    o = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
    L = np.where(live, (m + np.log2(np.where(live, l, 1.0))) * LN2, -np.inf)
    return o, L
