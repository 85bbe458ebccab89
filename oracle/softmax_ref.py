"""Plain fp64 reference for the row-wise softmax (test infrastructure only).

What it computes: for every row x of a [rows][cols] matrix, y_j = exp(x_j - max x) / sum_k
exp(x_k - max x), and the row's log-sum-exp max x + log sum_k exp(x_k - max x).  This is the
workload of page "Chapter 10 Writing and Benchmarking Custom Kernels", section 10.2.2 (the worked
example: row-wise softmax over a 4096 x 4096 float32 matrix, one block per row, the max
subtracted before exponentiating), computed in one pass over the row with the running
(max, sum) recurrence that the same section's closing question and page "Kernels -- fusion and
FlashAttention", section 3, describe: when a later tile raises the running max, the sum so far
is multiplied by exp(m_old - m_new) before the new terms are added.  The recurrence reaches the
plain softmax exactly (up to rounding), so ``softmax_rows`` is that plain definition written out;
``online_stats`` follows the recurrence step by step so that the tests can tie it to the plain
max and sum.

Readings where the pages are silent:
  * entries equal to -inf are masked: they get y = 0 (the page's masked load uses -inf as the
    fill value); a row whose entries are all -inf has no softmax and is rejected;
  * the log-sum-exp is in the natural log, as for attention.

Every function here is pinned in ``tests/test_oracle_softmax.py`` (closed forms, invariants,
scipy's softmax and logsumexp, and the recurrence against the plain statistics); nothing here is
"parity unpinned".
"""
from __future__ import annotations

import numpy as np


def softmax_rows(x):
    """(y, lse) for every row of x, float64.  y has x's shape, lse one value per row."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("x must be [rows][cols]")
    m = np.max(x, axis=1)
    if not np.all(np.isfinite(m)):
        raise ValueError("every row needs at least one finite entry")
    e = np.exp(x - m[:, None])          # exp(-inf) = 0 for masked entries
    s = np.sum(e, axis=1)
    return e / s[:, None], m + np.log(s)


def online_stats(row, tile: int):
    """The running (max, sum) of one row after streaming it in tiles of `tile` entries.

    Start from m = -inf, l = 0; for each tile t: m_new = max(m, max t); l = l * exp(m - m_new)
    + sum exp(t - m_new); m = m_new.  Returns (m, l); the softmax is exp(x - m) / l.
    """
    row = np.asarray(row, dtype=np.float64)
    m, l = -np.inf, 0.0
    for j0 in range(0, row.size, tile):
        t = row[j0:j0 + tile]
        m_new = max(m, float(np.max(t)))
        if m_new == -np.inf:            # nothing visible yet
            continue
        l = l * np.exp(m - m_new) + float(np.sum(np.exp(t - m_new)))
        m = m_new
    return m, l
