"""Plain fp64 reference for the fused elementwise chains (test infrastructure only).

What it computes:
  * GELU in the tanh form the page "Chapter 10 Writing and Benchmarking Custom Kernels",
    section 10.2.1 (the GeLU case study) prints in its kernel:
        gelu(x) = 0.5 x (1 + tanh(sqrt(2 / pi) (x + 0.044715 x^3)));
  * the bias -> GELU -> dropout chain of page "Fusion and IO-aware kernels" ("The idea in one
    minute" and the chain it fuses into one kernel): y = keep * gelu(x + bias) / (1 - p) over a
    [rows][cols] activation with one bias per column;
  * the dropout decisions from a counter-based generator, Philox4x32-10 (Salmon, Moraes, Dror and
    Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), which both this oracle and the
    GPU kernel implement from that published definition.

Readings where the pages are silent:
  * element e of the row-major activation draws a 16-bit value: half e % 2 (the low 16 bits for
    even e, the high 16 bits for odd e) of word (e % 8) // 2 of Philox4x32-10 applied to the
    counter (e // 8 low 32 bits, e // 8 high 32 bits, offset low, offset high) under the key
    (seed low, seed high), so one generator call serves eight elements;
  * it is dropped iff that value is below floor(p * 2^16) (an integer comparison, so both sides
    take the same decision exactly; the drop probability is p to within 2^-16), and kept
    elements are scaled by 1 / (1 - p); p in [0, 1).

Every function here is pinned in ``tests/test_oracle_elementwise.py`` (the generator's published
known-answer vectors, identities of the tanh form, scipy's logistic function, the p = 0 case and
the keep rate); nothing here is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

GELU_A = 0.044715
GELU_C = math.sqrt(2.0 / math.pi)

# Philox4x32 round multipliers and Weyl key increments (the SC 2011 paper's constants).
PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = 0xFFFFFFFF


def gelu_tanh(x):
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) in float64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(GELU_C * (x + GELU_A * x ** 3)))


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds on arrays of counters [n][4] and keys [n][2] (uint32 values).

    One round: (hi0, lo0) = M0 * c0 and (hi1, lo1) = M1 * c2 as 64-bit products; the new counter
    is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); then the key is bumped by (W0, W1).  The first
    of the ten Philox rounds uses the key as given; each later one uses it bumped once more.
    """
    c = np.array(counter, dtype=np.uint64).reshape(-1, 4)
    k = np.array(key, dtype=np.uint64).reshape(-1, 2)
    c0, c1, c2, c3 = (c[:, i].copy() for i in range(4))
    k0, k1 = k[:, 0].copy(), k[:, 1].copy()
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    mask = np.uint64(_MASK32)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & mask
            k1 = (k1 + np.uint64(PHILOX_W1)) & mask
        p0 = m0 * c0            # < 2^64: exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """Draws below this integer are dropped: floor(p * 2^16), for p in [0, 1)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(math.floor(p * 65536.0)), 0xFFFF)


def dropout_words(n: int, seed: int, offset: int, first: int = 0):
    """The 16-bit draws of elements first .. first + n - 1 (see the module docstring)."""
    e = np.arange(first, first + n, dtype=np.uint64)
    blk = e // np.uint64(8)
    ctr = np.stack([blk & np.uint64(_MASK32), blk >> np.uint64(32),
                    np.full_like(blk, offset & _MASK32), np.full_like(blk, (offset >> 32) & _MASK32)],
                   axis=1)
    key = np.tile(np.array([seed & _MASK32, (seed >> 32) & _MASK32], dtype=np.uint64), (n, 1))
    words = philox4x32_10(ctr, key)
    word = words[np.arange(n), ((e % np.uint64(8)) // np.uint64(2)).astype(np.int64)]
    shift = (e % np.uint64(2)) * np.uint64(16)
    return ((word.astype(np.uint64) >> shift) & np.uint64(0xFFFF)).astype(np.uint32)


def bias_gelu_dropout(x, bias, p: float, seed: int, offset: int, first_row: int = 0):
    """y = keep * gelu(x + bias) / (1 - p) for rows first_row.. of a [rows][cols] activation.

    Returns (y float64, keep bool); x holds the rows given, bias has one value per column.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    words = dropout_words(rows * cols, seed, offset, first=first_row * cols).reshape(rows, cols)
    keep = words >= np.uint32(dropout_threshold(p))
    g = gelu_tanh(x + np.asarray(bias, dtype=np.float64)[None, :])
    return np.where(keep, g / (1.0 - p), 0.0), keep
