"""Pins of the fp64 elementwise-chain oracle (CPU only): Philox4x32-10's published known-answer
vectors, identities of the tanh-form GELU, scipy's logistic function, and the dropout rules."""
import importlib.util
import math
import os

import numpy as np
import pytest
from scipy import special

from oracle import elementwise_ref as eref

# The mutation test re-runs this file against a copy of the oracle with one planted mistake.
_MUTANT = os.environ.get("FA_ORACLE_ELEMENTWISE_MUTANT_FILE")
if _MUTANT:
    _spec = importlib.util.spec_from_file_location("oracle_elementwise_mutant", _MUTANT)
    eref = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(eref)

# Known-answer vectors of Philox4x32-10 as published with the generator (Random123 distribution,
# kat_vectors): (counter, key) -> output, all words in hex.  Fixture file: tests/golden/.
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "philox4x32_10_kat.txt")


def _kat():
    out = []
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if line:
            w = [int(t, 16) for t in line]
            out.append((w[0:4], w[4:6], w[6:10]))
    return out


@pytest.mark.parametrize("ctr,key,expect", _kat())
def test_philox_known_answers(ctr, key, expect):
    got = eref.philox4x32_10([ctr], [key])[0]
    assert [int(v) for v in got] == expect


def test_gelu_identities():
    x = np.linspace(-8, 8, 1601)
    g = eref.gelu_tanh(x)
    # gelu(x) - gelu(-x) = x for the tanh form (0.5 x (1 + t) + 0.5 x (1 - t))
    assert np.max(np.abs(g - eref.gelu_tanh(-x) - x)) <= 1e-14
    # 0.5 (1 + tanh u) is the logistic function of 2u: compare with scipy's expit
    u = math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)
    assert np.max(np.abs(g - x * special.expit(2 * u))) <= 1e-14
    assert eref.gelu_tanh(0.0) == 0.0
    assert abs(eref.gelu_tanh(10.0) - 10.0) <= 1e-12 and abs(eref.gelu_tanh(-10.0)) <= 1e-12
    # at x = 1: sqrt(2/pi) * 1.044715 inside the tanh
    assert abs(eref.gelu_tanh(1.0) - 0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * 1.044715))) <= 1e-16
    # within the approximation's known distance of the exact (erf) GELU
    exact = 0.5 * x * (1 + special.erf(x / math.sqrt(2)))
    assert np.max(np.abs(g - exact)) <= 1e-3


def test_dropout_threshold():
    assert eref.dropout_threshold(0.0) == 0
    assert eref.dropout_threshold(0.5) == 2 ** 15
    assert eref.dropout_threshold(0.1) == math.floor(0.1 * 2 ** 16) == 6553
    assert eref.dropout_threshold(0.99999) == 65535
    with pytest.raises(ValueError):
        eref.dropout_threshold(1.0)


def test_dropout_words_follow_the_counter_layout():
    w = eref.dropout_words(24, seed=0x1234_5678_9ABC_DEF0, offset=7)
    for e in range(24):
        blk = e // 8
        word = int(eref.philox4x32_10([[blk, 0, 7, 0]], [[0x9ABCDEF0, 0x12345678]])[0][(e % 8) // 2])
        ref = (word >> 16) if e % 2 else (word & 0xFFFF)
        assert w[e] == ref
    # a window starting mid-stream sees the same words
    assert np.array_equal(eref.dropout_words(5, 99, 3, first=6), eref.dropout_words(11, 99, 3)[6:])


def test_bias_gelu_dropout_rules():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 64))
    b = rng.standard_normal(64)
    y0, keep0 = eref.bias_gelu_dropout(x, b, 0.0, seed=1, offset=0)
    assert keep0.all() and np.max(np.abs(y0 - eref.gelu_tanh(x + b))) == 0.0
    y, keep = eref.bias_gelu_dropout(x, b, 0.25, seed=1, offset=0)
    assert np.all(y[~keep] == 0.0)
    assert np.max(np.abs(y[keep] - eref.gelu_tanh(x + b)[keep] / 0.75)) <= 1e-15
    # rows first_row.. of a bigger activation use the same words as the full call
    yf, kf = eref.bias_gelu_dropout(np.vstack([x, x]), b, 0.25, seed=1, offset=0)
    y2, k2 = eref.bias_gelu_dropout(x, b, 0.25, seed=1, offset=0, first_row=8)
    assert np.array_equal(k2, kf[8:]) and np.array_equal(y2, yf[8:])


def test_keep_rate_matches_p():
    words = eref.dropout_words(200_000, seed=2024, offset=1)
    assert words.max() <= 0xFFFF
    for p in (0.1, 0.5, 0.9):
        kept = np.mean(words >= np.uint32(eref.dropout_threshold(p)))
        sigma = math.sqrt(p * (1 - p) / words.size)
        assert abs(kept - (1 - p)) <= 5 * sigma
    # different offsets give different streams
    assert not np.array_equal(eref.dropout_words(64, 1, 0), eref.dropout_words(64, 1, 1))
