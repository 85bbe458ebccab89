"""Pins of the fp64 row-softmax oracle (CPU only): closed forms, invariants, scipy's independent
softmax / logsumexp, and the running (max, sum) recurrence against the plain statistics."""
import importlib.util
import math
import os

import numpy as np
import pytest
from scipy import special

from oracle import softmax_ref as sref

# The mutation test re-runs this file against a copy of the oracle with one planted mistake.
_MUTANT = os.environ.get("FA_ORACLE_SOFTMAX_MUTANT_FILE")
if _MUTANT:
    _spec = importlib.util.spec_from_file_location("oracle_softmax_mutant", _MUTANT)
    sref = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(sref)

RNG = np.random.default_rng(77)


def test_constant_row_is_uniform():
    y, lse = sref.softmax_rows(np.full((3, 7), 2.5))
    assert np.allclose(y, 1.0 / 7, atol=1e-15, rtol=0)
    assert np.allclose(lse, 2.5 + math.log(7), atol=1e-14, rtol=0)


def test_two_entries_give_the_logistic():
    a, b = 1.7, -0.4
    y, lse = sref.softmax_rows(np.array([[a, b]]))
    assert abs(y[0, 0] - 1.0 / (1.0 + math.exp(b - a))) <= 1e-15
    assert abs(y[0, 1] - 1.0 / (1.0 + math.exp(a - b))) <= 1e-15
    assert abs(lse[0] - math.log(math.exp(a) + math.exp(b))) <= 1e-14


def test_single_column():
    y, lse = sref.softmax_rows(np.array([[3.0], [-50.0]]))
    assert np.array_equal(y, np.ones((2, 1)))
    assert np.array_equal(lse, np.array([3.0, -50.0]))


def test_matches_scipy():
    x = RNG.standard_normal((5, 301)) * 3
    y, lse = sref.softmax_rows(x)
    assert np.max(np.abs(y - special.softmax(x, axis=1))) <= 1e-15
    assert np.max(np.abs(lse - special.logsumexp(x, axis=1))) <= 1e-13


def test_rows_sum_to_one_and_shift_invariance():
    x = RNG.standard_normal((4, 129)) * 10
    y, lse = sref.softmax_rows(x)
    assert np.allclose(y.sum(axis=1), 1.0, atol=1e-14, rtol=0)
    c = np.array([[1000.0], [-1000.0], [0.5], [123.25]])
    y2, lse2 = sref.softmax_rows(x + c)
    assert np.max(np.abs(y2 - y)) <= 1e-13
    assert np.max(np.abs(lse2 - (lse + c[:, 0]))) <= 1e-10


def test_large_logits_do_not_overflow():
    x = np.array([[1000.0, 999.0, -1000.0]])
    y, lse = sref.softmax_rows(x)
    e = math.exp(-1.0)
    assert abs(y[0, 0] - 1 / (1 + e)) <= 1e-15 and abs(y[0, 1] - e / (1 + e)) <= 1e-15
    assert y[0, 2] == 0.0
    assert abs(lse[0] - (1000.0 + math.log1p(e))) <= 1e-12


def test_masked_entries_are_zero():
    x = np.array([[0.3, -np.inf, 1.1, -np.inf]])
    y, lse = sref.softmax_rows(x)
    assert y[0, 1] == 0.0 and y[0, 3] == 0.0
    ref, _ = sref.softmax_rows(np.array([[0.3, 1.1]]))
    assert np.max(np.abs(y[0, [0, 2]] - ref[0])) <= 1e-16
    with pytest.raises(ValueError):
        sref.softmax_rows(np.array([[-np.inf, -np.inf]]))


def test_online_recurrence_reaches_the_plain_statistics():
    row = np.concatenate([RNG.standard_normal(50), [40.0], RNG.standard_normal(70) * 5])
    for tile in (1, 3, 16, 64, 1000):
        m, l = sref.online_stats(row, tile)
        assert m == np.max(row)
        assert abs(l - np.sum(np.exp(row - row.max()))) <= 1e-12 * l
    # a row whose max arrives last forces the rescale of everything before it
    row = np.arange(20, dtype=np.float64)
    m, l = sref.online_stats(row, 4)
    assert m == 19.0 and abs(l - sum(math.exp(v - 19.0) for v in row)) <= 1e-14
    # masked leading tiles
    row = np.array([-np.inf, -np.inf, -np.inf, 2.0, 1.0])
    m, l = sref.online_stats(row, 2)
    assert m == 2.0 and abs(l - (1 + math.exp(-1.0))) <= 1e-15
