"""Pins of the fp64 backward oracle (CPU only).

The oracle writes the page's formulas (dS = P (dP - D), dQ = scale dS K, ...); these tests tie it
to things that do not use those formulas: central finite differences of the forward oracle,
closed forms, invariants of softmax attention, and float64 autograd of a plain formulation.
"""
import importlib.util
import os

import numpy as np
import pytest
import torch

from oracle import attention_bwd_ref as bref
from oracle import attention_ref as ref

# The mutation test re-runs this file against a copy of the backward oracle with one planted
# mistake.
_MUTANT = os.environ.get("FA_ORACLE_BWD_MUTANT_FILE")
if _MUTANT:
    _spec = importlib.util.spec_from_file_location("oracle_bwd_mutant", _MUTANT)
    bref = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(bref)

RNG = np.random.default_rng(2024)


def _rand(*shape):
    return RNG.standard_normal(shape)


def _loss(q, k, v, do, scale, causal):
    O, _ = ref.naive_attention_head(q, k, v, scale, causal)
    return float(np.sum(do * O))


@pytest.mark.parametrize("causal,Tq,Tk,d", [(False, 3, 4, 5), (True, 4, 4, 3), (True, 3, 6, 2),
                                            (False, 1, 1, 4), (False, 5, 2, 3)])
def test_gradients_match_central_differences(causal, Tq, Tk, d):
    q, k, v, do = _rand(Tq, d), _rand(Tk, d), _rand(Tk, d), _rand(Tq, d)
    scale = 0.7
    r = bref.backward_head(q, k, v, do, scale, causal)
    h = 1e-6
    for name, x, g in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, scale, causal) -
                        _loss(args_m["q"], args_m["k"], args_m["v"], do, scale, causal)) / (2 * h)
        assert np.max(np.abs(num - g)) <= 1e-7 * (1 + np.max(np.abs(g))), name


def test_matches_float64_autograd_of_plain_attention():
    Tq, Tk, d, scale = 7, 9, 4, 0.37
    q, k, v, do = _rand(Tq, d), _rand(Tk, d), _rand(Tk, d), _rand(Tq, d)
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        s = scale * tq @ tk.T
        if causal:
            s = s.masked_fill(~torch.from_numpy(ref.causal_visible(Tq, Tk)), float("-inf"))
        o = torch.softmax(s, dim=1) @ tv
        (o * torch.from_numpy(do)).sum().backward()
        r = bref.backward_head(q, k, v, do, scale, causal)
        for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
            assert np.max(np.abs(t.grad.numpy() - r[name])) <= 1e-12, (causal, name)


def test_single_key_closed_form():
    # one key: P = 1, O = V_0, so dV_0 = sum_i dO_i and dQ = dK = 0
    q, k, v, do = _rand(5, 3), _rand(1, 3), _rand(1, 3), _rand(5, 3)
    r = bref.backward_head(q, k, v, do, 1.3, False)
    assert np.allclose(r["dv"][0], do.sum(axis=0), atol=1e-14)
    assert np.max(np.abs(r["dq"])) <= 1e-14 and np.max(np.abs(r["dk"])) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    Tq, Tk, d, scale = 11, 11, 6, 0.41
    q, k, v, do = _rand(Tq, d), _rand(Tk, d), _rand(Tk, d), _rand(Tq, d)
    r = bref.backward_head(q, k, v, do, scale, causal)
    # rows of P sum to 1, so the value gradients add up to the summed output gradient
    assert np.allclose(r["dv"].sum(axis=0), do.sum(axis=0), atol=1e-12)
    # shifting every key by one vector changes each row's scores by a constant: no effect
    assert np.allclose(r["dk"].sum(axis=0), 0.0, atol=1e-12)
    # D_i = <dO_i, O_i> = sum_j P_ij dP_ij, and each row of dS sums to zero
    assert np.allclose(r["D"], np.sum(r["P"] * r["dP"], axis=1), atol=1e-12)
    assert np.allclose(r["dS"].sum(axis=1), 0.0, atol=1e-12)
    # scaling Q and K together: sum_i <q_i, dQ_i> = sum_j <k_j, dK_j>
    assert np.isclose(np.sum(q * r["dq"]), np.sum(k * r["dk"]), atol=1e-12)


def test_probabilities_rebuilt_from_lse():
    Tq, Tk, d, scale = 6, 8, 5, 0.5
    q, k, v, do = _rand(Tq, d), _rand(Tk, d), _rand(Tk, d), _rand(Tq, d)
    for causal in (False, True):
        r = bref.backward_head(q, k, v, do, scale, causal)
        P = bref.probabilities_from_lse(q, k, r["LSE"], scale, causal)
        assert np.max(np.abs(P - r["P"])) <= 1e-14


def test_abs_bounds_dominate_the_gradients():
    Tq, Tk, d, scale = 9, 13, 4, 0.6
    q, k, v, do = _rand(Tq, d), _rand(Tk, d), _rand(Tk, d), _rand(Tq, d)
    r = bref.backward_head(q, k, v, do, scale, True)
    a = bref.abs_bounds_head(r, q, k, do, scale)
    for name in ("dq", "dk", "dv"):
        assert np.all(np.abs(r[name]) <= a[name] + 1e-15)


def test_batched_wrapper_matches_heads():
    q, k, v, do = _rand(2, 3, 5, 4), _rand(2, 3, 7, 4), _rand(2, 3, 7, 4), _rand(2, 3, 5, 4)
    dq, dk, dv, D = bref.backward(q, k, v, do, 0.5, True)
    r = bref.backward_head(q[1, 2], k[1, 2], v[1, 2], do[1, 2], 0.5, True)
    assert np.array_equal(dq[1, 2], r["dq"]) and np.array_equal(dv[1, 2], r["dv"])
    assert np.array_equal(D[1, 2], r["D"])


def test_abs_bounds_are_attained_by_single_term_gradients():
    """Upper pin: where a gradient element is one product, or products of one sign, the bound
    equals |gradient| exactly, so an inflated bound (a wrong factor, |dP| for |dS|, a dropped
    probability) fails here.  One query row: dK_j = scale dS_1j q_1 and dV_j = P_1j dO_1 are
    single products.  Two keys with k_2 = -k_1: dS_i2 = -dS_i1, so dQ_i = 2 scale dS_i1 k_1 and
    |dQ_i| = |scale| (|dS_i1| + |dS_i2|) |k_1|, the bound."""
    d, scale = 5, -0.7
    q, v, do = _rand(1, d), _rand(2, d), _rand(1, d)
    k1 = _rand(1, d)
    k = np.concatenate([k1, -k1])
    r = bref.backward_head(q, k, v, do, scale, False)
    a = bref.abs_bounds_head(r, q, k, do, scale)
    for name in ("dq", "dk", "dv"):
        assert np.all(np.abs(a[name]) > 0)
        assert np.allclose(np.abs(r[name]), a[name], rtol=1e-12, atol=0), name
    # several query rows, same-sign upstream gradients: A_dv = P^T |dO| = dV exactly
    Tq, Tk = 7, 9
    q, k, v = _rand(Tq, d), _rand(Tk, d), _rand(Tk, d)
    do = np.abs(_rand(Tq, d))
    r = bref.backward_head(q, k, v, do, scale, True)
    a = bref.abs_bounds_head(r, q, k, do, scale)
    assert np.allclose(r["dv"], a["dv"], rtol=1e-12, atol=0)
