"""Pins of the fp64 oracle against what the pages and mathematics fix (CPU only).

Each pin is chosen so that a plausible mistake in the oracle fails at least one of them:
a dropped scale (causal row 0 LSE, hand example), a wrong sign in an exponent (sum-to-one,
shift invariance, hand example), an off-by-one or mis-aligned causal mask (Q = 0 gives
ln(#visible) per row), K and V swapped (equal keys -> mean of V, one-hot -> that V row, hand
example), log2 instead of ln (Q = 0, hand example), a missing rescale in the recurrence
(online vs two-pass on spiky scores), a wrong split-combine weight (split invariance).
"""
import importlib.util
import math
import os

import numpy as np
import pytest
import scipy.special

import seeded_inputs as si
from oracle import attention_ref as ref

# The mutation test re-runs this file against a copy of the oracle with one planted mistake.
_MUTANT = os.environ.get("FA_ORACLE_MUTANT_FILE")
if _MUTANT:
    _spec = importlib.util.spec_from_file_location("oracle_mutant", _MUTANT)
    ref = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(ref)

RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


def test_hand_worked_example():
    # d = 1, q = 1, keys 0, ln 2, ln 3, scale 1: exponentials 1, 2, 3 -> P = 1/6, 2/6, 3/6.
    q = np.array([[1.0]])
    k = np.array([[0.0], [math.log(2.0)], [math.log(3.0)]])
    v = np.array([[6.0], [0.0], [2.0]])
    O, LSE = ref.naive_attention_head(q, k, v, 1.0, causal=False)
    assert O[0, 0] == pytest.approx(2.0, abs=1e-14)        # (6*1 + 0*2 + 2*3) / 6
    assert LSE[0] == pytest.approx(math.log(6.0), abs=1e-14)
    # with scale 2 the exponentials are 1, 4, 9 -> O = (6 + 18) / 14
    O2, LSE2 = ref.naive_attention_head(q, k, v, 2.0, causal=False)
    assert O2[0, 0] == pytest.approx(24.0 / 14.0, abs=1e-14)
    assert LSE2[0] == pytest.approx(math.log(14.0), abs=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    S = 3.0 * _rand(37, 53)
    vis = ref.causal_visible(37, 53) if causal else None
    _, _, P = ref.softmax_attend(S, _rand(53, 8), vis)
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-12
    if causal:
        assert np.all(P[~vis] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_keys_give_mean_of_visible_values(causal):
    Tq, Tk, d = 19, 19, 16
    q = _rand(Tq, d)
    k = np.tile(_rand(1, d), (Tk, 1))
    v = _rand(Tk, d)
    O, _ = ref.naive_attention_head(q, k, v, 0.3, causal)
    if causal:
        expect = np.cumsum(v, axis=0) / np.arange(1, Tk + 1)[:, None]
    else:
        expect = np.tile(v.mean(axis=0), (Tq, 1))
    assert np.max(np.abs(O - expect)) <= 1e-12


@pytest.mark.parametrize("c", [700.0, -700.0])
def test_constant_shift_leaves_output_and_shifts_lse(c):
    S = 2.0 * _rand(23, 31)
    V = _rand(31, 8)
    vis = ref.causal_visible(23, 31)
    O0, L0, _ = ref.softmax_attend(S, V, vis)
    O1, L1, _ = ref.softmax_attend(S + c, V, vis)
    assert np.all(np.isfinite(O1))          # exp(700) overflows without the max subtraction
    assert np.max(np.abs(O1 - O0)) <= 1e-12
    assert np.max(np.abs((L1 - L0) - c)) <= 1e-9


def test_one_hot_dominant_score_selects_its_value_row():
    Tq, Tk, d = 11, 40, 8
    S = _rand(Tq, Tk)
    star = RNG.integers(0, Tk, size=Tq)
    S[np.arange(Tq), star] = S.max(axis=1) + 40.0
    V = _rand(Tk, d)
    O, _, _ = ref.softmax_attend(S, V)
    bound = Tk * math.exp(-40.0) * np.abs(V).max() * 2
    assert np.max(np.abs(O - V[star])) <= bound


@pytest.mark.parametrize("tile", [1, 3, 7, 128, 37])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_matches_two_pass(tile, causal):
    Tq, Tk, d = 5, 37, 8
    q, k, v = _rand(Tq, d), _rand(Tk, d), _rand(Tk, d)
    k[::9] *= 8.0                               # force running-max jumps
    O, L = ref.naive_attention_head(q, k, v, 0.7, causal)
    vis = ref.causal_visible(Tq, Tk)
    for i in range(Tq):
        o, lse = ref.online_softmax_row(q[i], k, v, 0.7, tile, vis[i] if causal else None)
        assert np.max(np.abs(o - O[i])) <= 1e-12
        assert abs(lse - L[i]) <= 1e-12


def test_single_key():
    q, k, v = _rand(4, 16), _rand(1, 16), _rand(1, 16)
    O, L = ref.naive_attention_head(q, k, v, 0.25, causal=False)
    assert np.array_equal(O, np.tile(v[0], (4, 1)))
    assert np.allclose(L, 0.25 * (q @ k[0]), atol=1e-14, rtol=0)


@pytest.mark.parametrize("Tq,Tk,causal", [(16, 16, True), (5, 21, True), (9, 13, False)])
def test_zero_queries_give_log_count_and_mean(Tq, Tk, causal):
    d = 8
    q, k, v = np.zeros((Tq, d)), _rand(Tk, d), _rand(Tk, d)
    O, L = ref.naive_attention_head(q, k, v, 0.5, causal)
    counts = np.arange(Tq) + (Tk - Tq) + 1 if causal else np.full(Tq, Tk)
    assert np.max(np.abs(L - np.log(counts))) <= 1e-13
    for i in range(Tq):
        assert np.max(np.abs(O[i] - v[:counts[i]].mean(axis=0))) <= 1e-13


def test_constant_value_rows():
    q, k = _rand(12, 8), _rand(30, 8)
    v = np.full((30, 8), 0.375)
    O, _ = ref.naive_attention_head(q, k, v, 0.9, causal=True)
    assert np.max(np.abs(O - 0.375)) <= 1e-14


def test_causal_row_zero_is_first_value_row():
    q, k, v = _rand(10, 8), _rand(10, 8), _rand(10, 8)
    O, L = ref.naive_attention_head(q, k, v, 0.125, causal=True)
    assert np.array_equal(O[0], v[0])
    assert L[0] == pytest.approx(0.125 * float(q[0] @ k[0]), abs=1e-14)


def test_joint_key_value_permutation_invariance():
    q, k, v = _rand(7, 8), _rand(29, 8), _rand(29, 8)
    perm = RNG.permutation(29)
    O0, L0 = ref.naive_attention_head(q, k, v, 0.4, causal=False)
    O1, L1 = ref.naive_attention_head(q, k[perm], v[perm], 0.4, causal=False)
    assert np.max(np.abs(O1 - O0)) <= 1e-13
    assert np.max(np.abs(L1 - L0)) <= 1e-13


def test_scipy_softmax_and_logsumexp():
    S = 4.0 * _rand(13, 17)
    V = _rand(17, 5)
    O, L, P = ref.softmax_attend(S, V)
    assert np.max(np.abs(P - scipy.special.softmax(S, axis=1))) <= 1e-14
    assert np.max(np.abs(L - scipy.special.logsumexp(S, axis=1))) <= 1e-12


def test_brute_force_loops_on_tiny_workload():
    wl = si.WORKLOADS["tiny_noncausal_b1_h2_t128_d64"]
    q, k, v = si.make_inputs(wl, seed=0)
    q, k, v = (si.bf16_bits_to_f64(x) for x in (q, k, v))
    O, L = ref.naive_attention(q, k, v, wl.scale, wl.causal)
    for h in range(wl.h):
        Ob, Lb = ref.scalar_attention_loops(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(),
                                            wl.scale, wl.causal)
        assert np.max(np.abs(Ob - O[0, h])) <= 1e-12
        assert np.max(np.abs(Lb - L[0, h])) <= 1e-12


def test_brute_force_loops_causal_rectangular():
    q, k, v = _rand(6, 4), _rand(9, 4), _rand(9, 4)
    O, L = ref.naive_attention_head(q, k, v, 0.5, causal=True)
    Ob, Lb = ref.scalar_attention_loops(q.tolist(), k.tolist(), v.tolist(), 0.5, True)
    assert np.max(np.abs(Ob - O)) <= 1e-13 and np.max(np.abs(Lb - L)) <= 1e-13


@pytest.mark.parametrize("Tk,splits", [(64, 1), (64, 2), (64, 16), (64, 64), (5, 4), (100, 7)])
def test_split_combine_equals_full_row(Tk, splits):
    d = 8
    q, k, v = _rand(d), _rand(Tk, d), _rand(Tk, d)
    k[::5] *= 8.0
    O, L = ref.naive_attention_head(q[None], k, v, 0.6, causal=False)
    parts = ref.split_kv_partials(q, k, v, 0.6, splits)
    assert len(parts) == splits
    o, lse = ref.combine_split_partials(parts)
    assert np.max(np.abs(o - O[0])) <= 1e-12
    assert abs(lse - L[0]) <= 1e-12


def test_split_kv_decode_shapes():
    q, k, v = _rand(2, 3, 8), _rand(2, 3, 20, 8), _rand(2, 3, 20, 8)
    O, L = ref.split_kv_decode(q, k, v, 0.5, 3, heads=[(1, 2), (0, 0)])
    O0, L0 = ref.naive_attention_head(q[1, 2][None], k[1, 2], v[1, 2], 0.5, False)
    assert np.max(np.abs(O[0] - O0[0])) <= 1e-12 and abs(L[0] - L0[0]) <= 1e-12


def test_sampled_rows_equal_full_rows():
    q, k, v = _rand(300, 16), _rand(300, 16), _rand(300, 16)
    O, L = ref.naive_attention_head(q, k, v, 0.25, causal=True, chunk=64)
    rows = np.array([0, 1, 63, 64, 299])
    Os, Ls = ref.naive_attention_head(q, k, v, 0.25, causal=True, rows=rows)
    assert np.array_equal(Os, O[rows]) and np.array_equal(Ls, L[rows])


def test_fully_masked_row_is_rejected():
    with pytest.raises(ValueError):
        ref.softmax_attend(np.zeros((1, 3)), np.zeros((3, 2)), np.zeros((1, 3), dtype=bool))
