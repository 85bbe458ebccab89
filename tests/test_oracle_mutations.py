"""Planted mistakes in a copy of the oracle must each fail at least one pin (CPU only).

Each mutant is a one-line edit of ``oracle/attention_ref.py`` written to a temporary file; the pin
suite ``tests/test_oracle.py`` is then run against it in a subprocess and must fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attention_ref.py")

MUTANTS = {
    "scale dropped": ("return float(scale) * (q @ k.T)", "return (q @ k.T)"),
    "causal mask off by one": ("<= (rows[:, None] + (Tk - Tq))", "< (rows[:, None] + (Tk - Tq))"),
    "causal mask top-left aligned": ("(rows[:, None] + (Tk - Tq))", "(rows[:, None] + 0)"),
    "keys used as values": ("softmax_attend(S, v, vis)", "softmax_attend(S, k[:, :v.shape[1]], vis)"),
    "log2 instead of ln": ("LSE = m[:, 0] + np.log(ell[:, 0])", "LSE = m[:, 0] + np.log2(ell[:, 0])"),
    "exponent sign flipped": ("P = np.exp(S - m)", "P = np.exp(-(S - m))"),
    "not normalised": ("    P /= ell\n", "    pass\n"),
    "max not subtracted": ("P = np.exp(S - m)", "P = np.exp(S)"),
    "recurrence output not rescaled": ("o[t] = o[t] * c + sum(", "o[t] = o[t] + sum("),
    "recurrence denominator not rescaled": ("ell = ell * c + sum(p.values())",
                                            "ell = ell + sum(p.values())"),
    "combine weight inverted": ("else math.exp(m - m_star)", "else math.exp(m_star - m)"),
    "split chunk drops a key": ("min(Tk, (s + 1) * chunk)", "min(Tk, (s + 1) * chunk - 1)"),
    "lse of split uses wrong max": ("return o / ell, m_star + math.log(ell)",
                                    "return o / ell, math.log(ell)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    path = tmp_path / "mutant.py"
    path.write_text(src.replace(old, new))
    env = dict(os.environ, FA_ORACLE_MUTANT_FILE=str(path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant '{name}' passed every pin:\n{r.stdout[-2000:]}"


BWD_SRC = os.path.join(ROOT, "oracle", "attention_bwd_ref.py")

BWD_MUTANTS = {
    "score gradient without D": ("dS = P * (dP - D[:, None])", "dS = P * dP"),
    "score gradient sign flipped": ("dS = P * (dP - D[:, None])", "dS = P * (D[:, None] - dP)"),
    "dQ without the scale": ("dq = float(scale) * (dS @ k)", "dq = (dS @ k)"),
    "dK from dO instead of Q": ("dk = float(scale) * (dS.T @ q)", "dk = float(scale) * (dS.T @ do)"),
    "dV from dS instead of P": ("dv = P.T @ do", "dv = dS.T @ do"),
    "D from dP instead of O": ("D = np.sum(do * O, axis=1)", "D = np.sum(dP, axis=1) / Tk"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name, tmp_path):
    old, new = BWD_MUTANTS[name]
    src = open(BWD_SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    path = tmp_path / "mutant_bwd.py"
    path.write_text(src.replace(old, new))
    env = dict(os.environ, FA_ORACLE_BWD_MUTANT_FILE=str(path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_bwd.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant '{name}' passed every pin:\n{r.stdout[-2000:]}"


SOFTMAX_SRC = os.path.join(ROOT, "oracle", "softmax_ref.py")
SOFTMAX_MUTANTS = {
    "no max subtraction": ("e = np.exp(x - m[:, None])", "e = np.exp(x)"),
    "sum over the wrong axis": ("s = np.sum(e, axis=1)", "s = np.sum(e, axis=0)[: e.shape[0]]"),
    "lse without the log": ("return e / s[:, None], m + np.log(s)", "return e / s[:, None], m + s"),
    "recurrence without the rescale": ("l = l * np.exp(m - m_new) + float(np.sum(np.exp(t - m_new)))",
                                       "l = l + float(np.sum(np.exp(t - m_new)))"),
    "recurrence rescale inverted": ("l = l * np.exp(m - m_new) + float(np.sum(np.exp(t - m_new)))",
                                    "l = l * np.exp(m_new - m) + float(np.sum(np.exp(t - m_new)))"),
}


@pytest.mark.parametrize("name", sorted(SOFTMAX_MUTANTS))
def test_softmax_mutant_is_caught(name, tmp_path):
    old, new = SOFTMAX_MUTANTS[name]
    src = open(SOFTMAX_SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    path = tmp_path / "mutant_softmax.py"
    path.write_text(src.replace(old, new))
    env = dict(os.environ, FA_ORACLE_SOFTMAX_MUTANT_FILE=str(path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_softmax.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant '{name}' passed every pin:\n{r.stdout[-2000:]}"


ELEMENTWISE_SRC = os.path.join(ROOT, "oracle", "elementwise_ref.py")
ELEMENTWISE_MUTANTS = {
    "gelu cubic coefficient": ("GELU_A = 0.044715", "GELU_A = 0.04715"),
    "gelu without the half": ("return 0.5 * x * (1.0 + np.tanh(", "return x * (1.0 + np.tanh("),
    "philox multipliers swapped": ("p0 = m0 * c0", "p0 = m1 * c0"),
    "philox key never bumped": ("k0 = (k0 + np.uint64(PHILOX_W0)) & mask", "k0 = k0"),
    "philox output order": ("c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0",
                            "c0, c1, c2, c3 = hi0 ^ c1 ^ k0, lo1, hi1 ^ c3 ^ k1, lo0"),
    "dropout without the rescale": ("np.where(keep, g / (1.0 - p), 0.0)", "np.where(keep, g, 0.0)"),
    "dropout decision inverted": ("keep = words >= np.uint32(dropout_threshold(p))",
                                  "keep = words < np.uint32(dropout_threshold(p))"),
    "words indexed by block": (
        "word = words[np.arange(n), ((e % np.uint64(8)) // np.uint64(2)).astype(np.int64)]",
        "word = words[np.arange(n), 0]"),
    "one half of each word": ("shift = (e % np.uint64(2)) * np.uint64(16)",
                              "shift = np.zeros_like(e)"),
    "32-bit threshold": ("return min(int(math.floor(p * 65536.0)), 0xFFFF)",
                         "return min(int(math.floor(p * 4294967296.0)), 0xFFFFFFFF)"),
}


@pytest.mark.parametrize("name", sorted(ELEMENTWISE_MUTANTS))
def test_elementwise_mutant_is_caught(name, tmp_path):
    old, new = ELEMENTWISE_MUTANTS[name]
    src = open(ELEMENTWISE_SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    path = tmp_path / "mutant_elementwise.py"
    path.write_text(src.replace(old, new))
    env = dict(os.environ, FA_ORACLE_ELEMENTWISE_MUTANT_FILE=str(path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_elementwise.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant '{name}' passed every pin:\n{r.stdout[-2000:]}"
