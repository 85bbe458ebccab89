"""Plain fp64 reference for the attention backward pass (test infrastructure only).

What it computes, per head: the gradients of the scalar sum(dO * O) with respect to Q, K and V,
where O = softmax(scale * Q K^T, masked) V is the forward of ``attention_ref``.  Written from the
page "Chapter 10 Writing and Benchmarking Custom Kernels", section 10.3.2 (backward-pass
recomputation): the upstream gradient of P is dO_i V_j^T, the per-row scalar D_i is the inner
product of dO_i and O_i, P can be rebuilt from the stored log-sum-exp as P_ij = exp(S_ij - L_i),
and the score gradient follows by substituting both into the softmax backward.

Readings where the pages are silent or their formulas are lost in the text:
  * the score gradient is dS_ij = P_ij (dP_ij - D_i) with dP = dO V^T (the softmax Jacobian
    applied to dP; the page's displayed formula is missing, its ingredients are as above);
  * the scores are scaled, S = scale * Q K^T, so dQ = scale * dS K and dK = scale * dS^T Q; and
    dV = P^T dO;
  * masked entries have P = 0 and therefore dS = 0; a query row with no visible key is rejected,
    as in the forward.

Every function here is pinned in ``tests/test_oracle_bwd.py`` (central finite differences of the
forward oracle, closed forms, invariants, and float64 autograd of an independent formulation).
"""
from __future__ import annotations

import numpy as np

from oracle import attention_ref as fwd


def backward_head(q, k, v, do, scale: float, causal: bool):
    """Gradients of sum(dO * O) for one head, float64.

    Returns a dict with dq [Tq][d], dk [Tk][d], dv [Tk][d], and the intermediates the page names:
    P [Tq][Tk], dP [Tq][Tk], D [Tq], dS [Tq][Tk], O [Tq][d], LSE [Tq].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    Tq, Tk = q.shape[0], k.shape[0]
    S = fwd.scores(q, k, scale)
    vis = fwd.causal_visible(Tq, Tk) if causal else None
    O, LSE, P = fwd.softmax_attend(S, v, vis)
    dP = do @ v.T                                  # dL/dP_ij = dO_i . V_j
    D = np.sum(do * O, axis=1)                     # D_i = <dO_i, O_i>
    dS = P * (dP - D[:, None])                     # softmax backward; zero where masked (P = 0)
    dq = float(scale) * (dS @ k)
    dk = float(scale) * (dS.T @ q)
    dv = P.T @ do
    return {"dq": dq, "dk": dk, "dv": dv, "P": P, "dP": dP, "D": D, "dS": dS, "O": O,
            "LSE": LSE}


def probabilities_from_lse(q, k, lse, scale: float, causal: bool):
    """P rebuilt from the stored log-sum-exp, P_ij = exp(S_ij - L_i) (page "Chapter 10 ...",
    section 10.3.2), with P = 0 on masked entries."""
    S = fwd.scores(q, k, scale)
    P = np.exp(S - np.asarray(lse, dtype=np.float64)[:, None])
    if causal:
        P[~fwd.causal_visible(q.shape[0], k.shape[0])] = 0.0
    return P


def backward(q, k, v, do, scale: float, causal: bool):
    """All heads: q, do [B][h][Tq][d], k, v [B][h][Tk][d] -> (dq, dk, dv, D) float64."""
    B, H = q.shape[:2]
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(v.shape, dtype=np.float64)
    D = np.empty(q.shape[:3], dtype=np.float64)
    for b in range(B):
        for h in range(H):
            r = backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
            dq[b, h], dk[b, h], dv[b, h], D[b, h] = r["dq"], r["dk"], r["dv"], r["D"]
    return dq, dk, dv, D


def abs_bounds_head(r, q, k, do, scale: float):
    """Sums of absolute values of the products that make up each gradient element:
    A_dv = P^T |dO|, A_dq = |scale| |dS| |K|, A_dk = |scale| |dS|^T |Q|.  A kernel that rounds
    each P_ij or dS_ij to a format with unit roundoff u (and accumulates exactly) errs by at most
    u * A in each element; the GPU tests build their tolerance from these."""
    absS = np.abs(r["dS"])
    return {"dv": r["P"].T @ np.abs(np.asarray(do, dtype=np.float64)),
            "dq": abs(float(scale)) * (absS @ np.abs(np.asarray(k, dtype=np.float64))),
            "dk": abs(float(scale)) * (absS.T @ np.abs(np.asarray(q, dtype=np.float64)))}
