"""Plain fp64 reference for attention forward and split-KV decode (test infrastructure only).

Parity pins: every function here is pinned by ``tests/test_oracle.py`` against closed forms,
invariants, scipy routines and brute force; nothing in this file is "parity unpinned".

Readings where the pages are silent (the same readings the GPU library documents):
  * scores are scaled before the softmax, and the log-sum-exp is over the scaled scores, in the
    natural log (page "Kernels — fusion and FlashAttention", §5, the Triton program stores
    m + log(l));
  * causal masking with Tq != Tk is bottom-right aligned: query i sits at absolute position
    i + (Tk - Tq) and sees key j iff j <= i + (Tk - Tq).  With Tq == Tk this is the usual
    lower-triangular mask with the diagonal kept (page "Chapter 10 Writing and Benchmarking Custom
    Kernels", §10.3.1 "What You Actually Decide in Practice", causal skipping of tiles above the
    diagonal);
  * a row with no visible key has no defined softmax; callers never request one (the library
    rejects causal with Tq > Tk), and this module raises if asked;
  * inputs are whatever float64 values the caller passes; the tests pass the exact bf16 values the
    GPU receives, and the float32 value of the scale.
"""
from __future__ import annotations

import math

import numpy as np


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for one head, float64.

    Page "Kernels — fusion and FlashAttention", §2 (scores, then mask, softmax, weight the values)
    and §3 (the per-tile score is q K_j^T / sqrt(d_head)); page "Chapter 10 ...", §10.3.1
    (S = Q K^T / sqrt(d)).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    return float(scale) * (q @ k.T)


def causal_visible(Tq: int, Tk: int, rows=None) -> np.ndarray:
    """Boolean visibility [len(rows)][Tk]: key j visible to query i iff j <= i + (Tk - Tq)."""
    rows = np.arange(Tq) if rows is None else np.asarray(rows)
    return np.arange(Tk)[None, :] <= (rows[:, None] + (Tk - Tq))


def softmax_attend(S: np.ndarray, V: np.ndarray, visible: np.ndarray | None = None):
    """Row softmax of a score matrix, then the weighted sum of value rows.

    Returns (O, LSE, P).  Masked entries get -inf before the softmax.  The row max is subtracted
    before exponentiating (page "Kernels — fusion and FlashAttention", §3: subtract the row max for
    stability, exponentiate, divide by the row sum); LSE = m + ln(sum) (same page, §5, and page
    "Chapter 10 ...", §10.3.2: L_i = m_i + log l_i).
    """
    S = np.array(S, dtype=np.float64, copy=True)
    V = np.asarray(V, dtype=np.float64)
    if visible is not None:
        S[~visible] = -np.inf
    m = S.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key; its softmax is undefined")
    P = np.exp(S - m)
    ell = P.sum(axis=1, keepdims=True)
    P /= ell
    O = P @ V
    LSE = m[:, 0] + np.log(ell[:, 0])
    return O, LSE, P


def naive_attention_head(q, k, v, scale: float, causal: bool, rows=None, chunk: int = 512):
    """Naive attention for one head: materialise S, mask, softmax, multiply by V.

    q [Tq][d], k and v [Tk][d] (float64 values).  ``rows`` selects a subset of query rows (each
    row's result depends only on that row of Q), used to sample large problems.  Rows are taken in
    chunks only to bound memory; every row is the full definition.
    Page "Kernels — fusion and FlashAttention", §2 (the naive data flow); page "Fusion and
    IO-aware kernels", "How it really works" (standard attention writes S, softmaxes it, multiplies
    by V).  Returns (O [n][d], LSE [n]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, Tk = q.shape[0], k.shape[0]
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    LSE = np.empty(rows.size, dtype=np.float64)
    for c0 in range(0, rows.size, chunk):
        r = rows[c0:c0 + chunk]
        S = scores(q[r], k, scale)
        vis = causal_visible(Tq, Tk, r) if causal else None
        O[c0:c0 + r.size], LSE[c0:c0 + r.size], _ = softmax_attend(S, v, vis)
    return O, LSE


def naive_attention(q, k, v, scale: float, causal: bool):
    """Naive attention over [B][h][T][d] float64 arrays; returns (O [B][h][Tq][d], LSE [B][h][Tq])."""
    q = np.asarray(q, dtype=np.float64)
    B, H, Tq, d = q.shape
    O = np.empty((B, H, Tq, v.shape[-1]), dtype=np.float64)
    LSE = np.empty((B, H, Tq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            O[b, h], LSE[b, h] = naive_attention_head(q[b, h], k[b, h], v[b, h], scale, causal)
    return O, LSE


def online_softmax_row(q_row, K, V, scale: float, tile: int, visible=None):
    """The online-softmax recurrence for one query row, streaming K/V in tiles of ``tile`` keys.

    Follows the per-row recurrence of page "Kernels — fusion and FlashAttention", §3: running max
    m, running denominator l and running output o start at (-inf, 0, 0); for each tile the running
    max is raised to cover the tile's scores, the old l and o are multiplied by the correction
    exp(m_old - m_new), the tile's shifted exponentials are added to l and their value-weighted sum
    to o; the output is o / l.  The log-sum-exp m + ln l is returned as well.  Written with scalar
    Python arithmetic per key so that it shares nothing with the vectorised two-pass path.
    Returns (o [d], lse).
    """
    q_row = [float(x) for x in q_row]
    Tk, d = len(K), len(q_row)
    m, ell = -math.inf, 0.0
    o = [0.0] * d
    for j0 in range(0, Tk, tile):
        idx = [j for j in range(j0, min(Tk, j0 + tile)) if visible is None or visible[j]]
        if not idx:
            continue
        s = {}
        for j in idx:
            acc = 0.0
            for t in range(d):
                acc += q_row[t] * float(K[j][t])
            s[j] = float(scale) * acc
        m_new = max(m, max(s.values()))
        c = math.exp(m - m_new) if m != -math.inf else 0.0
        p = {j: math.exp(s[j] - m_new) for j in idx}
        ell = ell * c + sum(p.values())
        for t in range(d):
            o[t] = o[t] * c + sum(p[j] * float(V[j][t]) for j in idx)
        m = m_new
    if ell == 0.0:
        raise ValueError("a query row has no visible key; its softmax is undefined")
    return np.array([x / ell for x in o]), m + math.log(ell)


def scalar_attention_loops(q, k, v, scale: float, causal: bool):
    """Brute force with pure-Python loops over one head (tiny inputs only).

    Two passes per row exactly as the definition reads: all scores, their max, the exponentials,
    their sum, the weighted sum of V rows.  Returns (O [Tq][d], LSE [Tq]).
    """
    Tq, Tk, d = len(q), len(k), len(q[0])
    O = np.zeros((Tq, d))
    LSE = np.zeros(Tq)
    for i in range(Tq):
        s = []
        for j in range(Tk):
            if causal and j > i + (Tk - Tq):
                continue
            s.append((j, float(scale) * sum(float(q[i][t]) * float(k[j][t]) for t in range(d))))
        mx = max(x for _, x in s)
        e = [(j, math.exp(x - mx)) for j, x in s]
        tot = sum(x for _, x in e)
        for t in range(d):
            O[i, t] = sum(w * float(v[j][t]) for j, w in e) / tot
        LSE[i] = mx + math.log(tot)
    return O, LSE


def split_kv_partials(q_row, K, V, scale: float, num_splits: int):
    """Per-chunk partial softmax state for one decode query (split-KV / FlashDecoding reading).

    Page "Fusion and IO-aware kernels", "Where it breaks": at decode the sequence is split across
    workers and the pieces are combined afterwards.  The sequence of Tk keys is cut into
    ``num_splits`` chunks of ceil(Tk / num_splits) keys (the last ones may be short or empty); each
    chunk reports its own max m_s, its denominator l_s = sum exp(s - m_s) and its unnormalised
    output o_s = sum exp(s - m_s) v.  An empty chunk reports (-inf, 0, 0).
    """
    q_row = np.asarray(q_row, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Tk = K.shape[0]
    chunk = -(-Tk // num_splits)
    parts = []
    for s in range(num_splits):
        lo, hi = s * chunk, min(Tk, (s + 1) * chunk)
        if lo >= hi:
            parts.append((-np.inf, 0.0, np.zeros(V.shape[1])))
            continue
        sc = float(scale) * (K[lo:hi] @ q_row)
        m = sc.max()
        p = np.exp(sc - m)
        parts.append((m, p.sum(), p @ V[lo:hi]))
    return parts


def combine_split_partials(parts):
    """Merge per-chunk (m_s, l_s, o_s) into the row's output and log-sum-exp.

    The merge is the rescale of page "Kernels — fusion and FlashAttention", §3: bring every chunk
    onto the common max m* = max_s m_s by the factor exp(m_s - m*), add the denominators and the
    outputs, divide.  Chunks with m_s = -inf carry weight 0.  Returns (o [d], lse).
    """
    m_star = max(m for m, _, _ in parts)
    if not np.isfinite(m_star):
        raise ValueError("every chunk is empty")
    ell = 0.0
    o = None
    for m, l_s, o_s in parts:
        w = 0.0 if m == -np.inf else math.exp(m - m_star)
        ell += w * l_s
        o = w * o_s if o is None else o + w * o_s
    return o / ell, m_star + math.log(ell)


def split_kv_decode(q, k, v, scale: float, num_splits: int, heads=None):
    """Split-KV decode over [B][h][d] queries and [B][h][Tk][d] caches, chunk by chunk.

    ``heads`` optionally lists (b, h) pairs to compute; returns (O, LSE) for those (or for all).
    """
    q = np.asarray(q)
    B, H = q.shape[0], q.shape[1]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    O = np.empty((len(heads), q.shape[-1]))
    LSE = np.empty(len(heads))
    for n, (b, h) in enumerate(heads):
        O[n], LSE[n] = combine_split_partials(
            split_kv_partials(q[b, h], k[b, h], v[b, h], scale, num_splits))
    return O, LSE
