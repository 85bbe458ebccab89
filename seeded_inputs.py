"""Seeded synthetic inputs for the attention forward and split-KV decode workloads.

This module is shared by the CPU oracle's tests and by the GPU path's tests and benchmark. It holds
none of the attention arithmetic: it only draws standard-normal float32 values and rounds them to
bfloat16, so that both sides consume the very same bf16 bits.

Generator (fixed so that any single head can be regenerated on its own):
  * every (tensor, batch b, head h) slice is drawn from numpy's PCG64 stream
    ``default_rng([seed, tensor_id, b, h])`` with ``standard_normal(dtype=float32)``, in row-major
    [T][d] order; tensor ids are Q=0, K=1, V=2, the key-spike mask stream is 3 and the output
    gradient dO of the backward workloads is 4 (standard normal like the others);
  * the row-softmax workload's fp32 matrix is drawn the same way, row by row, from stream
    ``[seed, 5, row]`` (float32 standard normal, not rounded to bf16);
  * the GELU workload's flat fp32 vector is stream ``[seed, 6]``; the bias-GELU-dropout
    activation [rows][cols] is stream ``[seed, 7]`` and its per-column bias ``[seed, 8]``, both
    rounded to bf16;
  * float32 -> bfloat16 is round-to-nearest-even on the bit pattern (inputs are finite);
  * the long-context workload scales a Bernoulli(1%) subset of key vectors by 8 (a power of two,
    so the scaling is exact in bf16); the subset of head (b, h) is ``random(T) < 0.01`` drawn from
    stream ``[seed, 3, b, h]``.

Arrays are returned as ``uint16`` bit patterns (bf16), shape [B][h][T][d] (decode query: [B][h][d]).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_KEY_SPIKES, TENSOR_DO, TENSOR_SOFTMAX = 0, 1, 2, 3, 4, 5
TENSOR_ELEMENTWISE, TENSOR_ACTIVATION, TENSOR_BIAS = 6, 7, 8


@dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, mask and input structure."""

    name: str
    B: int
    h: int
    Tq: int
    Tk: int
    d: int
    causal: bool
    decode: bool = False
    num_splits: int = 0
    key_spike_frac: float = 0.0
    key_spike_mult: float = 1.0

    @property
    def scale(self) -> float:
        """1/sqrt(d_head) rounded to float32, the value the kernel receives."""
        return float(np.float32(1.0 / math.sqrt(self.d)))


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_noncausal_b1_h2_t128_d64", 1, 2, 128, 128, 64, False),
        Workload("causal_b8_h32_t1024_d64", 8, 32, 1024, 1024, 64, True),
        Workload("causal_b8_h32_t4096_d128", 8, 32, 4096, 4096, 128, True),
        Workload("longctx_causal_b2_h32_t16384_d128_keyspikes", 2, 32, 16384, 16384, 128, True,
                 key_spike_frac=0.01, key_spike_mult=8.0),
        Workload("decode_b64_h32_tk8192_d128_s16", 64, 32, 1, 8192, 128, False, decode=True,
                 num_splits=16),
    )
}


def rne_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def head_normal_bits(seed: int, tensor_id: int, b: int, h: int, rows: int, d: int) -> np.ndarray:
    """The [rows][d] bf16 slice of one tensor for head (b, h)."""
    rng = np.random.default_rng([seed, tensor_id, b, h])
    return rne_bf16_bits(rng.standard_normal(rows * d, dtype=np.float32)).reshape(rows, d)


def key_spike_rows(seed: int, b: int, h: int, T: int, frac: float) -> np.ndarray:
    """Boolean [T]: which key vectors of head (b, h) are scaled up."""
    rng = np.random.default_rng([seed, TENSOR_KEY_SPIKES, b, h])
    return rng.random(T) < frac


def head_inputs(wl: Workload, seed: int, b: int, h: int):
    """(q, k, v) bf16 bit arrays of one head: q [Tq][d], k and v [Tk][d]."""
    q = head_normal_bits(seed, TENSOR_Q, b, h, wl.Tq, wl.d)
    k = head_normal_bits(seed, TENSOR_K, b, h, wl.Tk, wl.d)
    v = head_normal_bits(seed, TENSOR_V, b, h, wl.Tk, wl.d)
    if wl.key_spike_frac > 0.0:
        rows = key_spike_rows(seed, b, h, wl.Tk, wl.key_spike_frac)
        k[rows] = rne_bf16_bits(bf16_bits_to_f32(k[rows]) * np.float32(wl.key_spike_mult))
    return q, k, v


def _threads(threads: int | None) -> int:
    if threads:
        return threads
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(wl: Workload, seed: int = 0, threads: int | None = None):
    """Full (q, k, v) bf16 bit arrays.

    Shapes: q [B][h][Tq][d] ([B][h][d] for decode), k and v [B][h][Tk][d].
    """
    q = np.empty((wl.B, wl.h, wl.Tq, wl.d), dtype=np.uint16)
    k = np.empty((wl.B, wl.h, wl.Tk, wl.d), dtype=np.uint16)
    v = np.empty((wl.B, wl.h, wl.Tk, wl.d), dtype=np.uint16)

    def fill(bh):
        b, h = divmod(bh, wl.h)
        q[b, h], k[b, h], v[b, h] = head_inputs(wl, seed, b, h)

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(fill, range(wl.B * wl.h)))
    if wl.decode:
        q = q.reshape(wl.B, wl.h, wl.d)
    return q, k, v


def make_grad(wl: Workload, seed: int = 0, threads: int | None = None) -> np.ndarray:
    """The output gradient dO [B][h][Tq][d] (bf16 bits) of a backward workload."""
    do = np.empty((wl.B, wl.h, wl.Tq, wl.d), dtype=np.uint16)

    def fill(bh):
        b, h = divmod(bh, wl.h)
        do[b, h] = head_normal_bits(seed, TENSOR_DO, b, h, wl.Tq, wl.d)

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(fill, range(wl.B * wl.h)))
    return do


SOFTMAX_WORKLOAD = (4096, 4096)   # rows x cols, fp32 (the pages' row-softmax worked example)


def softmax_rows_input(rows: int, cols: int, seed: int = 0, row0: int = 0) -> np.ndarray:
    """Rows row0 .. row0 + rows - 1 of the [*, cols] fp32 softmax input (standard normal)."""
    out = np.empty((rows, cols), dtype=np.float32)
    for r in range(rows):
        rng = np.random.default_rng([seed, TENSOR_SOFTMAX, row0 + r])
        out[r] = rng.standard_normal(cols, dtype=np.float32)
    return out


GELU_WORKLOAD_N = 64_000_000          # fp32 elements (the pages' GeLU case study)
DROPOUT_WORKLOAD = (4096, 8192, 0.1)  # rows, cols, p: the pages' 4096 x 8192 bf16 activation


def elementwise_input(n: int, seed: int = 0) -> np.ndarray:
    """The flat fp32 GELU input (standard normal)."""
    return np.random.default_rng([seed, TENSOR_ELEMENTWISE]).standard_normal(n, dtype=np.float32)


def activation_input(rows: int, cols: int, seed: int = 0):
    """(x [rows][cols], bias [cols]) as bf16 bit patterns for the bias-GELU-dropout chain."""
    x = np.random.default_rng([seed, TENSOR_ACTIVATION]).standard_normal(rows * cols,
                                                                         dtype=np.float32)
    b = np.random.default_rng([seed, TENSOR_BIAS]).standard_normal(cols, dtype=np.float32)
    return rne_bf16_bits(x).reshape(rows, cols), rne_bf16_bits(b)


def custom_workload(B, h, Tq, Tk, d, causal, name="custom", **kw) -> Workload:
    """A workload of arbitrary shape drawn with the same generator (edge-shape tests)."""
    return Workload(name, B, h, Tq, Tk, d, causal, **kw)
