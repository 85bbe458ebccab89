"""GPU parity of the fused elementwise chains (GELU fp32 / bf16, bias-GELU-dropout bf16) against
the fp64 oracle, through the C ABI.

Tolerance, from the kernels' fp32 arithmetic: gelu(x) = x / (1 + 2^z) with
z = -2 sqrt(2/pi) log2(e) x (1 + 0.044715 x^2).  z carries a few roundings (relative 2^-22), the
exponential and the division a couple of ulps, and dy/dz is at most |x| ln2 / 4, so
    |y - gelu(x)| <= 2^-21 (|x| |z| + 2 |y|) + 2^-120,
plus half a bf16 ulp (2^-8 |y|) where the output is bf16.  The dropout mask is an integer
decision and must match the oracle exactly.  Full workloads run at the pages' sizes in the launch
configuration the benchmark times, with the oracle on sampled elements or rows.
"""
import math

import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import elementwise_ref as eref
from tests.gpu_support import log

pytestmark = pytest.mark.gpu

K1 = -2.0 * math.sqrt(2.0 / math.pi) * math.log2(math.e)


def _tol(xin, y_ref, bf16_out, scale=1.0):
    z = K1 * xin * (1.0 + 0.044715 * xin * xin)
    t = (2.0 ** -21 * (np.abs(xin) * np.abs(z) + 2 * np.abs(y_ref / scale))) * scale + 2.0 ** -120
    if scale != 1.0:
        t = t + 2.0 ** -23 * np.abs(y_ref)   # the fp32 rounding of the dropout factor
    if bf16_out:
        t = t + 2.0 ** -8 * np.abs(y_ref)
    return t


def _check(tag, xin, got, y_ref, bf16_out, scale=1.0):
    err = np.abs(got - y_ref)
    tol = _tol(xin, y_ref, bf16_out, scale)
    ratio = float(np.max(err / tol)) if err.size else 0.0
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"{tag}: {len(bad)} elements beyond tolerance, first {bad[0]}: "
                           f"x={xin.ravel()[bad[0][0]]} got={got.ravel()[bad[0][0]]} "
                           f"ref={y_ref.ravel()[bad[0][0]]}")
    log(f"[parity] {tag}: max|dy|={err.max():.2e} (x{ratio:.3f} of tol)")


def _bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1023, 4099, 1_000_003])
def test_gelu_f32_lengths(gpu, n):
    log(f"[case] gelu f32 n={n}")
    x = si.elementwise_input(n, seed=2) * np.float32(3.0)
    x[:3] = np.array([0.0, 40.0, -40.0], dtype=np.float32)[: min(3, n)]
    y = gpu.fa_gelu_f32(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    x64 = x.astype(np.float64)
    _check(f"gelu f32 n={n}", x64, y.cpu().numpy().astype(np.float64), eref.gelu_tanh(x64), False)


@pytest.mark.parametrize("n", [1, 7, 8, 9, 100_001])
def test_gelu_bf16_lengths(gpu, n):
    log(f"[case] gelu bf16 n={n}")
    xb = si.rne_bf16_bits(si.elementwise_input(n, seed=3) * np.float32(3.0))
    xg = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    y = gpu.fa_gelu_bf16(xg)
    torch.cuda.synchronize()
    x64 = si.bf16_bits_to_f64(xb)
    _check(f"gelu bf16 n={n}", x64, _bf16_to_f64(y), eref.gelu_tanh(x64), True)


def test_gelu_in_place(gpu):
    x = si.elementwise_input(10_000, seed=4)
    xg = torch.from_numpy(x).cuda()
    gpu.fa_gelu_f32(xg, y=xg)
    torch.cuda.synchronize()
    x64 = x.astype(np.float64)
    _check("gelu in place", x64, xg.cpu().numpy().astype(np.float64), eref.gelu_tanh(x64), False)


def test_gelu_f32_workload_full_size(gpu):
    n = si.GELU_WORKLOAD_N
    log(f"[case] gelu f32 workload n={n}")
    x = si.elementwise_input(n, seed=0)
    y = gpu.fa_gelu_f32(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    rng = np.random.default_rng(31)
    idx = np.unique(np.concatenate([np.arange(100), np.arange(n - 100, n),
                                    rng.integers(0, n, 2_000_000)]))
    x64 = x[idx].astype(np.float64)
    _check("gelu f32 64M sampled", x64, yc[idx].astype(np.float64), eref.gelu_tanh(x64), False)


def _dropout_case(gpu, rows, cols, p, seed, offset, tag, sample_rows=None):
    xb, bb = si.activation_input(rows, cols, seed=5)
    xg = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    bg = torch.from_numpy(bb.view(np.int16)).view(torch.bfloat16).cuda()
    y = gpu.fa_bias_gelu_dropout_bf16(xg, bg, p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    got = _bf16_to_f64(y)
    rows_ = np.arange(rows) if sample_rows is None else sample_rows
    b64 = si.bf16_bits_to_f64(bb)
    scale = 1.0 / (1.0 - p)
    kept_total, n_total = 0, 0
    for r in rows_:
        x64 = si.bf16_bits_to_f64(xb[r:r + 1])
        y_ref, keep = eref.bias_gelu_dropout(x64, b64, p, seed, offset, first_row=int(r))
        g = got[r:r + 1]
        assert np.all(g[~keep] == 0.0), f"{tag}: row {r}: a dropped element is not zero"
        if keep.any():
            # the kernel's factor is 1 / (1 - p) rounded to fp32: within 2^-24 of the exact one
            _check(f"{tag} row {r}", (x64 + b64[None, :])[keep], g[keep], y_ref[keep], True,
                   scale)
        kept_total += int(keep.sum())
        n_total += keep.size
    log(f"[parity] {tag}: mask exact on {len(rows_)} rows, kept {kept_total / n_total:.4f} "
        f"(1 - p = {1 - p:.4f})")


@pytest.mark.parametrize("rows,cols,p,seed,offset", [
    (3, 7, 0.1, 1, 0),                      # scalar path
    (4, 8, 0.5, 2, 5),
    (5, 1000, 0.1, 3, 2**33 + 7),           # vector path, offset above 32 bits
    (2, 1003, 0.9, 2**40 + 11, 1),          # scalar path, seed above 32 bits
    (6, 4096, 0.0, 9, 0),                   # p = 0: no drops
    (1, 2048, 0.3, 4, 3),                   # vector path, one row (its pair has no second row)
    (7, 24, 0.2, 6, 1),                     # vector path, odd row count, one lane per row
])
def test_bias_gelu_dropout_shapes(gpu, rows, cols, p, seed, offset):
    log(f"[case] bias-gelu-dropout {rows}x{cols} p={p} seed={seed} offset={offset}")
    _dropout_case(gpu, rows, cols, p, seed, offset, f"dropout {rows}x{cols} p={p}")


def test_bias_gelu_dropout_workload_full_size(gpu):
    rows, cols, p = si.DROPOUT_WORKLOAD
    log(f"[case] bias-gelu-dropout workload {rows}x{cols} p={p}")
    rng = np.random.default_rng(41)
    sample = np.unique(np.concatenate([[0, 1, rows - 1], rng.choice(rows, 29, replace=False)]))
    _dropout_case(gpu, rows, cols, p, 1234, 0, "dropout 4096x8192", sample_rows=sample)
