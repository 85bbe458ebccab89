"""GPU parity of the one-pass row softmax against the fp64 oracle, through the C ABI.

Tolerance, derived from the kernel's fp32 arithmetic: each output is exp2((x - m) log2 e) for the
lane's max m (the subtraction and the multiply round once each, the exponential is within an
ulp or two), times exp(m - M) / L with M the row max and L an fp32 sum of at most a few thousand
positive terms (relative error < 2^-16 for these row lengths).  So
    |y - y_ref| <= y_ref * (2^-21 (|x - M| + |M| + 1) + 2^-15) + 2^-40,
and |lse - lse_ref| <= 2^-22 |M| + 2^-15.  The full-size case runs the 4096 x 4096 workload in the
launch configuration the benchmark times, with the oracle on sampled rows.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import softmax_ref as sref
from tests.gpu_support import log

pytestmark = pytest.mark.gpu


def _check(tag, x, y, lse, rows=None):
    x = np.asarray(x, dtype=np.float64)
    rows = np.arange(x.shape[0]) if rows is None else rows
    y_ref, l_ref = sref.softmax_rows(x[rows])
    got = np.asarray(y, dtype=np.float64)[rows]
    M = np.max(x[rows], axis=1, keepdims=True)
    fin = np.isfinite(x[rows])
    dist = np.where(fin, np.abs(x[rows] - M), 0.0)
    # masked (-inf) entries must be exactly 0
    tol = np.where(fin, y_ref * (2.0 ** -21 * (dist + np.abs(M) + 1) + 2.0 ** -15) + 2.0 ** -40,
                   0.0)
    err = np.abs(got - y_ref)
    ratio = float(np.max(np.where(fin, err / np.where(fin, tol, 1.0), 0.0)))
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    assert np.all(err <= tol), f"{tag}: max err {err.max():.3e}, worst ratio {ratio:.3f}"
    if lse is not None:
        lg = np.asarray(lse, dtype=np.float64)[rows]
        lt = 2.0 ** -22 * np.abs(M[:, 0]) + 2.0 ** -15
        assert np.all(np.abs(lg - l_ref) <= lt), f"{tag}: lse beyond tolerance"
    log(f"[parity] softmax {tag}: max|dy|={err.max():.2e} (x{ratio:.3f} of tol)")


SHAPES = [(7, 1), (5, 3), (3, 63), (9, 257), (11, 260), (6, 4096), (2, 8192), (3, 8193),
          (2, 12000), (1, 100000), (13, 1000)]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_softmax_shapes(gpu, rows, cols):
    log(f"[case] softmax rows={rows} cols={cols}")
    x = si.softmax_rows_input(rows, cols, seed=3) * np.float32(2.0)
    xg = torch.from_numpy(x).cuda()
    y, lse = gpu.fa_softmax_rows(xg, with_lse=True)
    torch.cuda.synchronize()
    _check(f"{rows}x{cols}", x, y.cpu().numpy(), lse.cpu().numpy())


def test_softmax_large_logits_and_masks(gpu):
    log("[case] softmax large logits and -inf entries")
    rng = np.random.default_rng(9)
    x = rng.uniform(-1000, 1000, size=(8, 777)).astype(np.float32)
    x[1, ::3] = -np.inf                     # masked entries
    x[2, :] = -np.inf
    x[2, 500] = 3.0                         # a single visible entry
    x[3, :] = 123.5                         # constant row
    xg = torch.from_numpy(x).cuda()
    y, lse = gpu.fa_softmax_rows(xg, with_lse=True)
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    assert np.all(yc[1, ::3] == 0.0)
    assert yc[2, 500] == 1.0 and np.all(np.delete(yc[2], 500) == 0.0)
    _check("large/masked", x, yc, lse.cpu().numpy())


def test_softmax_unaligned_scalar_path(gpu):
    log("[case] softmax unaligned pointers (scalar path)")
    x = si.softmax_rows_input(5, 1025, seed=4)
    buf = torch.from_numpy(np.concatenate([[0.0], x.ravel()]).astype(np.float32)).cuda()
    xv = buf[1:].view(5, 1025)
    y, _ = gpu.fa_softmax_rows(xv)
    torch.cuda.synchronize()
    _check("unaligned", x, y.cpu().numpy(), None)


def test_softmax_workload_full_size(gpu):
    rows, cols = si.SOFTMAX_WORKLOAD
    log(f"[case] softmax workload {rows}x{cols}")
    x = si.softmax_rows_input(rows, cols, seed=0)
    xg = torch.from_numpy(x).cuda()
    y, lse = gpu.fa_softmax_rows(xg, with_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    sample = np.unique(np.concatenate([[0, 1, rows - 1], rng.choice(rows, 61, replace=False)]))
    _check("4096x4096 sampled", x, y.cpu().numpy(), lse.cpu().numpy(), rows=sample)
    # every row sums to one
    s = y.double().sum(dim=1).cpu().numpy()
    assert np.max(np.abs(s - 1.0)) <= 1e-5
