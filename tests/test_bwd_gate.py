"""The backward parity gate has teeth (CPU only, no GPU).

At the prefill workload's head shape (causal, T = 4096, d = 128) the per-element tolerance the GPU
tests apply (tests/gpu_support.bwd_tolerances) must accept the exact gradients after the output
rounding a correct kernel performs, and must reject a gradient that lost the contribution of one
64-key tile (dQ) or of one 256-query block (dK, dV): the mistakes a tiling bug would make.
"""
import numpy as np
import pytest

import seeded_inputs as si
from tests.gpu_support import BWD_FAC_BF16, bwd_tolerances


@pytest.fixture(scope="module")
def head():
    from oracle import attention_bwd_ref as bref
    wl = si.custom_workload(1, 1, 4096, 4096, 128, True)
    q, k, v = si.make_inputs(wl, seed=0, threads=8)
    do = si.make_grad(wl, seed=0, threads=8)
    x = [si.bf16_bits_to_f64(t[0, 0]) for t in (q, k, v, do)]
    r = bref.backward_head(*x, wl.scale, True)
    tol = bwd_tolerances(r, *x, wl.scale, BWD_FAC_BF16)
    return r, x, wl.scale, tol


def _bf16(a):
    return si.bf16_bits_to_f64(si.rne_bf16_bits(a.astype(np.float32)))


def test_rounded_exact_gradients_pass(head):
    r, _, _, tol = head
    for name in ("dq", "dk", "dv"):
        assert np.all(np.abs(_bf16(r[name]) - r[name]) <= tol[name]), name


@pytest.mark.parametrize("tile", [0, 17, 40, 63])
def test_dq_missing_one_key_tile_fails(head, tile):
    r, (q, k, v, do), scale, tol = head
    j = slice(64 * tile, 64 * tile + 64)
    dq_bad = r["dq"] - scale * (r["dS"][:, j] @ k[j])
    assert np.any(np.abs(_bf16(dq_bad) - r["dq"]) > tol["dq"])


@pytest.mark.parametrize("block", [0, 7, 15])
def test_dk_dv_missing_one_query_block_fail(head, block):
    r, (q, k, v, do), scale, tol = head
    i = slice(256 * block, 256 * block + 256)
    dk_bad = r["dk"] - scale * (r["dS"][i].T @ q[i])
    dv_bad = r["dv"] - r["P"][i].T @ do[i]
    assert np.any(np.abs(_bf16(dk_bad) - r["dk"]) > tol["dk"])
    assert np.any(np.abs(_bf16(dv_bad) - r["dv"]) > tol["dv"])
