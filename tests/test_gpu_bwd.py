"""GPU parity of the attention backward (dQ, dK, dV) against the fp64 oracle, through the C ABI.

The kernels take O (bf16) and LSE (fp32) as inputs; the parity cases feed them the oracle's own O
rounded to bf16 and LSE rounded to fp32, so each gradient element is gated by a tolerance derived
from the kernels' arithmetic (tests/gpu_support.py: bwd_tolerances).  The end-to-end cases feed
the GPU forward's outputs instead, with the forward's O error added to the bound.  Full workload
sizes run in the launch configuration the benchmark times, with the oracle on sampled heads.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from tests.gpu_support import (assert_bwd_bf16_is_rne_of_f32, check_bwd_head, log,
                               oracle_bwd_head, run_bwd, to_gpu, workload_inputs)

pytestmark = pytest.mark.gpu


def _small_case(B, h, Tq, Tk, d, causal, seed, scale=None):
    wl = si.custom_workload(B, h, Tq, Tk, d, causal, name=f"bwd_b{B}_h{h}_q{Tq}_k{Tk}_d{d}")
    q, k, v = si.make_inputs(wl, seed)
    do = si.make_grad(wl, seed)
    scale = wl.scale if scale is None else scale
    o = np.empty_like(q)
    lse = np.empty((B, h, Tq), dtype=np.float32)
    refs = {}
    for b in range(B):
        for hh in range(h):
            r, x64, o_bits, l32 = oracle_bwd_head(q[b, hh], k[b, hh], v[b, hh], do[b, hh], scale,
                                                  causal)
            refs[(b, hh)] = (r, x64)
            o[b, hh], lse[b, hh] = o_bits, l32
    return wl, scale, q, k, v, do, o, lse, refs


SMALL = [
    # B, h, Tq, Tk, d, causal
    (1, 2, 200, 200, 64, True),      # ragged, several tiles
    (1, 2, 130, 300, 128, False),    # Tq != Tk, ragged both ways
    (2, 1, 257, 257, 128, True),     # one row past a block
    (1, 1, 100, 333, 64, True),      # causal with Tq < Tk (bottom-right diagonal)
    (1, 1, 1, 1, 128, False),        # a single query and key
    (1, 1, 1, 70, 64, True),         # one query that sees every key
    (1, 3, 64, 64, 128, True),       # exactly one tile
    (1, 8, 256, 256, 128, True),     # head count on the XCD grouping
    (1, 8, 192, 448, 64, False),     # XCD grouping, non-causal, Tk > Tq
    (1, 2, 1024, 1024, 128, True),   # many tiles
    (1, 2, 600, 700, 128, True),     # several 256-query blocks, ragged, diagonal offset
    (2, 1, 513, 513, 64, False),     # two 256-query blocks plus one row
]


@pytest.mark.parametrize("B,h,Tq,Tk,d,causal", SMALL)
def test_bwd_parity_small(gpu, B, h, Tq, Tk, d, causal):
    tag = f"bwd B={B} h={h} Tq={Tq} Tk={Tk} d={d} causal={causal}"
    log(f"[case] {tag}")
    wl, scale, q, k, v, do, o, lse, refs = _small_case(B, h, Tq, Tk, d, causal, seed=5)
    res = run_bwd(gpu, q, k, v, o, do, lse, causal, scale)
    assert_bwd_bf16_is_rne_of_f32(res)
    for bh, (r, x64) in refs.items():
        check_bwd_head(tag, res, bh, r, x64, scale)


@pytest.mark.parametrize("scale", [-0.11, 0.5, 0.0])
def test_bwd_parity_scales(gpu, scale):
    tag = f"bwd scale={scale}"
    log(f"[case] {tag}")
    wl, scale, q, k, v, do, o, lse, refs = _small_case(1, 2, 150, 190, 64, True, seed=6,
                                                       scale=scale)
    res = run_bwd(gpu, q, k, v, o, do, lse, True, scale)
    for bh, (r, x64) in refs.items():
        check_bwd_head(tag, res, bh, r, x64, scale)


def test_bwd_is_deterministic(gpu):
    log("[case] bwd determinism")
    wl, scale, q, k, v, do, o, lse, refs = _small_case(1, 4, 300, 300, 128, True, seed=7)
    a = run_bwd(gpu, q, k, v, o, do, lse, True, scale, f32=False)
    b = run_bwd(gpu, q, k, v, o, do, lse, True, scale, f32=False)
    for name in ("dq16", "dk16", "dv16"):
        assert torch.equal(a[name].view(torch.int16), b[name].view(torch.int16)), name


def test_bwd_end_to_end_with_gpu_forward(gpu):
    """Forward on the GPU, its O and LSE into the backward; the bound adds the forward's O error
    (P rounded to bf16 before P V, normalised by the rounded sum, O rounded: <= 3u sum P|V|)."""
    B, h, T, d = 1, 2, 520, 128
    log(f"[case] bwd end-to-end B={B} h={h} T={T} d={d}")
    wl, scale, q, k, v, do, o_oracle, lse_oracle, refs = _small_case(B, h, T, T, d, True, seed=8)
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    o_gpu, lse_gpu = gpu.fa_fwd(qg, kg, vg, causal=True, scale=scale)
    res = run_bwd(gpu, qg, kg, vg, o_gpu, to_gpu(do), lse_gpu, True, scale)
    for bh, (r, x64) in refs.items():
        o_err = 3 * 2.0 ** -8 * (r["P"] @ np.abs(x64[2])) + 1e-6
        check_bwd_head("bwd e2e", res, bh, r, x64, scale, o_err=o_err)


def _full_size(gpu, name, sample_heads):
    """Full workload in the benchmark's launch configuration: O and LSE from the GPU forward for
    every head, replaced by the oracle's (rounded) values on the sampled heads, which are then
    checked element by element."""
    wl, q, k, v = workload_inputs(name)
    do = si.make_grad(wl, 0)
    qg, kg, vg, dog = to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(do)
    o_gpu, lse_gpu = gpu.fa_fwd(qg, kg, vg, causal=wl.causal, scale=wl.scale)
    refs = {}
    for (b, h) in sample_heads:
        log(f"[oracle] {name} head {(b, h)}")
        r, x64, o_bits, l32 = oracle_bwd_head(q[b, h], k[b, h], v[b, h], do[b, h], wl.scale,
                                              wl.causal)
        refs[(b, h)] = (r, x64)
        o_gpu[b, h] = to_gpu(o_bits)
        lse_gpu[b, h] = torch.from_numpy(l32).cuda()
    log(f"[gpu] {name} backward")
    res = run_bwd(gpu, qg, kg, vg, o_gpu, dog, lse_gpu, wl.causal, wl.scale)
    assert_bwd_bf16_is_rne_of_f32(res)
    for name_ in ("dq16", "dk16", "dv16"):
        assert bool(torch.isfinite(res[name_].float()).all()), name_
    for bh, (r, x64) in refs.items():
        check_bwd_head(name, res, bh, r, x64, wl.scale)


def test_bwd_causal_t1024_d64_full_size(gpu):
    _full_size(gpu, "causal_b8_h32_t1024_d64", [(0, 0), (4, 13), (7, 31)])


def test_bwd_causal_t4096_d128_full_size(gpu):
    _full_size(gpu, "causal_b8_h32_t4096_d128", [(0, 0), (5, 9)])


def test_bwd_persistent_schedule_more_pairs_than_cus(gpu):
    """111 heads (not a multiple of the 8 XCD groups) and 9 key blocks per head (an odd count:
    a middle block without a partner): 555 key-block pairs for the persistent dK/dV grid, and
    555 query blocks in dQ's eight item queues of unequal length (14 or 13 heads: workgroups
    take from other queues at the end).  Every gradient element is written (outputs start as
    NaN), and sampled heads, among them the last heads of several groups, match the oracle."""
    B, h, T, d = 3, 37, 1100, 128
    log(f"[case] bwd persistent B={B} h={h} T={T} d={d}")
    wl = si.custom_workload(B, h, T, T, d, True, name="bwd_persistent")
    q, k, v = si.make_inputs(wl, 31)
    do = si.make_grad(wl, 31)
    qg, kg, vg, dog = to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(do)
    o_gpu, lse_gpu = gpu.fa_fwd(qg, kg, vg, causal=True, scale=wl.scale)
    refs = {}
    for bh in (0, 7, 8, 55, 103, 104, 109, 110):
        b, hh = divmod(bh, h)
        r, x64, o_bits, l32 = oracle_bwd_head(q[b, hh], k[b, hh], v[b, hh], do[b, hh], wl.scale,
                                              True)
        refs[(b, hh)] = (r, x64)
        o_gpu[b, hh] = to_gpu(o_bits)
        lse_gpu[b, hh] = torch.from_numpy(l32).cuda()
    nan = float("nan")
    dq = torch.full_like(qg, nan)
    dk = torch.full_like(kg, nan)
    dv = torch.full_like(vg, nan)
    gpu.fa_bwd(qg, kg, vg, o_gpu, dog, lse_gpu, causal=True, scale=wl.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t.float()).all()), f"{name}: an element was not written"
    res = {"dq16": dq, "dk16": dk, "dv16": dv}
    for bh, (r, x64) in refs.items():
        check_bwd_head("bwd persistent", res, bh, r, x64, wl.scale)
