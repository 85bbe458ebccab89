"""GPU parity of the backward's layout and head-dimension variants (fa_bwd_strided).

Contiguous d = 64 / 128 tensors passed as strided views (e.g. [B][T][h][d] storage, or rows with
gaps) must give fa_bwd's gradients bit for bit: the kernels stage the same bytes into the same
on-chip tiles.  Other head dims (multiples of 8 up to 128, zero-padded on chip) are gated
against the fp64 oracle with the bf16-output tolerance of the backward tests.  Columns outside a
strided output's rows must stay untouched.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from tests.gpu_support import check_bwd_head, log, oracle_bwd_head, to_gpu

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1   # a bf16 NaN bit pattern no kernel writes


def _bthd(x):
    """[B][h][T][d] bf16 (bits or tensor) -> a [B][h][T][d] view of a [B][T][h][d] GPU tensor."""
    t = to_gpu(x) if isinstance(x, np.ndarray) else x
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def _gapped_out(B, h, T, d, extra):
    """A [B][h][T][d] bf16 view into a sentinel-filled [B][T][h][d + extra] buffer."""
    buf = torch.full((B, T, h, d + extra), SENTINEL, dtype=torch.int16, device="cuda")
    return buf, buf.view(torch.bfloat16)[..., :d].transpose(1, 2)


def _gap_untouched(buf, d):
    return bool(torch.all(buf[..., d:] == SENTINEL))


def _inputs(B, h, Tq, Tk, d, causal, seed):
    wl = si.custom_workload(B, h, Tq, Tk, d, causal, name=f"bwdlay_b{B}_h{h}_q{Tq}_k{Tk}_d{d}")
    q, k, v = si.make_inputs(wl, seed)
    do = si.make_grad(wl, seed)
    return wl, q, k, v, do


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_strided_equals_contiguous_bitwise(gpu, d, causal):
    B, h, Tq, Tk = 2, 3, 300, (300 if causal else 257)
    tag = f"bwd strided d={d} causal={causal}"
    log(f"[case] {tag}")
    wl, q, k, v, do = _inputs(B, h, Tq, Tk, d, causal, seed=21)
    qg, kg, vg, dog = (to_gpu(x) for x in (q, k, v, do))
    og, lse = gpu.fa_fwd(qg, kg, vg, causal=causal, scale=wl.scale)
    ref = gpu.fa_bwd(qg, kg, vg, og, dog, lse, causal=causal, scale=wl.scale)
    # [B][T][h][d] inputs; dq into a gapped [B][T][h][d + 8] buffer, dk / dv default (same
    # strides as k / v)
    dq_buf, dq_view = _gapped_out(B, h, Tq, d, 8)
    got = gpu.fa_bwd_strided(_bthd(qg), _bthd(kg), _bthd(vg), _bthd(og), _bthd(dog), lse,
                             causal=causal, scale=wl.scale, dq=dq_view)
    torch.cuda.synchronize()
    assert got[0].data_ptr() == dq_buf.data_ptr()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a.contiguous().view(torch.int16), b.view(torch.int16)), \
            f"{tag}: {name} differs from fa_bwd"
    assert _gap_untouched(dq_buf, d), f"{tag}: dq wrote outside its rows"
    log(f"[parity] {tag}: dq, dk, dv equal fa_bwd bit for bit")


@pytest.mark.parametrize("d", [8, 48, 80, 96, 120])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_padded_head_dims(gpu, d, causal):
    B, h, Tq, Tk = 1, 2, 200, (200 if causal else 333)
    tag = f"bwd d={d} causal={causal}"
    log(f"[case] {tag}")
    wl, q, k, v, do = _inputs(B, h, Tq, Tk, d, causal, seed=22)
    o = np.empty_like(q)
    lse = np.empty((B, h, Tq), dtype=np.float32)
    refs = {}
    for hh in range(h):
        r, x64, o_bits, l32 = oracle_bwd_head(q[0, hh], k[0, hh], v[0, hh], do[0, hh], wl.scale,
                                              causal)
        refs[hh] = (r, x64)
        o[0, hh], lse[0, hh] = o_bits, l32
    args = (to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(o), to_gpu(do), torch.from_numpy(lse).cuda())
    dq, dk, dv = gpu.fa_bwd_strided(*args, causal=causal, scale=wl.scale)
    # the contiguous entry point takes the same padded kernels for the same tensors
    same = gpu.fa_bwd(*args, causal=causal, scale=wl.scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), same):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), \
            f"{tag}: fa_bwd {name} differs from fa_bwd_strided"
    res = {"dq16": dq, "dk16": dk, "dv16": dv}
    for hh in range(h):
        check_bwd_head(tag, res, (0, hh), refs[hh][0], refs[hh][1], wl.scale)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_strided_padded_bthd(gpu, causal):
    """d = 80 in [B][T][h][d] storage, every output into a gapped buffer."""
    B, h, Tq, Tk, d = 2, 2, 150, (150 if causal else 221), 80
    tag = f"bwd bthd d={d} causal={causal}"
    log(f"[case] {tag}")
    wl, q, k, v, do = _inputs(B, h, Tq, Tk, d, causal, seed=23)
    o = np.empty_like(q)
    lse = np.empty((B, h, Tq), dtype=np.float32)
    refs = {}
    for b in range(B):
        for hh in range(h):
            r, x64, o_bits, l32 = oracle_bwd_head(q[b, hh], k[b, hh], v[b, hh], do[b, hh],
                                                  wl.scale, causal)
            refs[(b, hh)] = (r, x64)
            o[b, hh], lse[b, hh] = o_bits, l32
    bufs = [_gapped_out(B, h, T, d, 16) for T in (Tq, Tk, Tk)]
    dq, dk, dv = gpu.fa_bwd_strided(_bthd(q), _bthd(k), _bthd(v), _bthd(o), _bthd(do),
                                    torch.from_numpy(lse).cuda(), causal=causal, scale=wl.scale,
                                    dq=bufs[0][1], dk=bufs[1][1], dv=bufs[2][1])
    torch.cuda.synchronize()
    for buf, _ in bufs:
        assert _gap_untouched(buf, d), f"{tag}: an output wrote outside its rows"
    res = {"dq16": dq, "dk16": dk, "dv16": dv}
    for bh, (r, x64) in refs.items():
        check_bwd_head(tag, res, bh, r, x64, wl.scale)
