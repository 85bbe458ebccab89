"""GPU parity of the decode's layout and head-dimension variants (fa_decode_strided).

A strided KV cache (e.g. [B][Tk][h][d] storage) with d = 64 / 128 must give fa_decode's output
bit for bit; other head dims (multiples of 8 up to 128, zero-padded on chip) are gated against
the fp64 oracle like the decode tests (max|dO| <= 1e-2 on the bf16 output, max|dLSE| <= 1e-3).
Elements outside a strided output must stay untouched.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import attention_ref as ref
from tests.gpu_support import LSE_TOL, O_TOL, log, to_gpu

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1   # a bf16 NaN bit pattern no kernel writes


def _case(B, h, Tk, d, seed):
    wl = si.custom_workload(B, h, 1, Tk, d, False, decode=True, num_splits=5,
                            name=f"declay_b{B}_h{h}_k{Tk}_d{d}")
    q, k, v = si.make_inputs(wl, seed)
    return wl, q, k, v


def _kv_bthd(bits):
    """[B][h][Tk][d] bits -> a [B][h][Tk][d] view of a [B][Tk][h][d] GPU tensor."""
    return to_gpu(np.ascontiguousarray(bits.transpose(0, 2, 1, 3))).transpose(1, 2)


def _gapped_o(B, h, d, extra):
    """A [B][h][d] bf16 view into a sentinel-filled [B][h][d + extra] buffer."""
    buf = torch.full((B, h, d + extra), SENTINEL, dtype=torch.int16, device="cuda")
    return buf, buf.view(torch.bfloat16)[..., :d]


def _oracle_gate(tag, o, lse, q, k, v, scale):
    B, h = q.shape[:2]
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    worst_o = worst_l = 0.0
    for b in range(B):
        for hh in range(h):
            Or, Lr = ref.naive_attention_head(si.bf16_bits_to_f64(q[b, hh])[None],
                                              si.bf16_bits_to_f64(k[b, hh]),
                                              si.bf16_bits_to_f64(v[b, hh]), scale, False)
            worst_o = max(worst_o, float(np.max(np.abs(og[b, hh] - Or[0]))))
            worst_l = max(worst_l, abs(float(lg[b, hh]) - float(Lr[0])))
    log(f"[parity] {tag}: max|dO16|={worst_o:.3e} max|dLSE|={worst_l:.3e}")
    assert worst_o <= O_TOL and worst_l <= LSE_TOL


@pytest.mark.parametrize("d", [64, 128])
def test_decode_strided_equals_contiguous_bitwise(gpu, d):
    B, h, Tk = 2, 3, 777
    tag = f"decode strided d={d}"
    log(f"[case] {tag}")
    wl, q, k, v = _case(B, h, Tk, d, seed=31)
    qg = to_gpu(q)
    o_ref, l_ref = gpu.fa_decode(qg, to_gpu(k), to_gpu(v), num_splits=5, scale=wl.scale)
    buf, o_view = _gapped_o(B, h, d, 8)
    o, lse = gpu.fa_decode_strided(qg, _kv_bthd(k), _kv_bthd(v), num_splits=5, scale=wl.scale,
                                   o=o_view)
    torch.cuda.synchronize()
    assert torch.equal(o.contiguous().view(torch.int16), o_ref.view(torch.int16)), tag
    assert torch.equal(lse, l_ref), tag
    assert bool(torch.all(buf[..., d:] == SENTINEL)), f"{tag}: o written outside its rows"


@pytest.mark.parametrize("d", [8, 48, 80, 120])
def test_decode_padded_head_dims(gpu, d):
    B, h, Tk = 2, 2, 300
    tag = f"decode d={d}"
    log(f"[case] {tag}")
    wl, q, k, v = _case(B, h, Tk, d, seed=32)
    o, lse = gpu.fa_decode_strided(to_gpu(q), to_gpu(k), to_gpu(v), num_splits=5,
                                   scale=wl.scale)
    # the contiguous entry point takes the same padded kernels for the same tensors
    o2, lse2 = gpu.fa_decode(to_gpu(q), to_gpu(k), to_gpu(v), num_splits=5, scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(lse2, lse), \
        f"{tag}: fa_decode differs from fa_decode_strided"
    _oracle_gate(tag, o, lse, q, k, v, wl.scale)


def test_decode_strided_padded_bthd(gpu):
    B, h, Tk, d = 2, 3, 513, 80
    tag = f"decode bthd d={d}"
    log(f"[case] {tag}")
    wl, q, k, v = _case(B, h, Tk, d, seed=33)
    # q as a [B][h][d] view with gaps between heads
    qbuf = np.zeros((B, h, d + 16), dtype=np.uint16)
    qbuf[..., :d] = q
    qv = to_gpu(qbuf)[..., :d]
    buf, o_view = _gapped_o(B, h, d, 24)
    o, lse = gpu.fa_decode_strided(qv, _kv_bthd(k), _kv_bthd(v), num_splits=7, scale=wl.scale,
                                   o=o_view)
    torch.cuda.synchronize()
    assert bool(torch.all(buf[..., d:] == SENTINEL)), f"{tag}: o written outside its rows"
    _oracle_gate(tag, o, lse, q, k, v, wl.scale)
