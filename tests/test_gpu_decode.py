"""GPU parity of the split-KV decode against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import attention_ref as ref
from tests.gpu_support import (LSE_TOL, O_TOL, bf16_floor, log, lse_row_tolerance, to_gpu,
                               workload_inputs)

pytestmark = pytest.mark.gpu


def _oracle(q, k, v, scale, heads):
    O = np.empty((len(heads), q.shape[-1]))
    L = np.empty(len(heads))
    for n, (b, h) in enumerate(heads):
        o, l = ref.naive_attention_head(si.bf16_bits_to_f64(q[b, h])[None],
                                        si.bf16_bits_to_f64(k[b, h]),
                                        si.bf16_bits_to_f64(v[b, h]), scale, causal=False)
        O[n], L[n] = o[0], l[0]
    return O, L


def _gate(tag, o16, lse, O_ref, L_ref):
    d_o = float(np.max(np.abs(o16 - O_ref)))
    d_l = float(np.max(np.abs(lse - L_ref)))
    log(f"[parity] {tag}: max|dO16|={d_o:.3e} max|dLSE|={d_l:.3e} bf16 floor={bf16_floor(O_ref):.3e}")
    assert d_o <= O_TOL and d_l <= LSE_TOL


def test_decode_b64_h32_tk8192_full_size(gpu):
    wl, q, k, v = workload_inputs("decode_b64_h32_tk8192_d128_s16")
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    o, lse = gpu.fa_decode(qg, kg, vg, num_splits=wl.num_splits, scale=wl.scale)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(wl.B) for h in range(wl.h)]
    O_ref, L_ref = _oracle(q, k, v, wl.scale, heads)
    _gate(wl.name, o.float().cpu().numpy().reshape(-1, wl.d), lse.cpu().numpy().reshape(-1),
          O_ref, L_ref)


@pytest.mark.parametrize("B,h,Tk,d,S", [
    (1, 1, 1, 128, 1), (2, 3, 7, 64, 3), (2, 2, 5, 128, 4), (1, 4, 1000, 128, 16),
    (3, 2, 4097, 64, 7), (1, 1, 513, 128, 256), (2, 2, 300, 128, 256), (2, 2, 40, 128, 40), (1, 2, 100, 64, 1),
    # chunks that take the 8-wave split workgroup (d = 128: 129-256 keys, d = 64: 257-512),
    # the last chunk ragged
    (2, 3, 1599, 128, 8), (2, 2, 3199, 64, 8),
])
def test_decode_edge_shapes(gpu, B, h, Tk, d, S):
    wl = si.custom_workload(B, h, 1, Tk, d, False, decode=True, num_splits=S)
    q, k, v = si.make_inputs(wl, seed=21, threads=4)
    o, lse = gpu.fa_decode(to_gpu(q), to_gpu(k), to_gpu(v), num_splits=S, scale=wl.scale)
    torch.cuda.synchronize()
    heads = [(b, hh) for b in range(B) for hh in range(h)]
    O_ref, L_ref = _oracle(q, k, v, wl.scale, heads)
    _gate(f"decode B{B} h{h} Tk{Tk} d{d} S{S}", o.float().cpu().numpy().reshape(-1, d),
          lse.cpu().numpy().reshape(-1), O_ref, L_ref)


def test_split_count_invariance_and_forward_agreement(gpu):
    wl = si.custom_workload(2, 4, 1, 2000, 128, False, decode=True)
    q, k, v = si.make_inputs(wl, seed=22, threads=4)
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    outs = [gpu.fa_decode(qg, kg, vg, num_splits=S, scale=wl.scale) for S in (1, 2, 16, 61, 256)]
    of, lf = gpu.fa_fwd_o32(qg[:, :, None, :].contiguous(), kg, vg, causal=False, scale=wl.scale)
    torch.cuda.synchronize()
    for o, lse in outs:
        assert torch.max(torch.abs(o.float() - of[:, :, 0])).item() <= O_TOL
        assert torch.max(torch.abs(lse - lf[:, :, 0])).item() <= LSE_TOL
        assert torch.max(torch.abs(o.float() - outs[0][0].float())).item() <= O_TOL


def test_decode_large_scores(gpu):
    wl = si.custom_workload(1, 2, 1, 3000, 128, False, decode=True)
    q, k, v = si.make_inputs(wl, seed=23, threads=2)
    o, lse = gpu.fa_decode(to_gpu(q), to_gpu(k), to_gpu(v), num_splits=8, scale=12.0)
    torch.cuda.synchronize()
    O_ref, L_ref = _oracle(q, k, v, 12.0, [(0, 0), (0, 1)])
    assert np.max(np.abs(o.float().cpu().numpy().reshape(2, -1) - O_ref)) <= O_TOL
    # absolute per-row gate: LSE_TOL plus the fp32 rounding of scores this large
    err = np.abs(lse.cpu().numpy().reshape(-1) - L_ref)
    tol = np.array([lse_row_tolerance(si.bf16_bits_to_f64(q[0, h])[None],
                                      si.bf16_bits_to_f64(k[0, h]), 12.0, False, L_ref[h:h + 1])[0]
                    for h in range(2)])
    log(f"[parity] decode large scores: |LSE|={np.abs(L_ref)} |dLSE|={err} tol={tol}")
    assert np.all(err <= tol)


def test_decode_rejects_too_many_splits(gpu):
    q = torch.zeros((1, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 300, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu.FaError) as e:
        gpu.fa_decode(q, k, k, num_splits=300)
    assert e.value.status == gpu.FA_ERR_SPLITS


def test_decode_rejects_small_workspace_without_writing(gpu):
    q = torch.zeros((1, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.full((1, 1, 128), 2.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 1), 5.0, device="cuda")
    ws = torch.full((16,), 9, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu.FaError) as e:
        gpu.fa_decode(q, k, k, num_splits=4, o=o, lse=lse, workspace=ws)
    assert e.value.status == gpu.FA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(o == 2.0) and torch.all(lse == 5.0) and torch.all(ws == 9)
