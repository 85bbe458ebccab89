"""fa_decode_noalloc (partials in the library's static per-GPU array) against fa_decode (partials
in a caller workspace), through the C ABI: the same kernels read and write the same partials, so
the outputs must agree bit for bit, on two calls in a row, the second smaller than the first;
the first output is also checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import attention_ref as ref
from tests.gpu_support import LSE_TOL, O_TOL, log, to_gpu

pytestmark = pytest.mark.gpu


def _pair(gpu, B, h, Tk, d, S, seed):
    wl = si.custom_workload(B, h, 1, Tk, d, False, decode=True, num_splits=S)
    q, k, v = si.make_inputs(wl, seed=seed, threads=4)
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    log(f"[noalloc] B={B} h={h} Tk={Tk} d={d} S={S} seed={seed}")
    o_ref, l_ref = gpu.fa_decode(qg, kg, vg, num_splits=S, scale=wl.scale)
    o, lse = gpu.fa_decode_noalloc(qg, kg, vg, num_splits=S, scale=wl.scale)
    torch.cuda.synchronize()
    return (q, k, v, wl), (o, lse), (o_ref, l_ref)


def test_noalloc_decode_matches_workspace_decode_twice(gpu):
    # first call: the decode workload's shape with 16 splits (17 MB of partials)
    (q, k, v, wl), (o, lse), (o_ref, l_ref) = _pair(gpu, 64, 32, 8192, 128, 16, seed=31)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, l_ref)
    for b, h in [(0, 0), (17, 5), (63, 31)]:
        O, L = ref.naive_attention_head(si.bf16_bits_to_f64(q[b, h])[None],
                                        si.bf16_bits_to_f64(k[b, h]),
                                        si.bf16_bits_to_f64(v[b, h]), wl.scale, False)
        assert np.max(np.abs(o[b, h].float().cpu().numpy() - O[0])) <= O_TOL
        assert abs(float(lse[b, h]) - L[0]) <= LSE_TOL
    # second call, smaller: fewer heads and splits, a ragged chunk, padded head dim; the array
    # still holds the first call's partials beyond what this call writes
    (_, _, _, _), (o2, lse2), (o2_ref, l2_ref) = _pair(gpu, 3, 5, 1000, 80, 7, seed=32)
    assert torch.equal(o2.view(torch.int16), o2_ref.view(torch.int16))
    assert torch.equal(lse2, l2_ref)


def test_noalloc_decode_rejects_oversized_partials(gpu):
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((64, 32, 64, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.full((64, 32, 128), 2.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((64, 32), 5.0, device="cuda")
    with pytest.raises(gpu.FaError) as e:
        gpu.fa_decode_noalloc(q, k, k, num_splits=64, o=o, lse=lse)
    assert e.value.status == gpu.FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(o == 2.0) and torch.all(lse == 5.0)
