"""Shared helpers of the GPU parity tests: upload seeded inputs, run the library, compare with the
oracle.  Every GPU call goes through the C ABI via the package binding."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import seeded_inputs as si

O_TOL = 1e-2      # max |dO| on the kernel's fp32 output
LSE_TOL = 1e-3    # max |dLSE|


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> contiguous bf16 tensor on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def rne_bf16_of(t32: torch.Tensor) -> torch.Tensor:
    return t32.to(torch.bfloat16)


@functools.lru_cache(maxsize=4)
def workload_inputs(name: str, seed: int = 0):
    wl = si.WORKLOADS[name]
    log(f"[inputs] generating {name} seed={seed}")
    q, k, v = si.make_inputs(wl, seed)
    return wl, q, k, v


def run_fwd(fa, q, k, v, causal, scale, out32=True):
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    o16, l16 = fa.fa_fwd(qg, kg, vg, causal=causal, scale=scale)
    res = {"o16": o16, "lse16": l16}
    if out32:
        o32, l32 = fa.fa_fwd_o32(qg, kg, vg, causal=causal, scale=scale)
        res.update(o32=o32, lse32=l32)
    torch.cuda.synchronize()
    return res


def bf16_floor(o_ref: np.ndarray) -> float:
    """max |bf16(O_ref) - O_ref|: what rounding the exact output to bf16 alone costs."""
    r = si.bf16_bits_to_f64(si.rne_bf16_bits(o_ref.astype(np.float32)))
    return float(np.max(np.abs(r - o_ref))) if o_ref.size else 0.0


def check_rows(tag, o32_rows, lse_rows, o16_rows, o_ref, lse_ref):
    """Gate the fp32 output and LSE; bound the bf16 output by the fp32 gate plus its rounding."""
    d_o = float(np.max(np.abs(o32_rows - o_ref)))
    d_l = float(np.max(np.abs(lse_rows - lse_ref)))
    d_o16 = float(np.max(np.abs(o16_rows - o_ref)))
    floor = bf16_floor(o_ref)
    log(f"[parity] {tag}: max|dO32|={d_o:.3e} max|dLSE|={d_l:.3e} max|dO16|={d_o16:.3e} "
        f"bf16 floor={floor:.3e}")
    assert d_o <= O_TOL, f"{tag}: max|dO| {d_o} > {O_TOL}"
    assert d_l <= LSE_TOL, f"{tag}: max|dLSE| {d_l} > {LSE_TOL}"
    # O16 = RNE(O32) differs from O32 by at most half a bf16 ulp <= 2^-8 |O32|
    bound = O_TOL + 2.0 ** -8 * (np.abs(o_ref) + O_TOL)
    assert np.all(np.abs(o16_rows - o_ref) <= bound), f"{tag}: bf16 output beyond its bound"
    return d_o, d_l, d_o16


def assert_bf16_is_rne_of_f32(res):
    o16 = res["o16"]
    o32 = res["o32"]
    assert torch.equal(o16.view(torch.int16), rne_bf16_of(o32).view(torch.int16)), \
        "bf16 output is not the round-to-nearest-even of the fp32 output"
    assert torch.equal(res["lse16"], res["lse32"])
