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


def lse_row_tolerance(q64: np.ndarray, k64: np.ndarray, scale: float, causal: bool,
                      lse_ref: np.ndarray) -> np.ndarray:
    """Absolute per-row LSE tolerance for scores far from O(1), from fp32 score rounding.

    The kernels form s_ij = q_i . k_j in fp32 (bf16 products are exact; each of the d additions
    rounds, so |ds_ij| <= d u A_ij with A_ij = sum_c |q_ic k_jc| and u = 2^-24, whatever the
    summation order), then scale it, take the max and carry m + log l, each one fp32 rounding of
    a value of magnitude <= |scale| A_ij or |LSE_i|.  Since dLSE_i/dS_ij = P_ij >= 0 sums to one,
    |dLSE_i| <= max_j |dS_ij| over the visible keys.  Tolerance:
        LSE_TOL + (d + 4) u |scale| max_j A_ij + 4 u |LSE_i|.
    At O(1) scores the extra terms are ~1e-5 and LSE_TOL alone governs."""
    u = 2.0 ** -24
    d = q64.shape[-1]
    A = np.abs(q64) @ np.abs(k64).T
    if causal:
        Tq, Tk = A.shape
        vis = np.arange(Tk)[None, :] <= np.arange(Tq)[:, None] + (Tk - Tq)
        A = np.where(vis, A, 0.0)
    return LSE_TOL + (d + 4) * u * abs(float(scale)) * A.max(axis=1) + 4 * u * np.abs(lse_ref)


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


# ---- backward ----------------------------------------------------------------------------------
# Tolerance of a backward gradient element, derived from the kernels' arithmetic: P and dS are
# rounded to bf16 (unit roundoff u = 2^-8) as MFMA operands, the gradients are accumulated in fp32
# (at most a few thousand terms: < 2^-11 relative to the sum of absolute products A), and the
# bf16 outputs add one more rounding (<= u |x| <= u A).  So |gpu - exact| <= FAC * A with
# FAC = 2u + 2^-11 (bf16 outputs) or u + 2^-11 (fp32 outputs), plus the error that reaches dS
# through D_i = <dO_i, O_i> when O is given in bf16 (|dD_i| <= u_O sum_d |dO_id| |O_id|) and
# the fp32 rounding of dP - D (<= 2^-16 (sum_d |dO_id V_jd| + |D_i|)).
BWD_FAC_BF16 = 2.0 ** -7 + 2.0 ** -11
BWD_FAC_F32 = 2.0 ** -8 + 2.0 ** -11


def bwd_tolerances(r, q, k, v, do, scale, fac, o_err=None):
    """Per-element tolerances {dq, dk, dv} for one head from the oracle's intermediates r.

    ``o_err`` [Tq][d] bounds |O_given - O_exact| (default: bf16 rounding of the exact O)."""
    from oracle import attention_bwd_ref as bref
    A = bref.abs_bounds_head(r, q, k, do, scale)
    if o_err is None:
        o_err = 2.0 ** -8 * np.abs(r["O"])
    ado = np.abs(do)
    dD = np.sum(ado * o_err, axis=1)                          # |dD_i|
    E = np.sum(ado * np.abs(r["O"]), axis=1)                  # sum of |terms| of D_i
    G = ado @ np.abs(v).T + E[:, None]                        # magnitudes in dP - D
    err_ds = r["P"] * (dD[:, None] + 2.0 ** -16 * G)          # |error of dS_ij| beyond rounding
    s = abs(float(scale))
    return {"dq": fac * A["dq"] + s * (err_ds @ np.abs(k)) + 1e-7,
            "dk": fac * A["dk"] + s * (err_ds.T @ np.abs(q)) + 1e-7,
            "dv": fac * A["dv"] + 1e-7}


def oracle_bwd_head(q_bits, k_bits, v_bits, do_bits, scale, causal):
    """fp64 oracle backward of one head from bf16 bits, plus the O (bf16 bits, RNE) and LSE (fp32)
    the kernels take as inputs."""
    from oracle import attention_bwd_ref as bref
    q, k, v, do = (si.bf16_bits_to_f64(x) for x in (q_bits, k_bits, v_bits, do_bits))
    r = bref.backward_head(q, k, v, do, scale, causal)
    o_bits = si.rne_bf16_bits(r["O"].astype(np.float32))
    return r, (q, k, v, do), o_bits, r["LSE"].astype(np.float32)


def run_bwd(fa, q, k, v, o, do, lse, causal, scale, f32=True):
    """GPU backward through the C ABI; q, k, v, o, do bf16 bits, lse fp32 (numpy or torch)."""
    qg, kg, vg, og, dog = (x if isinstance(x, torch.Tensor) else to_gpu(x)
                           for x in (q, k, v, o, do))
    lg = lse if isinstance(lse, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(lse)).cuda()
    res = {}
    res["dq16"], res["dk16"], res["dv16"] = fa.fa_bwd(qg, kg, vg, og, dog, lg, causal=causal,
                                                      scale=scale)
    if f32:
        res["dq32"], res["dk32"], res["dv32"] = fa.fa_bwd_f32(qg, kg, vg, og, dog, lg,
                                                              causal=causal, scale=scale)
    torch.cuda.synchronize()
    return res


def check_bwd_head(tag, res, bh, r, x64, scale, o_err=None):
    """Gate one head's gradients (fp32 and bf16 outputs) against the oracle."""
    q, k, v, do = x64
    b, h = bh
    worst = {}
    for out, fac in (("32", BWD_FAC_F32), ("16", BWD_FAC_BF16)):
        if "dq" + out not in res:
            continue
        tol = bwd_tolerances(r, q, k, v, do, scale, fac, o_err)
        for name in ("dq", "dk", "dv"):
            got = res[name + out][b, h].float().cpu().numpy().astype(np.float64)
            err = np.abs(got - r[name])
            ratio = float(np.max(err / tol[name])) if err.size else 0.0
            worst[name + out] = (float(np.max(err)), ratio)
            assert np.all(np.isfinite(got)), f"{tag} {name}{out}: non-finite output"
            bad = np.argwhere(err > tol[name])
            assert bad.size == 0, (f"{tag} {name}{out}: {len(bad)} elements beyond tolerance, "
                                   f"first {tuple(bad[0])} err {err[tuple(bad[0])]:.3e} "
                                   f"tol {tol[name][tuple(bad[0])]:.3e}")
    log(f"[parity] {tag} head {bh}: " +
        " ".join(f"{k}: max|d|={a:.2e} (x{rr:.3f} of tol)" for k, (a, rr) in worst.items()))
    return worst


def assert_bwd_bf16_is_rne_of_f32(res):
    for name in ("dq", "dk", "dv"):
        assert torch.equal(res[name + "16"].view(torch.int16),
                           rne_bf16_of(res[name + "32"]).view(torch.int16)), \
            f"bf16 {name} is not the round-to-nearest-even of the fp32 {name}"
