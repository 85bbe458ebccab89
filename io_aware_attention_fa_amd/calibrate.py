"""Run the gfx950 calibration microbenchmarks (libfa_calib.so) and print one JSON object.

Measures the ceilings the attention kernels are held against: dense bf16 MFMA FLOP/s, v_exp_f32
rate, LDS read bandwidth (ds_read_b128 and ds_read_b64_tr_b16), MFMAs fed from LDS with random
data, fp32 atomic-add throughput, streaming HBM read bandwidth and the shader clock.
Usage: python -m io_aware_attention_fa_amd.calibrate
"""
from __future__ import annotations

import ctypes
import json
import os

import torch

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_calib.so")


def _time(fn, reps=5):
    fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps * 1e-3


def main():
    lib = ctypes.CDLL(LIB)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {"device": torch.cuda.get_device_properties(0).name, "cus": cus}

    clk = torch.zeros(3, dtype=torch.int64, device="cuda")
    lib.calib_clock(ctypes.c_void_p(clk.data_ptr()), 2_000_000, st)
    torch.cuda.synchronize()
    c = clk.cpu().tolist()
    res["sclk_mhz_from_memtime"] = c[0] / c[1] * 100.0 if c[1] else None

    out = torch.empty(cus * 16 * 256, dtype=torch.float32, device="cuda")
    for waves_per_simd, nacc in ((2, 1), (2, 2), (2, 4), (2, 8), (1, 2), (1, 4), (1, 8)):
        blocks = cus * waves_per_simd
        iters = 32000 // nacc
        t = _time(lambda: lib.calib_mfma(ctypes.c_void_p(out.data_ptr()), blocks, iters, nacc,
                                         ctypes.c_void_p(clk.data_ptr()), st))
        c = clk.cpu().tolist()
        res[f"mfma_bf16_tflops_{waves_per_simd}wave_{nacc}acc"] = (
            blocks * 4 * iters * nacc * 32768 / t / 1e12)
        res[f"mfma_sclk_mhz_{waves_per_simd}wave_{nacc}acc"] = c[0] / c[1] * 100.0 if c[1] else None

    blocks = cus * 8
    iters = 20000
    t = _time(lambda: lib.calib_exp(ctypes.c_void_p(out.data_ptr()), blocks, iters, st))
    res["exp2_per_s"] = blocks * 256 * iters * 16 / t

    for op, name in enumerate(("add_f32", "fma_f32", "dot2c_f32_bf16", "cvt_pk_bf16_f32",
                               "max3_f32")):
        t = _time(lambda: lib.calib_valu(ctypes.c_void_p(out.data_ptr()), blocks, iters, op, st))
        # wave-instructions per CU per clock at 2.4 GHz (4 SIMDs: 4.0 = one per SIMD per clock)
        insts = blocks * 4 * iters * 16
        res[f"valu_{name}_wave_insts_per_clk_per_cu"] = insts / t / cus / 2.4e9

    # MFMA waves and VALU waves sharing SIMDs: time each alone and together
    times = {}
    for mode, name in ((1, "mfma_only"), (2, "valu_only"), (0, "both")):
        times[name] = _time(lambda: lib.calib_coexec(ctypes.c_void_p(out.data_ptr()), cus, 8000,
                                                     16000, mode, st))
        res[f"coexec_ms_{name}"] = times[name] * 1e3
    res["coexec_overlap"] = ((times["mfma_only"] + times["valu_only"] - times["both"]) /
                             min(times["mfma_only"], times["valu_only"]))

    outu = out.view(torch.int32)
    blocks_l = cus * 2
    iters = 20000
    t = _time(lambda: lib.calib_lds_b128(ctypes.c_void_p(outu.data_ptr()), blocks_l, iters, st))
    bps = blocks_l * 256 * iters * 8 * 16 / t
    res["lds_b128_bytes_per_s"] = bps
    res["lds_b128_bytes_per_clk_per_cu_at_2400"] = bps / cus / 2.4e9
    t = _time(lambda: lib.calib_lds_tr(ctypes.c_void_p(outu.data_ptr()), blocks_l, iters, st))
    bps = blocks_l * 256 * iters * 8 * 8 / t
    res["lds_tr16_b64_bytes_per_s"] = bps
    res["lds_tr16_b64_bytes_per_clk_per_cu_at_2400"] = bps / cus / 2.4e9

    # MFMAs fed from LDS with random data (two waves per SIMD, one workgroup per CU): with and
    # without reuse of each A operand, and with 0, 48 or 80 vector instructions per 16 MFMAs
    iters = 4000
    for reuse in (1, 2):
        for nv in (0, 48, 80):
            t = _time(lambda: lib.calib_lds_mfma(ctypes.c_void_p(out.data_ptr()), cus, iters,
                                                 reuse, nv, st))
            flops = cus * 8 * iters * 16 * 32768
            res[f"lds_mfma_random_tflops_reuse{reuse}_valu{nv}"] = flops / t / 1e12

    # fp32 atomic adds without a return value, 256-byte runs per wave: payload bytes per second
    # into a 4 MiB (L2-sized) and a 512 MiB buffer
    for mib in (4, 512):
        nf = mib << 18   # floats
        acc = torch.zeros(nf, dtype=torch.float32, device="cuda")
        blocks_a, iters_a = cus * 8, 2000
        t = _time(lambda: lib.calib_atomic_add(ctypes.c_void_p(acc.data_ptr()), nf - 1, blocks_a,
                                               iters_a, st))
        res[f"atomic_add_f32_GBps_{mib}MiB"] = blocks_a * 256 * iters_a * 4 / t / 1e9
        del acc

    n = 4 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    for blocks_h in (cus * 4, cus * 8, cus * 16):
        t = _time(lambda: lib.calib_hbm_read(ctypes.c_void_p(src.data_ptr()), n // 16,
                                             ctypes.c_void_p(outu.data_ptr()), blocks_h, st))
        res[f"hbm_read_GBps_blocks{blocks_h}"] = n / t / 1e9
    t = _time(lambda: lib.calib_hbm_read_blocked(ctypes.c_void_p(src.data_ptr()),
                                                 ctypes.c_long(n // 16),
                                                 ctypes.c_void_p(outu.data_ptr()), st))
    res["hbm_read_GBps_blocked_128KB_per_16_waves"] = n / t / 1e9
    dst = torch.empty_like(src)
    t = _time(lambda: dst.copy_(src))
    res["torch_copy_GBps_read_plus_write"] = 2 * n / t / 1e9
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
