"""Benchmark of the attention hot path on one MI355X.

One step = one causal attention forward at B=8, h=32, T=4096, d_head=128 (bf16, fp32 accumulate)
plus one split-KV decode at B=64, h=32, Tk=8192, d_head=128 with 16 splits.  Inputs are seeded
synthetic N(0,1) bf16 tensors, resident in HBM before timing starts.  W warm-up steps, then K timed
steps between two device synchronisations; every library call is bracketed by HIP events on the
stream it is launched on, which gives each kernel's average duration.

Prints ONE JSON line on stdout (diagnostics go to stderr):
  value    = forward TFLOP/s (4*B*h*T*T*d/2 FLOPs / average forward duration)
  roofline = that kernel against the MI355X dense-bf16 MFMA peak
  decode   = decode HBM GB/s (K+V bytes / average decode duration) against the HBM peak
  cpu_baseline = the fp64 CPU oracle timed on a bounded sample of the same forward workload
  backward = the attention backward (dQ, dK, dV) on the forward workload, timed separately
             after the steps (not part of ms_per_step): TFLOP/s at 2.5x the forward's FLOPs,
             against the MFMA peak, with its own bounded CPU-oracle sample
  softmax  = the one-pass row softmax on a 4096 x 4096 fp32 matrix, timed separately: HBM GB/s
             (one read and one write of the matrix) against the HBM peak
  gelu, bias_gelu_dropout = the fused elementwise chains on the pages' workloads (64M fp32
             values; a 4096 x 8192 bf16 activation with p = 0.1), timed separately: HBM GB/s
  layouts  = the forward and backward on strided [B][T][h][d] tensors at the prefill shape, each
             timed in alternating rounds with the contiguous call (ratio reported), d_head = 80
             (20 heads, padded to 128 on chip; TFLOP/s of the true and of the padded d_head),
             and the decode on a [B][Tk][h][d] KV cache
  configs  = every forward configuration with its roofline and the oracle timed beside it:
             C1 (B=1 h=2 T=128 d=64 non-causal) as a latency; C2 (B=8 h=32 T=1024 d=64 causal)
             against both the MFMA and the HBM peak, warm and with a 512 MB flush between
             trials; C3 (the prefill above); C4 (B=2 h=32 T=16384 d=128 causal, 1% of keys x8)
             against the MFMA peak; C5 (the decode above)
  clock    = the GFX clock sampled (amdsmi) while the forward runs back to back, the CU count,
             and the forward's fraction of the MFMA peak at that clock
  host     = the CPUs the oracle ran on (affinity count, machine count, model, BLAS, threads)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PREFILL = "causal_b8_h32_t4096_d128"
DECODE = "decode_b64_h32_tk8192_d128_s16"
METRIC = "attention fwd TFLOP/s (% MFMA peak) at T=4096 causal; decode HBM GB/s (% peak)"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def upload(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def traffic_from_profiles(name):
    """HBM bytes per launch of a kernel, from the committed rocprofv3 counter summary, if any.

    The summary (profiles/traffic__<name>.txt) holds FETCH_SIZE / WRITE_SIZE per dispatch
    already scaled by the copy-kernel calibration factors, with the sha256 of the kernel sources
    it was taken on; if those sources have changed since, the figure is stale and this gives None.
    """
    import hashlib
    path = os.path.join(PROFILE_DIR, f"traffic__{name}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        key, sep, val = line.partition(":")
        if sep and key in ("sources", "sources_sha256", "hbm_bytes_per_launch"):
            fields[key] = val.strip()
    try:
        h = hashlib.sha256()
        for src in fields["sources"].split():
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() != fields["sources_sha256"]:
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def blas_threads():
    """(vendor, threads) of the BLAS numpy's matrix products run on."""
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            return (f"{pools[0].get('internal_api')} {pools[0].get('version')}",
                    int(max(p.get("num_threads", 1) for p in pools)))
    except Exception:  # pragma: no cover
        pass
    return ("unknown", os.cpu_count() or 1)


def host_info():
    """The host the CPU oracle runs on: CPUs visible to this process, CPUs of the machine, the
    CPU model and the BLAS numpy uses."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    vendor, threads = blas_threads()
    return {"affinity_cpus": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(),
            "cpu_model": model, "blas": vendor, "blas_threads": threads}


def oracle_runs(wl, heads, runs, get_head=None):
    """Seconds per run of the fp64 oracle over the listed (b, h) heads of a workload (input
    generation and the bf16 -> fp64 conversion are outside the timed region)."""
    import seeded_inputs as si
    from oracle import attention_ref as ref
    get_head = get_head or (lambda b, h: si.head_inputs(wl, 0, b, h))
    cached = [tuple(si.bf16_bits_to_f64(x) for x in get_head(b, h)) for b, h in heads]
    times = []
    for _ in range(runs):
        el = 0.0
        for q, k, v in cached:
            q2 = q.reshape(-1, wl.d)
            t0 = time.perf_counter()
            ref.naive_attention_head(q2, k, v, wl.scale, wl.causal)
            el += time.perf_counter() - t0
        times.append(el)
    return times


def oracle_baseline(wl, heads, runs, what, unit="TFLOP/s", get_head=None):
    """The oracle timed on a sample of heads, scaled to the metric's unit: TFLOP/s by the same
    FLOP formula as the GPU, or GB/s of K+V (decode)."""
    from io_aware_attention_fa_amd import costmodel as cm
    times = oracle_runs(wl, heads, runs, get_head)
    n = len(heads)
    if unit == "GB/s":
        work = n * wl.Tk * cm.decode_kv_bytes_per_token(wl.d) / 1e9
    else:
        work = cm.attention_flops(1, n, wl.Tq, wl.Tk, wl.d, wl.causal) / 1e12
    best = min(times)
    return {"value": work / best, "unit": unit, "cores": blas_threads()[1], "kind": "oracle",
            "runs_s": times, "seconds_per_head": best / n,
            "seconds_whole_workload_est": best / n * wl.B * wl.h,
            "sample": f"{n} of {wl.B * wl.h} heads of {wl.name}, {what}; {runs} run(s), best "
                      f"of {best:.3g} s of fp64 numpy"}


def sample_clock(torch, fn, seconds=1.5):
    """The GFX clock while fn runs back to back: amdsmi's gpu_metrics of this device sampled from
    a host thread every few ms over about ``seconds`` of launches (outside any timed region).
    Returns None if the metrics cannot be read."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception as e:  # pragma: no cover
        return {"mhz": None, "error": f"amdsmi unavailable: {e}"}
    try:
        pr = torch.cuda.get_device_properties(torch.cuda.current_device())
        bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
        hnd = amdsmi.amdsmi_get_processor_handle_from_bdf(bdf)

        def read():
            m = amdsmi.amdsmi_get_gpu_metrics_info(hnd)
            xs = m.get("current_gfxclks")
            if isinstance(xs, (list, tuple)):
                xs = [x for x in xs if isinstance(x, (int, float)) and 0 < x < 10000]
                if xs:
                    return sum(xs) / len(xs)
            x = m.get("current_gfxclk")
            return float(x) if isinstance(x, (int, float)) and 0 < x < 10000 else None

        if read() is None:
            return {"mhz": None, "error": "gpu_metrics hold no current GFX clock"}
        samples, stop = [], threading.Event()

        def poll():
            while not stop.is_set():
                v = read()
                if v is not None:
                    samples.append(v)
                time.sleep(0.004)

        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < 0.3:   # calls per batch: about 0.3 s of work
            fn()
            n += 1
            torch.cuda.synchronize()
        th = threading.Thread(target=poll, daemon=True)
        th.start()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
        stop.set()
        th.join()
        if not samples:
            return {"mhz": None, "error": "no samples"}
        samples.sort()
        return {"mhz": sum(samples) / len(samples), "median_mhz": samples[len(samples) // 2],
                "samples": len(samples), "bdf": bdf,
                "source": "amdsmi gpu_metrics current GFX clock (mean over XCDs), sampled "
                          "every ~4 ms during back-to-back launches"}
    except Exception as e:  # pragma: no cover
        return {"mhz": None, "error": f"{type(e).__name__}: {e}"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def cpu_baseline(seconds_budget: float):
    """Time the fp64 oracle on whole heads of the forward workload (same generator, seed 0)."""
    import numpy as np
    import seeded_inputs as si
    from io_aware_attention_fa_amd import costmodel as cm
    from oracle import attention_ref as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    wl = si.WORKLOADS[PREFILL]
    heads, elapsed = 0, 0.0
    while heads == 0 or (elapsed < seconds_budget and heads < wl.B * wl.h):
        b, h = divmod(heads, wl.h)
        q, k, v = si.head_inputs(wl, 0, b, h)
        q, k, v = si.bf16_bits_to_f64(q), si.bf16_bits_to_f64(k), si.bf16_bits_to_f64(v)
        t0 = time.perf_counter()
        ref.naive_attention_head(q, k, v, wl.scale, True)
        elapsed += time.perf_counter() - t0
        heads += 1
    flops = cm.attention_flops(1, heads, wl.Tq, wl.Tk, wl.d, True)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{heads} whole heads (4096x4096 causal, d=128) of {PREFILL}, "
                      f"{elapsed:.1f} s of fp64 numpy; FLOPs counted as 4*T*T*d/2 per head"}


def cpu_baseline_backward(seconds_budget: float):
    """Time the fp64 backward oracle on whole heads of the forward workload (bounded sample)."""
    import numpy as np  # noqa: F401
    import seeded_inputs as si
    from io_aware_attention_fa_amd import costmodel as cm
    from oracle import attention_bwd_ref as bref
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    wl = si.WORKLOADS[PREFILL]
    heads, elapsed = 0, 0.0
    while heads == 0 or (elapsed < seconds_budget and heads < wl.B * wl.h):
        b, h = divmod(heads, wl.h)
        q, k, v = si.head_inputs(wl, 0, b, h)
        do = si.head_normal_bits(0, si.TENSOR_DO, b, h, wl.Tq, wl.d)
        q, k, v, do = (si.bf16_bits_to_f64(x) for x in (q, k, v, do))
        t0 = time.perf_counter()
        bref.backward_head(q, k, v, do, wl.scale, True)
        elapsed += time.perf_counter() - t0
        heads += 1
    flops = cm.attention_bwd_flops(1, heads, wl.Tq, wl.Tk, wl.d, True)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{heads} whole heads (4096x4096 causal, d=128) of {PREFILL}, "
                      f"{elapsed:.1f} s of fp64 numpy; FLOPs counted as 2.5 x 4*T*T*d/2 per head"}


def measure_backward(args, fa, si, cm, torch, wp, pq, pk, pv, po, plse):
    """The attention backward on the forward workload: dO from the seeded generator, O and LSE
    from fa_fwd; warm-up, then timed calls bracketed by HIP events on the launch stream."""
    do = upload(si.make_grad(wp, seed=0))
    fa.fa_fwd(pq, pk, pv, causal=True, scale=wp.scale, o=po, lse=plse)
    dq, dk, dv = torch.empty_like(pq), torch.empty_like(pk), torch.empty_like(pv)
    ws = torch.empty(fa.fa_bwd_workspace_size(wp.B, wp.h, wp.Tq), dtype=torch.uint8,
                     device="cuda")

    def call():
        fa.fa_bwd(pq, pk, pv, po, do, plse, causal=True, scale=wp.scale, dq=dq, dk=dk, dv=dv,
                  workspace=ws)

    W, K = 3, max(1, args.bwd_steps)
    for _ in range(W):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in ev]
    ms = sum(t) / K
    flops = cm.attention_bwd_flops(wp.B, wp.h, wp.Tq, wp.Tk, wp.d, True)
    tflops = flops / (ms * 1e-3) / 1e12
    executed = cm.attention_bwd_executed_flops(wp.B, wp.h, wp.Tq, wp.Tk, wp.d, True)
    peak = cm.MI355X_PEAK_BF16_DENSE_FLOPS / 1e12
    eprint(f"[bench] backward avg {ms:.4f} ms  {tflops:.1f} TFLOP/s (2.5x fwd FLOPs)  "
           f"{100 * tflops / peak:.1f}% of {peak:.0f}; executed MFMA rate "
           f"{executed / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
    res = {"metric": "attention backward TFLOP/s (dQ, dK, dV; 2.5x forward FLOPs)",
           "value": tflops, "unit": "TFLOP/s", "steps": K, "warmup": W,
           "avg_ms": ms, "min_ms": min(t), "median_ms": sorted(t)[K // 2],
           "roofline": {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                        "frac": tflops / peak,
                        "traffic": traffic_from_profiles(f"fa_bwd__{PREFILL}")},
           "executed_mfma_tflops": executed / (ms * 1e-3) / 1e12,
           "config": {"B": wp.B, "h": wp.h, "T": wp.Tq, "d_head": wp.d, "causal": True,
                      "flops": flops, "executed_flops": executed,
                      "alg_bytes": cm.attention_bwd_io_bytes(wp.B, wp.h, wp.Tq, wp.Tk, wp.d)}}
    if not args.no_cpu_baseline:
        eprint("[bench] timing the CPU backward oracle on a sample")
        res["cpu_baseline"] = cpu_baseline_backward(min(args.cpu_seconds, 15.0))
    return res


def event_trials(torch, fn, warmup, trials, between=None):
    """Per-call durations (ms) of fn from HIP events recorded around each call on the launch
    stream; ``between`` (if given) is enqueued before each trial, outside its events."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(trials)]
    for a, b in ev:
        if between is not None:
            between()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return {"avg_ms": sum(t) / trials, "median_ms": t[trials // 2], "min_ms": t[0],
            "trials": trials}


def rooflines(cm, flops, nbytes, ms):
    """Achieved rates of one launch against the MFMA and the HBM peaks."""
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    pf = cm.MI355X_PEAK_BF16_DENSE_FLOPS / 1e12
    pb = cm.MI355X_PEAK_HBM_BYTES_PER_S / 1e9
    return ({"bound": "mfma", "achieved": tf, "peak": pf, "unit": "TFLOP/s", "frac": tf / pf,
             "traffic": None},
            {"bound": "hbm", "achieved": gbs, "peak": pb, "unit": "GB/s", "frac": gbs / pb,
             "traffic": None})


def measure_configs(args, fa, si, cm, torch):
    """The other forward configurations: the tiny non-causal case as a latency, B=8 h=32 T=1024
    d=64 causal against both rooflines (it sits near the ridge) with and without a 512 MB cache
    flush between trials, and the long-context B=2 h=32 T=16384 d=128 causal workload with key
    spikes as a fraction of the MFMA peak; each with the CPU oracle timed beside it."""
    res = {}
    cpu = not args.no_cpu_baseline
    # C1: latency of one call, and of 20 back-to-back calls between two events
    wl = si.WORKLOADS["tiny_noncausal_b1_h2_t128_d64"]
    q, k, v = si.make_inputs(wl, seed=0, threads=2)
    tq, tk, tv = upload(q), upload(k), upload(v)
    o = torch.empty_like(tq)
    lse = torch.empty((wl.B, wl.h, wl.Tq), dtype=torch.float32, device="cuda")
    call = lambda: fa.fa_fwd(tq, tk, tv, causal=False, scale=wl.scale, o=o, lse=lse)
    t = event_trials(torch, call, 20, 200)
    t["back_to_back_20_avg_ms"] = time_calls(torch, call, 5, 20)
    flops = cm.attention_flops(1, 2, 128, 128, 64, False)
    nbytes = cm.attention_io_bytes(1, 2, 128, 128, 64)
    r_f, r_b = rooflines(cm, flops, nbytes, t["median_ms"])
    c1 = {"metric": "attention fwd latency (one call, HIP events around the launch)",
          "value": t["median_ms"] * 1e3, "unit": "us", "higher_is_better": False,
          "roofline": {"bound": "latency", "achieved": t["median_ms"] * 1e3, "peak": None,
                       "unit": "us", "frac": None, "traffic": None,
                       "mfma_frac": r_f["frac"], "hbm_frac": r_b["frac"]},
          "timing": t, "config": {"workload": wl.name, "flops": flops, "alg_bytes": nbytes}}
    eprint(f"[bench] C1 {wl.name}: median {t['median_ms'] * 1e3:.1f} us per call, "
           f"{t['back_to_back_20_avg_ms'] * 1e3:.1f} us back to back")
    if cpu:
        c1["cpu_baseline"] = oracle_baseline(wl, [(0, 0), (0, 1)], 3, "whole workload")
        cb = c1["cpu_baseline"]
        cb["latency_ms"] = min(cb["runs_s"]) * 1e3
    res["C1"] = c1
    del tq, tk, tv, o, lse

    # C2: near the ridge; warm (inputs resident in the 256 MB MALL) and with a 512 MB write
    # between trials
    wl = si.WORKLOADS["causal_b8_h32_t1024_d64"]
    q, k, v = si.make_inputs(wl, seed=0)
    tq, tk, tv = upload(q), upload(k), upload(v)
    del q, k, v
    o = torch.empty_like(tq)
    lse = torch.empty((wl.B, wl.h, wl.Tq), dtype=torch.float32, device="cuda")
    call = lambda: fa.fa_fwd(tq, tk, tv, causal=True, scale=wl.scale, o=o, lse=lse)
    warm = event_trials(torch, call, 10, 100)
    flush = torch.empty(512 * 2**20, dtype=torch.uint8, device="cuda")
    cnt = [0]

    def scrub():
        cnt[0] += 1
        flush.fill_(cnt[0] & 0xff)

    cold = event_trials(torch, call, 3, 100, between=scrub)
    del flush
    flops = cm.attention_flops(wl.B, wl.h, wl.Tq, wl.Tk, wl.d, True)
    nbytes = cm.attention_io_bytes(wl.B, wl.h, wl.Tq, wl.Tk, wl.d)
    w_f, w_b = rooflines(cm, flops, nbytes, warm["avg_ms"])
    c_f, c_b = rooflines(cm, flops, nbytes, cold["avg_ms"])
    c2 = {"metric": "attention fwd TFLOP/s and HBM GB/s at the ridge (causal T=1024 d=64)",
          "value": w_f["achieved"], "unit": "TFLOP/s", "roofline": w_b,
          "roofline_mfma": w_f, "roofline_hbm": w_b, "timing": warm,
          "flushed": {"timing": cold, "roofline_mfma": c_f, "roofline_hbm": c_b,
                      "flush": "512 MB device write between trials (outside the events)"},
          "config": {"workload": wl.name, "flops": flops, "alg_bytes": nbytes}}
    eprint(f"[bench] C2 {wl.name}: {warm['avg_ms'] * 1e3:.1f} us  {w_f['achieved']:.0f} TFLOP/s "
           f"({100 * w_f['frac']:.1f}% MFMA)  {w_b['achieved']:.0f} GB/s "
           f"({100 * w_b['frac']:.1f}% HBM); flushed {cold['avg_ms'] * 1e3:.1f} us "
           f"({100 * c_f['frac']:.1f}% MFMA, {100 * c_b['frac']:.1f}% HBM)")
    if cpu:
        c2["cpu_baseline"] = oracle_baseline(wl, [divmod(i, wl.h) for i in range(0, 256, 4)], 3,
                                             "every 4th head")
    res["C2"] = c2
    del tq, tk, tv, o, lse
    torch.cuda.empty_cache()

    # C4: long context with key spikes
    wl = si.WORKLOADS["longctx_causal_b2_h32_t16384_d128_keyspikes"]
    q, k, v = si.make_inputs(wl, seed=0)
    tq, tk, tv = upload(q), upload(k), upload(v)
    del q, k, v
    o = torch.empty_like(tq)
    lse = torch.empty((wl.B, wl.h, wl.Tq), dtype=torch.float32, device="cuda")
    call = lambda: fa.fa_fwd(tq, tk, tv, causal=True, scale=wl.scale, o=o, lse=lse)
    t = event_trials(torch, call, 3, max(20, args.extra_steps))
    flops = cm.attention_flops(wl.B, wl.h, wl.Tq, wl.Tk, wl.d, True)
    nbytes = cm.attention_io_bytes(wl.B, wl.h, wl.Tq, wl.Tk, wl.d)
    r_f, r_b = rooflines(cm, flops, nbytes, t["avg_ms"])
    c4 = {"metric": "attention fwd TFLOP/s (% MFMA peak), causal T=16384 d=128, 1% keys x8",
          "value": r_f["achieved"], "unit": "TFLOP/s", "roofline": r_f, "roofline_hbm": r_b,
          "timing": t, "config": {"workload": wl.name, "flops": flops, "alg_bytes": nbytes}}
    eprint(f"[bench] C4 {wl.name}: {t['avg_ms']:.3f} ms  {r_f['achieved']:.0f} TFLOP/s "
           f"({100 * r_f['frac']:.1f}% MFMA)")
    if cpu:
        c4["cpu_baseline"] = oracle_baseline(wl, [(0, 0), (0, 11), (1, 5), (1, 30)], 1,
                                             "four whole heads")
    res["C4"] = c4
    del tq, tk, tv, o, lse
    torch.cuda.empty_cache()
    return res


def time_calls(torch, fn, warmup, steps):
    """Average milliseconds per call of `steps` back-to-back calls of fn, between two HIP events
    on the current stream (the stream the library launches on).  For kernels of tens of
    microseconds, one event pair per call would add its own overhead to every call."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def measure_softmax(args, fa, si, torch):
    """The row softmax on the pages' 4096 x 4096 fp32 matrix (seeded N(0,1) rows)."""
    from io_aware_attention_fa_amd import costmodel as cm
    rows, cols = si.SOFTMAX_WORKLOAD
    x = torch.from_numpy(si.softmax_rows_input(rows, cols, seed=0)).cuda()
    y = torch.empty_like(x)
    K = args.extra_steps or 100
    ms = time_calls(torch, lambda: fa.fa_softmax_rows(x, y=y), 3, K)
    nbytes = 2.0 * rows * cols * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    peak = cm.MI355X_PEAK_HBM_BYTES_PER_S / 1e9
    eprint(f"[bench] softmax {rows}x{cols} avg {ms * 1e3:.1f} us  {gbs:.0f} GB/s  "
           f"{100 * gbs / peak:.1f}% of HBM peak")
    res = {"metric": "row softmax HBM GB/s (one read + one write of the fp32 matrix)",
           "value": gbs, "unit": "GB/s", "steps": K, "warmup": 3, "avg_ms": ms,
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": peak, "unit": "GB/s",
                        "frac": gbs / peak,
                        "traffic": traffic_from_profiles(
                            f"fa_softmax_reg_kernel__softmax_{rows}x{cols}")},
           "config": {"rows": rows, "cols": cols, "dtype": "f32", "alg_bytes": nbytes}}
    if not args.no_cpu_baseline:
        import time as _t

        import numpy as np  # noqa: F401
        from oracle import softmax_ref as sref
        n, el = 0, 0.0
        while n == 0 or (el < min(args.cpu_seconds, 5.0) and n < rows):
            xs = si.softmax_rows_input(256, cols, seed=0, row0=n)
            t0 = _t.perf_counter()
            sref.softmax_rows(xs)
            el += _t.perf_counter() - t0
            n += 256
        res["cpu_baseline"] = {"value": 2.0 * n * cols * 4 / el / 1e9, "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{n} rows of the {rows}x{cols} matrix, {el:.2f} s of "
                                         "fp64 numpy (bytes counted as fp32 read + write)"}
    return res


def interleaved(torch, fns, warmup, steps, rounds=5):
    """Median per-call milliseconds of each of several calls, timed in alternating rounds
    (``steps`` back-to-back calls between two events per round), so that all of them see the
    same clock and thermal state."""
    import numpy as np
    t = {n: [] for n in fns}
    for _ in range(rounds):
        for n, f in fns.items():
            t[n].append(time_calls(torch, f, warmup, steps))
    return {n: float(np.median(v)) for n, v in t.items()}


def measure_layouts(args, fa, si, cm, torch, dec=None):
    """The forward and the backward on layout variants, each timed in alternating rounds with
    the contiguous [B][h][T][d] call on the same data: the prefill workload with the tensors in
    [B][T][h][d] (strided views), and d_head = 80 with 20 heads (B=8, T=4096, causal), the
    pages' padding example (reported against the true FLOPs and against the FLOPs of the
    128-wide kernel that runs it); with ``dec`` = (workload, q, k, v) of the decode, also the
    decode on the same KV cache stored as [B][Tk][h][d]."""
    import numpy as np
    peak = cm.MI355X_PEAK_BF16_DENSE_FLOPS / 1e12
    K = args.extra_steps or 10
    res = {}

    def bthd(t):
        return t.transpose(1, 2).contiguous().transpose(1, 2)

    # forward: [B][T][h][d] against contiguous, same values
    B, h, T, d = 8, 32, 4096, 128
    wl = si.custom_workload(B, h, T, T, d, True, name="bthd")
    q, k, v = si.make_inputs(wl, seed=0)
    cq, ck, cv = upload(q), upload(k), upload(v)
    del q, k, v
    sq, sk, sv = bthd(cq), bthd(ck), bthd(cv)
    co, so = torch.empty_like(cq), bthd(torch.empty_like(cq))
    lse = torch.empty((B, h, T), dtype=torch.float32, device="cuda")
    ms = interleaved(torch, {
        "contiguous": lambda: fa.fa_fwd(cq, ck, cv, causal=True, scale=wl.scale, o=co, lse=lse),
        "bthd": lambda: fa.fa_fwd_strided(sq, sk, sv, causal=True, scale=wl.scale, o=so,
                                          lse=lse)}, 3, K)
    flops = cm.attention_flops(B, h, T, T, d, True)
    tf = {n: flops / (m * 1e-3) / 1e12 for n, m in ms.items()}
    eprint(f"[bench] layout bthd: B={B} h={h} T={T} d={d} {ms['bthd']:.4f} ms {tf['bthd']:.1f} "
           f"TFLOP/s against contiguous {ms['contiguous']:.4f} ms {tf['contiguous']:.1f} "
           f"(ratio {ms['bthd'] / ms['contiguous']:.3f})")
    res["bthd"] = {"metric": "attention fwd TFLOP/s, causal, d_head=128, [B][T][h][d] q, k, v and o",
                   "value": tf["bthd"], "unit": "TFLOP/s", "steps": K, "warmup": 3,
                   "avg_ms": ms["bthd"], "contiguous_ms": ms["contiguous"],
                   "time_ratio_vs_contiguous": ms["bthd"] / ms["contiguous"],
                   "roofline": {"bound": "mfma", "achieved": tf["bthd"], "peak": peak,
                                "unit": "TFLOP/s", "frac": tf["bthd"] / peak, "traffic": None},
                   "config": {"B": B, "h": h, "T": T, "d_head": d, "causal": True,
                              "layout": "BTHD strided", "flops": flops,
                              "timing": "median of 5 rounds alternating with the contiguous call"}}

    # backward on the same data: [B][T][h][d] tensors against contiguous
    dob = si.make_grad(wl, seed=0)
    cdo = upload(dob)
    del dob
    sdo = bthd(cdo)
    fa.fa_fwd(cq, ck, cv, causal=True, scale=wl.scale, o=co, lse=lse)
    fa.fa_fwd_strided(sq, sk, sv, causal=True, scale=wl.scale, o=so, lse=lse)
    cg = [torch.empty_like(cq) for _ in range(3)]
    sg = [bthd(torch.empty_like(cq)) for _ in range(3)]
    ws = torch.empty(fa.fa_bwd_workspace_size(B, h, T), dtype=torch.uint8, device="cuda")
    ms = interleaved(torch, {
        "contiguous": lambda: fa.fa_bwd(cq, ck, cv, co, cdo, lse, causal=True, scale=wl.scale,
                                        dq=cg[0], dk=cg[1], dv=cg[2], workspace=ws),
        "bthd": lambda: fa.fa_bwd_strided(sq, sk, sv, so, sdo, lse, causal=True, scale=wl.scale,
                                          dq=sg[0], dk=sg[1], dv=sg[2], workspace=ws)},
        2, max(3, K // 3))
    bflops = cm.attention_bwd_flops(B, h, T, T, d, True)
    tfb = {n: bflops / (m * 1e-3) / 1e12 for n, m in ms.items()}
    eprint(f"[bench] layout bwd_bthd: {ms['bthd']:.4f} ms {tfb['bthd']:.1f} TFLOP/s (2.5x fwd "
           f"FLOPs) against contiguous {ms['contiguous']:.4f} ms {tfb['contiguous']:.1f} "
           f"(ratio {ms['bthd'] / ms['contiguous']:.3f})")
    res["bwd_bthd"] = {"metric": "attention backward TFLOP/s (2.5x forward FLOPs), causal, "
                                 "d_head=128, [B][T][h][d] tensors",
                       "value": tfb["bthd"], "unit": "TFLOP/s", "steps": max(3, K // 3),
                       "warmup": 2, "avg_ms": ms["bthd"], "contiguous_ms": ms["contiguous"],
                       "time_ratio_vs_contiguous": ms["bthd"] / ms["contiguous"],
                       "roofline": {"bound": "mfma", "achieved": tfb["bthd"], "peak": peak,
                                    "unit": "TFLOP/s", "frac": tfb["bthd"] / peak,
                                    "traffic": None},
                       "config": {"B": B, "h": h, "T": T, "d_head": d, "causal": True,
                                  "layout": "BTHD strided", "flops": bflops}}
    del cq, ck, cv, sq, sk, sv, co, so, lse, cdo, sdo, cg, sg, ws
    torch.cuda.empty_cache()

    # d_head = 80 (20 heads), padded to 128 on chip: forward and backward
    B, h, T, d = 8, 20, 4096, 80
    wl = si.custom_workload(B, h, T, T, d, True, name="d80")
    q, k, v = si.make_inputs(wl, seed=0)
    dob = si.make_grad(wl, seed=0)
    tq, tk, tv, tdo = upload(q), upload(k), upload(v), upload(dob)
    del q, k, v, dob
    o = torch.empty_like(tq)
    lse = torch.empty((B, h, T), dtype=torch.float32, device="cuda")
    gr = [torch.empty_like(tq) for _ in range(3)]
    ws = torch.empty(fa.fa_bwd_workspace_size(B, h, T), dtype=torch.uint8, device="cuda")
    fa.fa_fwd(tq, tk, tv, causal=True, scale=wl.scale, o=o, lse=lse)
    ms = interleaved(torch, {
        "fwd": lambda: fa.fa_fwd(tq, tk, tv, causal=True, scale=wl.scale, o=o, lse=lse),
        "bwd": lambda: fa.fa_bwd(tq, tk, tv, o, tdo, lse, causal=True, scale=wl.scale,
                                 dq=gr[0], dk=gr[1], dv=gr[2], workspace=ws)}, 2, max(3, K // 2))
    for key, m, fl, padded, what in (
            ("d80", ms["fwd"], cm.attention_flops(B, h, T, T, d, True),
             cm.attention_flops(B, h, T, T, 128, True), "attention fwd"),
            ("bwd_d80", ms["bwd"], cm.attention_bwd_flops(B, h, T, T, d, True),
             cm.attention_bwd_flops(B, h, T, T, 128, True), "attention backward")):
        tf_true = fl / (m * 1e-3) / 1e12
        tf_pad = padded / (m * 1e-3) / 1e12
        eprint(f"[bench] layout {key}: B={B} h={h} T={T} d={d} {m:.4f} ms  {tf_true:.1f} TFLOP/s "
               f"of d=80 ({100 * tf_true / peak:.1f}%), {tf_pad:.1f} TFLOP/s of the 128-wide "
               f"kernel's work ({100 * tf_pad / peak:.1f}%)")
        res[key] = {"metric": f"{what} TFLOP/s, causal, d_head=80 (padded to 128 on chip)",
                    "value": tf_true, "unit": "TFLOP/s", "avg_ms": m,
                    "padded_tflops": tf_pad, "padded_frac": tf_pad / peak,
                    "roofline": {"bound": "mfma", "achieved": tf_true, "peak": peak,
                                 "unit": "TFLOP/s", "frac": tf_true / peak, "traffic": None},
                    "config": {"B": B, "h": h, "T": T, "d_head": d, "causal": True,
                               "flops": fl, "padded_flops": padded}}
    del tq, tk, tv, tdo, o, lse, gr, ws
    torch.cuda.empty_cache()

    if dec is not None:
        wd, dq_, dk_, dv_ = dec
        kc = dk_.transpose(1, 2).contiguous().transpose(1, 2)   # [B][Tk][h][d] storage
        vc = dv_.transpose(1, 2).contiguous().transpose(1, 2)
        o = torch.empty_like(dq_)
        lse = torch.empty((wd.B, wd.h), dtype=torch.float32, device="cuda")
        ws = torch.empty(fa.fa_decode_workspace_size(wd.B, wd.h, wd.d, wd.num_splits),
                         dtype=torch.uint8, device="cuda")
        ms = interleaved(torch, {
            "contiguous": lambda: fa.fa_decode(dq_, dk_, dv_, num_splits=wd.num_splits,
                                               scale=wd.scale, o=o, lse=lse, workspace=ws),
            "bthd": lambda: fa.fa_decode_strided(dq_, kc, vc, num_splits=wd.num_splits,
                                                 scale=wd.scale, o=o, lse=lse, workspace=ws)},
            3, K)
        kv = wd.B * wd.h * wd.Tk * cm.decode_kv_bytes_per_token(wd.d)
        gbs = {n: kv / (m * 1e-3) / 1e9 for n, m in ms.items()}
        hbm = cm.MI355X_PEAK_HBM_BYTES_PER_S / 1e9
        eprint(f"[bench] layout decode_bthd: B={wd.B} h={wd.h} Tk={wd.Tk} d={wd.d} "
               f"S={wd.num_splits} {ms['bthd']:.4f} ms {gbs['bthd']:.0f} GB/s "
               f"({100 * gbs['bthd'] / hbm:.1f}%) against contiguous {gbs['contiguous']:.0f} "
               f"(ratio {ms['bthd'] / ms['contiguous']:.3f})")
        res["decode_bthd"] = {
            "metric": "decode HBM GB/s (K+V bytes / split+combine time), KV cache in [B][Tk][h][d]",
            "value": gbs["bthd"], "unit": "GB/s", "steps": K, "warmup": 3,
            "avg_ms": ms["bthd"], "contiguous_ms": ms["contiguous"],
            "time_ratio_vs_contiguous": ms["bthd"] / ms["contiguous"],
            "roofline": {"bound": "hbm", "achieved": gbs["bthd"], "peak": hbm, "unit": "GB/s",
                         "frac": gbs["bthd"] / hbm, "traffic": None},
            "config": {"B": wd.B, "h": wd.h, "Tk": wd.Tk, "d_head": wd.d,
                       "num_splits": wd.num_splits, "layout": "BTHD strided KV cache"}}
        del kc, vc, o, lse, ws
        torch.cuda.empty_cache()
    return res


def measure_elementwise(args, fa, si, torch):
    """GELU on the pages' 64M fp32 values and bias-GELU-dropout on a 4096 x 8192 bf16
    activation (p = 0.1); each HBM GB/s counts one read and one write of the tensor."""
    import numpy as np
    from io_aware_attention_fa_amd import costmodel as cm
    peak = cm.MI355X_PEAK_HBM_BYTES_PER_S / 1e9
    res = {}
    n = si.GELU_WORKLOAD_N
    xh = si.elementwise_input(n, seed=0)
    x = torch.from_numpy(xh).cuda()
    y = torch.empty_like(x)
    K = args.extra_steps or 50
    ms = time_calls(torch, lambda: fa.fa_gelu_f32(x, y=y), 5, K)
    nbytes = 8.0 * n
    gbs = nbytes / (ms * 1e-3) / 1e9
    eprint(f"[bench] gelu f32 n={n} avg {ms * 1e3:.1f} us  {gbs:.0f} GB/s  "
           f"{100 * gbs / peak:.1f}% of HBM peak")
    g = {"metric": "GELU (tanh form) HBM GB/s, one read + one write of 64M fp32 values",
         "value": gbs, "unit": "GB/s", "steps": K, "warmup": 5, "avg_ms": ms,
         "roofline": {"bound": "hbm", "achieved": gbs, "peak": peak, "unit": "GB/s",
                      "frac": gbs / peak,
                      "traffic": traffic_from_profiles("fa_gelu_f32_kernel__gelu_64M_f32")},
         "config": {"n": n, "dtype": "f32", "alg_bytes": nbytes}}
    if not args.no_cpu_baseline:
        from oracle import elementwise_ref as eref
        m = 4_000_000
        t0 = time.perf_counter()
        eref.gelu_tanh(xh[:m])
        el = time.perf_counter() - t0
        g["cpu_baseline"] = {"value": 8.0 * m / el / 1e9, "unit": "GB/s", "cores": 1,
                             "kind": "oracle",
                             "sample": f"the first {m} of the {n} values, {el:.2f} s of fp64 "
                                       "numpy (bytes counted as fp32 read + write)"}
    res["gelu"] = g
    del x, y
    rows, cols, p = si.DROPOUT_WORKLOAD
    xb, bb = si.activation_input(rows, cols, seed=0)
    xa = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    ba = torch.from_numpy(bb.view(np.int16)).view(torch.bfloat16).cuda()
    ya = torch.empty_like(xa)
    ms = time_calls(torch, lambda: fa.fa_bias_gelu_dropout_bf16(xa, ba, p=p, seed=1234, y=ya), 5,
                    K)
    nbytes = 4.0 * rows * cols
    gbs = nbytes / (ms * 1e-3) / 1e9
    eprint(f"[bench] bias-gelu-dropout {rows}x{cols} p={p} avg {ms * 1e3:.1f} us  {gbs:.0f} GB/s  "
           f"{100 * gbs / peak:.1f}% of HBM peak")
    d = {"metric": "bias-GELU-dropout HBM GB/s, one read + one write of the bf16 activation",
         "value": gbs, "unit": "GB/s", "steps": K, "warmup": 5, "avg_ms": ms,
         "roofline": {"bound": "hbm", "achieved": gbs, "peak": peak, "unit": "GB/s",
                      "frac": gbs / peak,
                      "traffic": traffic_from_profiles(
                          f"fa_bias_gelu_dropout_vec_kernel__dropout_{rows}x{cols}_bf16")},
         "config": {"rows": rows, "cols": cols, "p": p, "dtype": "bf16", "alg_bytes": nbytes}}
    if not args.no_cpu_baseline:
        from oracle import elementwise_ref as eref
        r = 64
        t0 = time.perf_counter()
        eref.bias_gelu_dropout(si.bf16_bits_to_f64(xb[:r]), si.bf16_bits_to_f64(bb), p, 1234, 0)
        el = time.perf_counter() - t0
        d["cpu_baseline"] = {"value": 4.0 * r * cols / el / 1e9, "unit": "GB/s", "cores": 1,
                             "kind": "oracle",
                             "sample": f"the first {r} rows of {rows}, {el:.2f} s of fp64 numpy "
                                       "with the Philox stream (bytes counted as bf16 read + "
                                       "write)"}
    res["bias_gelu_dropout"] = d
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["prefill", "decode", "backward", "softmax", "elementwise",
                                       "layouts", "configs"],
                    default=None,
                    help="run one half of the step (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the separately timed backward measurement")
    ap.add_argument("--bwd-steps", type=int, default=20)
    ap.add_argument("--extra-steps", type=int, default=0,
                    help="timed calls of each separately measured kernel (0: its default)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the separately timed softmax and elementwise measurements")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other forward configurations (T=128 latency, T=1024 at the "
                         "ridge, T=16384 long context)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the GFX clock under the forward")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        eprint("bench.py measures a single GPU; runs on several GPUs are not supported. "
               "Run with --gpus 1.")
        sys.exit(2)

    import torch

    import io_aware_attention_fa_amd as fa
    import seeded_inputs as si
    from io_aware_attention_fa_amd import costmodel as cm

    if not torch.cuda.is_available():
        eprint("bench.py needs a GPU")
        sys.exit(1)
    dev = torch.cuda.current_device()
    props = torch.cuda.get_device_properties(dev)
    eprint(f"[bench] device {props.name} CUs={props.multi_processor_count} lib={fa.LIB_PATH}")

    if args.copy_probe_mib:
        n = args.copy_probe_mib * 2**20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        eprint(f"[bench] copy probe of {n} bytes done")

    do_prefill = args.only in (None, "prefill")
    do_decode = args.only in (None, "decode")
    do_backward = args.only == "backward" or (args.only is None and not args.no_backward)
    do_softmax = args.only == "softmax" or (args.only is None and not args.no_extras)
    do_elementwise = args.only == "elementwise" or (args.only is None and not args.no_extras)
    do_layouts = args.only == "layouts" or (args.only is None and not args.no_extras)
    wp, wd = si.WORKLOADS[PREFILL], si.WORKLOADS[DECODE]

    t0 = time.perf_counter()
    if args.only == "softmax":
        sm = measure_softmax(args, fa, si, torch)
        out = {"metric": sm["metric"], "value": sm["value"], "unit": sm["unit"],
               "n_gpus": 1, "steps": sm["steps"], "warmup": sm["warmup"],
               "ms_per_step": sm["avg_ms"], "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": "f32", "data": "synthetic",
               "roofline": sm["roofline"], "config": {"workload": "softmax_rows_4096x4096_f32"},
               "cpu_baseline": sm.get("cpu_baseline")}
        print(json.dumps(out), flush=True)
        return

    if args.only == "configs":
        cf = measure_configs(args, fa, si, cm, torch)
        c4 = cf["C4"]
        out = {"metric": c4["metric"], "value": c4["value"], "unit": c4["unit"], "n_gpus": 1,
               "steps": c4["timing"]["trials"], "warmup": 3, "ms_per_step": c4["timing"]["avg_ms"],
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
               "data": "synthetic", "roofline": c4["roofline"],
               "config": {"workload": "longctx_causal_b2_h32_t16384_d128_keyspikes"},
               "cpu_baseline": c4.get("cpu_baseline"), "configs": cf}
        print(json.dumps(out), flush=True)
        return

    if args.only == "layouts":
        lay = measure_layouts(args, fa, si, cm, torch)
        b = lay["bthd"]
        out = {"metric": b["metric"], "value": b["value"], "unit": b["unit"], "n_gpus": 1,
               "steps": b["steps"], "warmup": b["warmup"], "ms_per_step": b["avg_ms"],
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
               "data": "synthetic", "roofline": b["roofline"],
               "config": {"workload": "causal_b8_h32_t4096_d128 in [B][T][h][d]"},
               "cpu_baseline": None, "layouts": lay}
        print(json.dumps(out), flush=True)
        return

    if args.only == "elementwise":
        ew = measure_elementwise(args, fa, si, torch)
        g = ew["gelu"]
        out = {"metric": g["metric"], "value": g["value"], "unit": g["unit"], "n_gpus": 1,
               "steps": g["steps"], "warmup": g["warmup"], "ms_per_step": g["avg_ms"],
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
               "data": "synthetic", "roofline": g["roofline"],
               "config": {"workload": "gelu_64M_f32 + bias_gelu_dropout_4096x8192_bf16"},
               "cpu_baseline": g.get("cpu_baseline"),
               "bias_gelu_dropout": ew["bias_gelu_dropout"]}
        print(json.dumps(out), flush=True)
        return

    if do_prefill or do_backward:
        q, k, v = si.make_inputs(wp, seed=0)
        pq, pk, pv = upload(q), upload(k), upload(v)
        po = torch.empty_like(pq)
        plse = torch.empty((wp.B, wp.h, wp.Tq), dtype=torch.float32, device="cuda")
        del q, k, v
    dec_host = None
    if do_decode:
        q, k, v = si.make_inputs(wd, seed=0)
        dq, dk, dv = upload(q), upload(k), upload(v)
        do = torch.empty_like(dq)
        dlse = torch.empty((wd.B, wd.h), dtype=torch.float32, device="cuda")
        ws = torch.empty(fa.fa_decode_workspace_size(wd.B, wd.h, wd.d, wd.num_splits),
                         dtype=torch.uint8, device="cuda")
        if not args.no_cpu_baseline:
            dec_host = (q, k, v)   # the oracle's sample reads the same bits
        del q, k, v
    torch.cuda.synchronize()
    eprint(f"[bench] inputs generated and resident in {time.perf_counter() - t0:.1f} s")


    if args.only == "backward":
        out = {"metric": "attention backward TFLOP/s (2.5x forward FLOPs), % MFMA peak",
               "n_gpus": 1, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
               "dtype": "bf16", "data": "synthetic"}
        bwd = measure_backward(args, fa, si, cm, torch, wp, pq, pk, pv, po, plse)
        out.update(value=bwd["value"], unit=bwd["unit"], roofline=bwd["roofline"],
                   steps=bwd["steps"], warmup=bwd["warmup"], ms_per_step=bwd["avg_ms"],
                   config={"workload": PREFILL, "backward": bwd["config"]},
                   cpu_baseline=bwd.get("cpu_baseline"))
        print(json.dumps(out), flush=True)
        return

    def step(evs=None, i=0):
        if do_prefill:
            if evs:
                evs["p0"][i].record()
            fa.fa_fwd(pq, pk, pv, causal=True, scale=wp.scale, o=po, lse=plse)
            if evs:
                evs["p1"][i].record()
        if do_decode:
            if evs:
                evs["d0"][i].record()
            fa.fa_decode(dq, dk, dv, num_splits=wd.num_splits, scale=wd.scale, o=do, lse=dlse,
                         workspace=ws)
            if evs:
                evs["d1"][i].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    evs = {key: [torch.cuda.Event(enable_timing=True) for _ in range(K)]
           for key in ("p0", "p1", "d0", "d1")}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(evs, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eprint(f"[bench] {K} steps in {wall * 1e3:.1f} ms")

    out = {"metric": METRIC, "n_gpus": 1, "steps": K, "warmup": args.warmup,
           "ms_per_step": wall / K * 1e3, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    config = {"workload": f"{PREFILL} + {DECODE}" if args.only is None else
              (PREFILL if do_prefill else DECODE)}

    if do_prefill:
        pt = [evs["p0"][i].elapsed_time(evs["p1"][i]) for i in range(K)]
        p_ms = sum(pt) / K
        flops = cm.attention_flops(wp.B, wp.h, wp.Tq, wp.Tk, wp.d, True)
        tflops = flops / (p_ms * 1e-3) / 1e12
        peak = cm.MI355X_PEAK_BF16_DENSE_FLOPS / 1e12
        out.update(value=tflops, unit="TFLOP/s")
        out["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                           "frac": tflops / peak,
                           "traffic": traffic_from_profiles(f"fa_fwd_kernel__{PREFILL}")}
        config.update(prefill={"B": wp.B, "h": wp.h, "T": wp.Tq, "d_head": wp.d, "causal": True,
                               "avg_ms": p_ms, "min_ms": min(pt), "median_ms": sorted(pt)[K // 2],
                               "alg_bytes": cm.attention_io_bytes(wp.B, wp.h, wp.Tq, wp.Tk, wp.d),
                               "flops": flops})
        eprint(f"[bench] prefill avg {p_ms:.4f} ms  {tflops:.1f} TFLOP/s  "
               f"{100 * tflops / peak:.1f}% of {peak:.0f}")
    if do_decode:
        dt = [evs["d0"][i].elapsed_time(evs["d1"][i]) for i in range(K)]
        d_ms = sum(dt) / K
        kv = wd.B * wd.h * wd.Tk * cm.decode_kv_bytes_per_token(wd.d)
        gbs = kv / (d_ms * 1e-3) / 1e9
        peak_gbs = cm.MI355X_PEAK_HBM_BYTES_PER_S / 1e9
        dec = {"metric": "decode HBM GB/s (K+V bytes / split+combine time)", "value": gbs,
               "unit": "GB/s",
               "roofline": {"bound": "hbm", "achieved": gbs, "peak": peak_gbs, "unit": "GB/s",
                            "frac": gbs / peak_gbs,
                            "traffic": traffic_from_profiles(
                                f"fa_decode_split_kernel__{DECODE}")},
               "avg_ms": d_ms, "min_ms": min(dt), "median_ms": sorted(dt)[K // 2],
               "config": {"B": wd.B, "h": wd.h, "Tk": wd.Tk, "d_head": wd.d,
                          "num_splits": wd.num_splits}}
        out["decode"] = dec
        eprint(f"[bench] decode avg {d_ms:.4f} ms  {gbs:.0f} GB/s  {100 * gbs / peak_gbs:.1f}%")
        if not do_prefill:
            out.update(value=gbs, unit="GB/s", roofline=dec["roofline"])
    out["config"] = config
    out["host"] = host_info()
    cus = props.multi_processor_count
    if do_prefill and not args.no_clock:
        clk = sample_clock(torch, lambda: fa.fa_fwd(pq, pk, pv, causal=True, scale=wp.scale,
                                                    o=po, lse=plse))
        clk["cus"] = cus
        clk["device"] = props.name
        if clk.get("mhz"):
            pk_clk = cm.bf16_peak_at_clock(clk["mhz"] * 1e6, cus) / 1e12
            clk["mfma_peak_at_clock_tflops"] = pk_clk
            clk["frac_at_clock"] = out["value"] / pk_clk
            out["roofline"]["frac_at_clock"] = out["value"] / pk_clk
            out["roofline"]["sclk_mhz"] = clk["mhz"]
            eprint(f"[bench] GFX clock under the forward: {clk['mhz']:.0f} MHz mean "
                   f"({clk['samples']} samples); MFMA peak at that clock {pk_clk:.0f} TFLOP/s, "
                   f"forward at {100 * clk['frac_at_clock']:.1f}% of it")
        else:
            eprint(f"[bench] GFX clock not measured: {clk.get('error')}")
        out["clock"] = clk
    else:
        out["clock"] = {"mhz": None, "cus": cus, "device": props.name}

    if do_prefill and not args.no_cpu_baseline:
        eprint("[bench] timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    configs = {}
    if do_prefill:
        configs["C3"] = {"workload": PREFILL, "value": out["value"], "unit": "TFLOP/s",
                         "roofline": out["roofline"], "cpu_baseline": out["cpu_baseline"]}
    if do_decode:
        c5 = {"workload": DECODE, "value": out["decode"]["value"], "unit": "GB/s",
              "roofline": out["decode"]["roofline"]}
        if dec_host is not None:
            eprint("[bench] timing the CPU decode oracle on a sample")
            hq, hk, hv = dec_host
            c5["cpu_baseline"] = oracle_baseline(
                wd, [divmod(i, wd.h) for i in range(0, wd.B * wd.h, 16)], 3, "every 16th head",
                unit="GB/s", get_head=lambda b, h: (hq[b, h], hk[b, h], hv[b, h]))
            out["decode"]["cpu_baseline"] = c5["cpu_baseline"]
            del hq, hk, hv, dec_host
        configs["C5"] = c5
    if args.only is None and not args.no_configs:
        configs.update(measure_configs(args, fa, si, cm, torch))
    if configs:
        out["configs"] = configs
    if do_backward:
        out["backward"] = measure_backward(args, fa, si, cm, torch, wp, pq, pk, pv, po, plse)
    if do_softmax:
        out["softmax"] = measure_softmax(args, fa, si, torch)
    if do_elementwise:
        out.update(measure_elementwise(args, fa, si, torch))
    if do_layouts:
        out["layouts"] = measure_layouts(args, fa, si, cm, torch,
                                         dec=(wd, dq, dk, dv) if do_decode else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
