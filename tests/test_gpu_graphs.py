"""The C-ABI entry points under HIP graph capture.

The library allocates nothing, synchronises nothing and records no memset: every entry point only
enqueues kernels on the caller's stream, so a caller can capture a whole step -- forward, backward,
decode and the fused row and elementwise kernels -- into one graph and replay it.  Each replay
below runs on fresh inputs copied into the captured buffers (eager work between replays), and its
outputs must equal those of the same calls made eagerly, bit for bit: every kernel here is
deterministic (no atomics, fixed reduction orders), so any difference would be a capture fault.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from tests.gpu_support import log, to_gpu

pytestmark = pytest.mark.gpu


def _inputs(seed):
    """One step's seeded inputs: prefill q/k/v/dO, a decode query and KV cache, fused-op data."""
    wl = si.custom_workload(2, 3, 700, 700, 128, True, name="graph_prefill")
    q, k, v = si.make_inputs(wl, seed, threads=4)
    do = si.make_grad(wl, seed)
    dwl = si.custom_workload(4, 4, 1, 2500, 128, False, decode=True, num_splits=8,
                             name="graph_decode")
    dq, dk, dv = si.make_inputs(dwl, seed + 100, threads=4)
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(300, 1000, generator=g)
    xb = torch.randn(256, 512, generator=g).to(torch.bfloat16)
    bias = torch.randn(512, generator=g).to(torch.bfloat16)
    return dict(q=to_gpu(q), k=to_gpu(k), v=to_gpu(v), do=to_gpu(do), dq_=to_gpu(dq),
                dk_=to_gpu(dk), dv_=to_gpu(dv), x=x.cuda(), xb=xb.cuda(), bias=bias.cuda())


def _step(fa, t, out, ws):
    """One pass over every entry point, writing into the given output buffers."""
    fa.fa_fwd(t["q"], t["k"], t["v"], causal=True, o=out["o"], lse=out["lse"])
    fa.fa_bwd(t["q"], t["k"], t["v"], out["o"], t["do"], out["lse"], causal=True,
              dq=out["dq"], dk=out["dk"], dv=out["dv"], workspace=ws["bwd"])
    fa.fa_decode(t["dq_"], t["dk_"], t["dv_"], num_splits=8, o=out["od"], lse=out["lsed"],
                 workspace=ws["dec"])
    fa.fa_softmax_rows(t["x"], y=out["y"], lse=out["ylse"], with_lse=True)
    fa.fa_gelu_f32(t["x"], y=out["g"])
    fa.fa_bias_gelu_dropout_bf16(t["xb"], t["bias"], p=0.1, seed=1234, offset=0, y=out["bgd"])


def _outputs(t):
    B, h, T, d = t["q"].shape
    Bd, hd, Tk, _ = t["dk_"].shape
    e = torch.empty
    return dict(o=torch.empty_like(t["q"]), lse=e((B, h, T), device="cuda"),
                dq=torch.empty_like(t["q"]), dk=torch.empty_like(t["k"]),
                dv=torch.empty_like(t["v"]), od=torch.empty_like(t["dq_"]),
                lsed=e((Bd, hd), device="cuda"), y=torch.empty_like(t["x"]),
                ylse=e((t["x"].shape[0],), device="cuda"), g=torch.empty_like(t["x"]),
                bgd=torch.empty_like(t["xb"]))


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


def test_graph_replays_equal_eager_calls(gpu):
    static = _inputs(seed=40)
    out = _outputs(static)
    B, h, T, d = static["q"].shape
    Bd, hd, _, _ = static["dk_"].shape
    ws = {"bwd": torch.empty(gpu.fa_bwd_workspace_size(B, h, T), dtype=torch.uint8,
                             device="cuda"),
          "dec": torch.empty(gpu.fa_decode_workspace_size(Bd, hd, d, 8), dtype=torch.uint8,
                             device="cuda")}
    # one eager pass first (nothing in the library needs it; it settles torch's own state)
    _step(gpu, static, out, ws)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(gpu, static, out, ws)
    torch.cuda.synchronize()

    for rep, seed in enumerate((41, 42, 43)):
        log(f"[case] graph replay {rep} seed={seed}")
        fresh = _inputs(seed)
        for name, tensor in fresh.items():
            static[name].copy_(tensor)
        graph.replay()
        torch.cuda.synchronize()
        replayed = {name: x.clone() for name, x in out.items()}
        # the same calls, eagerly, on the same inputs, into separate buffers
        eager_out = _outputs(fresh)
        eager_ws = {name: torch.empty_like(w) for name, w in ws.items()}
        _step(gpu, fresh, eager_out, eager_ws)
        torch.cuda.synchronize()
        for name in out:
            same = torch.equal(_bits(replayed[name]), _bits(eager_out[name]))
            assert same, f"replay {rep}: {name} differs from the eager call"
        assert np.isfinite(replayed["lse"].cpu().numpy()).all()
