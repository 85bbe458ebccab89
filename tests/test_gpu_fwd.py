"""GPU parity of the attention forward against the fp64 oracle, through the C ABI.

Gates: max|dO| <= 1e-2 on the kernel's fp32 output (same kernel, fp32 store), max|dLSE| <= 1e-3,
the bf16 output equal bit-for-bit to the round-to-nearest-even of the fp32 output, and the bf16
output within 1e-2 plus its own rounding of the oracle.  Full workload sizes run in the launch
configuration the benchmark times; the oracle checks sampled rows there.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import attention_ref as ref
from tests.gpu_support import (LSE_TOL, O_TOL, assert_bf16_is_rne_of_f32, check_rows, log,
                               lse_row_tolerance, run_fwd, to_gpu, workload_inputs)

pytestmark = pytest.mark.gpu


def _oracle_rows(q, k, v, wl, heads_rows):
    """Oracle (O, LSE) for {(b, h): rows}."""
    out = {}
    for (b, h), rows in heads_rows.items():
        out[(b, h)] = ref.naive_attention_head(si.bf16_bits_to_f64(q[b, h]),
                                               si.bf16_bits_to_f64(k[b, h]),
                                               si.bf16_bits_to_f64(v[b, h]), wl.scale, wl.causal,
                                               rows=rows)
    return out


def _check_sampled(tag, res, q, k, v, wl, heads_rows):
    o32 = res["o32"].cpu().numpy()
    l32 = res["lse32"].cpu().numpy()
    o16 = res["o16"].float().cpu().numpy()
    refs = _oracle_rows(q, k, v, wl, heads_rows)
    O_ref = np.concatenate([refs[bh][0] for bh in heads_rows])
    L_ref = np.concatenate([refs[bh][1] for bh in heads_rows])
    sel = lambda a: np.concatenate([a[b, h][rows] for (b, h), rows in heads_rows.items()])
    return check_rows(tag, sel(o32), sel(l32), sel(o16), O_ref, L_ref)


def test_tiny_noncausal_full(gpu):
    wl, q, k, v = workload_inputs("tiny_noncausal_b1_h2_t128_d64")
    res = run_fwd(gpu, q, k, v, wl.causal, wl.scale)
    assert_bf16_is_rne_of_f32(res)
    heads = {(0, h): np.arange(wl.Tq) for h in range(wl.h)}
    _check_sampled(wl.name, res, q, k, v, wl, heads)


def test_causal_t1024_d64_full_size(gpu):
    wl, q, k, v = workload_inputs("causal_b8_h32_t1024_d64")
    res = run_fwd(gpu, q, k, v, wl.causal, wl.scale)
    assert_bf16_is_rne_of_f32(res)
    rng = np.random.default_rng(11)
    heads = {(b, h): np.arange(wl.Tq) for b, h in [(0, 0), (3, 17), (7, 31)]}
    for _ in range(24):
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.h))
        heads.setdefault((b, h), np.sort(rng.choice(wl.Tq, 48, replace=False)))
    _check_sampled(wl.name, res, q, k, v, wl, heads)


def test_causal_t4096_d128_full_size(gpu):
    wl, q, k, v = workload_inputs("causal_b8_h32_t4096_d128")
    res = run_fwd(gpu, q, k, v, wl.causal, wl.scale)
    assert_bf16_is_rne_of_f32(res)
    rng = np.random.default_rng(12)
    heads = {(5, 9): np.arange(wl.Tq)}
    edge = np.array([0, 1, 127, 128, 129, 2047, 4094, 4095])
    for _ in range(16):
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.h))
        rows = np.unique(np.concatenate([edge, rng.choice(wl.Tq, 40, replace=False)]))
        heads.setdefault((b, h), rows)
    _check_sampled(wl.name, res, q, k, v, wl, heads)


def test_longctx_t16384_keyspikes_full_size(gpu):
    wl, q, k, v = workload_inputs("longctx_causal_b2_h32_t16384_d128_keyspikes")
    res = run_fwd(gpu, q, k, v, wl.causal, wl.scale)
    assert_bf16_is_rne_of_f32(res)
    rng = np.random.default_rng(13)
    heads = {}
    edge = np.array([0, 1, 2, 63, 64, 127, 128, 8191, 16382, 16383])
    for _ in range(12):
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.h))
        rows = np.unique(np.concatenate([edge, rng.choice(wl.Tq, 24, replace=False)]))
        heads.setdefault((b, h), rows)
    _check_sampled(wl.name, res, q, k, v, wl, heads)


EDGE_SHAPES = [
    # (B, h, Tq, Tk, d, causal)
    (1, 1, 1, 1, 64, False), (1, 1, 1, 1, 128, True), (2, 3, 7, 7, 64, True),
    (1, 2, 63, 63, 128, True), (1, 2, 127, 127, 64, False), (1, 2, 129, 129, 128, True),
    (2, 2, 1000, 1000, 64, True), (1, 1, 4097, 4097, 128, True), (1, 1, 4097, 4097, 64, False),
    (2, 2, 100, 333, 128, False), (2, 2, 333, 100, 64, False), (1, 3, 77, 200, 128, True),
    (1, 2, 1, 513, 128, True), (1, 2, 200, 200, 64, True), (3, 1, 64, 64, 128, True),
    (1, 1, 65, 1, 64, False), (1, 1, 256, 257, 128, True),
]


@pytest.mark.parametrize("B,h,Tq,Tk,d,causal", EDGE_SHAPES)
def test_edge_shapes(gpu, B, h, Tq, Tk, d, causal):
    wl = si.custom_workload(B, h, Tq, Tk, d, causal)
    q, k, v = si.make_inputs(wl, seed=5, threads=4)
    res = run_fwd(gpu, q, k, v, causal, wl.scale)
    assert_bf16_is_rne_of_f32(res)
    heads = {(b, hh): np.arange(Tq) for b in range(B) for hh in range(h)}
    _check_sampled(f"edge B{B} h{h} Tq{Tq} Tk{Tk} d{d} causal{int(causal)}", res, q, k, v, wl,
                   heads)


# Shapes with more (head, block-pair) items than CUs, so the kernel runs its persistent
# schedule: head counts not divisible by the 8 XCD groups, odd block counts (a middle block with
# no partner), causal with Tq < Tk, non-causal.
PERSISTENT_SHAPES = [
    (3, 37, 1100, 1100, 128, True), (3, 37, 1100, 1500, 64, True),
    (2, 45, 1300, 1300, 128, False), (1, 130, 1024, 1024, 64, True),
    # one key tile per item with more items than CUs (the launcher runs one block pair per
    # workgroup there, so the two-tile lookahead never has to reach past the next item)
    (8, 32, 4096, 64, 128, False), (32, 32, 64, 64, 64, True), (8, 32, 4096, 40, 64, False),
]


@pytest.mark.parametrize("B,h,Tq,Tk,d,causal", PERSISTENT_SHAPES)
def test_persistent_schedule_shapes(gpu, B, h, Tq, Tk, d, causal):
    wl = si.custom_workload(B, h, Tq, Tk, d, causal)
    q, k, v = si.make_inputs(wl, seed=21, threads=8)
    res = run_fwd(gpu, q, k, v, causal, wl.scale)
    assert_bf16_is_rne_of_f32(res)
    rng = np.random.default_rng(B * 1000 + h)
    edge = np.array([0, 1, 255, 256, 511, 512, Tq // 2, Tq - 2, Tq - 1])
    edge = edge[edge < Tq]
    heads = {}
    for bh in sorted({0, 1, 7, 8, 9, B * h // 2, B * h - 2, B * h - 1} |
                     set(rng.choice(B * h, 8, replace=False).tolist())):
        rows = np.unique(np.concatenate([edge, rng.choice(Tq, min(Tq, 24), replace=False)]))
        heads[divmod(int(bh), h)] = rows
    _check_sampled(f"persistent B{B} h{h} Tq{Tq} Tk{Tk} d{d} causal{int(causal)}", res, q, k, v,
                   wl, heads)
    # Every row of every item was written: its LSE lies between the row's largest visible score
    # and that plus ln(#visible keys) (scores in fp32 on the CPU, a bound, not the oracle).
    qf = torch.from_numpy(si.bf16_bits_to_f32(q)).reshape(B * h, Tq, d)
    kf = torch.from_numpy(si.bf16_bits_to_f32(k)).reshape(B * h, Tk, d)
    lse = res["lse32"].cpu().reshape(B * h, Tq)
    cnt = torch.full((Tq,), float(Tk))
    for i0 in range(0, B * h, 16):
        sc = torch.bmm(qf[i0:i0 + 16], kf[i0:i0 + 16].transpose(1, 2).contiguous()) * wl.scale
        if causal:
            vis = torch.arange(Tk)[None, :] <= torch.arange(Tq)[:, None] + (Tk - Tq)
            sc = sc.masked_fill(~vis, float("-inf"))
            cnt = vis.sum(1).float()
        mx = sc.amax(2)
        part = lse[i0:i0 + 16]
        assert torch.all(part >= mx - 1e-3), "an LSE below its row maximum: a row was not written"
        assert torch.all(part <= mx + torch.log(cnt)[None] + 1e-3), "an LSE above its bound"
    assert torch.isfinite(res["o32"]).all()


@pytest.mark.parametrize("d,causal", [(64, True), (64, False), (128, True)])
def test_key_spikes_raise_the_running_max(gpu, d, causal):
    """1% of the keys scaled x8 (the long-context recipe) at a size the oracle runs whole:
    the running max jumps many times per row, so the rescale path runs often."""
    wl = si.custom_workload(2, 3, 1500, 1500, d, causal, key_spike_frac=0.01,
                            key_spike_mult=8.0)
    q, k, v = si.make_inputs(wl, seed=23, threads=4)
    res = run_fwd(gpu, q, k, v, causal, wl.scale)
    o32 = res["o32"].cpu().numpy()
    l32 = res["lse32"].cpu().numpy()
    for bh in [(0, 0), (1, 2)]:
        o_ref, l_ref = ref.naive_attention_head(si.bf16_bits_to_f64(q[bh]),
                                                si.bf16_bits_to_f64(k[bh]),
                                                si.bf16_bits_to_f64(v[bh]), wl.scale, causal)
        d_o = float(np.max(np.abs(o32[bh] - o_ref)))
        d_l = float(np.max(np.abs(l32[bh] - l_ref)))
        log(f"[parity] keyspikes d={d} causal={causal} head {bh}: max|dO|={d_o:.3e} "
            f"max|dLSE|={d_l:.3e}")
        assert d_o <= O_TOL and d_l <= LSE_TOL


@pytest.mark.parametrize("d", [64, 128])
def test_causal_row_zero_is_exactly_first_value_row(gpu, d):
    wl = si.custom_workload(2, 4, 300, 300, d, True)
    q, k, v = si.make_inputs(wl, seed=8, threads=4)
    res = run_fwd(gpu, q, k, v, True, wl.scale)
    o16 = res["o16"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(o16[:, :, 0, :], v[:, :, 0, :])
    qf, kf = si.bf16_bits_to_f64(q), si.bf16_bits_to_f64(k)
    lse0 = wl.scale * np.einsum("bhd,bhd->bh", qf[:, :, 0], kf[:, :, 0])
    assert np.max(np.abs(res["lse32"].cpu().numpy()[:, :, 0] - lse0)) <= 1e-5


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,Tq,Tk", [(True, 300, 300), (True, 100, 357), (False, 130, 257)])
def test_zero_queries_give_log_count_and_mean(gpu, causal, Tq, Tk, d):
    wl = si.custom_workload(1, 2, Tq, Tk, d, causal)
    _, k, v = si.make_inputs(wl, seed=9, threads=2)
    q = np.zeros((1, 2, Tq, d), dtype=np.uint16)
    res = run_fwd(gpu, q, k, v, causal, wl.scale)
    counts = np.arange(Tq) + (Tk - Tq) + 1 if causal else np.full(Tq, Tk)
    lse = res["lse32"].cpu().numpy()
    assert np.max(np.abs(lse - np.log(counts)[None, None])) <= LSE_TOL
    vf = si.bf16_bits_to_f64(v)
    cum = np.cumsum(vf, axis=2) / np.arange(1, Tk + 1)[None, None, :, None]
    expect = cum[:, :, counts - 1, :]
    assert np.max(np.abs(res["o32"].cpu().numpy() - expect)) <= O_TOL


def test_constant_values_give_that_constant(gpu):
    wl = si.custom_workload(1, 2, 200, 200, 64, True)
    q, k, _ = si.make_inputs(wl, seed=10, threads=2)
    v = np.full_like(k, si.rne_bf16_bits(np.array([0.375], np.float32))[0])
    res = run_fwd(gpu, q, k, v, True, wl.scale)
    # O is normalised by the sum of the same bf16-rounded p the P V contraction used, so equal
    # value rows come back up to fp32 summation-order noise.
    err = np.abs(res["o32"].cpu().numpy() - 0.375)
    assert np.max(err) <= 0.375 * 2e-5
    assert np.all(err[:, :, 0] == 0.0)   # row 0 sees one key: p = 1 exactly


@pytest.mark.parametrize("d", [64, 128])
def test_large_scores_stay_finite_and_exact(gpu, d):
    """Scores in the hundreds: exp overflows unless the running max is subtracted."""
    wl = si.custom_workload(1, 2, 256, 256, d, True)
    q, k, v = si.make_inputs(wl, seed=14, threads=2)
    scale = 12.0
    res = run_fwd(gpu, q, k, v, True, scale)
    assert torch.isfinite(res["o32"]).all() and torch.isfinite(res["lse32"]).all()
    heads = {(0, h): np.arange(256) for h in range(2)}
    refs = {bh: ref.naive_attention_head(si.bf16_bits_to_f64(q[bh]), si.bf16_bits_to_f64(k[bh]),
                                         si.bf16_bits_to_f64(v[bh]), scale, True)
            for bh in heads}
    o32 = res["o32"].cpu().numpy()
    l32 = res["lse32"].cpu().numpy()
    for bh in heads:
        assert np.max(np.abs(o32[bh] - refs[bh][0])) <= O_TOL
        # |LSE| reaches several hundred here: the gate is absolute per row, LSE_TOL plus the fp32
        # rounding of scores of that size (lse_row_tolerance)
        tol = lse_row_tolerance(si.bf16_bits_to_f64(q[bh]), si.bf16_bits_to_f64(k[bh]), scale,
                                True, refs[bh][1])
        err = np.abs(l32[bh] - refs[bh][1])
        log(f"[parity] large scores d={d} head {bh}: max|LSE|={np.max(np.abs(refs[bh][1])):.1f} "
            f"max|dLSE|={np.max(err):.3e} max tol={np.max(tol):.3e} worst ratio "
            f"{np.max(err / tol):.3f}")
        assert np.all(err <= tol)


def test_run_to_run_bit_identical(gpu):
    wl, q, k, v = workload_inputs("causal_b8_h32_t1024_d64")
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    o1, l1 = gpu.fa_fwd(qg, kg, vg, causal=True, scale=wl.scale)
    o2, l2 = gpu.fa_fwd(qg, kg, vg, causal=True, scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_explicit_stream_and_preallocated_outputs(gpu):
    wl = si.custom_workload(1, 2, 129, 129, 128, True)
    q, k, v = si.make_inputs(wl, seed=15, threads=2)
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    s = torch.cuda.Stream()
    o = torch.empty_like(qg)
    lse = torch.empty((1, 2, 129), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        gpu.fa_fwd(qg, kg, vg, causal=True, scale=wl.scale, o=o, lse=lse, stream=s)
    s.synchronize()
    o_ref, l_ref = gpu.fa_fwd(qg, kg, vg, causal=True, scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, l_ref)


def test_rejected_call_leaves_device_outputs_untouched(gpu):
    qg = torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.full((1, 1, 16, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 1, 16), 7.0, device="cuda")
    kg = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu.FaError) as e:
        gpu.fa_fwd(qg, kg, kg, causal=True, scale=0.125, o=o, lse=lse)   # causal with Tq > Tk
    assert e.value.status == gpu.FA_ERR_CAUSAL_TQ_GT_TK
    torch.cuda.synchronize()
    assert torch.all(o == 3.0) and torch.all(lse == 7.0)


@pytest.mark.parametrize("d,causal,scale", [(128, True, -0.0883883), (64, False, -0.3),
                                           (128, False, 0.0), (64, True, -2.5)])
def test_negative_and_zero_scales(gpu, d, causal, scale):
    """A negative scale is applied on chip by negating Q (exact); zero gives uniform attention."""
    wl = si.custom_workload(2, 3, 300, 300, d, causal)
    q, k, v = si.make_inputs(wl, seed=17, threads=4)
    res = run_fwd(gpu, q, k, v, causal, scale)
    assert_bf16_is_rne_of_f32(res)
    heads = {(b, hh): np.arange(300) for b in range(2) for hh in range(3)}
    refs = {bh: ref.naive_attention_head(si.bf16_bits_to_f64(q[bh]), si.bf16_bits_to_f64(k[bh]),
                                         si.bf16_bits_to_f64(v[bh]), scale, causal)
            for bh in heads}
    o32 = res["o32"].cpu().numpy()
    l32 = res["lse32"].cpu().numpy()
    for bh in heads:
        d_o = float(np.max(np.abs(o32[bh] - refs[bh][0])))
        d_l = float(np.max(np.abs(l32[bh] - refs[bh][1])))
        assert d_o <= O_TOL and d_l <= LSE_TOL, (bh, d_o, d_l)
    log(f"[parity] scale={scale} d={d} causal={causal}: ok")
