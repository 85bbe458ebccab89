"""GPU parity of the forward's head-dimension and layout variants against the fp64 oracle.

Head dimensions that are multiples of 8 up to 128 run the 64- or 128-wide kernel with zero
padding on chip; strided tensors (e.g. [B][T][h][d], or rows with gaps) go through
fa_fwd_strided.  The oracle sees each head as a plain [T][d] array.  Gates as in the forward
tests: max|dO| <= 1e-2 on the fp32 output and max|dLSE| <= 1e-3; strided outputs are bf16 and
are allowed their rounding on top.  Columns outside a strided output's rows must stay untouched.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import attention_ref as ref
from tests.gpu_support import LSE_TOL, O_TOL, log, to_gpu

pytestmark = pytest.mark.gpu


def _oracle(q, k, v, b, h, scale, causal):
    return ref.naive_attention_head(si.bf16_bits_to_f64(q[b, h]), si.bf16_bits_to_f64(k[b, h]),
                                    si.bf16_bits_to_f64(v[b, h]), scale, causal)


@pytest.mark.parametrize("d", [8, 16, 24, 32, 48, 72, 80, 96, 112])
@pytest.mark.parametrize("causal", [False, True])
def test_padded_head_dims(gpu, d, causal):
    wl = si.custom_workload(1, 2, 200, 333 if not causal else 200, d, causal)
    log(f"[case] head dim d={d} causal={causal}")
    q, k, v = si.make_inputs(wl, seed=11)
    o, lse = gpu.fa_fwd_o32(to_gpu(q), to_gpu(k), to_gpu(v), causal=causal, scale=wl.scale)
    o16, lse16 = gpu.fa_fwd(to_gpu(q), to_gpu(k), to_gpu(v), causal=causal, scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o16.view(torch.int16), o.to(torch.bfloat16).view(torch.int16))
    for h in range(2):
        Or, Lr = _oracle(q, k, v, 0, h, wl.scale, causal)
        do = float(np.max(np.abs(o[0, h].cpu().numpy() - Or)))
        dl = float(np.max(np.abs(lse[0, h].cpu().numpy() - Lr)))
        log(f"[parity] d={d} causal={causal} head {h}: max|dO|={do:.2e} max|dLSE|={dl:.2e}")
        assert do <= O_TOL and dl <= LSE_TOL


def _bthd(bits):
    """[B][h][T][d] bf16 bits -> a [B][h][T][d] view of a [B][T][h][d] GPU tensor."""
    return to_gpu(np.ascontiguousarray(bits.transpose(0, 2, 1, 3))).transpose(1, 2)


def _padded_rows(bits, extra):
    """[B][h][T][d] -> a view of a [B][h][T][d + extra] GPU tensor (gaps between rows)."""
    B, H, T, d = bits.shape
    buf = np.zeros((B, H, T, d + extra), dtype=np.uint16)
    buf[..., :d] = bits
    return to_gpu(buf)[..., :d]


def _check_strided(tag, o, lse, q, k, v, wl, heads):
    for (b, h) in heads:
        Or, Lr = _oracle(q, k, v, b, h, wl.scale, wl.causal)
        og = o[b, h].float().cpu().numpy()
        do = float(np.max(np.abs(og - Or)))
        dl = float(np.max(np.abs(lse[b, h].cpu().numpy() - Lr)))
        bound = O_TOL + 2.0 ** -8 * (np.abs(Or) + O_TOL)
        log(f"[parity] {tag} head {(b, h)}: max|dO|={do:.2e} max|dLSE|={dl:.2e}")
        assert np.all(np.abs(og - Or) <= bound), f"{tag}: bf16 output beyond its bound"
        assert dl <= LSE_TOL


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bthd_layout(gpu, d, causal):
    wl = si.custom_workload(2, 3, 150, 150 if causal else 257, d, causal)
    log(f"[case] [B][T][h][d] layout d={d} causal={causal}")
    q, k, v = si.make_inputs(wl, seed=12)
    o_buf = torch.full((2, wl.Tq, 3, d), 7.0, dtype=torch.bfloat16, device="cuda")
    o_view = o_buf.transpose(1, 2)
    o, lse = gpu.fa_fwd_strided(_bthd(q), _bthd(k), _bthd(v), causal=causal, scale=wl.scale,
                                o=o_view)
    torch.cuda.synchronize()
    assert o.data_ptr() == o_buf.data_ptr()
    _check_strided(f"bthd d={d}", o, lse, q, k, v, wl, [(b, h) for b in range(2) for h in range(3)])


def test_mixed_layouts_and_row_gaps(gpu):
    """q in [B][T][h][d], k with 24-element gaps after each row, v contiguous, o with gaps: the
    gap elements of o must stay untouched."""
    wl = si.custom_workload(2, 2, 133, 200, 80, True)
    log("[case] mixed layouts and row gaps, d=80")
    q, k, v = si.make_inputs(wl, seed=13)
    o_buf = torch.full((2, 2, wl.Tq, 80 + 48), 3.0, dtype=torch.bfloat16, device="cuda")
    o, lse = gpu.fa_fwd_strided(_bthd(q), _padded_rows(k, 24), to_gpu(v), causal=True,
                                scale=wl.scale, o=o_buf[..., :80])
    torch.cuda.synchronize()
    assert bool((o_buf[..., 80:] == 3.0).all()), "the forward wrote outside its output rows"
    _check_strided("mixed d=80", o, lse, q, k, v, wl, [(b, h) for b in range(2) for h in range(2)])


@pytest.mark.parametrize("name,B,h,T,d", [("bthd_b8_h32_t4096_d128", 8, 32, 4096, 128),
                                           ("d80_b8_h20_t4096", 8, 20, 4096, 80)])
def test_layout_workloads_full_size(gpu, name, B, h, T, d):
    """The bench's layout workloads: the forward workload in [B][T][h][d], and the page's
    20 heads x 80 example, causal; the oracle on sampled heads and rows."""
    wl = si.custom_workload(B, h, T, T, d, True, name=name)
    log(f"[case] layout workload {name}")
    q, k, v = si.make_inputs(wl, seed=0)
    if d == 128:
        o, lse = gpu.fa_fwd_strided(_bthd(q), _bthd(k), _bthd(v), causal=True, scale=wl.scale)
    else:
        o, lse = gpu.fa_fwd(to_gpu(q), to_gpu(k), to_gpu(v), causal=True, scale=wl.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(51)
    for (b, hh) in [(0, 0), (B - 1, h - 1), (int(rng.integers(B)), int(rng.integers(h)))]:
        rows = np.unique(np.concatenate([[0, 1, 255, 256, T - 1], rng.choice(T, 40, replace=False)]))
        Or, Lr = ref.naive_attention_head(si.bf16_bits_to_f64(q[b, hh]), si.bf16_bits_to_f64(k[b, hh]),
                                          si.bf16_bits_to_f64(v[b, hh]), wl.scale, True, rows=rows)
        og = o[b, hh].float().cpu().numpy()[rows]
        bound = O_TOL + 2.0 ** -8 * (np.abs(Or) + O_TOL)
        assert np.all(np.abs(og - Or) <= bound), f"{name} head {(b, hh)}"
        assert float(np.max(np.abs(lse[b, hh].cpu().numpy()[rows] - Lr))) <= LSE_TOL
        log(f"[parity] {name} head {(b, hh)}: max|dO|={np.max(np.abs(og - Or)):.2e}")
