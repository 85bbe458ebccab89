"""Cost model pinned to the byte / FLOP figures the pages print (tests/golden/*.txt)."""
import math
import os

import pytest

from io_aware_attention_fa_amd import costmodel as cm

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _kv(name):
    out = {}
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            out[k] = float(v)
    return out


def _fusion_rows():
    rows = []
    for line in open(os.path.join(GOLD, "fusion_program_output.txt")):
        line = line.split("#")[0].strip()
        if line:
            rows.append(line.split())
    return rows


def test_fusion_program_chain_lines():
    hbm = 3.35e12
    n = 4096 * 8192
    chains = [r for r in _fusion_rows() if r[0] == "chain"]
    assert len(chains) == 2
    for kind, ops, unf, fus, unf_us, fus_us, ratio in chains:
        u, f = cm.elementwise_chain_bytes(n, int(ops))
        assert f"{u / 1e6:.0f}MB" == unf and f"{f / 1e6:.0f}MB" == fus
        assert f"{u / hbm * 1e6:.0f}" == unf_us and f"{f / hbm * 1e6:.0f}" == fus_us
        assert f"{u / f:.1f}" == ratio


def test_fusion_program_attention_lines():
    attn = [r for r in _fusion_rows() if r[0] == "attn"]
    assert len(attn) == 3
    for kind, seq, std, io, _, _, ratio in attn:
        seq = int(seq)
        s = cm.standard_attention_bytes(seq, 128, 32, 1)
        f = cm.io_aware_attention_bytes(seq, 128, 32, 1)
        assert f"{s / 1e9:.2f}GB" == std and f"{f / 1e9:.2f}GB" == io
        assert f"{s / f:.1f}" == ratio
        assert s / f == pytest.approx(1 + seq / 128)        # closed form: 1 + T / d


def test_rereads_make_the_io_aware_count_larger():
    lb = cm.io_aware_attention_bytes(16384, 128, 32, 1)
    rr = cm.io_aware_attention_bytes_with_rereads(16384, 128, 32, 1, q_block=128)
    assert rr == lb // 4 * (2 + 2 * 128)
    assert cm.standard_attention_bytes(16384, 128, 32, 1) / rr == pytest.approx(129 * 4 / 258)


def test_worked_example_tile_budget_and_traffic():
    g = _kv("worked_example_tiles.txt")
    t = cm.flash_tile_sram_bytes(64, 64, 128)
    for name in "QKVSO":
        assert t[name] / 1024 == g[f"tile_{name}_KiB"]
    assert t["stats"] / 1024 == g["stats_KiB"]
    assert abs(t["total"] / 1024 - g["total_KiB_approx"]) <= 1.0
    naive = cm.naive_attention_bytes_per_head(4096, 128)
    flash = cm.flash_attention_bytes_per_head(4096, 128)
    assert naive / 2**20 == g["naive_per_head_MiB"]
    assert flash / 2**20 == g["flash_per_head_MiB"]
    assert 32 * flash / 2**20 == g["flash_all_heads_MiB"]
    assert round(naive / flash) == g["reduction_x"]
    assert abs(32 * naive / 2**30 - g["naive_all_heads_GB_approx"]) <= 0.15
    hbm = g["hbm_bytes_per_s"]
    assert abs(32 * naive / hbm * 1e3 - g["naive_ms_approx"]) <= 0.1
    assert abs(32 * flash / hbm * 1e3 - g["flash_ms_approx"]) <= 0.005


def test_lesson_numbers():
    g = _kv("lesson_numbers.txt")
    act = 8 * 4096 * 4096 * 2
    assert round(act / 1e6) == g["activation_MB"]
    assert round(act / g["hbm_bytes_per_s"] * 1e6) == g["read_us"]
    assert abs(2 * act / g["hbm_bytes_per_s"] * 1e6 - g["read_write_us"]) <= 1.0
    T = cm.naive_oom_context(g["oom_hbm_bytes"], 8, 32)
    assert abs(T - g["oom_context_approx"]) <= 1000
    assert cm.naive_score_bytes(8, 32, int(T)) <= g["oom_hbm_bytes"]
    P = cm.backward_probability_bytes(4096, 32, 32)
    L = cm.backward_lse_bytes(4096, 32, 32)
    assert round(P / 1e9) == g["P_storage_GB_approx"]
    assert round(L / 2**20) == g["lse_storage_MB_approx"]
    assert abs(P / L - g["storage_reduction_x_approx"]) <= 100
    f = cm.backward_recompute_flops(4096, 128, 32)
    assert round(f / 1e9) == g["recompute_GFLOP"]
    assert round(f / g["quoted_bf16_flops"] * 1e3, 2) == g["recompute_ms_approx"]
    assert round(P / 32 / 3.35e12 * 1e3, 2) == g["saved_hbm_ms_approx"]


def test_prefill_and_decode_workload_formulas():
    f = cm.attention_flops(8, 32, 4096, 4096, 128, causal=True)
    assert f == pytest.approx(1.0995e12, rel=1e-4)
    assert cm.attention_io_bytes(8, 32, 4096, 4096, 128) == pytest.approx(1.078e9, rel=1e-3)
    assert cm.attention_flops(1, 2, 128, 128, 64, causal=False) == pytest.approx(8.39e6, rel=1e-3)
    kv = 64 * 32 * 8192 * cm.decode_kv_bytes_per_token(128)
    assert kv == pytest.approx(8.59e9, rel=1e-3)
    assert cm.decode_io_bytes(64, 32, 8192, 128) > kv
    assert cm.bf16_peak_at_clock(2.4e9) == pytest.approx(2.5166e15, rel=1e-4)
    assert cm.MI355X_PEAK_BF16_DENSE_FLOPS / cm.MI355X_PEAK_HBM_BYTES_PER_S == pytest.approx(312.5)
    assert math.isclose(cm.decode_workspace_bytes(64, 32, 128, 16), 64 * 32 * 16 * 130 * 4)


def test_backward_flops_and_bytes():
    f = cm.attention_flops(8, 32, 4096, 4096, 128, True)
    assert cm.attention_bwd_flops(8, 32, 4096, 4096, 128, True) == 2.5 * f
    assert cm.attention_bwd_executed_flops(8, 32, 4096, 4096, 128, True) == 3.5 * f
    # five contractions of 2*d FLOPs per pair, all pairs when not causal
    assert cm.attention_bwd_flops(1, 1, 3, 5, 8, False) == 5 * 2 * 8 * 3 * 5
    # Q, O, dO, dQ (Tq rows) and K, V, dK, dV (Tk rows) of d bf16, plus the fp32 LSE
    assert cm.attention_bwd_io_bytes(1, 1, 3, 5, 8) == 2 * 8 * (4 * 3 + 4 * 5) + 4 * 3
