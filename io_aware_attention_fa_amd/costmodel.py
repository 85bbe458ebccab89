"""Work and traffic accounting for the attention forward and split-KV decode, plus MI355X peaks.

Pure host arithmetic (no GPU, no oracle).  The benchmark uses it to turn measured times into
TFLOP/s, GB/s and roofline fractions; the tests pin it to the byte and FLOP figures the pages print.
"""
from __future__ import annotations

import math

# MI355X published peaks (dense, no structured sparsity) and unit counts.
MI355X_PEAK_BF16_DENSE_FLOPS = 2.5e15
MI355X_PEAK_HBM_BYTES_PER_S = 8.0e12
MI355X_COMPUTE_UNITS = 256
MI355X_XCDS = 8
MI355X_PEAK_SCLK_HZ = 2.4e9
MI355X_LDS_BYTES_PER_CU = 160 * 1024
# 256 CUs x 4 SIMDs x 1024 bf16 FLOP/clk (one 32x32x16 MFMA per 32 cycles) x 2.4 GHz.
MI355X_BF16_FLOPS_PER_CLK_PER_CU = 4096


def bf16_peak_at_clock(sclk_hz: float, cus: int = MI355X_COMPUTE_UNITS) -> float:
    """Dense bf16 MFMA peak at a given engine clock and CU count."""
    return cus * MI355X_BF16_FLOPS_PER_CLK_PER_CU * sclk_hz


def attention_flops(B, h, Tq, Tk, d, causal) -> float:
    """Algorithmic FLOPs of the forward: 4*B*h*Tq*Tk*d (two contractions), halved for causal.

    Two dense contractions per (query, key) pair, S = Q K^T and O += P V, each 2*d FLOPs (page
    "Chapter 10 Writing and Benchmarking Custom Kernels", §10.3.1: attention compute is the
    tile matmuls).  Causal keeps about half of the pairs.
    """
    f = 4.0 * B * h * Tq * Tk * d
    return f / 2.0 if causal else f


def attention_io_bytes(B, h, Tq, Tk, d, elem_bytes=2, lse_bytes=4) -> float:
    """Q, K, V read once, O and LSE written once: the IO-aware lower bound.

    Page "Fusion and IO-aware kernels", "Code": the IO-aware count reads Q, K, V and writes O once
    and calls itself a lower bound; the LSE (one fp32 per query row) is the forward's other output.
    """
    return (elem_bytes * B * h * d * (2 * Tq + 2 * Tk)) + lse_bytes * B * h * Tq


def attention_bwd_flops(B, h, Tq, Tk, d, causal) -> float:
    """Algorithmic FLOPs of the backward: five contractions per (query, key) pair, 2*d each.

    Page "Chapter 10 Writing and Benchmarking Custom Kernels", §10.3.2: the backward recomputes
    S = Q K^T and forms dP = dO V^T, dV = P^T dO, dK = dS^T Q and dQ = dS K, so it costs 2.5x the
    forward's two contractions; causal keeps about half of the pairs.
    """
    return 2.5 * attention_flops(B, h, Tq, Tk, d, causal)


def attention_bwd_executed_flops(B, h, Tq, Tk, d, causal) -> float:
    """MFMA FLOPs the two gradient kernels issue: S and dP are formed in both the key-block
    (dK, dV) and the query-block (dQ) kernel, so seven contractions instead of five."""
    return 3.5 * attention_flops(B, h, Tq, Tk, d, causal)


def attention_bwd_io_bytes(B, h, Tq, Tk, d, elem_bytes=2, lse_bytes=4) -> float:
    """Backward lower bound: Q, O, dO and K, V read once, LSE read once, dQ, dK, dV written once."""
    return elem_bytes * B * h * d * (4 * Tq + 4 * Tk) + lse_bytes * B * h * Tq


def decode_kv_bytes_per_token(d, elem_bytes=2) -> int:
    """K + V bytes of one cached token of one head: 2 * d * elem."""
    return 2 * d * elem_bytes


def decode_io_bytes(B, h, Tk, d, elem_bytes=2, lse_bytes=4) -> float:
    """Decode lower bound: the whole KV cache once, plus q read and o / LSE written."""
    return (B * h * Tk * decode_kv_bytes_per_token(d, elem_bytes)
            + elem_bytes * B * h * d * 2 + lse_bytes * B * h)


def decode_workspace_bytes(B, h, d, num_splits) -> int:
    """Bytes of per-chunk partials (m, l, o[d]) in fp32, written once and read once."""
    return 4 * B * h * num_splits * (d + 2)


# --- the pages' own accounting ------------------------------------------------------------------

def elementwise_chain_bytes(n, ops, elem_bytes=2):
    """(unfused, fused) HBM bytes of a chain of ``ops`` elementwise ops on n elements.

    Page "Fusion and IO-aware kernels", "Code": unfused, each op reads and writes the tensor;
    fused, it is read once and written once.
    """
    return ops * 2 * n * elem_bytes, 2 * n * elem_bytes


def standard_attention_bytes(seq, d, heads, batch, elem_bytes=2) -> int:
    """Q, K, V, O once plus four passes over the seq x seq score matrix (write S, read S,
    write P, read P), per the same program on page "Fusion and IO-aware kernels"."""
    bh = batch * heads
    return 4 * seq * d * elem_bytes * bh + 4 * seq * seq * elem_bytes * bh


def io_aware_attention_bytes(seq, d, heads, batch, elem_bytes=2) -> int:
    """Q, K, V, O once (the same program's IO-aware lower bound)."""
    return 4 * seq * d * elem_bytes * batch * heads


def io_aware_attention_bytes_with_rereads(seq, d, heads, batch, q_block, elem_bytes=2) -> int:
    """Q and O once, K and V once per query block of ``q_block`` rows (page "Fusion and IO-aware
    kernels", "Try it", exercise 1)."""
    bh = batch * heads
    n_blocks = math.ceil(seq / q_block)
    return (2 + 2 * n_blocks) * seq * d * elem_bytes * bh


def naive_score_bytes(B, h, T, elem_bytes=2) -> int:
    """One (B, h, T, T) score tensor (page "Kernels — fusion and FlashAttention", §2)."""
    return B * h * T * T * elem_bytes


def naive_oom_context(hbm_bytes, B, h, elem_bytes=2) -> float:
    """Context length at which one naive score tensor fills ``hbm_bytes``."""
    return math.sqrt(hbm_bytes / (B * h * elem_bytes))


def flash_tile_sram_bytes(Br, Bc, d, elem_bytes=2, stat_bytes=4) -> dict:
    """On-chip footprint of one FlashAttention tile set: Q, K, V, S, O tiles and m, l.

    Page "Chapter 10 ...", §10.3.1 "A Worked Example": Q, K, V and O tiles of (B x d) elements, a
    Br x Bc score tile and two per-row statistics.
    """
    t = {
        "Q": Br * d * elem_bytes,
        "K": Bc * d * elem_bytes,
        "V": Bc * d * elem_bytes,
        "S": Br * Bc * elem_bytes,
        "O": Br * d * elem_bytes,
        "stats": Br * stat_bytes * 2,
    }
    t["total"] = sum(t.values())
    return t


def naive_attention_bytes_per_head(N, d, elem_bytes=2) -> int:
    """Write S, read S, write P, read P, plus Q, K, V, O once (the same worked example)."""
    return 4 * N * N * elem_bytes + 4 * N * d * elem_bytes


def flash_attention_bytes_per_head(N, d, elem_bytes=2) -> int:
    """Q, K, V, O once (the same worked example)."""
    return 4 * N * d * elem_bytes


def backward_probability_bytes(N, H, layers, elem_bytes=2) -> int:
    """Storing P for the backward: N^2 per head per layer (page "Chapter 10 ...", §10.3.2)."""
    return N * N * H * layers * elem_bytes


def backward_lse_bytes(N, H, layers, lse_bytes=4) -> int:
    """Storing only L_i = m_i + log l_i in fp32 instead (same section)."""
    return N * H * layers * lse_bytes


def backward_recompute_flops(N, d, H) -> float:
    """Recomputing S = Q K^T for every tile of every head: 2 N^2 d H (same section)."""
    return 2.0 * N * N * d * H
