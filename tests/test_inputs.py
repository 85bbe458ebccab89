"""The seeded input generator (CPU): rounding, reproducibility and the key-spike structure."""
import numpy as np
import torch

import seeded_inputs as si


def test_rne_matches_torch_bfloat16_conversion():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.005859375, -1.00390625, 0.0, -0.0], np.float32)])
    ours = si.rne_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bf16_roundtrip_exact():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(si.rne_bf16_bits(si.bf16_bits_to_f32(bits)), bits)


def test_full_tensor_equals_per_head_slices():
    wl = si.custom_workload(2, 3, 5, 9, 64, True)
    q, k, v = si.make_inputs(wl, seed=3, threads=2)
    for b in range(2):
        for h in range(3):
            hq, hk, hv = si.head_inputs(wl, 3, b, h)
            assert np.array_equal(q[b, h], hq) and np.array_equal(k[b, h], hk)
            assert np.array_equal(v[b, h], hv)
    q2, _, _ = si.make_inputs(wl, seed=3, threads=1)
    assert np.array_equal(q, q2)
    q3, _, _ = si.make_inputs(wl, seed=4, threads=1)
    assert not np.array_equal(q, q3)


def test_key_spikes_exact_power_of_two():
    wl = si.custom_workload(1, 1, 4, 5000, 64, True, key_spike_frac=0.01, key_spike_mult=8.0)
    _, k, _ = si.head_inputs(wl, 0, 0, 0)
    base = si.head_normal_bits(0, si.TENSOR_K, 0, 0, 5000, 64)
    rows = si.key_spike_rows(0, 0, 0, 5000, 0.01)
    assert 20 <= rows.sum() <= 80
    assert np.array_equal(si.bf16_bits_to_f32(k[rows]), si.bf16_bits_to_f32(base[rows]) * 8)
    assert np.array_equal(k[~rows], base[~rows])


def test_decode_query_shape():
    wl = si.custom_workload(2, 2, 1, 33, 128, False, decode=True, num_splits=4)
    q, k, v = si.make_inputs(wl, seed=0, threads=1)
    assert q.shape == (2, 2, 128) and k.shape == (2, 2, 33, 128)


def test_named_workloads():
    w = si.WORKLOADS["causal_b8_h32_t4096_d128"]
    assert (w.B, w.h, w.Tq, w.Tk, w.d, w.causal) == (8, 32, 4096, 4096, 128, True)
    assert w.scale == float(np.float32(1 / np.sqrt(128)))
