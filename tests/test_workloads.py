"""The seeded input generator: determinism per row, bf16 rounding against
torch's own conversion, and the distribution each workload asks for."""
import numpy as np
import pytest
import torch

import workloads


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0]
    ours = workloads.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    np.testing.assert_array_equal(workloads.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_rows_are_deterministic_and_independent():
    w = workloads.WORKLOADS["tiny"]
    a = workloads.kv_row(w, 0, 1, workloads.TENSOR_K, 0)
    b = workloads.kv_row(w, 0, 1, workloads.TENSOR_K, 0)
    np.testing.assert_array_equal(a, b)
    c = workloads.kv_row(w, 0, 0, workloads.TENSOR_K, 0)
    assert not np.array_equal(a, c)
    full = workloads.kv_tensors(w, workloads.TENSOR_K)
    for loop in range(w.n_loops):
        np.testing.assert_array_equal(full[loop][0, 1], workloads.kv_row(w, 0, 1, workloads.TENSOR_K, loop))
    assert np.array_equal(full[-1], workloads.ref_tensor(w, workloads.TENSOR_K))


@pytest.mark.parametrize("name", ["tiny", "l4_b16_s4k", "heavy_tail"])
def test_residual_std_per_loop(name):
    w = workloads.WORKLOADS[name].with_batch(1).with_seq(512)
    xs = workloads.kv_rows_all_loops(w, 0, 0, workloads.TENSOR_V if name != "heavy_tail" else workloads.TENSOR_K)
    ref = workloads.bf16_bits_to_f32(xs[-1]).astype(np.float64)
    for loop in range(w.n_loops - 1):
        r = workloads.bf16_bits_to_f32(xs[loop]) - ref
        if name == "heavy_tail":
            r = np.delete(r, workloads.heavy_channels(w), axis=1)
        assert abs(r.std() / w.sigma[loop] - 1.0) < 0.05


def test_heavy_tail_channels_and_t4_values():
    w = workloads.WORKLOADS["heavy_tail"].with_batch(1).with_seq(2048)
    ch = workloads.heavy_channels(w)
    assert len(ch) == 4 and len(set(ch.tolist())) == 4
    k = workloads.bf16_bits_to_f32(workloads.kv_row(w, 0, 0, workloads.TENSOR_K, 3)).astype(np.float64)
    others = np.delete(k, ch, axis=1)
    assert abs(k[:, ch].std() / others.std() - 20.0) < 1.5
    v = workloads.bf16_bits_to_f32(workloads.kv_row(w, 0, 0, workloads.TENSOR_V, 3)).astype(np.float64)
    # Student-t with 4 dof: variance 2, excess kurtosis well above a Gaussian's
    assert 1.6 < v.var() < 2.6
    kurt = ((v - v.mean()) ** 4).mean() / v.var() ** 2
    assert kurt > 4.0


def test_peak_batch_sigma_is_geometric():
    s = workloads.WORKLOADS["peak_batch"].sigma
    assert s[-1] == 0.0
    np.testing.assert_allclose(s[6], 0.05)
    np.testing.assert_allclose(s[0], 0.2)
    ratios = np.array(s[:6]) / np.array(s[1:7])
    np.testing.assert_allclose(ratios, 4 ** (1 / 6))


def test_packed_rows():
    w = workloads.WORKLOADS["peak_batch"].with_batch(1).with_seq(64)
    words, scales = workloads.packed_row(w, 0, 0, 0, 0)
    assert words.shape == (64, 16) and words.dtype == np.uint32  # INT4 loop
    sv = scales.view(np.float16).astype(np.float64)
    assert sv.min() >= 0.2 * 0.0099 and sv.max() <= 0.2 * 0.1001  # INT4: 1.5 / 7.5 of INT2's range
    words1, s1 = workloads.packed_row(w, 0, 0, 0, 1)
    assert words1.shape == (64, 8)  # INT2 loop
    sv1 = s1.view(np.float16).astype(np.float64)
    assert sv1.min() >= 0.0099 and sv1.max() <= 0.1001


def test_peak_batch_bytes_per_sequence():
    """Per-sequence byte counts of the peak-batch workload (8 loops, 4 KV heads,
    head_dim 128, 16,384 positions): the residual cache (INT4 loop 0, INT2
    loops 1-6, the bf16 reference), the bf16 cache of every loop, and what an
    all-loop encode call holds on the device (all states plus its outputs).
    Counted by hand: 65,536 vectors per tensor and sequence; a vector costs
    256 B of bf16, 64 B of INT4 or 32 B of INT2 codes and 8 B of scales."""
    w = workloads.WORKLOADS["peak_batch"].with_batch(workloads.PEAK_TILE)
    vec = 2 * 4 * 16384  # K and V
    residual = vec * (64 + 8 + 6 * (32 + 8))
    assert workloads.cache_bytes_per_sequence(w, w.bits, with_reference=False) == residual == 40_894_464
    assert workloads.cache_bytes_per_sequence(w, w.bits) == residual + vec * 256 == 74_448_896
    assert workloads.bf16_cache_bytes_per_sequence(w, w.n_loops) == 8 * vec * 256 == 268_435_456
    assert workloads.encode_bytes_per_sequence(w) == 268_435_456 + 40_894_464
    # batches that fit 200 GB, rounded down to a multiple of the eight drawn entries
    assert workloads.peak_batch(74_448_896) == 2680
    assert workloads.peak_batch(268_435_456) == 744
    assert workloads.peak_batch(268_435_456 + 40_894_464) == 640
