"""The comparison helpers that read the GPU's outputs (tests/rq_parity.py) are
test code of their own, so that no oracle function takes the GPU's output.
Here they are pinned to the oracle on host data."""
import numpy as np
import pytest

import oracle
import workloads
from rq_parity import host_f64, recon_error, unpack_words


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_unpack_words_inverts_the_oracle_packing(bits, d):
    rng = np.random.default_rng(bits * d)
    codes = rng.integers(0, 1 << bits, size=(3, 5, d))
    words = oracle.pack_codes(codes, bits)
    np.testing.assert_array_equal(unpack_words(words, bits), codes)
    np.testing.assert_array_equal(unpack_words(words, bits), oracle.unpack_codes(words, bits))


def test_recon_error_and_host_conversion_match_the_oracle():
    rng = np.random.default_rng(7)
    ref = workloads.f32_to_bf16_bits(rng.standard_normal((4, 64)).astype(np.float32))
    x = workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(ref) + 0.1 * rng.standard_normal((4, 64))).astype(np.float32))
    np.testing.assert_array_equal(host_f64(x), oracle.bf16_to_f64(x))
    xh = oracle.bf16_to_f64(x) + 0.01 * rng.standard_normal((4, 64))
    assert recon_error(xh, x, ref) == pytest.approx(oracle.reconstruction_error(xh, x, ref), rel=1e-12)
