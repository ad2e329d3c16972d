"""Pins for packing, encode and reconstruction: hand-derived closed forms in
tests/golden/closed_forms.json, exact reconstruction of a zero residual, and
the orthogonality identity |x_hat - x| = |s q - y|."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads


@pytest.fixture(scope="module")
def golden(golden_dir):
    with open(os.path.join(golden_dir, "closed_forms.json")) as f:
        return json.load(f)


def test_packing_worked_words(golden):
    p = golden["packing"]
    c2 = np.tile([0, 1, 2, 3], 4)[None]
    assert oracle.pack_codes(c2, 2)[0, 0] == p["int2_0123"]
    assert oracle.pack_codes(np.arange(8)[None], 4)[0, 0] == p["int4_01234567"]
    assert oracle.pack_codes(np.full((1, 16), 2), 2)[0, 0] == p["int2_zero_group"]
    assert oracle.pack_codes(np.full((1, 8), 8), 4)[0, 0] == p["int4_zero_group"]
    assert oracle.pack_codes(np.arange(4)[None], 8)[0, 0] == p["int8_0123"]
    np.testing.assert_array_equal(oracle.pack_codes((np.arange(32) % 8)[None], 3)[0], p["int3_mod8"])


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_round_trip(bits):
    c = np.random.default_rng(2).integers(0, 2 ** bits, size=(10, 128))
    w = oracle.pack_codes(c, bits)
    assert w.shape == (10, 128 * bits // 32) and w.dtype == np.uint32
    np.testing.assert_array_equal(oracle.unpack_codes(w, bits), c)


def _x_bits(case):
    d = case["head_dim"]
    x = np.zeros(d, dtype=np.uint16)
    if "x_nonzero" in case:
        for k, v in case["x_nonzero"].items():
            x[int(k)] = v
    elif case["x_pattern"] == "plus_eighth_then_minus_eighth":
        x[: d // 2] = 0x3E00   # +0.125
        x[d // 2:] = 0xBE00    # -0.125
    elif case["x_pattern"] == "minus_eighth_then_plus_eighth":
        x[: d // 2] = 0xBE00
        x[d // 2:] = 0x3E00
    return x


def test_golden_closed_forms(golden):
    for case in golden["cases"]:
        d, bits = case["head_dim"], case["bits"]
        x = _x_bits(case)[None]
        ref = np.zeros_like(x)
        words, scales = oracle.encode(x, ref, bits)
        np.testing.assert_array_equal(words[0], np.array(case["words"], dtype=np.uint32), err_msg=case["name"])
        np.testing.assert_array_equal(scales[0], np.array(case["scale_bits"], dtype=np.uint16), err_msg=case["name"])
        xh = oracle.reconstruct(ref, words, scales, bits)[0]
        if "x_hat_nonzero" in case:
            expect = np.zeros(d)
            for k, v in case["x_hat_nonzero"].items():
                expect[int(k)] = v
            np.testing.assert_allclose(xh, expect, atol=1e-14, err_msg=case["name"])
        else:
            # one nonzero rotated coordinate (peak_y) in group 1, group 0 all zero
            e = case["sq_error"]
            s16 = oracle.f16_to_f64(np.array(case["scale_bits"][1:2], dtype=np.uint16))[0]
            err2 = (e["peak_level"] * s16 - e["peak_y"]) ** 2 + e["rest_count"] * (e["rest_level"] * s16) ** 2
            got = np.sum((xh - oracle.bf16_to_f64(x[0])) ** 2)
            assert abs(got - err2) < 1e-13


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_zero_residual_reconstructs_exactly(bits, d):
    ref = workloads.f32_to_bf16_bits(np.random.default_rng(5).standard_normal((20, d)).astype(np.float32))
    words, scales = oracle.encode(ref, ref, bits)
    # every code is 2^(b-1): 0b10, 0b1000, 0x80; INT3 0b100 = low plane 0, bit 2 set
    if bits == 3:
        assert np.all(words[:, : d // 16] == 0) and np.all(words[:, d // 16:] == 0xFFFFFFFF)
    else:
        assert np.all(words == {2: 0xAAAAAAAA, 4: 0x88888888, 8: 0x80808080}[bits])
    assert np.all(scales == 0)
    xh = oracle.reconstruct(ref, words, scales, bits)
    np.testing.assert_array_equal(xh, oracle.bf16_to_f64(ref))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_error_equals_rotated_domain_error(bits):
    """|x_hat - x| = |s16 q - y| because H is orthogonal; the error splits over groups."""
    rng = np.random.default_rng(11)
    ref = workloads.f32_to_bf16_bits(rng.standard_normal((30, 128)).astype(np.float32))
    x = workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(ref) + 0.1 * rng.standard_normal((30, 128))).astype(np.float32))
    words, scales = oracle.encode(x, ref, bits)
    xh = oracle.reconstruct(ref, words, scales, bits)
    y = oracle.rotate(oracle.bf16_to_f64(x) - oracle.bf16_to_f64(ref))
    z = oracle.dequantize(words, scales, bits, 128)
    np.testing.assert_allclose(np.linalg.norm(xh - oracle.bf16_to_f64(x), axis=1),
                               np.linalg.norm(z - y, axis=1), rtol=1e-12)


def test_quality_on_gaussian_residuals():
    """Self-consistency on iid Gaussian residuals: INT4 beats INT2, both far
    below the residual's own norm, and the LS fit beats the absmax step."""
    rng = np.random.default_rng(12)
    ref = workloads.f32_to_bf16_bits(rng.standard_normal((2000, 128)).astype(np.float32))
    x = workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(ref) + 0.2 * rng.standard_normal((2000, 128))).astype(np.float32))
    errs = {}
    for bits in (2, 4):
        w, s = oracle.encode(x, ref, bits)
        errs[bits] = oracle.reconstruction_error(oracle.reconstruct(ref, w, s, bits), x, ref)
    assert 0.35 < errs[2] < 0.45
    assert 0.06 < errs[4] < 0.12
    # absmax step alone (no LS refit) is worse
    y = oracle.rotate(oracle.bf16_to_f64(x) - oracle.bf16_to_f64(ref)).reshape(2000, 4, 32)
    codes, s0 = oracle.assign_codes(y, 2)
    e_abs = np.linalg.norm(y - s0[..., None] * (codes - 1.5)) / np.linalg.norm(y)
    assert e_abs > errs[2] + 0.02


def test_error_ordering_and_fine_grid_limit():
    """On iid Gaussian residuals the error falls with every added bit, and at
    INT8 it meets the fine-quantization limit: a uniform step D = m / 127.5
    leaves an error of variance D^2 / 12 per coordinate, so the relative error
    is sqrt(E[m^2] / (12 * 127.5^2)) with m the absmax of 32 unit Gaussians
    (estimated here by sampling, without the codec)."""
    rng = np.random.default_rng(13)
    ref = workloads.f32_to_bf16_bits(rng.standard_normal((1000, 128)).astype(np.float32))
    x = workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(ref) + 0.2 * rng.standard_normal((1000, 128))).astype(np.float32))
    y = oracle.rotate(oracle.bf16_to_f64(x) - oracle.bf16_to_f64(ref)).reshape(-1, 32)
    errs = {}
    for bits in (2, 3, 4, 8):
        w, s = oracle.encode(x, ref, bits)
        errs[bits] = oracle.reconstruction_error(oracle.reconstruct(ref, w, s, bits), x, ref)
    assert errs[2] > errs[3] > errs[4] > errs[8]
    m2 = np.mean(np.max(np.abs(y), axis=1) ** 2) / np.mean(y ** 2)
    limit = np.sqrt(m2 / (12 * 127.5 ** 2))
    assert abs(errs[8] / limit - 1.0) < 0.05, (errs[8], limit)


def test_rotation_spreads_outlier_channels():
    """On K with a few x20 channels the rotated INT2 residual is far more
    accurate than quantizing the unrotated residual."""
    w = workloads.WORKLOADS["heavy_tail"].with_batch(1).with_seq(256)
    xs = workloads.kv_rows_all_loops(w, 0, 0, workloads.TENSOR_K)
    x, ref = xs[0], xs[-1]
    words, scales = oracle.encode(x, ref, 2)
    e_rot = oracle.reconstruction_error(oracle.reconstruct(ref, words, scales, 2), x, ref)
    r = (oracle.bf16_to_f64(x) - oracle.bf16_to_f64(ref)).reshape(-1, 4, 32)
    codes, s = oracle.quantize_groups(r, 2)
    e_plain = np.linalg.norm(r - s[..., None] * (codes - 1.5)) / np.linalg.norm(r)
    assert e_rot < 0.5 * e_plain


def test_final_loop_is_the_reference():
    ref = np.array([[0x3F80, 0x4000]], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.reconstruct(ref, None, None, 0), [[1.0, 2.0]])


def test_rotation_only_baseline_is_the_zero_reference_case():
    """The rotation-only baseline quantizes H x itself. With a zero reference,
    encode's reconstruction error of x equals its rotated-domain error, and on
    loop states close to the final loop the residual codec is far more
    accurate at the same bit width (the ResidualQuant abstract's claim against
    the rotation-based baseline)."""
    rng = np.random.default_rng(7)
    ref = workloads.f32_to_bf16_bits(rng.standard_normal((200, 128)).astype(np.float32))
    x = workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(ref) +
                                    0.1 * rng.standard_normal((200, 128))).astype(np.float32))
    zero = np.zeros_like(ref)
    w0, s0 = oracle.encode(x, zero, 2)
    xh0 = oracle.reconstruct(zero, w0, s0, 2)
    y = oracle.rotate(oracle.bf16_to_f64(x))
    q = oracle.dequantize(w0, s0, 2, 128)
    np.testing.assert_allclose(np.linalg.norm(xh0 - oracle.bf16_to_f64(x)), np.linalg.norm(q - y), rtol=1e-10)
    w1, s1 = oracle.encode(x, ref, 2)
    xh1 = oracle.reconstruct(ref, w1, s1, 2)
    xf = oracle.bf16_to_f64(x)
    e_rot = np.linalg.norm(xh0 - xf) / np.linalg.norm(xf)
    e_res = np.linalg.norm(xh1 - xf) / np.linalg.norm(xf)
    assert e_res < 0.2 * e_rot
