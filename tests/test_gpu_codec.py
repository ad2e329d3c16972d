"""GPU parity of rq_encode and rq_reconstruct against the CPU oracle."""
import numpy as np
import pytest
import torch

import looped_transformer_kv_rq_amd as rq
import oracle
import workloads
from rq_parity import (RECON_TOL, compare_codes, recon_error, to_dev, to_host_u16, to_host_words)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _encode_gpu(xs_bits, ref_bits, bits):
    xs = [to_dev(x) for x in xs_bits]
    ref = to_dev(ref_bits)
    codes, scales = rq.encode(xs, ref, bits)
    torch.cuda.synchronize()
    return [to_host_words(c) for c in codes], [to_host_u16(s) for s in scales]


def _random_case(b, h, s, d, sigma=0.1, seed=0):
    rng = np.random.default_rng(seed)
    ref = workloads.f32_to_bf16_bits(rng.standard_normal((b, h, s, d)).astype(np.float32))
    x = workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(ref) + sigma * rng.standard_normal((b, h, s, d))).astype(np.float32))
    return x, ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("s", [1, 37, 300])
def test_encode_small_shapes(d, bits, s):
    print(f"encode d={d} bits={bits} s={s}", flush=True)
    x, ref = _random_case(2, 3, s, d, seed=s + d + bits)
    gw, gs = _encode_gpu([x], ref, [bits])
    ow, os_ = oracle.encode(x, ref, bits)
    compare_codes(gw[0], gs[0], ow, os_, x, ref, bits)


def test_encode_tiny_workload_all_loops_and_tensors():
    w = workloads.WORKLOADS["tiny"]
    for tensor in (workloads.TENSOR_K, workloads.TENSOR_V):
        xs = workloads.kv_tensors(w, tensor)
        bits = list(w.bits[:-1])
        gw, gs = _encode_gpu(xs[:-1], xs[-1], bits)
        for l, bl in enumerate(bits):
            ow, os_ = oracle.encode(xs[l], xs[-1], bl)
            compare_codes(gw[l], gs[l], ow, os_, xs[l], xs[-1], bl)


def test_encode_mixed_bits_in_one_call_equals_separate_calls():
    x0, ref = _random_case(1, 2, 129, 128, sigma=0.2, seed=1)
    x1, _ = _random_case(1, 2, 129, 128, sigma=0.05, seed=2)
    gw, gs = _encode_gpu([x0, x1, x0], ref, [4, 2, 2])
    a, sa = _encode_gpu([x0], ref, [4])
    b, sb = _encode_gpu([x1], ref, [2])
    np.testing.assert_array_equal(gw[0], a[0])
    np.testing.assert_array_equal(gs[0], sa[0])
    np.testing.assert_array_equal(gw[1], b[0])
    np.testing.assert_array_equal(gs[1], sb[0])
    ow, os_ = oracle.encode(x0, ref, 2)
    compare_codes(gw[2], gs[2], ow, os_, x0, ref, 2)


@pytest.mark.parametrize("bits", [2, 4])
def test_encode_zero_residual_and_zero_groups(bits):
    rng = np.random.default_rng(3)
    ref = workloads.f32_to_bf16_bits(rng.standard_normal((1, 1, 8, 64)).astype(np.float32))
    x = ref.copy()
    # vector 1: residual H e_32 (+-1/8): rotated group 0 exactly zero, group 1 nonzero
    r = np.where(np.arange(64) < 32, 0.125, -0.125).astype(np.float32)
    x[0, 0, 1] = workloads.f32_to_bf16_bits(np.zeros(64, np.float32) + r)
    ref[0, 0, 1] = 0
    gw, gs = _encode_gpu([x], ref, [bits])
    ow, os_ = oracle.encode(x, ref, bits)
    np.testing.assert_array_equal(gw[0], ow)
    np.testing.assert_array_equal(gs[0], os_)
    zero_word = 0xAAAAAAAA if bits == 2 else 0x88888888
    assert np.all(gw[0][0, 0, 0] == zero_word) and np.all(gs[0][0, 0, 0] == 0)


def test_encode_scale_saturates():
    ref = np.zeros((1, 1, 2, 64), dtype=np.uint16)
    x = workloads.f32_to_bf16_bits(np.full((1, 1, 2, 64), 3.0e5, dtype=np.float32))
    gw, gs = _encode_gpu([x], ref, [2])
    ow, os_ = oracle.encode(x, ref, 2)
    np.testing.assert_array_equal(gs[0], os_)
    assert np.all(os_[..., 0] == 0x7BFF)


def test_encode_deterministic_and_overwrites_sentinels():
    x, ref = _random_case(2, 2, 257, 128, seed=9)
    xs, r = [to_dev(x)], to_dev(ref)
    codes = [torch.full((2, 2, 257, 8), -1, dtype=torch.int32, device=DEV)]
    scales = [torch.full((2, 2, 257, 4), float("nan"), dtype=torch.float16, device=DEV)]
    rq.encode_into(xs, r, [2], codes, scales)
    c2, s2 = rq.encode(xs, r, [2])
    torch.cuda.synchronize()
    assert torch.equal(codes[0], c2[0]) and torch.equal(scales[0].view(torch.int16), s2[0].view(torch.int16))
    assert not torch.isnan(scales[0]).any()


@pytest.mark.parametrize("name,rows", [("l4_b16_s4k", [(0, 0), (15, 7), (7, 3)]),
                                       ("heavy_tail", [(0, 0), (31, 5)]),
                                       ("mixed_s32k", [(3, 2)]),
                                       ("peak_batch", [(0, 0), (3, 3)])])
def test_encode_full_size_sampled_rows(name, rows):
    """The launch configuration the benchmark times, checked on sampled rows."""
    w = workloads.WORKLOADS[name]
    if name == "peak_batch":
        w = w.with_batch(4)
    print(f"encode full {name} rows={rows}", flush=True)
    for tensor in (workloads.TENSOR_K, workloads.TENSOR_V):
        xs = workloads.kv_tensors(w, tensor)
        bits = list(w.bits[:-1])
        xd = [to_dev(x) for x in xs]
        del xs
        codes, scales = rq.encode(xd[:-1], xd[-1], bits)
        torch.cuda.synchronize()
        for (b, h) in rows:
            rows_bits = workloads.kv_rows_all_loops(w, b, h, tensor)
            for l, bl in enumerate(bits):
                ow, os_ = oracle.encode(rows_bits[l], rows_bits[-1], bl)
                gw = to_host_words(codes[l][b, h])
                gs = to_host_u16(scales[l][b, h])
                compare_codes(gw, gs, ow, os_, rows_bits[l], rows_bits[-1], bl)
        del xd, codes, scales
        torch.cuda.empty_cache()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [0, 2, 3, 4, 8])
def test_reconstruct_matches_oracle_on_oracle_codes(d, bits):
    x, ref = _random_case(2, 2, 70, d, sigma=0.2, seed=bits + d)
    if bits:
        ow, os_ = oracle.encode(x, ref, bits)
        codes = torch.from_numpy(ow.view(np.int32)).to(DEV)
        scales = to_dev(os_, torch.float16)
    else:
        ow = os_ = codes = scales = None
    expect = oracle.reconstruct(ref, ow, os_, bits)
    got = rq.reconstruct(to_dev(ref), codes, scales, bits).cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, expect, rtol=0, atol=2e-6 * max(1.0, np.abs(expect).max()))
    gotb = to_host_u16(rq.reconstruct(to_dev(ref), codes, scales, bits, out_dtype=torch.bfloat16))
    expb = oracle.f64_to_bf16(expect)
    # bf16 rounding of an fp32 value vs of the fp64 value: equal or one bf16 ulp apart at a tie
    assert np.all(np.abs(gotb.astype(np.int32) - expb.astype(np.int32)) <= 1)
    assert np.mean(gotb == expb) > 0.999


@pytest.mark.parametrize("name", ["tiny", "heavy_tail"])
def test_reconstruction_error_end_to_end(name):
    w = workloads.WORKLOADS[name]
    if name == "heavy_tail":
        w = w.with_batch(2).with_seq(1024)
    for tensor in (workloads.TENSOR_K, workloads.TENSOR_V):
        xs = workloads.kv_tensors(w, tensor)
        bits = list(w.bits[:-1])
        xd = [to_dev(x) for x in xs]
        codes, scales = rq.encode(xd[:-1], xd[-1], bits)
        for l, bl in enumerate(bits):
            xh = rq.reconstruct(xd[-1], codes[l], scales[l], bl).cpu().numpy().astype(np.float64)
            e_gpu = recon_error(xh, xs[l], xs[-1])
            ow, os_ = oracle.encode(xs[l], xs[-1], bl)
            e_orc = oracle.reconstruction_error(oracle.reconstruct(xs[-1], ow, os_, bl), xs[l], xs[-1])
            assert abs(e_gpu - e_orc) <= RECON_TOL, (name, tensor, l, e_gpu, e_orc)
            assert e_gpu < (0.5 if bl == 2 else 0.15)
