"""GPU parity of the rotation-only baseline (rq_encode_rotonly /
rq_reconstruct_rotonly): the codec with an all-zero reference, against the
oracle's encode and reconstruct with a zero reference."""
import numpy as np
import pytest
import torch

import looped_transformer_kv_rq_amd as rq
import oracle
import workloads
from rq_parity import compare_codes, host_f64, to_dev, to_host_u16, to_host_words

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _states(b, h, s, d, n, seed):
    rng = np.random.default_rng(seed)
    return [workloads.f32_to_bf16_bits(rng.standard_normal((b, h, s, d)).astype(np.float32)) for _ in range(n)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("s", [1, 45, 300])
def test_rotonly_encode_matches_oracle_with_zero_reference(d, s):
    print(f"rotonly encode d={d} s={s}", flush=True)
    bits = [2, 4, 2]
    xs = _states(2, 3, s, d, len(bits), seed=d + s)
    zero = np.zeros_like(xs[0])
    codes, scales = rq.encode_rotonly([to_dev(x) for x in xs], bits)
    torch.cuda.synchronize()
    for x, c, sc, bl in zip(xs, codes, scales, bits):
        ow, os_ = oracle.encode(x, zero, bl)
        compare_codes(to_host_words(c), to_host_u16(sc), ow, os_, x, zero, bl)


def test_rotonly_equals_encode_against_zero_reference():
    xs = _states(1, 2, 130, 128, 2, seed=9)
    xd = [to_dev(x) for x in xs]
    c1, s1 = rq.encode_rotonly(xd, [2, 4])
    c2, s2 = rq.encode(xd, torch.zeros_like(xd[0]), [2, 4])
    for a, b in zip(c1, c2):
        assert torch.equal(a, b)
    for a, b in zip(s1, s2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_rotonly_reconstruct_matches_oracle(d, bits):
    x = _states(2, 2, 70, d, 1, seed=3 * d + bits)[0]
    zero = np.zeros_like(x)
    ow, os_ = oracle.encode(x, zero, bits)
    codes = torch.from_numpy(ow.view(np.int32)).to(DEV)
    scales = to_dev(os_, torch.float16)
    expect = oracle.reconstruct(zero, ow, os_, bits)
    got = rq.reconstruct_rotonly(codes, scales, bits).cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, expect, rtol=0, atol=2e-6 * max(1.0, np.abs(expect).max()))
    # bf16 output: the RNE rounding of the fp32 value, within one bf16 ulp of the
    # oracle's rounding (values near zero may round across it, so compare values)
    gotb = host_f64(to_host_u16(rq.reconstruct_rotonly(codes, scales, bits, out_dtype=torch.bfloat16)))
    expb = oracle.bf16_to_f64(oracle.f64_to_bf16(expect))
    tol = 2.0 ** -7 * np.abs(expect) + 2e-6 * max(1.0, np.abs(expect).max())  # one bf16 ulp
    assert np.all(np.abs(gotb - expb) <= tol)


def test_rotonly_full_size_sampled_rows():
    """The launch the benchmark's rotation-only leg times (all 4 loops of l4_b16_s4k's K)."""
    w = workloads.WORKLOADS["l4_b16_s4k"]
    xs = workloads.kv_tensors(w, workloads.TENSOR_K)
    bits = [2] * w.n_loops
    codes, scales = rq.encode_rotonly([to_dev(x) for x in xs], bits)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (15, 7)]:
        rows = workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_K)
        zero = np.zeros_like(rows[0])
        for l in range(w.n_loops):
            ow, os_ = oracle.encode(rows[l], zero, 2)
            compare_codes(to_host_words(codes[l][b, h]), to_host_u16(scales[l][b, h]), ow, os_, rows[l], zero, 2)
