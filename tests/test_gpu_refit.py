"""GPU parity of rq_encode_refit (code / LS-scale alternation after the first
fit) against the oracle's encode with the same number of refits."""
import ctypes

import numpy as np
import pytest
import torch

import looped_transformer_kv_rq_amd as rq
import oracle
import workloads
from rq_parity import RECON_TOL, compare_codes_refit, recon_error, to_dev, to_host_u16, to_host_words

pytestmark = pytest.mark.gpu


def _case(b, h, s, d, sigma, seed):
    rng = np.random.default_rng(seed)
    ref = workloads.f32_to_bf16_bits(rng.standard_normal((b, h, s, d)).astype(np.float32))
    x = workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(ref) +
                                    sigma * rng.standard_normal((b, h, s, d))).astype(np.float32))
    return x, ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("refits", [1, 3])
def test_refit_matches_oracle(d, bits, refits):
    print(f"refit d={d} bits={bits} refits={refits}", flush=True)
    x, ref = _case(2, 3, 77, d, 0.2, seed=d + 10 * bits + refits)
    codes, scales = rq.encode([to_dev(x)], to_dev(ref), [bits], refits=refits)
    torch.cuda.synchronize()
    ow, os_ = oracle.encode(x, ref, bits, refits=refits)
    compare_codes_refit(to_host_words(codes[0]), to_host_u16(scales[0]), ow, os_, x, ref, bits, refits)


def test_refit_zero_equals_plain_encode():
    """rq_encode_refit with refits = 0 is rq_encode, bit for bit."""
    x, ref = _case(1, 2, 130, 128, 0.1, seed=4)
    xd, rd = to_dev(x), to_dev(ref)
    c1, s1 = rq.encode([xd], rd, [2])
    c2 = torch.empty_like(c1[0])
    s2 = torch.empty_like(s1[0])
    lib = rq._load()
    shp = rq._Shape(*x.shape)
    st = lib.rq_encode_refit(ctypes.byref(shp), 1, rq._ptr_array([xd]), (ctypes.c_int32 * 1)(2), rq._ptr(rd),
                             rq._ptr_array([c2]), rq._ptr_array([s2]), 0, rq._stream(xd.device, None))
    assert st == rq.RQ_OK
    torch.cuda.synchronize()
    assert torch.equal(c1[0], c2) and torch.equal(s1[0].view(torch.int16), s2.view(torch.int16))


def test_refit_lowers_the_reconstruction_error():
    w = workloads.WORKLOADS["tiny"]
    for tensor in (workloads.TENSOR_K, workloads.TENSOR_V):
        xs = workloads.kv_tensors(w, tensor)
        xd = [to_dev(x) for x in xs]
        bits = list(w.bits[:-1])
        for l, bl in enumerate(bits):
            e = {}
            for k in (0, 2):
                c, s = rq.encode([xd[l]], xd[-1], [bl], refits=k)
                xh = rq.reconstruct(xd[-1], c[0], s[0], bl).cpu().numpy().astype(np.float64)
                e[k] = recon_error(xh, xs[l], xs[-1])
                ow, os_ = oracle.encode(xs[l], xs[-1], bl, refits=k)
                e_orc = oracle.reconstruction_error(oracle.reconstruct(xs[-1], ow, os_, bl), xs[l], xs[-1])
                assert abs(e[k] - e_orc) <= RECON_TOL
            assert e[2] < e[0]


def test_refit_full_size_sampled_rows():
    """The launch the benchmark's refit leg times (K of l4_b16_s4k, two refits)."""
    w = workloads.WORKLOADS["l4_b16_s4k"]
    xs = workloads.kv_tensors(w, workloads.TENSOR_K)
    bits = list(w.bits[:-1])
    xd = [to_dev(x) for x in xs]
    codes, scales = rq.encode(xd[:-1], xd[-1], bits, refits=2)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (9, 5)]:
        rows = workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_K)
        for l, bl in enumerate(bits):
            ow, os_ = oracle.encode(rows[l], rows[-1], bl, refits=2)
            compare_codes_refit(to_host_words(codes[l][b, h]), to_host_u16(scales[l][b, h]), ow, os_,
                                rows[l], rows[-1], bl, 2)
