"""CPU check of the decode's numeric envelope (the operand roundings that
rq.h states for rq_decode_attn), on encoder outputs whose residual is as large
as the reference: a model of those roundings, written here from their
statement, evaluated in NumPy against the oracle's fp64 attention.

The modelled roundings: the rotated query Hq enters the residual scores as an
fp16 pair hi + lo of its fp32 value; every residual PV weight is the softmax
weight times the fp16 scale, rounded once to fp16 (INT8 at half the weight,
its levels doubled); the reference parts stay exact (bf16 products of stored
values, P within 2^-16). Scores, softmax and sums are taken in fp64 here, below
the kernel's fp32, so the check covers the operand roundings only.

It pins two statements of the envelope: rows stay within 2e-3 of fp64 at
every width 2, 3, 4, 8, Gaussian and heavy-tailed; and a row's error stays
below its leading-term bound 2^-11 * max_t |v_hat_t - v_ref,t| / max |out|.
A single fp16 query operand, without the lo part, is shown to make the
heavy-tailed INT8 rows' error several times larger."""
import numpy as np
import pytest

import oracle
import workloads

def _model_rows(w, kx, vx, q_bits, query_lo=True):
    """Per row (b, q head) of loop 0: (row error against fp64, leading-term bound)."""
    bits, d, g = w.bits[0], w.head_dim, w.group_size
    h_mat = oracle.hadamard(d)
    scale = 1.0 / np.sqrt(d)
    errs, bounds = [], []
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            kr, vr = kx[-1][b, h], vx[-1][b, h]
            kw, ks = oracle.encode(kx[0][b, h], kr, bits)
            vw, vs = oracle.encode(vx[0][b, h], vr, bits)
            k_hat = oracle.reconstruct(kr, kw, ks, bits)
            v_hat = oracle.reconstruct(vr, vw, vs, bits)
            q = oracle.bf16_to_f64(q_bits[0, b, h * g:(h + 1) * g])
            exact = oracle.attention(q, k_hat, v_hat, scale)
            k_lev = oracle.unpack_codes(kw, bits) - oracle.level_offset(bits)
            v_lev = oracle.unpack_codes(vw, bits) - oracle.level_offset(bits)
            k_s = np.repeat(oracle.f16_to_f64(ks), 32, -1)
            # the rotated query: fp32, then fp16 hi (+ fp16 lo of the remainder)
            qt32 = (q @ h_mat).astype(np.float32)
            hi = qt32.astype(np.float16)
            qt = hi.astype(np.float64)
            if query_lo:
                qt = qt + (qt32 - hi.astype(np.float32)).astype(np.float16).astype(np.float64)
            z = (q @ oracle.bf16_to_f64(kr).T + qt @ (k_s * k_lev).T) * scale
            p = np.exp(z - z.max(-1, keepdims=True))
            v_s = oracle.f16_to_f64(vs)
            half = 0.5 if bits == 8 else 1.0
            ps = (p[:, :, None] * half * v_s[None]).astype(np.float16).astype(np.float64) / half
            o_res = np.einsum("gtk,tk->gk", np.repeat(ps, 32, -1), v_lev) @ h_mat
            out = (p @ oracle.bf16_to_f64(vr) + o_res) / p.sum(-1, keepdims=True)
            peak = np.abs(exact).max(-1)
            errs.append(np.abs(out - exact).max(-1) / peak)
            bounds.append(2.0 ** -11 * np.abs(v_hat - oracle.bf16_to_f64(vr)).max() / peak)
    return np.concatenate(errs), np.concatenate(bounds)


def _workload(bits, heavy):
    # 2 KV / 8 query heads, head_dim 128, 384 positions; residual sigma 1.0 as
    # large as the reference's, loop 1 the reference
    return workloads.Workload("envelope_model", 60 + bits, 2, 1, 2, 8, 128, 384, (bits, 0), (1.0, 0.0), heavy)


@pytest.mark.parametrize("heavy", [False, True])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_modelled_roundings_stay_inside_the_envelope(bits, heavy):
    w = _workload(bits, heavy)
    kx, vx = workloads.kv_tensors(w, workloads.TENSOR_K), workloads.kv_tensors(w, workloads.TENSOR_V)
    err, bound = _model_rows(w, kx, vx, workloads.q_tensor(w))
    assert err.max() <= 2e-3
    assert np.all(err <= bound)


def test_the_query_lo_part_cuts_the_heavy_tailed_int8_error():
    """Without the lo part of the rotated query, the heavy-tailed INT8 rows'
    largest error is several times that with it (the reason the kernel carries
    the pair; with a truncated P s as well it passed 2e-3)."""
    w = workloads.Workload("envelope_model", 68, 2, 2, 2, 8, 128, 1500, (8, 0), (1.0, 0.0), True)
    kx, vx = workloads.kv_tensors(w, workloads.TENSOR_K), workloads.kv_tensors(w, workloads.TENSOR_V)
    q = workloads.q_tensor(w)
    err_pair, _ = _model_rows(w, kx, vx, q)
    err_one, _ = _model_rows(w, kx, vx, q, query_lo=False)
    assert err_one.max() > 3 * err_pair.max()
