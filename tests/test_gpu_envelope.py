"""GPU parity of the encode -> fused decode chain on encoder-produced residuals:
the numeric envelope of the decode, and the benchmark's own launches at full
size.

* Residuals as large as the reference (sigma_res = sigma_ref) at every width
  2, 3, 4 and 8, Gaussian and heavy-tailed (4 of 128 K channels x20 in the
  reference and in the residual, V ~ Student-t(4)), for one 16-row block, two
  argument sets and 20-row blocks (the byte-table decode). A CPU emulation of
  the decode's roundings put the heavy-tailed INT2 rows at 3.0e-3 with an fp16
  rotated query alone; with the hi + lo split it is below 2.5e-4.
* The heavy_tail and mixed_s32k workloads at full size, in the launch
  configuration the benchmark times: rq_encode_kv of K and V (one launch), the
  codes of sampled rows against the oracle's encode, those rows' codes then
  replaced by the oracle's on the device (a code rounded to the other side of
  a decision boundary would move that token's score), and the decode of all
  loops against the oracle's decode of its own codes.

No oracle input comes from the GPU: the oracle sees the generator's data and
its own codes only."""
import numpy as np
import pytest
import torch

import looped_transformer_kv_rq_amd as rq
import oracle
import workloads
from rq_parity import assert_attn_close, compare_codes, to_dev, to_host_u16, to_host_words, words_to_dev

pytestmark = pytest.mark.gpu


def _encode_kv(kd, vd, bits, shape, d):
    """rq_encode_kv into fresh outputs; returns (kc, ks, vc, vs)."""
    kc = [torch.empty(shape + (d * b // 32,), dtype=torch.int32, device="cuda") for b in bits]
    vc = [torch.empty_like(t) for t in kc]
    ks = [torch.empty(shape + (d // 32,), dtype=torch.float16, device="cuda") for _ in bits]
    vs = [torch.empty_like(t) for t in ks]
    rq.encode_kv_into(kd[:-1], vd[:-1], kd[-1], vd[-1], bits, kc, ks, vc, vs)
    torch.cuda.synchronize()
    return kc, ks, vc, vs


def _check_and_substitute(rows, w, bits, kc, ks, vc, vs, k_rows, v_rows):
    """Codes of the sampled rows against the oracle's encode; then the oracle's
    codes replace the GPU's there. Returns {(b, h, l): (okw, oks, ovw, ovs)}."""
    orc = {}
    for (b, h) in rows:
        k_st, v_st = k_rows(b, h), v_rows(b, h)
        for l, bl in enumerate(bits):
            okw, oks = oracle.encode(k_st[l], k_st[-1], bl)
            ovw, ovs = oracle.encode(v_st[l], v_st[-1], bl)
            compare_codes(to_host_words(kc[l][b, h]), to_host_u16(ks[l][b, h]), okw, oks, k_st[l], k_st[-1], bl)
            compare_codes(to_host_words(vc[l][b, h]), to_host_u16(vs[l][b, h]), ovw, ovs, v_st[l], v_st[-1], bl)
            kc[l][b, h] = words_to_dev(okw)
            ks[l][b, h] = to_dev(oks, torch.float16)
            vc[l][b, h] = words_to_dev(ovw)
            vs[l][b, h] = to_dev(ovs, torch.float16)
            orc[(b, h, l)] = (okw, oks, ovw, ovs)
    return orc


def _oracle_row(w, b, h, q_bits, k_st, v_st, orc):
    """The oracle's decode of every loop for one (b, kv head) row: [L, G, D]."""
    g = w.group_size
    out = np.empty((w.n_loops, g, w.head_dim))
    for l in range(w.n_loops):
        if w.bits[l]:
            okw, oks, ovw, ovs = orc[(b, h, l)]
            k = oracle.reconstruct(k_st[-1], okw, oks, w.bits[l])
            v = oracle.reconstruct(v_st[-1], ovw, ovs, w.bits[l])
        else:
            k, v = oracle.bf16_to_f64(k_st[-1]), oracle.bf16_to_f64(v_st[-1])
        q = oracle.bf16_to_f64(q_bits[l, b, h * g:(h + 1) * g])
        out[l] = oracle.attention(q, k, v, 1.0 / np.sqrt(w.head_dim))
    return out


@pytest.mark.parametrize("heavy", [False, True])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("hq", [8, 32, 40])
def test_residual_as_large_as_reference(bits, heavy, hq):
    """sigma_res = sigma_ref = 1 (the rotation-only regime's magnitude); loops
    (bits, 2, 0). hq = 8: one 16-row block (G = 4); hq = 32: two argument sets
    of 16 rows (G = 16); hq = 40: 20-row blocks (G = 20), the byte-table PV."""
    print(f"envelope bits={bits} heavy={heavy} hq={hq}", flush=True)
    w = workloads.Workload("envelope", 60 + bits, 3, 2, 2, hq, 128, 1500, (bits, 2, 0), (1.0, 1.0, 0.0), heavy)
    kx, vx = workloads.kv_tensors(w, workloads.TENSOR_K), workloads.kv_tensors(w, workloads.TENSOR_V)
    kd, vd = [to_dev(x) for x in kx], [to_dev(x) for x in vx]
    res_bits = list(w.bits[:-1])
    kc, ks, vc, vs = _encode_kv(kd, vd, res_bits, (w.batch, w.n_kv_heads, w.seq_len), w.head_dim)
    rows = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    orc = _check_and_substitute(rows, w, res_bits, kc, ks, vc, vs,
                                lambda b, h: [x[b, h] for x in kx], lambda b, h: [x[b, h] for x in vx])
    q_bits = workloads.q_tensor(w)
    views = [rq.LoopView(bl, kc[l], ks[l], vc[l], vs[l]) for l, bl in enumerate(res_bits)] + [rq.LoopView(0)]
    out = rq.decode_attn(to_dev(q_bits), kd[-1], vd[-1], views).cpu().numpy()
    g = w.group_size
    for (b, h) in rows:
        want = _oracle_row(w, b, h, q_bits, [x[b, h] for x in kx], [x[b, h] for x in vx], orc)
        assert_attn_close(out[:, b, h * g:(h + 1) * g], want)


@pytest.mark.parametrize("name,rows", [("heavy_tail", [(0, 0), (13, 4), (31, 7)]),
                                       ("mixed_s32k", [(0, 3), (7, 7)])])
def test_encode_kv_then_decode_full_size(name, rows):
    """The benchmark's step at full size: rq_encode_kv (K and V, one launch),
    then rq_decode_attn over all loops with the automatic split count."""
    w = workloads.WORKLOADS[name]
    print(f"full-size chain {name} rows={rows}", flush=True)
    res_bits = [b for b in w.bits if b]
    kd = [to_dev(x) for x in workloads.kv_tensors(w, workloads.TENSOR_K)]
    vd = [to_dev(x) for x in workloads.kv_tensors(w, workloads.TENSOR_V)]
    kc, ks, vc, vs = _encode_kv(kd, vd, res_bits, (w.batch, w.n_kv_heads, w.seq_len), w.head_dim)
    orc = _check_and_substitute(rows, w, res_bits, kc, ks, vc, vs,
                                lambda b, h: workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_K),
                                lambda b, h: workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_V))
    q_bits = workloads.q_tensor(w)
    views = [rq.LoopView(bl, kc[l], ks[l], vc[l], vs[l]) for l, bl in enumerate(res_bits)] + [rq.LoopView(0)]
    out = rq.decode_attn(to_dev(q_bits), kd[-1], vd[-1], views).cpu().numpy()
    g = w.group_size
    for (b, h) in rows:
        want = _oracle_row(w, b, h, q_bits, workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_K),
                           workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_V), orc)
        assert_attn_close(out[:, b, h * g:(h + 1) * g], want)
    del kd, vd, kc, ks, vc, vs
    torch.cuda.empty_cache()
