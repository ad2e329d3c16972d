"""GPU parity of the INT3 and INT8 widths in the fused decode, and of the
per-(layer, loop) width table (rq_encode_layers), against the oracle.

The encoders, reconstruct, refit, append and rotation-only tests cover the new
widths in their own files (their width parametrisations include 3 and 8)."""
import numpy as np
import pytest
import torch

import looped_transformer_kv_rq_amd as rq
import oracle
import workloads
from rq_parity import assert_attn_close, compare_codes, to_dev, to_host_u16, to_host_words, words_to_dev
from test_gpu_decode import _all_rows, _run_case

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------- decode, random packed codes
# Random code words reach every code value of every width; the scales are
# fp16 values in [0.01, 0.1].

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [(8, 3, 2, 0), (3, 3, 3, 0), (8, 8, 0), (4, 3, 0), (8, 4, 3, 2, 0), (8, 2, 2, 0),
                                  (8, 8, 2, 0), (8, 8, 8, 8)])
@pytest.mark.parametrize("hq", [8, 16])
def test_decode_wide_tables(d, bits, hq):
    """G = 4 (one 16-row block per launch) and 8 (two blocks once there are
    three or more loops), every width order, both head sizes. At D = 128 and
    G = 4 the INT8 tables stage 20-30 KB per wave and tile: (8, 3, 2, 0) and
    (8, 8, 0) run six-wave blocks, (8, 2, 2, 0) seven, (8, 8, 2, 0) four (one
    block per CU). (8, 8, 8, 8) has no reference-only loop; at D = 128 its
    loops need two launches (three loops, then one), at D = 64 one launch of
    seven-wave blocks. With 131 positions (5 tiles) some waves get no tile."""
    print(f"decode wide d={d} bits={bits} hq={hq}", flush=True)
    n = len(bits)
    sig = tuple([0.1] * (n - 1) + [0.0])
    w = workloads.Workload("wide", 95, n, 2, 2, hq, d, 131, bits, sig)
    _run_case(w, range(n), _all_rows(w))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("s", [1, 63, 65, 200])
def test_decode_wide_ragged_lengths(d, s):
    w = workloads.Workload("wide_ragged", 96, 3, 2, 2, 8, d, s, (8, 3, 0), (0.2, 0.1, 0.0))
    _run_case(w, range(3), _all_rows(w))


def test_decode_wide_one_loop_and_split_counts():
    w = workloads.Workload("wide_splits", 97, 3, 1, 2, 8, 128, 1000, (3, 8, 0), (0.1, 0.1, 0.0))
    for loop in range(3):
        _run_case(w, [loop], _all_rows(w))
    for n in (1, 3, 16):
        _run_case(w, range(3), _all_rows(w), n_splits=n)


# --------------------------------------------------------------------------- decode after a GPU encode

def _states(b, h, s, d, sigmas, seed):
    rng = np.random.default_rng(seed)
    ref = workloads.f32_to_bf16_bits(rng.standard_normal((b, h, s, d)).astype(np.float32))
    xs = [workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(ref) + sg * rng.standard_normal(
        (b, h, s, d))).astype(np.float32)) for sg in sigmas]
    return xs + [ref]


def _oracle_decode(q_bits, ks, vs, bits, enc_k, enc_v):
    """Oracle decode over the oracle's reconstruction from its own codes."""
    k_hat, v_hat = [], []
    for l, bl in enumerate(bits):
        if bl:
            k_hat.append(oracle.reconstruct(ks[-1], *enc_k[l], bl))
            v_hat.append(oracle.reconstruct(vs[-1], *enc_v[l], bl))
        else:
            k_hat.append(oracle.bf16_to_f64(ks[-1]))
            v_hat.append(oracle.bf16_to_f64(vs[-1]))
    return oracle.decode_attn(q_bits, k_hat, v_hat)


@pytest.mark.parametrize("d", [64, 128])
def test_encode_then_decode_wide(d):
    """GPU encode of K and V at (8, 3, 4), compared with the oracle's encode
    (codes bit-exact away from a decision boundary, scales within one ulp).
    The device codes are then replaced by the oracle's, so the fused decode
    runs on exactly the oracle's inputs, and its output is compared with the
    oracle's decode of those codes."""
    bits = (8, 3, 4, 0)
    b, h, hq, s = 2, 2, 8, 257
    ks = _states(b, h, s, d, (0.2, 0.1, 0.05), seed=d)
    vs = _states(b, h, s, d, (0.2, 0.1, 0.05), seed=d + 1)
    kd, vd = [to_dev(x) for x in ks], [to_dev(x) for x in vs]
    kc, kss = rq.encode(kd[:-1], kd[-1], bits[:-1])
    vc, vss = rq.encode(vd[:-1], vd[-1], bits[:-1])
    torch.cuda.synchronize()
    enc_k, enc_v = [], []
    for l, bl in enumerate(bits[:-1]):
        okw, oks = oracle.encode(ks[l], ks[-1], bl)
        ovw, ovs = oracle.encode(vs[l], vs[-1], bl)
        compare_codes(to_host_words(kc[l]), to_host_u16(kss[l]), okw, oks, ks[l], ks[-1], bl)
        compare_codes(to_host_words(vc[l]), to_host_u16(vss[l]), ovw, ovs, vs[l], vs[-1], bl)
        kc[l].copy_(words_to_dev(okw))
        kss[l].copy_(to_dev(oks, torch.float16))
        vc[l].copy_(words_to_dev(ovw))
        vss[l].copy_(to_dev(ovs, torch.float16))
        enc_k.append((okw, oks))
        enc_v.append((ovw, ovs))
    views = [rq.LoopView(bl, kc[l], kss[l], vc[l], vss[l]) for l, bl in enumerate(bits[:-1])] + [rq.LoopView(0)]
    q = workloads.f32_to_bf16_bits(np.random.default_rng(7).standard_normal((4, b, hq, d)).astype(np.float32))
    out = rq.decode_attn(to_dev(q), kd[-1], vd[-1], views).cpu().numpy()
    assert_attn_close(out, _oracle_decode(q, ks, vs, bits, enc_k, enc_v))


# --------------------------------------------------------------------------- per-(layer, loop) table

def test_encode_layers_equals_per_layer_encodes():
    table = [(8, 4, 2), (3, 3, 2), (2, 8, 3)]
    layers = [_states(2, 2, 70, 128, (0.2, 0.1, 0.05), seed=30 + l) for l in range(3)]
    dev = [[to_dev(x) for x in st] for st in layers]
    codes, scales = rq.encode_layers([st[:-1] for st in dev], [st[-1] for st in dev], table)
    for l, row in enumerate(table):
        c1, s1 = rq.encode(dev[l][:-1], dev[l][-1], row)
        for i, bl in enumerate(row):
            assert torch.equal(codes[l][i], c1[i])
            assert torch.equal(scales[l][i].view(torch.int16), s1[i].view(torch.int16))
            ow, os_ = oracle.encode(layers[l][i], layers[l][-1], bl)
            compare_codes(to_host_words(codes[l][i]), to_host_u16(scales[l][i]), ow, os_, layers[l][i],
                          layers[l][-1], bl)


def test_layer_table_full_size_sampled_rows():
    """The launches the benchmark's layer-table leg times: every layer of
    LAYER_BITS_L4 encoded over the K and V states of l4_b16_s4k (one call for
    all layers), then each layer's decode with its row of the table."""
    w = workloads.WORKLOADS["l4_b16_s4k"]
    table = workloads.LAYER_BITS_L4
    rows = [(0, 0), (11, 6)]
    q_bits = workloads.q_tensor(w)
    qd = to_dev(q_bits)
    enc = {}
    oenc = {}  # the oracle's own codes of the sampled rows
    for tensor in (workloads.TENSOR_K, workloads.TENSOR_V):
        xs = workloads.kv_tensors(w, tensor)
        xd = [to_dev(x) for x in xs]
        codes, scales = rq.encode_layers([xd[:-1]] * len(table), [xd[-1]] * len(table),
                                         [row[:-1] for row in table])
        torch.cuda.synchronize()
        for (b, h) in rows:
            st = workloads.kv_rows_all_loops(w, b, h, tensor)
            for l, row in enumerate(table):
                for i, bl in enumerate(row[:-1]):
                    ow, os_ = oracle.encode(st[i], st[-1], bl)
                    oenc[(tensor, l, i, b, h)] = (ow, os_)
                    compare_codes(to_host_words(codes[l][i][b, h]), to_host_u16(scales[l][i][b, h]), ow, os_,
                                  st[i], st[-1], bl)
                    # the decode below runs on the oracle's codes for this row: a code
                    # rounded to the other side of a decision boundary (allowed above)
                    # would move that token's score
                    codes[l][i][b, h] = words_to_dev(ow)
                    scales[l][i][b, h] = to_dev(os_, torch.float16)
        enc[tensor] = (xd[-1], codes, scales)
        del xd
    kref, kc, ksc = enc[workloads.TENSOR_K]
    vref, vc, vsc = enc[workloads.TENSOR_V]
    g = w.group_size
    for l, row in enumerate(table):
        views = [rq.LoopView(bl, kc[l][i], ksc[l][i], vc[l][i], vsc[l][i]) for i, bl in enumerate(row[:-1])]
        out = rq.decode_attn(qd, kref, vref, views + [rq.LoopView(0)]).cpu().numpy()
        for (b, h) in rows:
            k_st = workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_K)
            v_st = workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_V)
            scale = 1.0 / np.sqrt(w.head_dim)
            for i, bl in enumerate(row):
                if bl:
                    k = oracle.reconstruct(k_st[-1], *oenc[(workloads.TENSOR_K, l, i, b, h)], bl)
                    v = oracle.reconstruct(v_st[-1], *oenc[(workloads.TENSOR_V, l, i, b, h)], bl)
                else:
                    k, v = oracle.bf16_to_f64(k_st[-1]), oracle.bf16_to_f64(v_st[-1])
                q = oracle.bf16_to_f64(q_bits[i, b, h * g:(h + 1) * g])
                assert_attn_close(out[i, b, h * g:(h + 1) * g], oracle.attention(q, k, v, scale))
    del enc, kc, vc, ksc, vsc
    torch.cuda.empty_cache()


def test_int8_layer_mixed_s32k_sampled_row():
    """The INT8 layer of the bench's width table at its own size: the (8, 4, 2,
    0) row of LAYER_BITS_L4 over the mixed_s32k states (B = 8, 8 / 32 heads,
    32K positions), encoded by rq_encode, then decoded with the automatic plan
    the bench times (six-wave blocks, 4 splits). One sampled (b, kv head) row:
    codes against the oracle, then the oracle's codes substituted and every
    loop's rows decoded against the oracle's attention."""
    w = workloads.WORKLOADS["mixed_s32k"]
    row = workloads.LAYER_BITS_L4[0]
    assert tuple(row) == (8, 4, 2, 0)
    assert rq.decode_splits(w.batch, w.n_kv_heads, w.seq_len, w.head_dim, w.n_q_heads, w.n_loops,
                            bits=list(row)) == 4
    b, h = 5, 3
    print(f"int8 layer mixed_s32k row ({b}, {h})", flush=True)
    q_bits = workloads.q_tensor(w)
    enc, oenc = {}, {}
    for tensor in (workloads.TENSOR_K, workloads.TENSOR_V):
        xs = workloads.kv_tensors(w, tensor)
        xd = [to_dev(x) for x in xs]
        del xs
        codes, scales = rq.encode(xd[:-1], xd[-1], list(row[:-1]))
        torch.cuda.synchronize()
        st = workloads.kv_rows_all_loops(w, b, h, tensor)
        for i, bl in enumerate(row[:-1]):
            ow, os_ = oracle.encode(st[i], st[-1], bl)
            oenc[(tensor, i)] = (ow, os_)
            compare_codes(to_host_words(codes[i][b, h]), to_host_u16(scales[i][b, h]), ow, os_, st[i], st[-1], bl)
            codes[i][b, h] = words_to_dev(ow)
            scales[i][b, h] = to_dev(os_, torch.float16)
        enc[tensor] = (xd[-1], codes, scales)
        del xd
    kref, kc, ksc = enc[workloads.TENSOR_K]
    vref, vc, vsc = enc[workloads.TENSOR_V]
    views = [rq.LoopView(bl, kc[i], ksc[i], vc[i], vsc[i]) for i, bl in enumerate(row[:-1])] + [rq.LoopView(0)]
    out = rq.decode_attn(to_dev(q_bits), kref, vref, views).cpu().numpy()
    k_st = workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_K)
    v_st = workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_V)
    g = w.group_size
    scale = 1.0 / np.sqrt(w.head_dim)
    for i, bl in enumerate(row):
        if bl:
            k = oracle.reconstruct(k_st[-1], *oenc[(workloads.TENSOR_K, i)], bl)
            v = oracle.reconstruct(v_st[-1], *oenc[(workloads.TENSOR_V, i)], bl)
        else:
            k, v = oracle.bf16_to_f64(k_st[-1]), oracle.bf16_to_f64(v_st[-1])
        q = oracle.bf16_to_f64(q_bits[i, b, h * g:(h + 1) * g])
        assert_attn_close(out[i, b, h * g:(h + 1) * g], oracle.attention(q, k, v, scale))
    del enc, kc, vc, ksc, vsc, kref, vref
    torch.cuda.empty_cache()
