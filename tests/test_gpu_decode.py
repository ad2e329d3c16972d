"""GPU parity of rq_decode_attn (fused reconstruct + decode attention) and of
the bf16 baseline, against the CPU oracle."""
import numpy as np
import pytest
import torch

import looped_transformer_kv_rq_amd as rq
import oracle
import workloads
from rq_parity import assert_attn_close, to_dev, words_to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _packed_cache(w, loops=None):
    """Generator-made decode inputs: bf16 refs and random packed codes/scales per residual loop."""
    loops = range(w.n_loops) if loops is None else loops
    kref = workloads.ref_tensor(w, workloads.TENSOR_K)
    vref = workloads.ref_tensor(w, workloads.TENSOR_V)
    res = {}
    for l in loops:
        if w.bits[l]:
            res[l] = (workloads.packed_tensors(w, 0, l), workloads.packed_tensors(w, 1, l))
    return kref, vref, res


def _views(w, loops, res):
    views = []
    for l in loops:
        if w.bits[l]:
            (kw, ks), (vw, vs) = res[l]
            views.append(rq.LoopView(w.bits[l], words_to_dev(kw), to_dev(ks, torch.float16),
                                     words_to_dev(vw), to_dev(vs, torch.float16)))
        else:
            views.append(rq.LoopView(0))
    return views


def _oracle_rows(w, loops, q_bits, kref, vref, res, rows):
    """Oracle decode for sampled (b, kv_head) rows: [len(loops), len(rows), G, D]."""
    g = w.group_size
    out = np.empty((len(loops), len(rows), g, w.head_dim))
    scale = 1.0 / np.sqrt(w.head_dim)
    for i, l in enumerate(loops):
        for j, (b, h) in enumerate(rows):
            if w.bits[l]:
                (kw, ks), (vw, vs) = res[l]
                k = oracle.reconstruct(kref[b, h], kw[b, h], ks[b, h], w.bits[l])
                v = oracle.reconstruct(vref[b, h], vw[b, h], vs[b, h], w.bits[l])
            else:
                k, v = oracle.bf16_to_f64(kref[b, h]), oracle.bf16_to_f64(vref[b, h])
            q = oracle.bf16_to_f64(q_bits[i, b, h * g:(h + 1) * g])
            out[i, j] = oracle.attention(q, k, v, scale)
    return out


def _gpu_rows(out, rows, g):
    return np.stack([np.stack([out[i, b, h * g:(h + 1) * g] for (b, h) in rows]) for i in range(out.shape[0])])


def _run_case(w, loops, rows, n_splits=0):
    kref, vref, res = _packed_cache(w, loops)
    q_all = workloads.q_tensor(w)
    q_bits = q_all[list(loops)]
    out = rq.decode_attn(to_dev(q_bits), to_dev(kref), to_dev(vref), _views(w, loops, res), n_splits=n_splits)
    torch.cuda.synchronize()
    got = _gpu_rows(out.cpu().numpy(), rows, w.group_size)
    ref = _oracle_rows(w, loops, q_bits, kref, vref, res, rows)
    return assert_attn_close(got, ref)


def _all_rows(w):
    return [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]


def test_decode_tiny_all_loops():
    w = workloads.WORKLOADS["tiny"]
    _run_case(w, range(w.n_loops), _all_rows(w))


@pytest.mark.parametrize("loop", [0, 3])
def test_decode_tiny_one_loop(loop):
    w = workloads.WORKLOADS["tiny"]
    _run_case(w, [loop], _all_rows(w))


@pytest.mark.parametrize("bits", [(4, 4, 2, 0), (4, 4, 4, 0)])
@pytest.mark.parametrize("s,n_splits", [(131, 0), (1000, 0), (1000, 3)])
def test_decode_int4_heavy_tables(bits, s, n_splits):
    """16 query rows whose INT2 / INT4 loops stage more than 20 KB per wave and
    tile at D = 128, so two 4-wave blocks do not fit a CU: the call runs
    seven-wave blocks over prepared query records instead of rotating the
    queries in the kernel."""
    print(f"decode int4-heavy bits={bits} s={s} n_splits={n_splits}", flush=True)
    n = len(bits)
    w = workloads.Workload("int4_heavy", 91, n, 2, 2, 8, 128, s, bits, tuple([0.2] * (n - 1) + [0.0]))
    _run_case(w, range(n), _all_rows(w), n_splits=n_splits)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("s", [1, 63, 65, 200])
def test_decode_ragged_lengths(d, s):
    w = workloads.Workload("ragged", 90, 3, 2, 2, 8, d, s, (4, 2, 0), (0.2, 0.1, 0.0))
    _run_case(w, range(3), _all_rows(w))


@pytest.mark.parametrize("hq,hkv,n_loops", [(4, 4, 4), (16, 2, 4), (32, 1, 2), (12, 4, 8), (12, 2, 5), (20, 2, 3)])
def test_decode_head_groupings(hq, hkv, n_loops):
    """G = 1, 8, 32, 3, 6 and 10; more than 32 rows per kv head splits the launch over loops.
    G = 6 with 5 loops and G = 10 with 3 loops fit 32 rows but not two sets of at most 16
    (2 and 1 loops per set), so those launches split over loops."""
    bits = tuple([4] + [2] * (n_loops - 2) + [0])
    sig = tuple([0.1] * (n_loops - 1) + [0.0])
    w = workloads.Workload("groups", 91, n_loops, 2, hkv, hq, 128, 300, bits, sig)
    _run_case(w, range(n_loops), _all_rows(w))


def _constant_words(shape, d, bits, c):
    """Code words [..., d*bits/32] holding code c at every coordinate (the
    layouts of oracle.pack_codes, written out for a constant)."""
    if bits == 3:
        lo = sum((c & 3) << (2 * j) for j in range(16))
        hi = 0xFFFFFFFF if c & 4 else 0
        words = np.empty(shape + (3 * d // 32,), dtype=np.uint32)
        words[..., : d // 16] = lo
        words[..., d // 16:] = hi
        return words
    return np.full(shape + (d * bits // 32,), sum(c << (bits * j) for j in range(32 // bits)), dtype=np.uint32)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("hq", [8, 40])
def test_decode_constant_v_codes(bits, hq):
    """Every V code of the residual loop set to one value: the lowest, the
    highest and the first positive level. The residual part of each output is
    then that level times the scale-weighted softmax sum of each group, which a
    decode that forms levels as 2^b (1 + c/2^b) minus an offset must cancel
    exactly. G = 4 runs one 16-row block; G = 20 two (the byte-table levels)."""
    w = workloads.Workload("constv", 98, 2, 1, 2, hq, 128, 150, (bits, 0), (0.2, 0.0))
    kref, vref, res = _packed_cache(w, [0, 1])
    (kw, ks), (vw, vs) = res[0]
    q_bits = workloads.q_tensor(w)
    rows = _all_rows(w)
    for c in (0, (1 << bits) - 1, 1 << (bits - 1)):
        print(f"constant V codes bits={bits} hq={hq} c={c}", flush=True)
        cres = {0: ((kw, ks), (_constant_words(vw.shape[:-1], w.head_dim, bits, c), vs))}
        out = rq.decode_attn(to_dev(q_bits), to_dev(kref), to_dev(vref), _views(w, [0, 1], cres))
        torch.cuda.synchronize()
        got = _gpu_rows(out.cpu().numpy(), rows, w.group_size)
        assert_attn_close(got, _oracle_rows(w, [0, 1], q_bits, kref, vref, cres, rows))


def test_decode_split_counts_agree():
    w = workloads.Workload("splits", 92, 2, 1, 2, 8, 128, 1000, (2, 0), (0.1, 0.0))
    for n in (1, 3, 16):
        _run_case(w, range(2), _all_rows(w), n_splits=n)


def test_decode_repeatable_and_overwrites():
    w = workloads.Workload("det", 93, 2, 2, 2, 8, 64, 500, (2, 0), (0.1, 0.0))
    kref, vref, res = _packed_cache(w)
    q = to_dev(workloads.q_tensor(w))
    views = _views(w, range(2), res)
    k, v = to_dev(kref), to_dev(vref)
    out = torch.full((2, 2, 8, 64), float("nan"), device=DEV)
    rq.decode_attn(q, k, v, views, out=out)
    again = rq.decode_attn(q, k, v, views)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, again)


def test_decode_end_to_end_after_gpu_encode():
    """GPU encode -> GPU decode against oracle encode -> oracle decode (tiny workload)."""
    w = workloads.WORKLOADS["tiny"]
    ks, vs = workloads.kv_tensors(w, 0), workloads.kv_tensors(w, 1)
    bits = list(w.bits[:-1])
    kd, vd = [to_dev(x) for x in ks], [to_dev(x) for x in vs]
    kc, ksc = rq.encode(kd[:-1], kd[-1], bits)
    vc, vsc = rq.encode(vd[:-1], vd[-1], bits)
    views = [rq.LoopView(bits[l], kc[l], ksc[l], vc[l], vsc[l]) for l in range(len(bits))] + [rq.LoopView(0)]
    q_bits = workloads.q_tensor(w)
    out = rq.decode_attn(to_dev(q_bits), kd[-1], vd[-1], views).cpu().numpy()
    khat, vhat = [], []
    for l in range(w.n_loops):
        if w.bits[l]:
            kw, kss = oracle.encode(ks[l], ks[-1], w.bits[l])
            vw, vss = oracle.encode(vs[l], vs[-1], w.bits[l])
            khat.append(oracle.reconstruct(ks[-1], kw, kss, w.bits[l]))
            vhat.append(oracle.reconstruct(vs[-1], vw, vss, w.bits[l]))
        else:
            khat.append(oracle.bf16_to_f64(ks[-1]))
            vhat.append(oracle.bf16_to_f64(vs[-1]))
    assert_attn_close(out, oracle.decode_attn(q_bits, khat, vhat))


@pytest.mark.parametrize("name,rows", [("l4_b16_s4k", [(0, 0), (15, 7)]),
                                       ("mixed_s32k", [(0, 0), (7, 7)]),
                                       ("heavy_tail", [(31, 0)]),
                                       ("peak_batch", [(0, 0), (3, 3)])])
def test_decode_full_size_sampled_rows(name, rows):
    w = workloads.WORKLOADS[name]
    if name == "peak_batch":
        w = w.with_batch(4)
    print(f"decode full {name} rows={rows}", flush=True)
    _run_case(w, range(w.n_loops), rows)


def test_decode_per_loop_calls_match_all_loop_call():
    w = workloads.Workload("perloop", 94, 4, 2, 2, 8, 128, 777, (4, 2, 2, 0), (0.2, 0.1, 0.05, 0.0))
    kref, vref, res = _packed_cache(w)
    q_bits = workloads.q_tensor(w)
    k, v = to_dev(kref), to_dev(vref)
    views = _views(w, range(4), res)
    full = rq.decode_attn(to_dev(q_bits), k, v, views).cpu().numpy()
    for l in range(4):
        one = rq.decode_attn(to_dev(q_bits[l:l + 1]), k, v, [views[l]]).cpu().numpy()
        np.testing.assert_allclose(one[0], full[l], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("name", ["tiny", "l4_b16_s4k"])
def test_bf16_baseline(name):
    w = workloads.WORKLOADS[name]
    if name == "l4_b16_s4k":
        w = w.with_batch(2).with_seq(1500)
    ks, vs = workloads.kv_tensors(w, 0), workloads.kv_tensors(w, 1)
    q_bits = workloads.q_tensor(w)
    out = rq.decode_attn_bf16(to_dev(q_bits), [to_dev(x) for x in ks], [to_dev(x) for x in vs]).cpu().numpy()
    expect = oracle.decode_attn(q_bits, [oracle.bf16_to_f64(x) for x in ks], [oracle.bf16_to_f64(x) for x in vs])
    assert_attn_close(out, expect)


@pytest.mark.parametrize("hq,hkv,d,n_loops", [(4, 4, 128, 2), (16, 2, 64, 3), (32, 1, 128, 2), (24, 8, 64, 1)])
def test_bf16_baseline_head_groupings(hq, hkv, d, n_loops):
    """G = 1, 8, 32 (two 16-row MFMA blocks) and 3, both head sizes, a ragged length."""
    bits = tuple([2] * (n_loops - 1) + [0])
    sig = tuple([0.1] * (n_loops - 1) + [0.0])
    w = workloads.Workload("bf16_groups", 94, n_loops, 2, hkv, hq, d, 257, bits, sig)
    ks, vs = workloads.kv_tensors(w, 0), workloads.kv_tensors(w, 1)
    q_bits = workloads.q_tensor(w)
    out = rq.decode_attn_bf16(to_dev(q_bits), [to_dev(x) for x in ks], [to_dev(x) for x in vs]).cpu().numpy()
    expect = oracle.decode_attn(q_bits, [oracle.bf16_to_f64(x) for x in ks], [oracle.bf16_to_f64(x) for x in vs])
    assert_attn_close(out, expect)


def test_final_loop_rq_equals_bf16_on_reference():
    w = workloads.Workload("final", 95, 1, 2, 2, 8, 128, 333, (0,), (0.0,))
    kref, vref = workloads.ref_tensor(w, 0), workloads.ref_tensor(w, 1)
    q = to_dev(workloads.q_tensor(w))
    a = rq.decode_attn(q, to_dev(kref), to_dev(vref), [rq.LoopView(0)])
    b = rq.decode_attn_bf16(q, [to_dev(kref)], [to_dev(vref)])
    torch.cuda.synchronize()
    np.testing.assert_allclose(a.cpu().numpy(), b.cpu().numpy(), rtol=1e-6, atol=1e-7)
