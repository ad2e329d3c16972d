"""The peak-batch workload at its largest batch, against the oracle on sampled
rows: the residual cache of 8 loops (INT4 loop 0, INT2 loops 1-6, bf16
reference) filling about 200 GB of HBM, and the bf16-KV baseline at its own
largest batch. These are the largest launches the library runs here (row
offsets past 2^31 elements). The batch is built on the device by repeating
eight host-drawn entries, so row (b, h) holds the generator's row (b % 8, h)."""
import numpy as np
import pytest
import torch

import looped_transformer_kv_rq_amd as rq
import oracle
import workloads
from rq_parity import assert_attn_close, compare_codes, to_dev, to_host_u16, to_host_words, words_to_dev

pytestmark = pytest.mark.gpu


def _budget():
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    return min(workloads.PEAK_CACHE_BUDGET, free - 16 * 2**30)


def _rows(batch):
    return [(0, 0), (batch - 1, 3), (batch // 2 + 3, 1), (1029 % batch, 2)]


def _q(q8, batch):
    return torch.stack([workloads.tile_batch(to_dev(q8[l]), batch) for l in range(q8.shape[0])])


def test_peak_batch_rq_decode_sampled_rows():
    w8 = workloads.WORKLOADS["peak_batch"].with_batch(workloads.PEAK_TILE)
    batch = workloads.peak_batch(workloads.cache_bytes_per_sequence(w8, w8.bits), _budget())
    print(f"peak batch rq: B = {batch}", flush=True)
    assert batch >= 8 * workloads.PEAK_TILE
    kref8 = workloads.ref_tensor(w8, workloads.TENSOR_K)
    vref8 = workloads.ref_tensor(w8, workloads.TENSOR_V)
    res8 = {l: (workloads.packed_tensors(w8, 0, l), workloads.packed_tensors(w8, 1, l))
            for l in range(w8.n_loops) if w8.bits[l]}
    q8 = workloads.q_tensor(w8)
    tile = workloads.tile_batch
    kref, vref = tile(to_dev(kref8), batch), tile(to_dev(vref8), batch)
    views = []
    for l in range(w8.n_loops):
        if w8.bits[l]:
            (kw, ks), (vw, vs) = res8[l]
            views.append(rq.LoopView(w8.bits[l], tile(words_to_dev(kw), batch), tile(to_dev(ks, torch.float16), batch),
                                     tile(words_to_dev(vw), batch), tile(to_dev(vs, torch.float16), batch)))
        else:
            views.append(rq.LoopView(0))
    out = rq.decode_attn(_q(q8, batch), kref, vref, views)
    torch.cuda.synchronize()
    g = w8.group_size
    rows = _rows(batch)
    got = np.stack([np.stack([out[l, b, h * g:(h + 1) * g].cpu().numpy() for (b, h) in rows])
                    for l in range(w8.n_loops)])
    del out, views, kref, vref
    torch.cuda.empty_cache()
    want = np.empty_like(got, dtype=np.float64)
    scale = 1.0 / np.sqrt(w8.head_dim)
    for j, (b, h) in enumerate(rows):
        t = b % workloads.PEAK_TILE
        for l in range(w8.n_loops):
            if w8.bits[l]:
                (kw, ks), (vw, vs) = res8[l]
                k = oracle.reconstruct(kref8[t, h], kw[t, h], ks[t, h], w8.bits[l])
                v = oracle.reconstruct(vref8[t, h], vw[t, h], vs[t, h], w8.bits[l])
            else:
                k, v = oracle.bf16_to_f64(kref8[t, h]), oracle.bf16_to_f64(vref8[t, h])
            want[l, j] = oracle.attention(oracle.bf16_to_f64(q8[l, t, h * g:(h + 1) * g]), k, v, scale)
    assert_attn_close(got, want)


def test_peak_batch_bf16_baseline_sampled_rows():
    """Every loop's K_l / V_l is its own allocation holding the reference's values."""
    w8 = workloads.WORKLOADS["peak_batch"].with_batch(workloads.PEAK_TILE)
    batch = workloads.peak_batch(workloads.bf16_cache_bytes_per_sequence(w8, w8.n_loops), _budget())
    print(f"peak batch bf16: B = {batch}", flush=True)
    assert batch >= 8 * workloads.PEAK_TILE
    kref8 = workloads.ref_tensor(w8, workloads.TENSOR_K)
    vref8 = workloads.ref_tensor(w8, workloads.TENSOR_V)
    q8 = workloads.q_tensor(w8)
    kd, vd = to_dev(kref8), to_dev(vref8)
    ks = [workloads.tile_batch(kd, batch) for _ in range(w8.n_loops)]
    vs = [workloads.tile_batch(vd, batch) for _ in range(w8.n_loops)]
    out = rq.decode_attn_bf16(_q(q8, batch), ks, vs)
    torch.cuda.synchronize()
    g = w8.group_size
    rows = _rows(batch)
    got = np.stack([np.stack([out[l, b, h * g:(h + 1) * g].cpu().numpy() for (b, h) in rows])
                    for l in range(w8.n_loops)])
    del out, ks, vs
    torch.cuda.empty_cache()
    want = np.empty_like(got, dtype=np.float64)
    scale = 1.0 / np.sqrt(w8.head_dim)
    for j, (b, h) in enumerate(rows):
        t = b % workloads.PEAK_TILE
        k, v = oracle.bf16_to_f64(kref8[t, h]), oracle.bf16_to_f64(vref8[t, h])
        for l in range(w8.n_loops):
            want[l, j] = oracle.attention(oracle.bf16_to_f64(q8[l, t, h * g:(h + 1) * g]), k, v, scale)
    assert_attn_close(got, want)


def test_peak_batch_encode_kv_sampled_rows():
    """rq_encode_kv of the seven residual loops of K and V in one launch, at the
    largest batch whose bf16 states and packed outputs fit the budget (element
    offsets past 2^32 in every state tensor), the launch the benchmark times:
    codes and scales of sampled rows against the oracle's."""
    w8 = workloads.WORKLOADS["peak_batch"].with_batch(workloads.PEAK_TILE)
    batch = workloads.peak_batch(workloads.encode_bytes_per_sequence(w8), _budget())
    print(f"peak batch encode: B = {batch}", flush=True)
    assert batch >= 8 * workloads.PEAK_TILE
    res = [l for l in range(w8.n_loops) if w8.bits[l]]
    bits = [w8.bits[l] for l in res]
    tile = workloads.tile_batch
    st = {}
    for tensor in (workloads.TENSOR_K, workloads.TENSOR_V):
        xs8 = workloads.kv_tensors(w8, tensor)
        st[tensor] = [tile(to_dev(x), batch) for x in xs8]
        del xs8
    shp = (batch, w8.n_kv_heads, w8.seq_len)
    codes = {t: [torch.empty(shp + (w8.head_dim * b // 32,), dtype=torch.int32, device="cuda") for b in bits]
             for t in st}
    scales = {t: [torch.empty(shp + (w8.head_dim // 32,), dtype=torch.float16, device="cuda") for _ in bits]
              for t in st}
    K, V = workloads.TENSOR_K, workloads.TENSOR_V
    rq.encode_kv_into([st[K][l] for l in res], [st[V][l] for l in res], st[K][-1], st[V][-1], bits,
                      codes[K], scales[K], codes[V], scales[V])
    torch.cuda.synchronize()
    rows = _rows(batch)
    got = {(t, i, b, h): (to_host_words(codes[t][i][b, h]), to_host_u16(scales[t][i][b, h]))
           for t in st for i in range(len(bits)) for (b, h) in rows}
    del st, codes, scales
    torch.cuda.empty_cache()
    for (b, h) in rows:
        for t in (K, V):
            row = workloads.kv_rows_all_loops(w8, b % workloads.PEAK_TILE, h, t)
            for i, l in enumerate(res):
                ow, os_ = oracle.encode(row[l], row[-1], bits[i])
                compare_codes(*got[(t, i, b, h)], ow, os_, row[l], row[-1], bits[i])
