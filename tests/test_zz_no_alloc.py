"""rq_decode_attn_noalloc (the decode for callers that cannot allocate)
against rq_decode_attn with its own workspace: the same kernels and split
plan, so the outputs must be identical. Two calls in a row, the second with a
smaller input, so the second reads the scratch the first left behind."""
import numpy as np
import pytest
import torch

import looped_transformer_kv_rq_amd as rq
import workloads
from rq_parity import to_dev, words_to_dev

pytestmark = pytest.mark.gpu


def _case(w):
    """Generator-made residual cache of workload w (random packed codes)."""
    kref = to_dev(workloads.ref_tensor(w, workloads.TENSOR_K))
    vref = to_dev(workloads.ref_tensor(w, workloads.TENSOR_V))
    views = []
    for l in range(w.n_loops):
        if w.bits[l]:
            (kw, ks), (vw, vs) = workloads.packed_tensors(w, 0, l), workloads.packed_tensors(w, 1, l)
            views.append(rq.LoopView(w.bits[l], words_to_dev(kw), to_dev(ks, torch.float16), words_to_dev(vw),
                                     to_dev(vs, torch.float16)))
        else:
            views.append(rq.LoopView(0))
    return to_dev(workloads.q_tensor(w)), kref, vref, views


def test_noalloc_equals_decode_attn_twice_second_smaller():
    big = workloads.Workload("noalloc_big", 81, 4, 4, 8, 32, 128, 3000, (4, 2, 2, 0), (0.2, 0.1, 0.05, 0.0))
    small = workloads.Workload("noalloc_small", 82, 3, 2, 2, 8, 64, 777, (8, 3, 0), (0.2, 0.1, 0.0))
    need = [rq.decode_workspace_bytes(w.batch, w.n_kv_heads, w.seq_len, w.head_dim, w.n_q_heads, w.n_loops)
            for w in (big, small)]
    assert need[0] > need[1] and need[0] <= rq.NOALLOC_SCRATCH_BYTES
    for w in (big, small):
        print(f"noalloc {w.name}", flush=True)
        q, kref, vref, views = _case(w)
        want = rq.decode_attn(q, kref, vref, views)
        out = torch.full_like(want, float("nan"))
        got = rq.decode_attn_noalloc(q, kref, vref, views, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.isfinite(got).all()
        assert torch.equal(got, want)
        # an explicit split count, as rq_decode_attn with the same count
        want3 = rq.decode_attn(q, kref, vref, views, n_splits=3)
        got3 = rq.decode_attn_noalloc(q, kref, vref, views, n_splits=3)
        torch.cuda.synchronize()
        assert torch.equal(got3, want3)


def test_noalloc_equals_decode_attn_with_many_wave_blocks():
    """An INT8 table whose 16-row blocks run six waves and whose automatic plan
    counts rounds of 256 blocks: the scratch holds that plan's partials too."""
    w = workloads.Workload("noalloc_wide", 84, 4, 4, 4, 16, 128, 2000, (8, 4, 2, 0), (0.2, 0.1, 0.05, 0.0))
    assert rq.decode_splits(w.batch, w.n_kv_heads, w.seq_len, w.head_dim, w.n_q_heads, w.n_loops,
                            bits=list(w.bits)) != rq.decode_splits(w.batch, w.n_kv_heads, w.seq_len, w.head_dim,
                                                                  w.n_q_heads, w.n_loops)
    print(f"noalloc {w.name}", flush=True)
    q, kref, vref, views = _case(w)
    want = rq.decode_attn(q, kref, vref, views)
    got = rq.decode_attn_noalloc(q, kref, vref, views)
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    assert torch.equal(got, want)


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    """A call whose workspace would exceed the scratch is refused before any
    launch, and the output is left as it was."""
    w = workloads.Workload("noalloc_huge", 83, 2, 64, 8, 256, 64, 4096, (2, 0), (0.1, 0.0))
    splits = 4
    assert rq.decode_splits(w.batch, w.n_kv_heads, w.seq_len, w.head_dim, w.n_q_heads, w.n_loops, splits) == splits
    need = rq.decode_workspace_bytes(w.batch, w.n_kv_heads, w.seq_len, w.head_dim, w.n_q_heads, w.n_loops,
                                     n_splits=splits)
    assert need > rq.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((w.n_loops, w.batch, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((w.batch, w.n_kv_heads, w.seq_len, w.head_dim), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((w.batch, w.n_kv_heads, w.seq_len, w.head_dim * 2 // 32), dtype=torch.int32, device="cuda")
    scales = torch.zeros((w.batch, w.n_kv_heads, w.seq_len, w.head_dim // 32), dtype=torch.float16, device="cuda")
    views = [rq.LoopView(2, codes, scales, codes, scales), rq.LoopView(0)]
    out = torch.full((w.n_loops, w.batch, w.n_q_heads, w.head_dim), 7.0, device="cuda")
    with pytest.raises(rq.RQError) as e:
        rq.decode_attn_noalloc(q, k, k, views, n_splits=splits, out=out)
    assert e.value.status == rq.RQ_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
