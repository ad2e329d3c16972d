"""GPU parity of the block-paged serving step (rq_decode_attn_paged,
rq_encode_append_paged) against the oracle, and of the contiguous varlen
decode when the cache past each prefix holds non-finite bits.

Paged tensors are [n_blocks, Hkv, P, row]; the tests scatter a dense cache
into shuffled blocks, leave every block and position outside the cache
filled with NaN / Inf bit patterns, and compare with the oracle's decode
over the dense cache the table describes (oracle.gather_pages)."""
import numpy as np
import pytest
import torch

import looped_transformer_kv_rq_amd as rq
import oracle
import workloads
from rq_parity import assert_attn_close, compare_codes, to_dev, to_host_u16, to_host_words, words_to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16_NAN, F16_INF = 0x7FC0, 0x7C00


def _bf16(rng, shape, scale=1.0):
    return workloads.f32_to_bf16_bits((scale * rng.standard_normal(shape)).astype(np.float32))


def _dense_cache(rng, B, H, S, d, bits_per_loop):
    kref, vref = _bf16(rng, (B, H, S, d)), _bf16(rng, (B, H, S, d))
    res = {}
    for l, bl in enumerate(bits_per_loop):
        if bl:
            kx = workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(kref) + 0.2 * rng.standard_normal(
                kref.shape)).astype(np.float32))
            vx = workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(vref) + 0.2 * rng.standard_normal(
                vref.shape)).astype(np.float32))
            res[l] = (oracle.encode(kx, kref, bl), oracle.encode(vx, vref, bl))
    return kref, vref, res


def _table(rng, B, max_blocks, lens, P, spare):
    """Shuffled physical blocks for the positions below each length; -1 for the rest."""
    need = [(int(n) + P - 1) // P for n in lens]
    perm = rng.permutation(sum(need) + spare)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        for j in range(need[b]):
            table[b, j] = perm[k]
            k += 1
    return table, len(perm)


def _dense_from_pages(pages, table, P, S):
    """Dense [B, H, S, ...] copy of a paged cache read back from the device:
    position t of sequence b from block table[b, t // P]; unmapped blocks stay zero."""
    out = np.zeros((table.shape[0], pages.shape[1], S) + pages.shape[3:], dtype=pages.dtype)
    for b in range(table.shape[0]):
        for j in range(S // P):
            if 0 <= table[b, j] < pages.shape[0]:
                out[b, :, j * P:(j + 1) * P] = pages[table[b, j]]
    return out


def _scatter(dense, table, lens, P, n_blocks, fill):
    """Paged copy of dense [B, H, S, row]: positions below lens[b] only; the rest is `fill`."""
    B, H, S = dense.shape[:3]
    pages = np.full((n_blocks, H, P) + dense.shape[3:], fill, dtype=dense.dtype)
    for b in range(B):
        for t in range(int(lens[b])):
            pages[table[b, t // P], :, t % P] = dense[b, :, t]
    return pages


def _hat(kref, vref, res, bits_per_loop):
    kh, vh = [], []
    for l, bl in enumerate(bits_per_loop):
        if bl:
            (kw, ks), (vw, vs) = res[l]
            kh.append(oracle.reconstruct(kref, kw, ks, bl))
            vh.append(oracle.reconstruct(vref, vw, vs, bl))
        else:
            kh.append(oracle.bf16_to_f64(kref))
            vh.append(oracle.bf16_to_f64(vref))
    return kh, vh


# hq = 8 (G = 4) with 8 loops and hq = 16 (G = 8) with 4 loops: 32 query rows
# per kv head, so the launch runs two 16-row argument sets
@pytest.mark.parametrize("d,P,bits_per_loop,tail,hq", [
    (128, 64, (2, 4, 0), 0, 8), (128, 128, (2, 2, 0), 1, 8), (64, 64, (8, 3, 0), 2, 8), (128, 256, (4, 2, 2, 0), 1, 8),
    (128, 64, (2, 4, 2, 2, 2, 2, 2, 0), 1, 8), (64, 128, (8, 3, 2, 0), 0, 16), (128, 64, (8, 2, 2, 0), 1, 8),
    (128, 128, (4, 4, 2, 0), 1, 8)])
def test_paged_decode_matches_oracle(d, P, bits_per_loop, tail, hq):
    print(f"paged d={d} P={P} bits={bits_per_loop} tail={tail} hq={hq}", flush=True)
    rng = np.random.default_rng(d + P + tail + hq)
    L, B, H, max_blocks = len(bits_per_loop), 6, 2, 4
    S = max_blocks * P
    lens = np.array([0, 1, P - 1, P, P + 1, S], dtype=np.int32)
    kref, vref, res = _dense_cache(rng, B, H, S, d, bits_per_loop)
    table, n_blocks = _table(rng, B, max_blocks, lens, P, spare=2)
    views = []
    for l, bl in enumerate(bits_per_loop):
        if bl:
            (kw, ks), (vw, vs) = res[l]
            pk = [_scatter(kw, table, lens, P, n_blocks, 0xFFFFFFFF), _scatter(ks, table, lens, P, n_blocks, F16_INF)]
            pv = [_scatter(vw, table, lens, P, n_blocks, 0xFFFFFFFF), _scatter(vs, table, lens, P, n_blocks, F16_INF)]
            views.append(rq.LoopView(bl, words_to_dev(pk[0]), to_dev(pk[1], torch.float16), words_to_dev(pv[0]),
                                     to_dev(pv[1], torch.float16)))
        else:
            views.append(rq.LoopView(0))
    kp = _scatter(kref, table, lens, P, n_blocks, BF16_NAN)
    vp = _scatter(vref, table, lens, P, n_blocks, BF16_NAN)
    q = _bf16(rng, (L, B, hq, d))
    tk = tv = None
    if tail:
        tk = [_bf16(rng, (B, H, tail, d)) for _ in range(L)]
        tv = [_bf16(rng, (B, H, tail, d)) for _ in range(L)]
    out = rq.decode_attn_paged(to_dev(q), to_dev(kp), to_dev(vp), views, torch.from_numpy(table).to(DEV),
                               seq_lens=torch.from_numpy(lens).to(DEV),
                               tail_k=None if tk is None else [to_dev(x) for x in tk],
                               tail_v=None if tv is None else [to_dev(x) for x in tv]).cpu().numpy()
    assert np.all(np.isfinite(out))
    # the oracle reads the dense cache the table describes
    assert np.array_equal(oracle.gather_pages(kp, table, P, S)[1, :, :1], kref[1, :, :1])
    kh, vh = _hat(kref, vref, res, bits_per_loop)
    expect = oracle.decode_attn_varlen(q, kh, vh, lens, tk, tv)
    if not tail:
        assert np.all(out[:, 0] == 0)  # sequence 0 has no position at all
        assert_attn_close(out[:, 1:], expect[:, 1:])
    else:
        assert_attn_close(out, expect)


@pytest.mark.parametrize("d,P,bits_per_loop,tail,hq", [
    (128, 64, (2, 4, 0), 0, 8), (128, 128, (4, 2, 2, 0), 1, 8), (64, 64, (8, 3, 0), 1, 8),
    (128, 64, (2, 4, 2, 2, 2, 2, 2, 0), 0, 8), (128, 128, (8, 4, 2, 0), 1, 8)])
def test_paged_decode_missing_block_inside_prefix(d, P, bits_per_loop, tail, hq):
    """Table entries that are not blocks (-1, and one past n_blocks) inside
    [0, seq_lens[b]): their positions take no weight, as the oracle's
    pages_present reading says; sequence 2's every block is missing."""
    print(f"paged holes d={d} P={P} bits={bits_per_loop} tail={tail} hq={hq}", flush=True)
    rng = np.random.default_rng(7 * d + P + tail)
    L, B, H, max_blocks = len(bits_per_loop), 4, 2, 4
    S = max_blocks * P
    lens = np.array([S, 3 * P - 5, 2 * P, P + 40], dtype=np.int32)
    kref, vref, res = _dense_cache(rng, B, H, S, d, bits_per_loop)
    table, n_blocks = _table(rng, B, max_blocks, np.full(B, S), P, spare=1)
    table[0, 1] = -1
    table[1, 0] = -1
    table[1, 2] = n_blocks + 3  # not a block either
    table[2, :] = -1
    table[3, 1] = -1  # the block holding the last, partial tile
    present = oracle.pages_present(table, P, n_blocks, S)
    assert not present[0, P] and present[0, 2 * P] and not present[1, 0] and not present[3, P]
    views = []
    for l, bl in enumerate(bits_per_loop):
        if bl:
            (kw, ks), (vw, vs) = res[l]
            pk = [_scatter_present(kw, table, lens, P, n_blocks, 0xFFFFFFFF),
                  _scatter_present(ks, table, lens, P, n_blocks, F16_INF)]
            pv = [_scatter_present(vw, table, lens, P, n_blocks, 0xFFFFFFFF),
                  _scatter_present(vs, table, lens, P, n_blocks, F16_INF)]
            views.append(rq.LoopView(bl, words_to_dev(pk[0]), to_dev(pk[1], torch.float16), words_to_dev(pv[0]),
                                     to_dev(pv[1], torch.float16)))
        else:
            views.append(rq.LoopView(0))
    kp = _scatter_present(kref, table, lens, P, n_blocks, BF16_NAN)
    vp = _scatter_present(vref, table, lens, P, n_blocks, BF16_NAN)
    q = _bf16(rng, (L, B, hq, d))
    tk = tv = None
    if tail:
        tk = [_bf16(rng, (B, H, tail, d)) for _ in range(L)]
        tv = [_bf16(rng, (B, H, tail, d)) for _ in range(L)]
    out = rq.decode_attn_paged(to_dev(q), to_dev(kp), to_dev(vp), views, torch.from_numpy(table).to(DEV),
                               seq_lens=torch.from_numpy(lens).to(DEV),
                               tail_k=None if tk is None else [to_dev(x) for x in tk],
                               tail_v=None if tv is None else [to_dev(x) for x in tv]).cpu().numpy()
    assert np.all(np.isfinite(out))
    kh, vh = _hat(kref, vref, res, bits_per_loop)
    expect = oracle.decode_attn_varlen(q, kh, vh, lens, tk, tv, present=present)
    if not tail:
        assert np.all(out[:, 2] == 0)  # sequence 2 has no position at all
    assert_attn_close(out, expect)


def _scatter_present(dense, table, lens, P, n_blocks, fill):
    """Paged copy of dense [B, H, S, row] for positions below lens[b] whose
    table entry is a block; everything else is `fill`."""
    B, H, S = dense.shape[:3]
    pages = np.full((n_blocks, H, P) + dense.shape[3:], fill, dtype=dense.dtype)
    for b in range(B):
        for t in range(int(lens[b])):
            blk = int(table[b, t // P])
            if 0 <= blk < n_blocks:
                pages[blk, :, t % P] = dense[b, :, t]
    return pages


@pytest.mark.parametrize("bits_per_loop,hq", [((2, 2, 0), 8), ((4, 2, 2, 2, 2, 2, 2, 0), 8)])
def test_paged_equals_contiguous_varlen(bits_per_loop, hq):
    """The same cache, dense or scattered into shuffled blocks: identical results
    (the 8-loop case runs two argument sets)."""
    rng = np.random.default_rng(5)
    B, H, d, P, max_blocks = 3, 2, 128, 128, 3
    S = P * max_blocks
    lens = np.array([S, 200, 77], dtype=np.int32)
    kref, vref, res = _dense_cache(rng, B, H, S, d, bits_per_loop)
    table, n_blocks = _table(rng, B, max_blocks, np.full(B, S), P, spare=1)
    q = to_dev(_bf16(rng, (len(bits_per_loop), B, hq, d)))
    dense_views, paged_views = [], []
    for l, bl in enumerate(bits_per_loop):
        if bl:
            (kw, ks), (vw, vs) = res[l]
            dense_views.append(rq.LoopView(bl, words_to_dev(kw), to_dev(ks, torch.float16), words_to_dev(vw),
                                           to_dev(vs, torch.float16)))
            full = np.full(B, S)
            paged_views.append(rq.LoopView(
                bl, words_to_dev(_scatter(kw, table, full, P, n_blocks, 0)),
                to_dev(_scatter(ks, table, full, P, n_blocks, 0), torch.float16),
                words_to_dev(_scatter(vw, table, full, P, n_blocks, 0)),
                to_dev(_scatter(vs, table, full, P, n_blocks, 0), torch.float16)))
        else:
            dense_views.append(rq.LoopView(0))
            paged_views.append(rq.LoopView(0))
    full = np.full(B, S)
    lens_d = torch.from_numpy(lens).to(DEV)
    a = rq.decode_attn_varlen(q, to_dev(kref), to_dev(vref), dense_views, seq_lens=lens_d)
    b = rq.decode_attn_paged(q, to_dev(_scatter(kref, table, full, P, n_blocks, 0)),
                             to_dev(_scatter(vref, table, full, P, n_blocks, 0)), paged_views,
                             torch.from_numpy(table).to(DEV), seq_lens=lens_d)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("bits", [(2, 4), (8, 3)])
def test_paged_append_writes_exactly_the_new_positions(bits):
    rng = np.random.default_rng(sum(bits))
    B, H, d, P, max_blocks, t_new = 4, 2, 128, 64, 3, 3
    S = P * max_blocks
    bits = list(bits)
    ref_new = _bf16(rng, (B, H, t_new, d))
    xs = [workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(ref_new) + 0.2 * rng.standard_normal(
        ref_new.shape)).astype(np.float32)) for _ in bits]
    # sequence 0 crosses from block 0 into block 1; sequence 2 runs past the capacity;
    # sequence 3's second block is not there (-1)
    pos = np.array([P - 2, 5, S - 1, P - 1], dtype=np.int32)
    table = np.array([[4, 0, 7], [2, 5, 6], [1, 3, 8], [9, -1, 10]], dtype=np.int32)
    n_blocks = 11
    codes = [torch.full((n_blocks, H, P, d * b // 32), 0x5A5A5A5A, dtype=torch.int32, device=DEV) for b in bits]
    scales = [torch.full((n_blocks, H, P, d // 32), 7.0, dtype=torch.float16, device=DEV) for _ in bits]
    ref_pages = torch.full((n_blocks, H, P, d), 3.0, dtype=torch.bfloat16, device=DEV)
    rq.encode_append_paged([to_dev(x) for x in xs], to_dev(ref_new), bits, torch.from_numpy(pos).to(DEV),
                           torch.from_numpy(table).to(DEV), ref_pages, codes, scales)
    torch.cuda.synchronize()
    written = np.zeros((n_blocks, P), dtype=bool)
    where = {}
    for b in range(B):
        for t in range(t_new):
            p = int(pos[b]) + t
            if 0 <= p < S and table[b, p // P] >= 0:
                blk, off = int(table[b, p // P]), p % P
                written[blk, off] = True
                where[(b, t)] = (blk, off)
    assert len(where) == B * t_new - 2 - 2  # two past the capacity, two into the missing block
    rp = to_host_u16(ref_pages)
    for (b, t), (blk, off) in where.items():
        np.testing.assert_array_equal(rp[blk, :, off], ref_new[b, :, t])
    sentinel = to_host_u16(torch.full((1,), 3.0, dtype=torch.bfloat16))[0]
    assert np.all(rp.transpose(0, 2, 1, 3)[~written] == sentinel)
    for i, bl in enumerate(bits):
        cw, cs = to_host_words(codes[i]), to_host_u16(scales[i])
        assert np.all(cw.transpose(0, 2, 1, 3)[~written] == 0x5A5A5A5A)
        ow, os_ = oracle.encode(xs[i], ref_new, bl)
        for (b, t), (blk, off) in where.items():
            compare_codes(cw[blk, :, off], cs[blk, :, off], ow[b, :, t], os_[b, :, t], xs[i][b, :, t],
                          ref_new[b, :, t], bl)


def test_paged_serving_steps_append_then_decode():
    """Prefill into pages with one append of every sequence's prefix, then three
    decode steps that attend over the pages plus the current position's bf16
    loop states and append that position."""
    rng = np.random.default_rng(43)
    bits = [2, 4]
    L = len(bits) + 1
    B, H, d, hq, P, max_blocks = 3, 2, 128, 8, 64, 3
    S = P * max_blocks
    lens = np.array([5, 63, 120], dtype=np.int32)
    kref_all, vref_all = _bf16(rng, (B, H, S, d)), _bf16(rng, (B, H, S, d))
    kl = [workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(kref_all) + 0.15 * rng.standard_normal(
        kref_all.shape)).astype(np.float32)) for _ in bits] + [kref_all]
    vl = [workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(vref_all) + 0.15 * rng.standard_normal(
        vref_all.shape)).astype(np.float32)) for _ in bits] + [vref_all]
    table_np, n_blocks = _table(rng, B, max_blocks, np.full(B, S), P, spare=0)
    table = torch.from_numpy(table_np).to(DEV)
    kc = [torch.zeros((n_blocks, H, P, d * b // 32), dtype=torch.int32, device=DEV) for b in bits]
    ks = [torch.zeros((n_blocks, H, P, d // 32), dtype=torch.float16, device=DEV) for _ in bits]
    vc = [torch.zeros_like(t) for t in kc]
    vs = [torch.zeros_like(t) for t in ks]
    kref_p = torch.zeros((n_blocks, H, P, d), dtype=torch.bfloat16, device=DEV)
    vref_p = torch.zeros_like(kref_p)
    n0 = int(lens.max())
    zero = torch.zeros(B, dtype=torch.int32, device=DEV)
    for src, codes, scales, refp in ((kl, kc, ks, kref_p), (vl, vc, vs, vref_p)):
        rq.encode_append_paged([to_dev(x[:, :, :n0]) for x in src[:-1]], to_dev(src[-1][:, :, :n0]), bits, zero,
                               table, refp, codes, scales)
    views = [rq.LoopView(b, kc[i], ks[i], vc[i], vs[i]) for i, b in enumerate(bits)] + [rq.LoopView(0)]
    # the oracle's cache: its own encode of every loop's whole history, dense
    khat = [oracle.reconstruct(kl[-1], *oracle.encode(kl[i], kl[-1], bl), bl) for i, bl in enumerate(bits)]
    vhat = [oracle.reconstruct(vl[-1], *oracle.encode(vl[i], vl[-1], bl), bl) for i, bl in enumerate(bits)]
    khat.append(oracle.bf16_to_f64(kl[-1]))
    vhat.append(oracle.bf16_to_f64(vl[-1]))
    lens_now = lens.copy()
    for step in range(3):
        q = _bf16(rng, (L, B, hq, d))
        tail_k = [np.stack([kl[l][b, :, lens_now[b]:lens_now[b] + 1] for b in range(B)]) for l in range(L)]
        tail_v = [np.stack([vl[l][b, :, lens_now[b]:lens_now[b] + 1] for b in range(B)]) for l in range(L)]
        out = rq.decode_attn_paged(to_dev(q), kref_p, vref_p, views, table,
                                   seq_lens=torch.from_numpy(lens_now).to(DEV),
                                   tail_k=[to_dev(x) for x in tail_k], tail_v=[to_dev(x) for x in tail_v])
        expect = oracle.decode_attn_varlen(q, khat, vhat, lens_now, tail_k, tail_v)
        assert_attn_close(out.cpu().numpy(), expect)
        pos = torch.from_numpy(lens_now).to(DEV)
        for codes, scales, refp, tail in ((kc, ks, kref_p, tail_k), (vc, vs, vref_p, tail_v)):
            rq.encode_append_paged([to_dev(tail[l]) for l in range(len(bits))], to_dev(tail[-1]), bits, pos, table,
                                   refp, codes, scales)
        lens_now = lens_now + 1
    torch.cuda.synchronize()
    kr = _dense_from_pages(to_host_u16(kref_p), table_np, P, S)
    for b in range(B):
        n = int(lens_now[b])
        np.testing.assert_array_equal(kr[b, :, :n], kl[-1][b, :, :n])
        for i, bl in enumerate(bits):
            cw = _dense_from_pages(to_host_words(kc[i]), table_np, P, S)
            cs = _dense_from_pages(to_host_u16(ks[i]), table_np, P, S)
            ow, os_ = oracle.encode(kl[i][b, :, :n], kl[-1][b, :, :n], bl)
            compare_codes(cw[b, :, :n], cs[b, :, :n], ow, os_, kl[i][b, :, :n], kl[-1][b, :, :n], bl)


def test_varlen_ignores_non_finite_bits_past_each_prefix():
    """Contiguous cache: positions at and past seq_lens[b] hold NaN / Inf bit
    patterns; they take no weight and cannot reach the output."""
    rng = np.random.default_rng(17)
    bits_per_loop = (2, 4, 0)
    B, H, S, d = 4, 2, 256, 128
    lens = np.array([1, 63, 100, 255], dtype=np.int32)
    kref, vref, res = _dense_cache(rng, B, H, S, d, bits_per_loop)
    kh, vh = _hat(kref, vref, res, bits_per_loop)
    past = np.arange(S)[None, :] >= lens[:, None]  # [B, S]
    mask = past[:, None, :]
    kref[np.broadcast_to(mask, kref.shape[:3])] = BF16_NAN
    vref[np.broadcast_to(mask, vref.shape[:3])] = BF16_NAN
    views = []
    for l, bl in enumerate(bits_per_loop):
        if bl:
            (kw, ks), (vw, vs) = res[l]
            kw, ks, vw, vs = kw.copy(), ks.copy(), vw.copy(), vs.copy()
            for arr, val in ((ks, F16_INF), (vs, F16_INF)):
                arr[np.broadcast_to(mask, arr.shape[:3])] = val
            views.append(rq.LoopView(bl, words_to_dev(kw), to_dev(ks, torch.float16), words_to_dev(vw),
                                     to_dev(vs, torch.float16)))
        else:
            views.append(rq.LoopView(0))
    q = _bf16(rng, (3, B, 8, d))
    out = rq.decode_attn_varlen(to_dev(q), to_dev(kref), to_dev(vref), views,
                                seq_lens=torch.from_numpy(lens).to(DEV)).cpu().numpy()
    assert np.all(np.isfinite(out))
    assert_attn_close(out, oracle.decode_attn_varlen(q, kh, vh, lens))


def test_serving_step_full_size_sampled_rows():
    """The launches the benchmark's serving legs time, at full size: the
    l4_b16_s4k cache encoded on the GPU, prefix lengths drawn in [S/2, S) as
    the benchmark draws them, one bf16 tail position per loop, decoded over the
    dense cache and over a copy in 512 shuffled blocks of 128 positions;
    sampled (batch, kv head) rows against the oracle: their codes, then their
    decode over the oracle's codes."""
    w = workloads.WORKLOADS["l4_b16_s4k"]
    bits = [b for b in w.bits if b]
    P, nbs = 128, w.seq_len // 128
    kx = [to_dev(x) for x in workloads.kv_tensors(w, workloads.TENSOR_K)]
    vx = [to_dev(x) for x in workloads.kv_tensors(w, workloads.TENSOR_V)]
    kc, ks = rq.encode(kx[:-1], kx[-1], bits)
    vc, vs = rq.encode(vx[:-1], vx[-1], bits)
    torch.cuda.synchronize()
    rows = [(0, 0), (7, 3), (15, 7)]
    # The GPU's codes of the sampled rows against the oracle's own encode. Then
    # those rows take the oracle's codes, so the decodes below run on exactly the
    # oracle's inputs there: a code the two round to opposite sides of a decision
    # boundary (allowed above) moves that token's score by up to s/sqrt(D).
    orc = {}
    for (b, h) in rows:
        k_st = workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_K)
        v_st = workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_V)
        for l, bl in enumerate(bits):  # the residual loops are loops 0 .. L-2, in order
            okw, oks = oracle.encode(k_st[l], k_st[-1], bl)
            ovw, ovs = oracle.encode(v_st[l], v_st[-1], bl)
            compare_codes(to_host_words(kc[l][b, h]), to_host_u16(ks[l][b, h]), okw, oks, k_st[l], k_st[-1], bl)
            compare_codes(to_host_words(vc[l][b, h]), to_host_u16(vs[l][b, h]), ovw, ovs, v_st[l], v_st[-1], bl)
            kc[l][b, h] = words_to_dev(okw)
            ks[l][b, h] = to_dev(oks, torch.float16)
            vc[l][b, h] = words_to_dev(ovw)
            vs[l][b, h] = to_dev(ovs, torch.float16)
            orc[(b, h, l)] = (okw, oks, ovw, ovs)
    views = [rq.LoopView(b, kc[i], ks[i], vc[i], vs[i]) for i, b in enumerate(bits)] + [rq.LoopView(0)]
    lens = np.random.default_rng(w.seed).integers(w.seq_len // 2, w.seq_len, size=w.batch).astype(np.int32)
    lens_d = torch.from_numpy(lens).to(DEV)
    tk = [x[:, :, :1].contiguous() for x in kx]
    tv = [x[:, :, :1].contiguous() for x in vx]
    q_bits = workloads.q_tensor(w)
    q = to_dev(q_bits)
    dense = rq.decode_attn_varlen(q, kx[-1], vx[-1], views, seq_lens=lens_d, tail_k=tk, tail_v=tv).cpu().numpy()
    perm = torch.from_numpy(np.random.default_rng(w.seed + 1).permutation(w.batch * nbs)).to(DEV)
    table = perm.view(w.batch, nbs).to(torch.int32).contiguous()

    def paged(t):
        blocks = t.view(w.batch, w.n_kv_heads, nbs, P, t.shape[-1]).permute(0, 2, 1, 3, 4)
        blocks = blocks.reshape(w.batch * nbs, w.n_kv_heads, P, t.shape[-1])
        out = torch.empty_like(blocks)
        out[perm] = blocks
        return out

    pviews = [rq.LoopView(b, paged(kc[i]), paged(ks[i]), paged(vc[i]), paged(vs[i])) for i, b in enumerate(bits)]
    pviews.append(rq.LoopView(0))
    pag = rq.decode_attn_paged(q, paged(kx[-1]), paged(vx[-1]), pviews, table, seq_lens=lens_d, tail_k=tk,
                               tail_v=tv).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(dense, pag)  # the same cache, dense or paged: identical results
    g = w.group_size
    for (b, h) in rows:
        n = int(lens[b])
        k_st = workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_K)
        v_st = workloads.kv_rows_all_loops(w, b, h, workloads.TENSOR_V)
        for l in range(w.n_loops):
            if w.bits[l]:
                okw, oks, ovw, ovs = orc[(b, h, l)]
                k = oracle.reconstruct(k_st[-1], okw, oks, w.bits[l])
                v = oracle.reconstruct(v_st[-1], ovw, ovs, w.bits[l])
            else:
                k, v = oracle.bf16_to_f64(k_st[-1]), oracle.bf16_to_f64(v_st[-1])
            k = np.concatenate([k[:n], oracle.bf16_to_f64(k_st[l][:1])])
            v = np.concatenate([v[:n], oracle.bf16_to_f64(v_st[l][:1])])
            qq = oracle.bf16_to_f64(q_bits[l, b, h * g:(h + 1) * g])
            assert_attn_close(dense[l, b, h * g:(h + 1) * g], oracle.attention(qq, k, v, 1.0 / np.sqrt(w.head_dim)))
    del kx, vx, kc, ks, vc, vs
    torch.cuda.empty_cache()
