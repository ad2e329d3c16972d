"""GPU parity of the serving-loop entry points: rq_encode_append (new
positions into a cache at per-sequence positions) and rq_decode_attn_varlen
(per-sequence prefix lengths plus bf16 tail positions), against the oracle."""
import numpy as np
import pytest
import torch

import looped_transformer_kv_rq_amd as rq
import oracle
import workloads
from rq_parity import assert_attn_close, compare_codes, to_dev, to_host_u16, to_host_words, words_to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf16(rng, shape, scale=1.0):
    return workloads.f32_to_bf16_bits((scale * rng.standard_normal(shape)).astype(np.float32))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("t_new", [1, 3])
@pytest.mark.parametrize("bits", [(2, 4), (8, 3)])
def test_append_writes_exactly_the_new_positions(d, t_new, bits):
    print(f"append d={d} t_new={t_new} bits={bits}", flush=True)
    rng = np.random.default_rng(d + t_new)
    B, H, S = 4, 2, 40
    bits = list(bits)
    ref_new = _bf16(rng, (B, H, t_new, d))
    xs = [workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(ref_new) + 0.2 * rng.standard_normal(
        ref_new.shape)).astype(np.float32)) for _ in bits]
    pos = np.array([0, 17, S - 2, -1], dtype=np.int32)  # the last two run past / start before the cache
    codes = [torch.full((B, H, S, d * b // 32), 0x5A5A5A5A, dtype=torch.int32, device=DEV) for b in bits]
    scales = [torch.full((B, H, S, d // 32), 7.0, dtype=torch.float16, device=DEV) for _ in bits]
    ref_cache = torch.full((B, H, S, d), 3.0, dtype=torch.bfloat16, device=DEV)
    rq.encode_append([to_dev(x) for x in xs], to_dev(ref_new), bits, torch.from_numpy(pos).to(DEV), ref_cache,
                     codes, scales)
    torch.cuda.synchronize()
    rc = to_host_u16(ref_cache)
    sentinel_ref = to_host_u16(torch.full((1,), 3.0, dtype=torch.bfloat16))[0]
    written = np.zeros((B, S), dtype=bool)
    for b in range(B):
        for t in range(t_new):
            p = int(pos[b]) + t
            if 0 <= p < S:
                written[b, p] = True
                np.testing.assert_array_equal(rc[b, :, p], ref_new[b, :, t])
    assert np.all(rc.transpose(0, 2, 1, 3)[~written] == sentinel_ref)
    for i, bl in enumerate(bits):
        cw = to_host_words(codes[i])
        cs = to_host_u16(scales[i])
        assert np.all(cw.transpose(0, 2, 1, 3)[~written] == 0x5A5A5A5A)
        assert np.all(cs.transpose(0, 2, 1, 3)[~written] == to_host_u16(torch.full((1,), 7.0, dtype=torch.float16))[0])
        ow, os_ = oracle.encode(xs[i], ref_new, bl)
        for b in range(B):
            for t in range(t_new):
                p = int(pos[b]) + t
                if 0 <= p < S:
                    compare_codes(cw[b, :, p], cs[b, :, p], ow[b, :, t], os_[b, :, t], xs[i][b, :, t],
                                  ref_new[b, :, t], bl)


def _cache(rng, B, H, S, d, bits_per_loop):
    """Oracle-encoded cache: bf16 refs, and per residual loop the oracle's codes."""
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


def _views(res, bits_per_loop):
    out = []
    for l, bl in enumerate(bits_per_loop):
        if bl:
            (kw, ks), (vw, vs) = res[l]
            out.append(rq.LoopView(bl, words_to_dev(kw), to_dev(ks, torch.float16), words_to_dev(vw),
                                   to_dev(vs, torch.float16)))
        else:
            out.append(rq.LoopView(0))
    return out


@pytest.mark.parametrize("d,hq,tail,bits_per_loop", [
    (128, 8, 0, (4, 2, 0)), (128, 8, 1, (4, 2, 0)), (64, 16, 3, (4, 2, 0)), (128, 4, 2, (4, 2, 0)),
    (128, 8, 1, (8, 2, 2, 0)), (128, 8, 0, (8, 4, 2, 0)), (128, 8, 1, (4, 4, 4, 0))])
def test_varlen_decode_matches_oracle(d, hq, tail, bits_per_loop):
    """The last three cases run seven- and six-wave blocks (INT8, and three
    INT4 loops) over length-balanced splits."""
    print(f"varlen d={d} hq={hq} tail={tail} bits={bits_per_loop}", flush=True)
    rng = np.random.default_rng(d + hq + tail + (0 if len(bits_per_loop) == 3 else 100 + bits_per_loop[1]))
    L, B, H, S = len(bits_per_loop), 7, 2, 200
    lens = np.array([0, 1, 63, 64, 65, 131, 200], dtype=np.int32)
    kref, vref, res = _cache(rng, B, H, S, d, bits_per_loop)
    q = _bf16(rng, (L, B, hq, d))
    tk = tv = None
    if tail:
        tk = [_bf16(rng, (B, H, tail, d)) for _ in range(L)]
        tv = [_bf16(rng, (B, H, tail, d)) for _ in range(L)]
    out = rq.decode_attn_varlen(to_dev(q), to_dev(kref), to_dev(vref), _views(res, bits_per_loop),
                                seq_lens=torch.from_numpy(lens).to(DEV),
                                tail_k=None if tk is None else [to_dev(x) for x in tk],
                                tail_v=None if tv is None else [to_dev(x) for x in tv]).cpu().numpy()
    kh, vh = _hat(kref, vref, res, bits_per_loop)
    expect = oracle.decode_attn_varlen(q, kh, vh, lens, tk, tv)
    if not tail:
        assert np.all(out[:, 0] == 0)  # sequence 0 has no position at all
        assert_attn_close(out[:, 1:], expect[:, 1:])
    else:
        assert_attn_close(out, expect)


@pytest.mark.parametrize("case", ["many_rows", "one_long", "rows_past_target"])
@pytest.mark.parametrize("tail", [0, 1])
def test_varlen_balanced_splits_match_oracle(case, tail):
    """The automatic split plan of a ragged decode balances its splits over the
    actual lengths. many_rows: 70 sequences (more than one 64-wide scan chunk),
    lengths from 0 to the capacity. one_long: one sequence at the capacity and
    fifteen short ones, so the long row's split count reaches its cap and its
    splits grow instead. rows_past_target: 300 sequences x 2 KV heads, more
    (batch, kv head) rows than the 512 blocks a launch aims at, so every
    sequence keeps one split."""
    print(f"varlen balanced case={case} tail={tail}", flush=True)
    rng = np.random.default_rng(7 + tail + {"many_rows": 0, "one_long": 100, "rows_past_target": 200}[case])
    if case == "many_rows":
        bits_per_loop, B, H, S, d, hq = [4, 2, 0], 70, 2, 512, 128, 8
        lens = rng.integers(0, S + 1, size=B).astype(np.int32)
        lens[:4] = [0, S, 1, 64]
    elif case == "rows_past_target":
        bits_per_loop, B, H, S, d, hq = [2, 0], 300, 2, 192, 64, 4
        lens = rng.integers(0, S + 1, size=B).astype(np.int32)
        lens[:3] = [0, S, 65]
    else:
        bits_per_loop, B, H, S, d, hq = [2, 0], 16, 4, 4096, 64, 16
        lens = np.array([S, 0, 1, 5, 63, 64, 65, 100, 2, 3, 40, 17, 0, 9, 128, 33], dtype=np.int32)
    L = len(bits_per_loop)
    kref, vref, res = _cache(rng, B, H, S, d, bits_per_loop)
    q = _bf16(rng, (L, B, hq, d))
    tk = tv = None
    if tail:
        tk = [_bf16(rng, (B, H, tail, d)) for _ in range(L)]
        tv = [_bf16(rng, (B, H, tail, d)) for _ in range(L)]
    out = rq.decode_attn_varlen(to_dev(q), to_dev(kref), to_dev(vref), _views(res, bits_per_loop),
                                seq_lens=torch.from_numpy(lens).to(DEV),
                                tail_k=None if tk is None else [to_dev(x) for x in tk],
                                tail_v=None if tv is None else [to_dev(x) for x in tv]).cpu().numpy()
    kh, vh = _hat(kref, vref, res, bits_per_loop)
    expect = oracle.decode_attn_varlen(q, kh, vh, lens, tk, tv)
    empty = (lens == 0) if not tail else np.zeros(B, dtype=bool)
    assert np.all(out[:, empty] == 0)  # a sequence with no position at all
    assert_attn_close(out[:, ~empty], expect[:, ~empty])


def test_varlen_with_full_lengths_equals_the_plain_decode():
    rng = np.random.default_rng(31)
    bits_per_loop = [2, 2, 0]
    B, H, S, d = 2, 2, 300, 128
    kref, vref, res = _cache(rng, B, H, S, d, bits_per_loop)
    q = to_dev(_bf16(rng, (3, B, 8, d)))
    views = _views(res, bits_per_loop)
    a = rq.decode_attn(q, to_dev(kref), to_dev(vref), views)
    b = rq.decode_attn_varlen(q, to_dev(kref), to_dev(vref), views,
                              seq_lens=torch.full((B,), S, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_serving_steps_append_then_decode():
    """Three decode steps of a looped model's serving loop. Each step attends
    over the encoded prefix plus the current position's bf16 loop states as
    the tail, then appends that position to the cache."""
    rng = np.random.default_rng(41)
    bits = [2, 2]                 # residual loops; the final loop is the reference
    L = len(bits) + 1
    B, H, S_cap, d, hq = 3, 2, 96, 128, 8
    lens = np.array([5, 40, 64], dtype=np.int32)
    # full history of every loop's K and V, bf16, for S_cap positions
    kref_all, vref_all = _bf16(rng, (B, H, S_cap, d)), _bf16(rng, (B, H, S_cap, d))
    kl = [workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(kref_all) + 0.15 * rng.standard_normal(
        kref_all.shape)).astype(np.float32)) for _ in bits] + [kref_all]
    vl = [workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(vref_all) + 0.15 * rng.standard_normal(
        vref_all.shape)).astype(np.float32)) for _ in bits] + [vref_all]
    # device cache, filled for each sequence's prefix by appending it
    kc = [torch.zeros((B, H, S_cap, d * b // 32), dtype=torch.int32, device=DEV) for b in bits]
    ks = [torch.zeros((B, H, S_cap, d // 32), dtype=torch.float16, device=DEV) for _ in bits]
    vc = [torch.zeros_like(t) for t in kc]
    vs = [torch.zeros_like(t) for t in ks]
    kref_c = torch.zeros((B, H, S_cap, d), dtype=torch.bfloat16, device=DEV)
    vref_c = torch.zeros_like(kref_c)
    n0 = int(lens.max())
    zero = torch.zeros(B, dtype=torch.int32, device=DEV)
    for tensor, src, codes, scales, refc in (("k", kl, kc, ks, kref_c), ("v", vl, vc, vs, vref_c)):
        rq.encode_append([to_dev(x[:, :, :n0]) for x in src[:-1]], to_dev(src[-1][:, :, :n0]), bits, zero, refc,
                         codes, scales)
    views = [rq.LoopView(b, kc[i], ks[i], vc[i], vs[i]) for i, b in enumerate(bits)] + [rq.LoopView(0)]
    # the oracle's cache: its own encode of every loop's whole history (each step
    # attends over the prefix of it that the GPU cache holds by then)
    khat = [oracle.reconstruct(kl[-1], *oracle.encode(kl[i], kl[-1], bl), bl) for i, bl in enumerate(bits)]
    vhat = [oracle.reconstruct(vl[-1], *oracle.encode(vl[i], vl[-1], bl), bl) for i, bl in enumerate(bits)]
    khat.append(oracle.bf16_to_f64(kl[-1]))
    vhat.append(oracle.bf16_to_f64(vl[-1]))
    lens_now = lens.copy()
    for step in range(3):
        q = _bf16(rng, (L, B, hq, d))
        tail_k = [np.stack([kl[l][b, :, lens_now[b]:lens_now[b] + 1] for b in range(B)]) for l in range(L)]
        tail_v = [np.stack([vl[l][b, :, lens_now[b]:lens_now[b] + 1] for b in range(B)]) for l in range(L)]
        out = rq.decode_attn_varlen(to_dev(q), kref_c, vref_c, views, seq_lens=torch.from_numpy(lens_now).to(DEV),
                                    tail_k=[to_dev(x) for x in tail_k], tail_v=[to_dev(x) for x in tail_v])
        expect = oracle.decode_attn_varlen(q, khat, vhat, lens_now, tail_k, tail_v)
        assert_attn_close(out.cpu().numpy(), expect)
        # the step's position is now complete: encode it into the cache
        pos = torch.from_numpy(lens_now).to(DEV)
        for src, codes, scales, refc, tail in (("k", kc, ks, kref_c, tail_k), ("v", vc, vs, vref_c, tail_v)):
            rq.encode_append([to_dev(tail[l]) for l in range(len(bits))], to_dev(tail[-1]), bits, pos, refc,
                             codes, scales)
        lens_now = lens_now + 1
    # the appended positions hold what a whole-prefix encode gives
    torch.cuda.synchronize()
    for b in range(B):
        n = int(lens_now[b])
        for i, bl in enumerate(bits):
            ow, os_ = oracle.encode(kl[i][b, :, :n], kl[-1][b, :, :n], bl)
            compare_codes(to_host_words(kc[i][b, :, :n]), to_host_u16(ks[i][b, :, :n]), ow, os_,
                          kl[i][b, :, :n], kl[-1][b, :, :n], bl)
