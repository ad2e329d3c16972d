"""Pins for the oracle's decode attention: brute force on tiny shapes, the
special cases S=1, equal keys and zero query, permutation invariance and the
GQA head mapping."""
import math

import numpy as np
import pytest

import oracle
import workloads


def _brute(q, k, v):
    """Explicit softmax with Python floats, scale 1/sqrt(D)."""
    d = len(q)
    z = [sum(q[i] * kt[i] for i in range(d)) / math.sqrt(d) for kt in k]
    e = [math.exp(zt) for zt in z]
    tot = sum(e)
    return [sum(e[t] * v[t][i] for t in range(len(k))) / tot for i in range(d)]


@pytest.mark.parametrize("s", [1, 2, 5, 8])
def test_matches_brute_force(s):
    rng = np.random.default_rng(s)
    d = 8
    q = rng.standard_normal((3, d))
    k = rng.standard_normal((s, d)) * 2
    v = rng.standard_normal((s, d))
    out = oracle.attention(q, k, v, 1.0 / math.sqrt(d))
    for r in range(3):
        np.testing.assert_allclose(out[r], _brute(list(q[r]), k.tolist(), v.tolist()), rtol=1e-12, atol=1e-14)


def test_special_cases():
    rng = np.random.default_rng(0)
    d = 16
    v = rng.standard_normal((6, d))
    k = rng.standard_normal((6, d))
    q = rng.standard_normal((2, d))
    # one position: the output is that position's value
    np.testing.assert_allclose(oracle.attention(q, k[:1], v[:1], 0.25), np.repeat(v[:1], 2, 0), atol=1e-15)
    # all keys equal, or a zero query: the mean of the values
    kk = np.repeat(k[:1], 6, 0)
    np.testing.assert_allclose(oracle.attention(q, kk, v, 0.25), np.repeat(v.mean(0, keepdims=True), 2, 0), atol=1e-14)
    np.testing.assert_allclose(oracle.attention(np.zeros((1, d)), k, v, 0.25), v.mean(0, keepdims=True), atol=1e-14)
    # permutation of positions does not change the result
    perm = rng.permutation(6)
    np.testing.assert_allclose(oracle.attention(q, k[perm], v[perm], 0.25), oracle.attention(q, k, v, 0.25), atol=1e-14)


def test_gqa_head_mapping():
    """Query head h reads kv head h // G (consecutive query heads share a kv head)."""
    n_loops, batch, hkv, g, d = 1, 1, 3, 2, 8
    k = [np.zeros((batch, hkv, 1, d))]
    v = [np.zeros((batch, hkv, 1, d))]
    for h in range(hkv):
        v[0][0, h, 0, :] = h + 1
    q = np.zeros((n_loops, batch, hkv * g, d), dtype=np.uint16)
    out = oracle.decode_attn(q, k, v)
    for h in range(hkv * g):
        assert np.all(out[0, 0, h] == h // g + 1)


def test_decode_scale_and_loops():
    rng = np.random.default_rng(4)
    n_loops, batch, hkv, g, d, s = 2, 1, 1, 2, 8, 5
    q_bits = (rng.integers(0x3C00, 0x4000, size=(n_loops, batch, hkv * g, d))).astype(np.uint16)
    k = [rng.standard_normal((batch, hkv, s, d)) for _ in range(n_loops)]
    v = [rng.standard_normal((batch, hkv, s, d)) for _ in range(n_loops)]
    out = oracle.decode_attn(q_bits, k, v)
    q = oracle.bf16_to_f64(q_bits)
    for l in range(n_loops):
        for h in range(hkv * g):
            np.testing.assert_allclose(out[l, 0, h], _brute(list(q[l, 0, h]), k[l][0, 0].tolist(), v[l][0, 0].tolist()), rtol=1e-12)


def _bf16(rng, shape):
    return workloads.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def test_varlen_moving_a_position_into_the_tail_changes_nothing():
    """Attention is over a set of positions: position n-1 of the prefix and the
    same key/value given as a one-position tail give the same output."""
    rng = np.random.default_rng(21)
    L, B, Hkv, Hq, S, D = 2, 3, 2, 4, 9, 16
    q = _bf16(rng, (L, B, Hq, D))
    kb = [_bf16(rng, (B, Hkv, S, D)) for _ in range(L)]
    vb = [_bf16(rng, (B, Hkv, S, D)) for _ in range(L)]
    kh = [oracle.bf16_to_f64(x) for x in kb]
    vh = [oracle.bf16_to_f64(x) for x in vb]
    lens = np.array([9, 4, 1])
    full = oracle.decode_attn_varlen(q, kh, vh, lens)
    tk = [np.stack([kb[l][b, :, lens[b] - 1:lens[b]] for b in range(B)]) for l in range(L)]
    tv = [np.stack([vb[l][b, :, lens[b] - 1:lens[b]] for b in range(B)]) for l in range(L)]
    moved = oracle.decode_attn_varlen(q, kh, vh, lens - 1, tk, tv)
    np.testing.assert_allclose(moved, full, rtol=1e-12, atol=1e-14)
    # every position of the cache: the plain decode
    np.testing.assert_allclose(oracle.decode_attn_varlen(q, kh, vh, np.full(B, S)), oracle.decode_attn(q, kh, vh),
                               rtol=0, atol=0)


def test_varlen_special_cases():
    rng = np.random.default_rng(22)
    L, B, Hkv, Hq, S, D = 1, 2, 1, 2, 5, 8
    q = _bf16(rng, (L, B, Hq, D))
    kh = [oracle.bf16_to_f64(_bf16(rng, (B, Hkv, S, D)))]
    vh = [oracle.bf16_to_f64(_bf16(rng, (B, Hkv, S, D)))]
    tk = [_bf16(rng, (B, Hkv, 1, D))]
    tv = [_bf16(rng, (B, Hkv, 1, D))]
    # no cached position and no tail: a zero row; one tail position only: its value
    out = oracle.decode_attn_varlen(q, kh, vh, np.array([0, 0]))
    assert np.all(out == 0)
    out = oracle.decode_attn_varlen(q, kh, vh, np.array([0, 0]), tk, tv)
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(out[0, b, h], oracle.bf16_to_f64(tv[0][b, 0, 0]), rtol=1e-15)
    # one cached position: its value
    out = oracle.decode_attn_varlen(q, kh, vh, np.array([1, 1]))
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(out[0, b, h], vh[0][b, 0, 0], rtol=1e-15)


def test_gather_pages_worked_example():
    """Two sequences, blocks of two positions: sequence 0 uses blocks 2 then 0,
    sequence 1 uses block 1 and an entry that is not a block (-1)."""
    pages = np.arange(3 * 1 * 2).reshape(3, 1, 2)  # block k holds positions (2k, 2k+1) of value
    table = np.array([[2, 0], [1, -1]])
    got = oracle.gather_pages(pages, table, 2, 4)
    np.testing.assert_array_equal(got[0, 0], [4, 5, 0, 1])
    np.testing.assert_array_equal(got[1, 0], [2, 3, 0, 0])


def test_gather_pages_inverts_a_scatter():
    rng = np.random.default_rng(3)
    B, H, S, P, D = 3, 2, 256, 64, 5
    dense = rng.standard_normal((B, H, S, D))
    perm = rng.permutation(B * S // P + 2)  # two spare blocks
    table = perm[: B * S // P].reshape(B, S // P)
    pages = np.full((len(perm), H, P, D), np.nan)
    for b in range(B):
        for j in range(S // P):
            pages[table[b, j]] = dense[b, :, j * P:(j + 1) * P]
    np.testing.assert_array_equal(oracle.gather_pages(pages, table, P, S), dense)


def test_missing_block_takes_no_weight_worked_example():
    """A table entry that is not a block removes its positions from the
    softmax. Blocks of one position, D = 2, scale 1: q = (1, 0); keys
    (0, 0), (ln 3, 0) and (100, 0); values (1, 0), (0, 1) and (5, 5). The third
    position's block is missing (-1), so the weights are 1 : 3 and the output
    is (1/4, 3/4). Attending to a zero-filled third position would give
    weights 1 : 3 : 1 and (1/5, 3/5) instead."""
    table = np.array([[0, 1, -1]])
    present = oracle.pages_present(table, 1, 2, 3)
    np.testing.assert_array_equal(present, [[True, True, False]])
    k = [np.array([[[[0.0, 0.0], [math.log(3.0), 0.0], [100.0, 0.0]]]])]
    v = [np.array([[[[1.0, 0.0], [0.0, 1.0], [5.0, 5.0]]]])]
    q = np.array([[[[0x3F80, 0x0000]]]], dtype=np.uint16)  # bf16 (1, 0)
    out = oracle.decode_attn_varlen(q, k, v, np.array([3]), scale=1.0, present=present)
    np.testing.assert_allclose(out[0, 0, 0], [0.25, 0.75], rtol=1e-14)
    # the zero-filled cache gather_pages builds is not what the decode attends to
    pages = np.stack([k[0][0, :, 0], k[0][0, :, 1]])  # [2 blocks, Hkv = 1, D] -> one position per block
    kz = [oracle.gather_pages(pages[:, :, None, :], table, 1, 3)]
    vz = [oracle.gather_pages(np.stack([v[0][0, :, 0], v[0][0, :, 1]])[:, :, None, :], table, 1, 3)]
    zero_filled = oracle.decode_attn_varlen(q, kz, vz, np.array([3]), scale=1.0)
    np.testing.assert_allclose(zero_filled[0, 0, 0], [0.2, 0.6], rtol=1e-14)


def test_missing_blocks_equal_a_compacted_cache():
    """Leaving positions out equals attending over the cache with them deleted;
    a sequence whose every position is missing and has no tail is zero; with
    a tail it is the tail alone."""
    rng = np.random.default_rng(23)
    L, B, Hkv, Hq, S, D, P = 2, 3, 2, 4, 12, 8, 2
    q = _bf16(rng, (L, B, Hq, D))
    kh = [oracle.bf16_to_f64(_bf16(rng, (B, Hkv, S, D))) for _ in range(L)]
    vh = [oracle.bf16_to_f64(_bf16(rng, (B, Hkv, S, D))) for _ in range(L)]
    table = np.array([[0, -1, 2, 3, 7, 5], [-1, -1, -1, -1, -1, -1], [4, 6, 99, 1, 8, 9]])
    present = oracle.pages_present(table, P, 10, S)
    lens = np.array([11, 12, 9])
    got = oracle.decode_attn_varlen(q, kh, vh, lens, present=present)
    for b in range(B):
        keep = [t for t in range(lens[b]) if present[b, t]]
        kc = [x[b:b + 1, :, keep] for x in kh]
        vc = [x[b:b + 1, :, keep] for x in vh]
        want = oracle.decode_attn_varlen(q[:, b:b + 1], kc, vc, np.array([len(keep)]))
        np.testing.assert_allclose(got[:, b:b + 1], want, rtol=1e-12, atol=1e-14)
    assert np.all(got[:, 1] == 0)
    tk = [_bf16(rng, (B, Hkv, 1, D)) for _ in range(L)]
    tv = [_bf16(rng, (B, Hkv, 1, D)) for _ in range(L)]
    with_tail = oracle.decode_attn_varlen(q, kh, vh, lens, tk, tv, present=present)
    for l in range(L):
        for h in range(Hq):
            np.testing.assert_allclose(with_tail[l, 1, h], oracle.bf16_to_f64(tv[l][1, h // (Hq // Hkv), 0]),
                                       rtol=1e-15)
