"""Host-side checks of the C ABI: the library loads and exports every entry
point include/rq.h declares, size queries work, and every argument check
fails before any HIP call (no GPU is touched: each call below is rejected by
validation)."""
import ctypes
import os
import re

import pytest

import looped_transformer_kv_rq_amd as rq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(rq.library_path()), reason="librq.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(rq.library_path())
    names = declared_functions()
    assert {"rq_encode", "rq_reconstruct", "rq_encode_refit", "rq_encode_append", "rq_decode_attn_varlen",
            "rq_decode_attn_varlen_workspace", "rq_encode_rotonly", "rq_reconstruct_rotonly", "rq_decode_attn",
            "rq_decode_attn_bf16", "rq_encode_layers", "rq_encode_append_paged", "rq_decode_attn_paged",
            "rq_decode_attn_workspace", "rq_decode_attn_splits", "rq_status_str", "rq_format_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in rq.h but not exported"


def test_status_strings_and_version():
    lib = rq._load()
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.rq_status_str(st)
    assert lib.rq_status_str(123) == b"unknown status"
    assert rq.format_version() == 1


def test_workspace_and_split_queries():
    # 16 x 8 rows of 4096 tokens: enough splits for ~512 blocks, each a multiple of 64 tokens
    n = rq.decode_splits(16, 8, 4096, 128, 32, 4)
    assert n == 4
    # split partials (m, l, reference and residual outputs) + one 528-byte rotated-query record per
    # row (fp16 hi and lo parts of 128 coordinates, 4 group offsets)
    part = 4 * 16 * 32 * n * (2 * 128 + 2) * 4
    assert rq.decode_workspace_bytes(16, 8, 4096, 128, 32, 4) == (part + 255) // 256 * 256 + 4 * 16 * 32 * 528
    assert rq.decode_splits(1, 1, 1, 64, 1, 1) == 1
    assert rq.decode_splits(1, 1, 1000, 64, 1, 1, n_splits=3) == 3
    assert rq.decode_splits(1, 1, 100, 64, 1, 1, n_splits=50) == 2  # never below one 64-token tile
    assert rq.decode_workspace_bytes(1, 1, 1, 96, 1, 1) == 0       # unsupported head_dim
    assert rq.decode_workspace_bytes(1, 2, 1, 64, 3, 1) == 0       # Hq % Hkv != 0
    assert rq.decode_workspace_bytes(1, 1, 1, 64, 1, 9) == 0       # too many loops
    # one (batch, kv head) row of bf16 K must stay below 2^31 bytes
    assert rq.decode_workspace_bytes(1, 1, 2 ** 24 - 1, 64, 1, 1) > 0
    assert rq.decode_workspace_bytes(1, 1, 2 ** 24, 64, 1, 1) == 0
    assert rq.decode_workspace_bytes(1, 1, 2 ** 23, 128, 1, 1) == 0


def test_varlen_workspace_of_the_length_balanced_plan():
    # Ragged decode, automatic splits: up to 2 * ceil(512 / rows) + 1 prefix records per row
    # (rows = B * Hkv = 64 here: 17), one tail record, the query records, then one int32 split
    # count per sequence.
    B, H, S, D, HQ, L = 8, 8, 32768, 128, 32, 4
    part = L * B * HQ * (17 + 1) * (2 * D + 2) * 4
    expect = (part + 255) // 256 * 256 + L * B * HQ * 528 + 4 * B
    assert rq.decode_varlen_workspace_bytes(B, H, S, D, HQ, L, 0, 1) == expect
    # an explicit split count keeps the plain plan: n_splits prefix records and the tail record
    part4 = L * B * HQ * (4 + 1) * (2 * D + 2) * 4
    assert rq.decode_varlen_workspace_bytes(B, H, S, D, HQ, L, 4, 1) == (part4 + 255) // 256 * 256 + L * B * HQ * 528
    # the cap never exceeds the sequence's 64-position units
    part1 = 1 * 2 * 1 * 1 * (2 * 64 + 2) * 4
    assert rq.decode_varlen_workspace_bytes(2, 1, 64, 64, 1, 1, 0, 0) == (part1 + 255) // 256 * 256 + 2 * 1 * 272 + 8


def _shape(b=1, h=1, s=4, d=64):
    return rq._Shape(b, h, s, d)


FAKE = 0x10000  # never dereferenced: each call fails validation first


def _ptrs(*vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def test_encode_argument_checks():
    lib = rq._load()
    bits = (ctypes.c_int32 * 1)(2)
    x, c, s = _ptrs(FAKE), _ptrs(FAKE), _ptrs(FAKE)
    ok = dict(x=x, bits=bits, ref=FAKE, codes=c, scales=s)

    def call(shape=_shape(), n=1, **kw):
        a = {**ok, **kw}
        return lib.rq_encode(shape if shape is None else ctypes.byref(shape), n, a["x"], a["bits"], a["ref"],
                             a["codes"], a["scales"], None)

    assert call(shape=None) == rq.RQ_EINVAL
    assert call(shape=_shape(s=0)) == rq.RQ_EINVAL
    assert call(shape=_shape(d=96)) == rq.RQ_EUNSUPPORTED
    assert call(n=0) == rq.RQ_EINVAL
    assert call(n=9) == rq.RQ_EINVAL
    assert call(ref=None) == rq.RQ_EINVAL
    assert call(x=_ptrs(0)) == rq.RQ_EINVAL
    for b in (0, 1, 5, 6, 7, 16):  # widths are 2, 3, 4 and 8
        assert call(bits=(ctypes.c_int32 * 1)(b)) == rq.RQ_EUNSUPPORTED
    assert call(ref=FAKE + 8) == rq.RQ_EALIGN
    assert call(scales=_ptrs(FAKE + 2)) == rq.RQ_EALIGN


def test_reconstruct_argument_checks():
    lib = rq._load()
    sh = ctypes.byref(_shape())
    assert lib.rq_reconstruct(None, 2, FAKE, FAKE, FAKE, 0, FAKE, None) == rq.RQ_EINVAL
    assert lib.rq_reconstruct(sh, 5, FAKE, FAKE, FAKE, 0, FAKE, None) == rq.RQ_EUNSUPPORTED
    assert lib.rq_reconstruct(sh, 1, FAKE, FAKE, FAKE, 0, FAKE, None) == rq.RQ_EUNSUPPORTED
    assert lib.rq_reconstruct(sh, 2, FAKE, FAKE, FAKE, 7, FAKE, None) == rq.RQ_EUNSUPPORTED
    assert lib.rq_reconstruct(sh, 2, FAKE, None, FAKE, 0, FAKE, None) == rq.RQ_EINVAL
    assert lib.rq_reconstruct(sh, 2, FAKE, FAKE, FAKE, 0, None, None) == rq.RQ_EINVAL
    assert lib.rq_reconstruct(sh, 2, FAKE + 4, FAKE, FAKE, 0, FAKE, None) == rq.RQ_EALIGN


def test_rotonly_argument_checks():
    lib = rq._load()
    sh = ctypes.byref(_shape())
    bits = (ctypes.c_int32 * 1)(2)
    x, c, s = _ptrs(FAKE), _ptrs(FAKE), _ptrs(FAKE)
    assert lib.rq_encode_rotonly(None, 1, x, bits, c, s, None) == rq.RQ_EINVAL
    assert lib.rq_encode_rotonly(sh, 0, x, bits, c, s, None) == rq.RQ_EINVAL
    assert lib.rq_encode_rotonly(sh, 1, _ptrs(0), bits, c, s, None) == rq.RQ_EINVAL
    assert lib.rq_encode_rotonly(sh, 1, x, (ctypes.c_int32 * 1)(0), c, s, None) == rq.RQ_EUNSUPPORTED
    assert lib.rq_encode_rotonly(sh, 1, _ptrs(FAKE + 8), bits, c, s, None) == rq.RQ_EALIGN
    # the reference-based encoders still require their reference
    assert lib.rq_encode(sh, 1, x, bits, None, c, s, None) == rq.RQ_EINVAL
    assert lib.rq_encode_refit(sh, 1, x, bits, None, c, s, 1, None) == rq.RQ_EINVAL
    assert lib.rq_encode_refit(sh, 1, x, bits, FAKE, c, s, -1, None) == rq.RQ_EINVAL
    assert lib.rq_encode_refit(sh, 1, x, bits, FAKE, c, s, 17, None) == rq.RQ_EINVAL
    assert lib.rq_encode_refit(sh, 1, x, (ctypes.c_int32 * 1)(5), FAKE, c, s, 2, None) == rq.RQ_EUNSUPPORTED
    assert lib.rq_reconstruct_rotonly(sh, 0, FAKE, FAKE, 0, FAKE, None) == rq.RQ_EUNSUPPORTED
    assert lib.rq_reconstruct_rotonly(sh, 2, None, FAKE, 0, FAKE, None) == rq.RQ_EINVAL
    assert lib.rq_reconstruct_rotonly(sh, 2, FAKE, FAKE, 5, FAKE, None) == rq.RQ_EUNSUPPORTED
    assert lib.rq_reconstruct_rotonly(sh, 2, FAKE, FAKE, 0, FAKE + 4, None) == rq.RQ_EALIGN
    assert lib.rq_reconstruct(sh, 2, None, FAKE, FAKE, 0, FAKE, None) == rq.RQ_EINVAL


def test_append_and_varlen_argument_checks():
    lib = rq._load()
    sh = ctypes.byref(_shape(b=2, h=2, s=64, d=64))
    bits = (ctypes.c_int32 * 1)(2)
    x, c, s = _ptrs(FAKE), _ptrs(FAKE), _ptrs(FAKE)
    ap = lib.rq_encode_append
    assert ap(sh, 1, 0, x, bits, FAKE, FAKE, FAKE, c, s, None) == rq.RQ_EINVAL        # t_new = 0
    assert ap(sh, 1, 1, x, bits, FAKE, None, FAKE, c, s, None) == rq.RQ_EINVAL        # no positions
    assert ap(sh, 1, 1, x, bits, FAKE, FAKE, None, c, s, None) == rq.RQ_EINVAL        # no reference cache
    assert ap(sh, 1, 1, x, (ctypes.c_int32 * 1)(0), FAKE, FAKE, FAKE, c, s, None) == rq.RQ_EUNSUPPORTED
    assert ap(sh, 1, 1, x, bits, FAKE, FAKE, FAKE + 2, c, s, None) == rq.RQ_EALIGN
    ws = lib.rq_decode_attn_varlen_workspace
    assert ws(sh, 4, 2, 0, 1) > ws(sh, 4, 2, 0, 0) >= lib.rq_decode_attn_workspace(sh, 4, 2, 0)
    assert ws(sh, 4, 2, 1, 0) == lib.rq_decode_attn_workspace(sh, 4, 2, 1)  # an explicit split count
    assert ws(sh, 4, 2, 0, -1) == 0
    need = ws(sh, 4, 2, 0, 1)
    views = (rq._LoopView * 2)()
    views[0].bits, views[0].k_codes, views[0].k_scales, views[0].v_codes, views[0].v_scales = 2, FAKE, FAKE, FAKE, FAKE
    tk = _ptrs(FAKE, FAKE)

    def call(lens=FAKE, tail=1, tkk=tk, tvv=tk, wsb=need):
        return lib.rq_decode_attn_varlen(sh, 4, 2, FAKE, FAKE, FAKE, views, lens, tail, tkk, tvv, 0.125, 0, FAKE,
                                         FAKE, wsb, None)

    assert call(tail=-1) == rq.RQ_EINVAL
    assert call(tkk=None) == rq.RQ_EINVAL
    assert call(tvv=_ptrs(FAKE, 0)) == rq.RQ_EINVAL
    assert call(lens=FAKE + 4) == rq.RQ_EALIGN
    assert call(tvv=_ptrs(FAKE, FAKE + 8)) == rq.RQ_EALIGN
    assert call(wsb=need - 1) == rq.RQ_EWORKSPACE   # the tail's records need room


def test_decode_argument_checks():
    lib = rq._load()
    sh = _shape(b=1, h=2, s=64, d=64)
    need = lib.rq_decode_attn_workspace(ctypes.byref(sh), 4, 2, 0)
    assert need > 0
    views = (rq._LoopView * 2)()
    views[0].bits, views[0].k_codes, views[0].k_scales, views[0].v_codes, views[0].v_scales = 2, FAKE, FAKE, FAKE, FAKE
    views[1].bits = 0

    def call(hq=4, n=2, q=FAKE, v=views, scale=0.125, splits=0, out=FAKE, ws=FAKE, wsb=need):
        return lib.rq_decode_attn(ctypes.byref(sh), hq, n, q, FAKE, FAKE, v, scale, splits, out, ws, wsb, None)

    assert call(hq=3) == rq.RQ_EINVAL            # Hq % Hkv != 0
    assert call(hq=2 * 33) == rq.RQ_EUNSUPPORTED  # more than 32 query heads per kv head
    assert call(n=9) == rq.RQ_EINVAL
    assert call(q=None) == rq.RQ_EINVAL
    assert call(scale=float("nan")) == rq.RQ_EINVAL
    assert call(splits=-1) == rq.RQ_EINVAL
    assert call(ws=None) == rq.RQ_EWORKSPACE
    assert call(wsb=need - 1) == rq.RQ_EWORKSPACE
    assert call(out=FAKE + 4) == rq.RQ_EALIGN
    bad = (rq._LoopView * 2)()
    bad[0].bits = 5
    assert call(v=bad) == rq.RQ_EUNSUPPORTED
    bad[0].bits = 2  # residual loop without its code pointers
    assert call(v=bad) == rq.RQ_EINVAL
    bf = lib.rq_decode_attn_bf16
    k = _ptrs(FAKE, FAKE)
    assert bf(ctypes.byref(sh), 4, 2, FAKE, k, _ptrs(FAKE, 0), 0.125, 0, FAKE, FAKE, need, None) == rq.RQ_EINVAL
    assert bf(ctypes.byref(sh), 4, 2, FAKE, k, k, 0.125, 0, FAKE, FAKE, 16, None) == rq.RQ_EWORKSPACE


def test_python_side_rejects_cpu_tensors():
    import torch
    ref = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rq.encode([ref], ref, [2])
    with pytest.raises(ValueError):
        rq.encode([ref], ref, [3])


def test_encode_layers_argument_checks():
    """Every layer's arguments are checked before the first launch: a bad entry
    in the last layer fails the call although the first layer is valid."""
    lib = rq._load()
    sh = ctypes.byref(_shape())
    enc = lib.rq_encode_layers
    x2, c2, s2 = _ptrs(FAKE, FAKE, FAKE, FAKE), _ptrs(FAKE, FAKE, FAKE, FAKE), _ptrs(FAKE, FAKE, FAKE, FAKE)
    refs = _ptrs(FAKE, FAKE)
    good = (ctypes.c_int32 * 4)(8, 3, 4, 2)
    assert enc(sh, 0, 2, x2, good, refs, c2, s2, None) == rq.RQ_EINVAL            # no layers
    assert enc(sh, 4097, 1, x2, good, refs, c2, s2, None) == rq.RQ_EINVAL         # above RQ_MAX_LAYERS
    assert enc(sh, 2, 0, x2, good, refs, c2, s2, None) == rq.RQ_EINVAL            # no loops
    assert enc(sh, 2, 9, x2, good, refs, c2, s2, None) == rq.RQ_EINVAL            # above RQ_MAX_LOOPS
    assert enc(None, 2, 2, x2, good, refs, c2, s2, None) == rq.RQ_EINVAL
    assert enc(sh, 2, 2, x2, None, refs, c2, s2, None) == rq.RQ_EINVAL
    assert enc(sh, 2, 2, x2, good, None, c2, s2, None) == rq.RQ_EINVAL
    assert enc(sh, 2, 2, x2, good, _ptrs(FAKE, 0), c2, s2, None) == rq.RQ_EINVAL   # layer 1 has no reference
    assert enc(sh, 2, 2, x2, (ctypes.c_int32 * 4)(2, 2, 2, 5), refs, c2, s2, None) == rq.RQ_EUNSUPPORTED
    assert enc(sh, 2, 2, x2, (ctypes.c_int32 * 4)(2, 2, 2, 0), refs, c2, s2, None) == rq.RQ_EUNSUPPORTED
    assert enc(sh, 2, 2, _ptrs(FAKE, FAKE, FAKE, 0), good, refs, c2, s2, None) == rq.RQ_EINVAL
    assert enc(sh, 2, 2, x2, good, refs, c2, _ptrs(FAKE, FAKE, FAKE, FAKE + 2), None) == rq.RQ_EALIGN
    assert enc(sh, 2, 2, x2, good, _ptrs(FAKE, FAKE + 8), c2, s2, None) == rq.RQ_EALIGN


def test_paged_argument_checks():
    lib = rq._load()
    P, max_blocks = 64, 4
    sh = ctypes.byref(_shape(b=2, h=2, s=P * max_blocks, d=64))
    good = rq._Pages(FAKE, max_blocks, P, 16)
    views = (rq._LoopView * 2)()
    views[0].bits, views[0].k_codes, views[0].k_scales, views[0].v_codes, views[0].v_scales = 8, FAKE, FAKE, FAKE, FAKE
    need = lib.rq_decode_attn_varlen_workspace(sh, 4, 2, 0, 0)

    def dec(pages=good, shape=sh):
        pg = None if pages is None else ctypes.byref(pages)
        return lib.rq_decode_attn_paged(shape, 4, 2, FAKE, FAKE, FAKE, views, pg, None, 0, None, None, 0.125, 0,
                                        FAKE, FAKE, need, None)

    assert dec(pages=None) == rq.RQ_EINVAL
    assert dec(pages=rq._Pages(0, max_blocks, P, 16)) == rq.RQ_EINVAL            # no block table
    assert dec(pages=rq._Pages(FAKE, max_blocks, 96, 16)) == rq.RQ_EUNSUPPORTED   # not a power of two
    assert dec(pages=rq._Pages(FAKE, max_blocks, 32, 16)) == rq.RQ_EUNSUPPORTED   # below 64
    assert dec(pages=rq._Pages(FAKE, 0, P, 16)) == rq.RQ_EINVAL
    assert dec(pages=rq._Pages(FAKE, max_blocks, P, 0)) == rq.RQ_EINVAL
    assert dec(pages=rq._Pages(FAKE, max_blocks - 1, P, 16)) == rq.RQ_EINVAL      # capacity != seq_len
    assert dec(pages=rq._Pages(FAKE + 4, max_blocks, P, 16)) == rq.RQ_EALIGN
    bits = (ctypes.c_int32 * 1)(3)
    x, c, s = _ptrs(FAKE), _ptrs(FAKE), _ptrs(FAKE)

    def app(pages=good, t_new=1):
        pg = None if pages is None else ctypes.byref(pages)
        return lib.rq_encode_append_paged(sh, pg, 1, t_new, x, bits, FAKE, FAKE, FAKE, c, s, None)

    assert app(pages=None) == rq.RQ_EINVAL
    assert app(t_new=0) == rq.RQ_EINVAL
    assert app(pages=rq._Pages(FAKE, max_blocks, 100, 16)) == rq.RQ_EUNSUPPORTED
    assert app(pages=rq._Pages(FAKE, 3, P, 16)) == rq.RQ_EINVAL


def test_kv_entry_points_check_both_tensors():
    """rq_encode_kv and the K+V appends reject a bad argument on either tensor
    before any HIP call (each returns the status the single-tensor call gives)."""
    lib = rq._load()
    bits = (ctypes.c_int32 * 1)(2)
    good = dict(kx=_ptrs(FAKE), vx=_ptrs(FAKE), kref=FAKE, vref=FAKE, kc=_ptrs(FAKE), ks=_ptrs(FAKE), vc=_ptrs(FAKE),
                vs=_ptrs(FAKE))

    def enc(shape=_shape(), **kw):
        a = {**good, **kw}
        return lib.rq_encode_kv(ctypes.byref(shape), 1, a["kx"], a["vx"], bits, a["kref"], a["vref"], a["kc"],
                                a["ks"], a["vc"], a["vs"], None)

    assert enc(kref=None) == rq.RQ_EINVAL
    assert enc(vref=None) == rq.RQ_EINVAL
    assert enc(vx=_ptrs(0)) == rq.RQ_EINVAL
    assert enc(vs=_ptrs(FAKE + 2)) == rq.RQ_EALIGN
    assert enc(kc=_ptrs(FAKE + 4)) == rq.RQ_EALIGN
    assert enc(shape=_shape(d=96)) == rq.RQ_EUNSUPPORTED

    sh = _shape(b=2, h=2, s=256, d=64)

    def app(**kw):
        a = {**good, **kw}
        return lib.rq_encode_append_kv(ctypes.byref(sh), 1, 1, a["kx"], a["vx"], bits, a["kref"], a["vref"], FAKE,
                                       FAKE, a.get("vcache", FAKE), a["kc"], a["ks"], a["vc"], a["vs"], None)

    assert app(vref=None) == rq.RQ_EINVAL
    assert app(vcache=FAKE + 8) == rq.RQ_EALIGN
    assert app(vc=_ptrs(0)) == rq.RQ_EINVAL
    pages = rq._Pages(FAKE, 4, 64, 16)

    def papp(pg=pages, **kw):
        a = {**good, **kw}
        p = None if pg is None else ctypes.byref(pg)
        return lib.rq_encode_append_paged_kv(ctypes.byref(sh), p, 1, 1, a["kx"], a["vx"], bits, a["kref"], a["vref"],
                                             FAKE, FAKE, FAKE, a["kc"], a["ks"], a["vc"], a["vs"], None)

    assert papp(pg=None) == rq.RQ_EINVAL
    assert papp(pg=rq._Pages(FAKE, 4, 96, 16)) == rq.RQ_EUNSUPPORTED
    assert papp(vs=_ptrs(FAKE + 2)) == rq.RQ_EALIGN


def test_noalloc_argument_checks_and_size_limit():
    """rq_decode_attn_noalloc: rq_decode_attn's checks (no workspace argument),
    and a call whose workspace would exceed RQ_NOALLOC_SCRATCH_BYTES is
    RQ_EWORKSPACE; every case fails before any HIP call."""
    lib = rq._load()
    views = (rq._LoopView * 2)()
    views[0].bits, views[0].k_codes, views[0].k_scales, views[0].v_codes, views[0].v_scales = 2, FAKE, FAKE, FAKE, FAKE

    def call(shape, hq=4, n=2, q=FAKE, out=FAKE, splits=0, vs=views):
        return lib.rq_decode_attn_noalloc(ctypes.byref(shape), hq, n, q, FAKE, FAKE, vs, 0.125, splits, out, None)

    sh = _shape(b=2, h=2, s=64, d=64)
    assert call(sh, q=None) == rq.RQ_EINVAL
    assert call(sh, hq=3) == rq.RQ_EINVAL
    assert call(sh, n=9) == rq.RQ_EINVAL
    assert call(sh, splits=-1) == rq.RQ_EINVAL
    assert call(_shape(b=2, h=2, s=64, d=96)) == rq.RQ_EUNSUPPORTED
    assert call(sh, out=FAKE + 4) == rq.RQ_EALIGN
    bad = (rq._LoopView * 2)()
    bad[0].bits = 5
    assert call(sh, vs=bad) == rq.RQ_EUNSUPPORTED
    # the largest size: 4 loops x 64 batch x 32 query heads x 16 splits needs more than 32 MiB
    big = _shape(b=64, h=8, s=8192, d=128)
    need = lib.rq_decode_attn_workspace(ctypes.byref(big), 32, 2, 16)
    assert need > rq.NOALLOC_SCRATCH_BYTES
    assert call(big, hq=32, n=2, splits=16) == rq.RQ_EWORKSPACE


def test_build_refuses_register_spills():
    """The build's spill guard reads the compiler's resource-usage remarks."""
    from looped_transformer_kv_rq_amd import build as b

    log = "\n".join([
        "x.hip:1:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark: Function Name: _Z3barPf [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 20 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert b.scratch_users(log) == [("_Z3barPf", 20)]


def _modelled_splits(rows, seq_len, round_blocks):
    """The automatic split count's rule written out: a request of c splits
    becomes splits of whole 64-token units (as few as hold the positions); of
    c = 1 .. 64, the one whose split count n has the least modelled time
    ceil(rows * n / round) * (1 / n + 6 * 64 / seq_len), the first on ties."""
    units = -(-seq_len // 64)
    best, best_n = None, 1
    for c in range(1, 65):
        c = min(c, units)
        tps = -(-(-(-seq_len // c)) // 64) * 64
        n = -(-seq_len // tps)
        t = -(-rows * n // round_blocks) * (1.0 / n + 6.0 * 64 / seq_len)
        if best is None or t < best * (1 - 1e-9):
            best, best_n = t, n
    return best_n


def test_automatic_splits_fill_whole_rounds():
    """The automatic split count follows the rounds of resident blocks: 512 for one
    16-row set, 1,024 for paired sets (more than 16 query rows per kv head, at most
    16 heads each), 256 for 32-row blocks. The sweep points of the 16-row kernel
    stay (4 splits at 16 x 8 rows of 4K, 8 at 8 x 8 rows of 32K), and the peak-batch
    cache (10,720 rows of 16K positions, 32 rows per kv head) takes 2 splits: 21
    rounds of half-length blocks instead of 11 rounds whose last one is half empty."""
    assert rq.decode_splits(16, 8, 4096, 128, 32, 4) == 4
    assert rq.decode_splits(8, 8, 32768, 128, 32, 4) == 8
    assert rq.decode_splits(32, 8, 8192, 128, 32, 4) == 2
    assert rq.decode_splits(2680, 4, 16384, 128, 16, 8) == 2
    assert rq.decode_splits(744, 4, 16384, 128, 16, 8) == 1
    # a paired launch at a small batch fills 1,024 slots, not 512
    assert rq.decode_splits(4, 4, 16384, 128, 16, 8) * 16 == 1024
    cases = [(b, h, s, g, nl) for b in (1, 3, 8, 16, 64, 300, 1072, 2680) for h in (1, 4, 8)
             for s in (64, 1000, 4096, 16384) for g, nl in ((4, 4), (4, 8), (16, 2), (20, 1), (32, 2))]
    for b, h, s, g, nl in cases:
        round_blocks = 256 if g > 16 else (1024 if g * nl > 16 else 512)
        got = rq.decode_splits(b, h, s, 128, g * h, nl)
        assert got == _modelled_splits(b * h, s, round_blocks), (b, h, s, g, nl, got)


def _wave_tile_bytes_d128(bits):
    """LDS one wave stages per 32-token tile at D = 128: the V tile (8 rows of
    1,024 bytes, each with a 128-byte pad), then each residual loop's K and V
    codes (32 tokens x 128 b / 8 bytes each) and fp16 scales (32 tokens x 4
    groups x 2 bytes each)."""
    return 8 * 1152 + sum(256 * (128 * b // 32) + 128 * 4 for b in bits if b)


def test_automatic_splits_follow_the_widths():
    """A 16-row call whose first launch stages more than 20 KB per wave and tile
    (an INT8 loop beside others) holds one block per CU, so its rounds are 256
    blocks: the INT8 layers of the mixed_s32k states take 4 splits, not 8. The
    first launch holds the call's loops, in order, while four waves' tiles fit
    160 KB. The workspace query sizes for the larger of the two plans."""
    assert rq.decode_splits(8, 8, 32768, 128, 32, 4, bits=[8, 4, 2, 0]) == 4
    assert rq.decode_splits(8, 8, 32768, 128, 32, 4, bits=[8, 8, 2, 0]) == 4
    assert rq.decode_splits(8, 8, 32768, 128, 32, 4, bits=[4, 3, 2, 0]) == 8
    assert rq.decode_splits(8, 8, 32768, 128, 32, 4, bits=[4, 2, 2, 0]) == 8
    assert rq.decode_splits(8, 8, 32768, 128, 32, 4, bits=[0, 0, 0, 0]) == 8
    assert rq.decode_splits(8, 8, 32768, 128, 32, 4, bits=[8, 4, 2, 7]) == 0  # not a width
    with pytest.raises(ValueError):
        rq.decode_splits(8, 8, 32768, 128, 32, 4, bits=[8, 4, 2])
    tables = ([8, 4, 2, 0], [8, 2, 2, 0], [4, 4, 4, 4], [8, 8, 8, 8, 8, 8, 8, 8], [2] * 8, [3, 8, 0, 0],
              [4, 3, 2, 0], [8, 0, 0, 0])
    for b in (1, 3, 8, 16, 48, 300):
        for h in (1, 4, 8):
            for s in (64, 1000, 4096, 32768):
                for bits in tables:
                    nl = len(bits)
                    g = 16 // nl
                    first = []
                    for w in bits:
                        if first and 4 * _wave_tile_bytes_d128(first + [w]) > 160 * 1024:
                            break
                        first.append(w)
                    one_per_cu = 8 * _wave_tile_bytes_d128(first) > 160 * 1024
                    want = _modelled_splits(b * h, s, 256 if one_per_cu else 512)
                    got = rq.decode_splits(b, h, s, 128, g * h, nl, bits=bits)
                    assert got == want, (b, h, s, bits, got, want)
                    # the workspace holds either plan's split partials
                    n_ws = max(_modelled_splits(b * h, s, 512), _modelled_splits(b * h, s, 256))
                    part = nl * b * g * h * n_ws * (2 * 128 + 2) * 4
                    assert rq.decode_workspace_bytes(b, h, s, 128, g * h, nl) == \
                        (part + 255) // 256 * 256 + nl * b * g * h * 528, (b, h, s, nl)
