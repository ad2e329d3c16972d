"""Python face of librq, the MI355X ResidualQuant hot path.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in include/rq.h. PyTorch provides device memory and streams.
The names follow the C entry points (rq_encode -> encode, ...).

bf16 tensors are torch.bfloat16, fp16 scales torch.float16, packed code
words torch.int32 (the bit patterns of the uint32 words).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import NamedTuple, Optional, Sequence

import torch

__all__ = [
    "LoopView", "RQError", "encode", "encode_into", "reconstruct", "decode_attn", "decode_attn_bf16",
    "encode_rotonly", "reconstruct_rotonly", "encode_append", "decode_attn_varlen", "encode_layers",
    "encode_append_paged", "decode_attn_paged",
    "decode_varlen_workspace_bytes",
    "decode_workspace_bytes", "decode_splits", "format_version", "library_path", "decode_attn_noalloc",
    "NOALLOC_SCRATCH_BYTES",
    "RQ_OK", "RQ_EINVAL", "RQ_EUNSUPPORTED", "RQ_EALIGN", "RQ_EWORKSPACE", "RQ_EHIP", "MAX_LOOPS",
    "WIDTHS",
]

RQ_OK, RQ_EINVAL, RQ_EUNSUPPORTED, RQ_EALIGN, RQ_EWORKSPACE, RQ_EHIP = 0, -1, -2, -3, -4, -5
RQ_OUT_F32, RQ_OUT_BF16 = 0, 1
MAX_LOOPS = 8
MAX_LAYERS = 4096
NOALLOC_SCRATCH_BYTES = 32 << 20  # RQ_NOALLOC_SCRATCH_BYTES
GROUP = 32
WIDTHS = (2, 3, 4, 8)  # residual code widths

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librq.so")
_lib = None


class RQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib.rq_status_str(status).decode() if _lib else status} (status {status})")


class _Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class _LoopView(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p)]


class _Pages(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("n_blocks", ctypes.c_int32)]


class LoopView(NamedTuple):
    """One loop of the cache for decode_attn. bits = 0: the reference loop."""
    bits: int
    k_codes: Optional[torch.Tensor] = None
    k_scales: Optional[torch.Tensor] = None
    v_codes: Optional[torch.Tensor] = None
    v_scales: Optional[torch.Tensor] = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"librq.so is not built ({_LIB_PATH}); run `python -m looped_transformer_kv_rq_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    PP = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "rq_encode": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, PP, ctypes.POINTER(I32), P, PP, PP, P]),
        "rq_reconstruct": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, P, P, P, I32, P, P]),
        "rq_encode_refit": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, PP, ctypes.POINTER(I32), P, PP, PP, I32, P]),
        "rq_encode_append": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, I32, PP, ctypes.POINTER(I32), P, P, P, PP,
                                             PP, P]),
        "rq_decode_attn_varlen_workspace": (SZ, [ctypes.POINTER(_Shape), I32, I32, I32, I32]),
        "rq_decode_attn_varlen": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, I32, P, P, P, ctypes.POINTER(_LoopView),
                                                 P, I32, PP, PP, F, I32, P, P, SZ, P]),
        "rq_encode_rotonly": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, PP, ctypes.POINTER(I32), PP, PP, P]),
        "rq_encode_layers": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, I32, PP, ctypes.POINTER(I32), PP, PP, PP,
                                            P]),
        "rq_encode_append_paged": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.POINTER(_Pages), I32, I32, PP,
                                                  ctypes.POINTER(I32), P, P, P, PP, PP, P]),
        "rq_decode_attn_paged": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, I32, P, P, P, ctypes.POINTER(_LoopView),
                                                ctypes.POINTER(_Pages), P, I32, PP, PP, F, I32, P, P, SZ, P]),
        "rq_reconstruct_rotonly": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, P, P, I32, P, P]),
        "rq_decode_attn_splits": (I32, [ctypes.POINTER(_Shape), I32, I32, ctypes.POINTER(I32), I32]),
        "rq_decode_attn_workspace": (SZ, [ctypes.POINTER(_Shape), I32, I32, I32]),
        "rq_decode_attn": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, I32, P, P, P, ctypes.POINTER(_LoopView),
                                          F, I32, P, P, SZ, P]),
        "rq_decode_attn_bf16": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, I32, P, PP, PP, F, I32, P, P, SZ, P]),
        "rq_decode_attn_noalloc": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, I32, P, P, P,
                                                  ctypes.POINTER(_LoopView), F, I32, P, P]),
        "rq_encode_kv": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, PP, PP, ctypes.POINTER(I32), P, P, PP, PP, PP,
                                        PP, P]),
        "rq_encode_append_kv": (ctypes.c_int, [ctypes.POINTER(_Shape), I32, I32, PP, PP, ctypes.POINTER(I32), P, P,
                                               P, P, P, PP, PP, PP, PP, P]),
        "rq_encode_append_paged_kv": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.POINTER(_Pages), I32, I32, PP,
                                                     PP, ctypes.POINTER(I32), P, P, P, P, P, PP, PP, PP, PP, P]),
        "rq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "rq_format_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def format_version() -> int:
    return _load().rq_format_version()


# ---------------------------------------------------------------------------
# argument checks (dtype / device / layout) before the FFI call
# ---------------------------------------------------------------------------

def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape_of(t: torch.Tensor) -> _Shape:
    if t.dim() != 4:
        raise ValueError("KV tensors are [batch, n_kv_heads, seq_len, head_dim]")
    b, h, s, d = t.shape
    return _Shape(b, h, s, d)


def _stream(device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _check(status: int, what: str):
    if status != RQ_OK:
        raise RQError(status, what)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def encode_into(xs: Sequence[torch.Tensor], ref: torch.Tensor, bits: Sequence[int],
                codes: Sequence[torch.Tensor], scales: Sequence[torch.Tensor], stream=None, refits: int = 0) -> None:
    """rq_encode (rq_encode_refit when refits > 0) into caller-provided outputs."""
    lib = _load()
    shp = _shape_of(ref)
    b, h, s, d = ref.shape
    _need(ref, "ref", torch.bfloat16, ref.shape)
    n = len(xs)
    if not (len(bits) == len(codes) == len(scales) == n):
        raise ValueError("xs, bits, codes and scales must have one entry per loop")
    for i in range(n):
        _need(xs[i], f"xs[{i}]", torch.bfloat16, ref.shape, ref.device)
        _need(codes[i], f"codes[{i}]", torch.int32, (b, h, s, d * int(bits[i]) // 32), ref.device)
        _need(scales[i], f"scales[{i}]", torch.float16, (b, h, s, d // GROUP), ref.device)
    bits_arr = (ctypes.c_int32 * n)(*[int(x) for x in bits])
    if refits:
        st = lib.rq_encode_refit(ctypes.byref(shp), n, _ptr_array(xs), bits_arr, _ptr(ref), _ptr_array(codes),
                                 _ptr_array(scales), int(refits), _stream(ref.device, stream))
        _check(st, "rq_encode_refit")
    else:
        st = lib.rq_encode(ctypes.byref(shp), n, _ptr_array(xs), bits_arr, _ptr(ref), _ptr_array(codes),
                           _ptr_array(scales), _stream(ref.device, stream))
        _check(st, "rq_encode")


def _check_loop_outputs(xs, ref, bits, codes, scales, rows, what):
    """Shapes of one tensor's loop states and outputs: rows = the leading [B, Hkv, S] of codes / scales."""
    b, h, s, d = ref.shape
    n = len(xs)
    if not (len(bits) == len(codes) == len(scales) == n):
        raise ValueError(f"{what}: xs, bits, codes and scales must have one entry per loop")
    for i in range(n):
        _need(xs[i], f"{what} xs[{i}]", torch.bfloat16, ref.shape, ref.device)
        _need(codes[i], f"{what} codes[{i}]", torch.int32, rows + (d * int(bits[i]) // 32,), ref.device)
        _need(scales[i], f"{what} scales[{i}]", torch.float16, rows + (d // GROUP,), ref.device)


def encode_kv_into(kx: Sequence[torch.Tensor], vx: Sequence[torch.Tensor], k_ref: torch.Tensor, v_ref: torch.Tensor,
                   bits: Sequence[int], k_codes: Sequence[torch.Tensor], k_scales: Sequence[torch.Tensor],
                   v_codes: Sequence[torch.Tensor], v_scales: Sequence[torch.Tensor], stream=None) -> None:
    """rq_encode_kv: encode_into for K and V in one launch (bit-identical to two encode_into calls)."""
    lib = _load()
    _need(k_ref, "k_ref", torch.bfloat16, k_ref.shape)
    _need(v_ref, "v_ref", torch.bfloat16, k_ref.shape, k_ref.device)
    rows = tuple(k_ref.shape[:3])
    _check_loop_outputs(kx, k_ref, bits, k_codes, k_scales, rows, "K")
    _check_loop_outputs(vx, v_ref, bits, v_codes, v_scales, rows, "V")
    n = len(kx)
    bits_arr = (ctypes.c_int32 * n)(*[int(x) for x in bits])
    st = lib.rq_encode_kv(ctypes.byref(_shape_of(k_ref)), n, _ptr_array(kx), _ptr_array(vx), bits_arr, _ptr(k_ref),
                          _ptr(v_ref), _ptr_array(k_codes), _ptr_array(k_scales), _ptr_array(v_codes),
                          _ptr_array(v_scales), _stream(k_ref.device, stream))
    _check(st, "rq_encode_kv")


def encode(xs: Sequence[torch.Tensor], ref: torch.Tensor, bits: Sequence[int], stream=None, refits: int = 0):
    """Encode loops xs[i] (bf16 [B,Hkv,S,D]) against the final-loop ref, with `refits`
    extra code / LS-scale alternations. Returns (codes, scales): per loop int32
    [B,Hkv,S,D*bits/32] and fp16 [B,Hkv,S,D/32]."""
    if ref.dim() != 4:
        raise ValueError("ref must be [batch, n_kv_heads, seq_len, head_dim]")
    b, h, s, d = ref.shape
    for x in bits:
        if int(x) not in WIDTHS:
            raise ValueError(f"encode bit widths must be in {WIDTHS}")
    codes = [torch.empty((b, h, s, d * int(x) // 32), dtype=torch.int32, device=ref.device) for x in bits]
    scales = [torch.empty((b, h, s, d // GROUP), dtype=torch.float16, device=ref.device) for _ in bits]
    encode_into(xs, ref, bits, codes, scales, stream, refits)
    return codes, scales


def encode_rotonly(xs: Sequence[torch.Tensor], bits: Sequence[int], stream=None):
    """Rotation-only baseline: quantize each state xs[i] (bf16 [B,Hkv,S,D]) directly
    after the rotation, with no reference. Returns (codes, scales) as encode()."""
    lib = _load()
    if len(xs) == 0 or len(xs) != len(bits):
        raise ValueError("xs and bits must have one entry per state")
    x0 = xs[0]
    shp = _shape_of(x0)
    b, h, s, d = x0.shape
    for x in bits:
        if int(x) not in WIDTHS:
            raise ValueError(f"bit widths must be in {WIDTHS}")
    codes = [torch.empty((b, h, s, d * int(x) // 32), dtype=torch.int32, device=x0.device) for x in bits]
    scales = [torch.empty((b, h, s, d // GROUP), dtype=torch.float16, device=x0.device) for _ in bits]
    for i, x in enumerate(xs):
        _need(x, f"xs[{i}]", torch.bfloat16, x0.shape, x0.device)
    n = len(xs)
    bits_arr = (ctypes.c_int32 * n)(*[int(x) for x in bits])
    st = lib.rq_encode_rotonly(ctypes.byref(shp), n, _ptr_array(xs), bits_arr, _ptr_array(codes),
                               _ptr_array(scales), _stream(x0.device, stream))
    _check(st, "rq_encode_rotonly")
    return codes, scales


def reconstruct_rotonly(codes: torch.Tensor, scales: torch.Tensor, bits: int, out_dtype: torch.dtype = torch.float32,
                        out: Optional[torch.Tensor] = None, stream=None):
    """Rotation-only state: out = H (s * q)."""
    lib = _load()
    if bits not in WIDTHS:
        raise ValueError(f"bits must be in {WIDTHS}")
    if codes.dim() != 4:
        raise ValueError("codes must be [batch, n_kv_heads, seq_len, head_dim*bits/32]")
    b, h, s, w = codes.shape
    d = w * 32 // bits
    shp = _Shape(b, h, s, d)
    _need(codes, "codes", torch.int32, (b, h, s, w))
    _need(scales, "scales", torch.float16, (b, h, s, d // GROUP), codes.device)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((b, h, s, d), dtype=out_dtype, device=codes.device)
    _need(out, "out", out_dtype, (b, h, s, d), codes.device)
    kind = RQ_OUT_F32 if out_dtype == torch.float32 else RQ_OUT_BF16
    st = lib.rq_reconstruct_rotonly(ctypes.byref(shp), int(bits), _ptr(codes), _ptr(scales), kind, _ptr(out),
                                    _stream(codes.device, stream))
    _check(st, "rq_reconstruct_rotonly")
    return out


def reconstruct(ref: torch.Tensor, codes: Optional[torch.Tensor], scales: Optional[torch.Tensor], bits: int,
                out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None, stream=None):
    """x_hat = ref + H (s * q); bits = 0 returns a copy of ref. float32 or bfloat16 output."""
    lib = _load()
    shp = _shape_of(ref)
    _need(ref, "ref", torch.bfloat16, ref.shape)
    b, h, s, d = ref.shape
    if bits:
        _need(codes, "codes", torch.int32, (b, h, s, d * bits // 32), ref.device)
        _need(scales, "scales", torch.float16, (b, h, s, d // GROUP), ref.device)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty(ref.shape, dtype=out_dtype, device=ref.device)
    _need(out, "out", out_dtype, ref.shape, ref.device)
    kind = RQ_OUT_F32 if out_dtype == torch.float32 else RQ_OUT_BF16
    st = lib.rq_reconstruct(ctypes.byref(shp), int(bits), _ptr(ref), _ptr(codes if bits else None),
                            _ptr(scales if bits else None), kind, _ptr(out), _stream(ref.device, stream))
    _check(st, "rq_reconstruct")
    return out


def decode_splits(batch: int, n_kv_heads: int, seq_len: int, head_dim: int, n_q_heads: int, n_loops: int,
                  n_splits: int = 0, bits: Optional[Sequence[int]] = None) -> int:
    """Split count of a decode call; bits: the loops' widths (None: widths that fit two blocks per CU)."""
    shp = _Shape(batch, n_kv_heads, seq_len, head_dim)
    arr = None
    if bits is not None:
        if len(bits) != n_loops:
            raise ValueError("bits needs one width per loop")
        arr = (ctypes.c_int32 * n_loops)(*bits)
    return _load().rq_decode_attn_splits(ctypes.byref(shp), n_q_heads, n_loops, arr, n_splits)


def decode_workspace_bytes(batch: int, n_kv_heads: int, seq_len: int, head_dim: int, n_q_heads: int,
                           n_loops: int, n_splits: int = 0) -> int:
    shp = _Shape(batch, n_kv_heads, seq_len, head_dim)
    return _load().rq_decode_attn_workspace(ctypes.byref(shp), n_q_heads, n_loops, n_splits)


def _workspace(ref, n_q_heads, n_loops, n_splits, workspace):
    b, h, s, d = ref.shape
    need = decode_workspace_bytes(b, h, s, d, n_q_heads, n_loops, n_splits)
    if need == 0:
        raise RQError(RQ_EINVAL, "decode workspace query")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=ref.device)
    return workspace


def _loop_views(loops, n_loops, k_ref):
    b, h, s, d = k_ref.shape
    if len(loops) != n_loops:
        raise ValueError("one LoopView per loop of q")
    views = (_LoopView * n_loops)()
    for i, lv in enumerate(loops):
        views[i].bits = int(lv.bits)
        if lv.bits:
            _need(lv.k_codes, f"loops[{i}].k_codes", torch.int32, (b, h, s, d * lv.bits // 32), k_ref.device)
            _need(lv.v_codes, f"loops[{i}].v_codes", torch.int32, (b, h, s, d * lv.bits // 32), k_ref.device)
            _need(lv.k_scales, f"loops[{i}].k_scales", torch.float16, (b, h, s, d // GROUP), k_ref.device)
            _need(lv.v_scales, f"loops[{i}].v_scales", torch.float16, (b, h, s, d // GROUP), k_ref.device)
            views[i].k_codes = lv.k_codes.data_ptr()
            views[i].k_scales = lv.k_scales.data_ptr()
            views[i].v_codes = lv.v_codes.data_ptr()
            views[i].v_scales = lv.v_scales.data_ptr()
    return views


def decode_varlen_workspace_bytes(batch: int, n_kv_heads: int, s_cap: int, head_dim: int, n_q_heads: int,
                                  n_loops: int, n_splits: int = 0, tail_len: int = 0) -> int:
    shp = _Shape(batch, n_kv_heads, s_cap, head_dim)
    return _load().rq_decode_attn_varlen_workspace(ctypes.byref(shp), n_q_heads, n_loops, n_splits, tail_len)


def decode_attn_varlen(q: torch.Tensor, k_ref: torch.Tensor, v_ref: torch.Tensor, loops: Sequence[LoopView],
                       seq_lens: Optional[torch.Tensor] = None, tail_k: Optional[Sequence[torch.Tensor]] = None,
                       tail_v: Optional[Sequence[torch.Tensor]] = None, softmax_scale: Optional[float] = None,
                       n_splits: int = 0, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Decode over a partly filled cache [B, Hkv, S_cap, D]: sequence b attends to its first
    seq_lens[b] positions (int32 device [B]; None = all) and then to the bf16 tail positions
    tail_k[i] / tail_v[i] ([B, Hkv, T, D] per loop; None = no tail)."""
    lib = _load()
    shp = _shape_of(k_ref)
    b, h, s, d = k_ref.shape
    n_loops, _, hq, _ = q.shape
    _need(q, "q", torch.bfloat16, (n_loops, b, hq, d), k_ref.device)
    _need(k_ref, "k_ref", torch.bfloat16, k_ref.shape)
    _need(v_ref, "v_ref", torch.bfloat16, k_ref.shape, k_ref.device)
    views = _loop_views(loops, n_loops, k_ref)
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32, (b,), k_ref.device)
    tail_len = 0
    tk = tv = None
    if tail_k is not None or tail_v is not None:
        if tail_k is None or tail_v is None or len(tail_k) != n_loops or len(tail_v) != n_loops:
            raise ValueError("tail_k and tail_v need one bf16 [B, Hkv, T, D] tensor per loop")
        tail_len = tail_k[0].shape[2]
        for i in range(n_loops):
            _need(tail_k[i], f"tail_k[{i}]", torch.bfloat16, (b, h, tail_len, d), k_ref.device)
            _need(tail_v[i], f"tail_v[{i}]", torch.bfloat16, (b, h, tail_len, d), k_ref.device)
        tk, tv = _ptr_array(tail_k), _ptr_array(tail_v)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((n_loops, b, hq, d), dtype=torch.float32, device=k_ref.device)
    _need(out, "out", torch.float32, (n_loops, b, hq, d), k_ref.device)
    need = decode_varlen_workspace_bytes(b, h, s, d, hq, n_loops, n_splits, tail_len)
    if need == 0:
        raise RQError(RQ_EINVAL, "decode workspace query")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=k_ref.device)
    st = lib.rq_decode_attn_varlen(ctypes.byref(shp), hq, n_loops, _ptr(q), _ptr(k_ref), _ptr(v_ref), views,
                                   _ptr(seq_lens), int(tail_len), tk, tv, float(softmax_scale), int(n_splits),
                                   _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(k_ref.device, stream))
    _check(st, "rq_decode_attn_varlen")
    return out


def _pages_of(block_table: torch.Tensor, block_size: int, n_blocks: int, batch: int, device) -> _Pages:
    if block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError("block_table must be int32 [batch, max_blocks]")
    _need(block_table, "block_table", torch.int32, tuple(block_table.shape), device)
    return _Pages(block_table.data_ptr(), block_table.shape[1], int(block_size), int(n_blocks))


def decode_attn_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, loops: Sequence[LoopView],
                      block_table: torch.Tensor, seq_lens: Optional[torch.Tensor] = None,
                      tail_k: Optional[Sequence[torch.Tensor]] = None, tail_v: Optional[Sequence[torch.Tensor]] = None,
                      softmax_scale: Optional[float] = None, n_splits: int = 0, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """decode_attn_varlen over a block-paged cache: k_pages, v_pages bf16 [n_blocks, Hkv, P, D] and
    the loop views' codes / scales [n_blocks, Hkv, P, ...]; block_table int32 device [B, max_blocks]
    (position t of sequence b is in block block_table[b, t // P] at offset t % P). Tails stay
    dense [B, Hkv, T, D]."""
    lib = _load()
    n_blocks, h, p, d = k_pages.shape
    n_loops, b, hq, _ = q.shape
    _need(q, "q", torch.bfloat16, (n_loops, b, hq, d), k_pages.device)
    _need(k_pages, "k_pages", torch.bfloat16, k_pages.shape)
    _need(v_pages, "v_pages", torch.bfloat16, k_pages.shape, k_pages.device)
    pages = _pages_of(block_table, p, n_blocks, b, k_pages.device)
    s_cap = pages.max_blocks * p
    shp = _Shape(b, h, s_cap, d)
    views = _loop_views(loops, n_loops, k_pages)
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32, (b,), k_pages.device)
    tail_len = 0
    tk = tv = None
    if tail_k is not None or tail_v is not None:
        if tail_k is None or tail_v is None or len(tail_k) != n_loops or len(tail_v) != n_loops:
            raise ValueError("tail_k and tail_v need one bf16 [B, Hkv, T, D] tensor per loop")
        tail_len = tail_k[0].shape[2]
        for i in range(n_loops):
            _need(tail_k[i], f"tail_k[{i}]", torch.bfloat16, (b, h, tail_len, d), k_pages.device)
            _need(tail_v[i], f"tail_v[{i}]", torch.bfloat16, (b, h, tail_len, d), k_pages.device)
        tk, tv = _ptr_array(tail_k), _ptr_array(tail_v)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((n_loops, b, hq, d), dtype=torch.float32, device=k_pages.device)
    _need(out, "out", torch.float32, (n_loops, b, hq, d), k_pages.device)
    need = decode_varlen_workspace_bytes(b, h, s_cap, d, hq, n_loops, n_splits, tail_len)
    if need == 0:
        raise RQError(RQ_EINVAL, "decode workspace query")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=k_pages.device)
    st = lib.rq_decode_attn_paged(ctypes.byref(shp), hq, n_loops, _ptr(q), _ptr(k_pages), _ptr(v_pages), views,
                                  ctypes.byref(pages), _ptr(seq_lens), int(tail_len), tk, tv, float(softmax_scale),
                                  int(n_splits), _ptr(out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(k_pages.device, stream))
    _check(st, "rq_decode_attn_paged")
    return out


def encode_append_paged(xs: Sequence[torch.Tensor], ref_new: torch.Tensor, bits: Sequence[int], pos: torch.Tensor,
                        block_table: torch.Tensor, ref_pages: torch.Tensor, codes: Sequence[torch.Tensor],
                        scales: Sequence[torch.Tensor], stream=None) -> None:
    """encode_append into a block-paged cache: ref_pages bf16 [n_blocks, Hkv, P, D], codes[i] /
    scales[i] [n_blocks, Hkv, P, ...], block_table int32 device [B, max_blocks]."""
    lib = _load()
    b, h, t, d = ref_new.shape
    n_blocks, _, p, _ = ref_pages.shape
    _need(ref_new, "ref_new", torch.bfloat16, ref_new.shape)
    _need(ref_pages, "ref_pages", torch.bfloat16, (n_blocks, h, p, d), ref_new.device)
    _need(pos, "pos", torch.int32, (b,), ref_new.device)
    pages = _pages_of(block_table, p, n_blocks, b, ref_new.device)
    n = len(xs)
    if not (len(bits) == len(codes) == len(scales) == n):
        raise ValueError("xs, bits, codes and scales must have one entry per loop")
    for i in range(n):
        _need(xs[i], f"xs[{i}]", torch.bfloat16, ref_new.shape, ref_new.device)
        _need(codes[i], f"codes[{i}]", torch.int32, (n_blocks, h, p, d * int(bits[i]) // 32), ref_new.device)
        _need(scales[i], f"scales[{i}]", torch.float16, (n_blocks, h, p, d // GROUP), ref_new.device)
    shp = _Shape(b, h, pages.max_blocks * p, d)
    bits_arr = (ctypes.c_int32 * n)(*[int(x) for x in bits])
    st = lib.rq_encode_append_paged(ctypes.byref(shp), ctypes.byref(pages), n, t, _ptr_array(xs), bits_arr,
                                    _ptr(ref_new), _ptr(pos), _ptr(ref_pages), _ptr_array(codes), _ptr_array(scales),
                                    _stream(ref_new.device, stream))
    _check(st, "rq_encode_append_paged")


def encode_append(xs: Sequence[torch.Tensor], ref_new: torch.Tensor, bits: Sequence[int], pos: torch.Tensor,
                  ref_cache: torch.Tensor, codes: Sequence[torch.Tensor], scales: Sequence[torch.Tensor],
                  stream=None) -> None:
    """Encode new positions (xs[i], ref_new: bf16 [B, Hkv, T, D]) into a cache of capacity S_cap at
    positions pos[b] + t (pos: int32 device [B]); ref_new is copied into ref_cache [B, Hkv, S_cap, D]."""
    lib = _load()
    b, h, t, d = ref_new.shape
    _need(ref_new, "ref_new", torch.bfloat16, ref_new.shape)
    _need(ref_cache, "ref_cache", torch.bfloat16, (b, h, ref_cache.shape[2], d), ref_new.device)
    s_cap = ref_cache.shape[2]
    _need(pos, "pos", torch.int32, (b,), ref_new.device)
    n = len(xs)
    if not (len(bits) == len(codes) == len(scales) == n):
        raise ValueError("xs, bits, codes and scales must have one entry per loop")
    for i in range(n):
        _need(xs[i], f"xs[{i}]", torch.bfloat16, ref_new.shape, ref_new.device)
        _need(codes[i], f"codes[{i}]", torch.int32, (b, h, s_cap, d * int(bits[i]) // 32), ref_new.device)
        _need(scales[i], f"scales[{i}]", torch.float16, (b, h, s_cap, d // GROUP), ref_new.device)
    shp = _Shape(b, h, s_cap, d)
    bits_arr = (ctypes.c_int32 * n)(*[int(x) for x in bits])
    st = lib.rq_encode_append(ctypes.byref(shp), n, t, _ptr_array(xs), bits_arr, _ptr(ref_new), _ptr(pos),
                              _ptr(ref_cache), _ptr_array(codes), _ptr_array(scales), _stream(ref_new.device, stream))
    _check(st, "rq_encode_append")


def encode_append_kv(kx: Sequence[torch.Tensor], vx: Sequence[torch.Tensor], k_ref_new: torch.Tensor,
                     v_ref_new: torch.Tensor, bits: Sequence[int], pos: torch.Tensor, k_ref_cache: torch.Tensor,
                     v_ref_cache: torch.Tensor, k_codes: Sequence[torch.Tensor], k_scales: Sequence[torch.Tensor],
                     v_codes: Sequence[torch.Tensor], v_scales: Sequence[torch.Tensor], stream=None) -> None:
    """rq_encode_append_kv: encode_append for K and V in one launch (bit-identical to two calls)."""
    lib = _load()
    b, h, t, d = k_ref_new.shape
    _need(k_ref_new, "k_ref_new", torch.bfloat16, k_ref_new.shape)
    _need(v_ref_new, "v_ref_new", torch.bfloat16, k_ref_new.shape, k_ref_new.device)
    s_cap = k_ref_cache.shape[2]
    _need(k_ref_cache, "k_ref_cache", torch.bfloat16, (b, h, s_cap, d), k_ref_new.device)
    _need(v_ref_cache, "v_ref_cache", torch.bfloat16, (b, h, s_cap, d), k_ref_new.device)
    _need(pos, "pos", torch.int32, (b,), k_ref_new.device)
    _check_loop_outputs(kx, k_ref_new, bits, k_codes, k_scales, (b, h, s_cap), "K")
    _check_loop_outputs(vx, v_ref_new, bits, v_codes, v_scales, (b, h, s_cap), "V")
    n = len(kx)
    shp = _Shape(b, h, s_cap, d)
    bits_arr = (ctypes.c_int32 * n)(*[int(x) for x in bits])
    st = lib.rq_encode_append_kv(ctypes.byref(shp), n, t, _ptr_array(kx), _ptr_array(vx), bits_arr, _ptr(k_ref_new),
                                 _ptr(v_ref_new), _ptr(pos), _ptr(k_ref_cache), _ptr(v_ref_cache),
                                 _ptr_array(k_codes), _ptr_array(k_scales), _ptr_array(v_codes), _ptr_array(v_scales),
                                 _stream(k_ref_new.device, stream))
    _check(st, "rq_encode_append_kv")


def encode_append_paged_kv(kx: Sequence[torch.Tensor], vx: Sequence[torch.Tensor], k_ref_new: torch.Tensor,
                           v_ref_new: torch.Tensor, bits: Sequence[int], pos: torch.Tensor, block_table: torch.Tensor,
                           k_ref_pages: torch.Tensor, v_ref_pages: torch.Tensor, k_codes: Sequence[torch.Tensor],
                           k_scales: Sequence[torch.Tensor], v_codes: Sequence[torch.Tensor],
                           v_scales: Sequence[torch.Tensor], stream=None) -> None:
    """rq_encode_append_paged_kv: encode_append_paged for K and V in one launch (bit-identical to two calls)."""
    lib = _load()
    b, h, t, d = k_ref_new.shape
    n_blocks, _, p, _ = k_ref_pages.shape
    _need(k_ref_new, "k_ref_new", torch.bfloat16, k_ref_new.shape)
    _need(v_ref_new, "v_ref_new", torch.bfloat16, k_ref_new.shape, k_ref_new.device)
    _need(k_ref_pages, "k_ref_pages", torch.bfloat16, (n_blocks, h, p, d), k_ref_new.device)
    _need(v_ref_pages, "v_ref_pages", torch.bfloat16, (n_blocks, h, p, d), k_ref_new.device)
    _need(pos, "pos", torch.int32, (b,), k_ref_new.device)
    pages = _pages_of(block_table, p, n_blocks, b, k_ref_new.device)
    _check_loop_outputs(kx, k_ref_new, bits, k_codes, k_scales, (n_blocks, h, p), "K")
    _check_loop_outputs(vx, v_ref_new, bits, v_codes, v_scales, (n_blocks, h, p), "V")
    n = len(kx)
    shp = _Shape(b, h, pages.max_blocks * p, d)
    bits_arr = (ctypes.c_int32 * n)(*[int(x) for x in bits])
    st = lib.rq_encode_append_paged_kv(ctypes.byref(shp), ctypes.byref(pages), n, t, _ptr_array(kx), _ptr_array(vx),
                                       bits_arr, _ptr(k_ref_new), _ptr(v_ref_new), _ptr(pos), _ptr(k_ref_pages),
                                       _ptr(v_ref_pages), _ptr_array(k_codes), _ptr_array(k_scales),
                                       _ptr_array(v_codes), _ptr_array(v_scales), _stream(k_ref_new.device, stream))
    _check(st, "rq_encode_append_paged_kv")


def encode_layers(xs: Sequence[Sequence[torch.Tensor]], refs: Sequence[torch.Tensor],
                  bits_table: Sequence[Sequence[int]], stream=None):
    """Encode several layers' caches with a per-(layer, loop) bit table: xs[l][i] is loop i of
    layer l and refs[l] its final loop (bf16 [B, Hkv, S, D], one shape for all layers);
    bits_table[l][i] in WIDTHS. Returns (codes, scales) indexed [l][i] as encode()."""
    lib = _load()
    n_layers = len(refs)
    if n_layers == 0 or len(xs) != n_layers or len(bits_table) != n_layers:
        raise ValueError("xs, refs and bits_table must have one entry per layer")
    n = len(xs[0])
    if any(len(row) != n for row in xs) or any(len(row) != n for row in bits_table):
        raise ValueError("every layer must have the same number of loops")
    r0 = refs[0]
    shp = _shape_of(r0)
    b, h, s, d = r0.shape
    codes, scales = [], []
    for l in range(n_layers):
        _need(refs[l], f"refs[{l}]", torch.bfloat16, r0.shape, r0.device)
        for i in range(n):
            if int(bits_table[l][i]) not in WIDTHS:
                raise ValueError(f"bit widths must be in {WIDTHS}")
            _need(xs[l][i], f"xs[{l}][{i}]", torch.bfloat16, r0.shape, r0.device)
        codes.append([torch.empty((b, h, s, d * int(x) // 32), dtype=torch.int32, device=r0.device)
                      for x in bits_table[l]])
        scales.append([torch.empty((b, h, s, d // GROUP), dtype=torch.float16, device=r0.device)
                       for _ in bits_table[l]])
    flat = lambda rows: [t for row in rows for t in row]  # noqa: E731  (layer-major)
    bits_arr = (ctypes.c_int32 * (n_layers * n))(*[int(x) for row in bits_table for x in row])
    st = lib.rq_encode_layers(ctypes.byref(shp), n_layers, n, _ptr_array(flat(xs)), bits_arr, _ptr_array(refs),
                              _ptr_array(flat(codes)), _ptr_array(flat(scales)), _stream(r0.device, stream))
    _check(st, "rq_encode_layers")
    return codes, scales


def decode_attn(q: torch.Tensor, k_ref: torch.Tensor, v_ref: torch.Tensor, loops: Sequence[LoopView],
                softmax_scale: Optional[float] = None, n_splits: int = 0, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Fused reconstruct + single-query decode attention over the residual cache.
    q: bf16 [n_loops, B, Hq, D]; returns float32 [n_loops, B, Hq, D]."""
    lib = _load()
    shp = _shape_of(k_ref)
    b, h, s, d = k_ref.shape
    if q.dim() != 4:
        raise ValueError("q must be [n_loops, batch, n_q_heads, head_dim]")
    n_loops, _, hq, _ = q.shape
    _need(q, "q", torch.bfloat16, (n_loops, b, hq, d), k_ref.device)
    _need(k_ref, "k_ref", torch.bfloat16, k_ref.shape)
    _need(v_ref, "v_ref", torch.bfloat16, k_ref.shape, k_ref.device)
    views = _loop_views(loops, n_loops, k_ref)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((n_loops, b, hq, d), dtype=torch.float32, device=k_ref.device)
    _need(out, "out", torch.float32, (n_loops, b, hq, d), k_ref.device)
    workspace = _workspace(k_ref, hq, n_loops, n_splits, workspace)
    st = lib.rq_decode_attn(ctypes.byref(shp), hq, n_loops, _ptr(q), _ptr(k_ref), _ptr(v_ref), views,
                            float(softmax_scale), int(n_splits), _ptr(out), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(k_ref.device, stream))
    _check(st, "rq_decode_attn")
    return out


def decode_attn_noalloc(q: torch.Tensor, k_ref: torch.Tensor, v_ref: torch.Tensor, loops: Sequence[LoopView],
                        softmax_scale: Optional[float] = None, n_splits: int = 0, out: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """rq_decode_attn_noalloc: decode_attn without a workspace argument; the
    library's static device scratch (NOALLOC_SCRATCH_BYTES per GPU) holds the
    split partials. With `out` given, the call allocates no device memory.
    Calls on one GPU must not overlap (they share the scratch)."""
    lib = _load()
    shp = _shape_of(k_ref)
    b, h, s, d = k_ref.shape
    if q.dim() != 4:
        raise ValueError("q must be [n_loops, batch, n_q_heads, head_dim]")
    n_loops, _, hq, _ = q.shape
    _need(q, "q", torch.bfloat16, (n_loops, b, hq, d), k_ref.device)
    _need(k_ref, "k_ref", torch.bfloat16, k_ref.shape)
    _need(v_ref, "v_ref", torch.bfloat16, k_ref.shape, k_ref.device)
    views = _loop_views(loops, n_loops, k_ref)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((n_loops, b, hq, d), dtype=torch.float32, device=k_ref.device)
    _need(out, "out", torch.float32, (n_loops, b, hq, d), k_ref.device)
    st = lib.rq_decode_attn_noalloc(ctypes.byref(shp), hq, n_loops, _ptr(q), _ptr(k_ref), _ptr(v_ref), views,
                                    float(softmax_scale), int(n_splits), _ptr(out), _stream(k_ref.device, stream))
    _check(st, "rq_decode_attn_noalloc")
    return out


def decode_attn_bf16(q: torch.Tensor, k: Sequence[torch.Tensor], v: Sequence[torch.Tensor],
                     softmax_scale: Optional[float] = None, n_splits: int = 0, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The uncompressed baseline: loop i attends over its own bf16 K/V (k[i], v[i])."""
    lib = _load()
    n_loops, _, hq, _ = q.shape
    if len(k) != n_loops or len(v) != n_loops:
        raise ValueError("one K and one V per loop of q")
    shp = _shape_of(k[0])
    b, h, s, d = k[0].shape
    _need(q, "q", torch.bfloat16, (n_loops, b, hq, d), k[0].device)
    for i in range(n_loops):
        _need(k[i], f"k[{i}]", torch.bfloat16, k[0].shape, k[0].device)
        _need(v[i], f"v[{i}]", torch.bfloat16, k[0].shape, k[0].device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((n_loops, b, hq, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (n_loops, b, hq, d), q.device)
    workspace = _workspace(k[0], hq, n_loops, n_splits, workspace)
    st = lib.rq_decode_attn_bf16(ctypes.byref(shp), hq, n_loops, _ptr(q), _ptr_array(k), _ptr_array(v),
                                 float(softmax_scale), int(n_splits), _ptr(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(q.device, stream))
    _check(st, "rq_decode_attn_bf16")
    return out
