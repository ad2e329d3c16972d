"""Seeded synthetic inputs for the ResidualQuant hot path.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark. It holds no part of the method's arithmetic: it only draws
random numbers and rounds them to the storage formats (bf16 / fp16 bit
patterns) that both sides consume.

Workloads follow the five synthetic configurations of the ResidualQuant study
(a looped Transformer whose final-loop K/V is the reference and whose earlier
loops differ from it by a small residual; ResidualQuant abstract). Every
(batch, kv_head) row has its own PCG64 stream keyed by
``[seed, b, h, tensor, loop]`` so that any row can be regenerated without
building the whole tensor.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

TENSOR_K = 0
TENSOR_V = 1
TENSOR_Q = 2
TENSOR_PACKED_K = 3
TENSOR_PACKED_V = 4

GROUP = 32  # storage group of one fp16 scale (head_dim elements per scale)


@dataclass(frozen=True)
class Workload:
    """One synthetic configuration. ``bits[l]`` is the residual width of loop
    ``l`` (0 marks the final loop, stored as the bf16 reference)."""

    name: str
    index: int
    n_loops: int
    batch: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    seq_len: int
    bits: tuple
    sigma: tuple
    heavy_tailed: bool = False

    @property
    def seed(self) -> int:
        return 20261007 + self.index

    @property
    def group_size(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_batch(self, batch: int) -> "Workload":
        return replace(self, batch=batch)

    def with_seq(self, seq_len: int) -> "Workload":
        return replace(self, seq_len=seq_len)


def _sigma_geometric(n_loops: int) -> tuple:
    # distance d = L-1-l from the final loop; 0.05 at d=1 growing to 0.2 at d=L-1
    out = []
    for l in range(n_loops):
        d = n_loops - 1 - l
        out.append(0.0 if d == 0 else 0.05 * 4.0 ** ((d - 1) / (n_loops - 2)))
    return tuple(out)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 1, 2, 8, 64, 256, (2, 2, 2, 0), (0.1, 0.075, 0.05, 0.0)),
    "l4_b16_s4k": Workload("l4_b16_s4k", 2, 4, 16, 8, 32, 128, 4096, (2, 2, 2, 0), (0.2, 0.1, 0.05, 0.0)),
    "mixed_s32k": Workload("mixed_s32k", 3, 4, 8, 8, 32, 128, 32768, (4, 2, 2, 0), (0.2, 0.1, 0.05, 0.0)),
    "heavy_tail": Workload("heavy_tail", 4, 4, 32, 8, 32, 128, 8192, (2, 2, 2, 0), (0.2, 0.1, 0.05, 0.0), True),
    "peak_batch": Workload("peak_batch", 5, 8, 4, 4, 16, 128, 16384, (4, 2, 2, 2, 2, 2, 2, 0), _sigma_geometric(8)),
}

# A per-(layer, loop) width table for four layers of the l4_b16_s4k shape. The
# pages fill such a table by calibration, which is out of scope; this one is
# synthetic: wider codes in earlier layers and in loops far from the final
# loop, every width once. Row l is layer l's bits per loop (0: the reference).
LAYER_BITS_L4 = ((8, 4, 2, 0), (4, 3, 2, 0), (3, 3, 2, 0), (2, 2, 2, 0))

HEAVY_SCALE = 20.0
HEAVY_CHANNELS = 4


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns
    the 16-bit patterns. Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def heavy_channels(w: Workload) -> np.ndarray:
    """Indices of the K channels scaled x20 in the heavy-tailed workload."""
    return np.sort(np.random.default_rng(w.seed).choice(w.head_dim, HEAVY_CHANNELS, replace=False))


def _rng(w: Workload, b: int, h: int, tensor: int, loop: int) -> np.random.Generator:
    return np.random.default_rng([w.seed, b, h, tensor, loop])


def _ref_f32(w: Workload, b: int, h: int, tensor: int) -> np.ndarray:
    rng = _rng(w, b, h, tensor, w.n_loops - 1)
    shape = (w.seq_len, w.head_dim)
    if w.heavy_tailed and tensor == TENSOR_V:
        x = rng.standard_t(4, size=shape).astype(np.float32)
    else:
        x = rng.standard_normal(shape, dtype=np.float32)
    if w.heavy_tailed and tensor == TENSOR_K:
        x[:, heavy_channels(w)] *= np.float32(HEAVY_SCALE)
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _noise_f32(w: Workload, b: int, h: int, tensor: int, loop: int) -> np.ndarray:
    rng = _rng(w, b, h, tensor, loop)
    shape = (w.seq_len, w.head_dim)
    if w.heavy_tailed and tensor == TENSOR_V:
        n = rng.standard_t(4, size=shape).astype(np.float32)
    else:
        n = rng.standard_normal(shape, dtype=np.float32)
    if w.heavy_tailed and tensor == TENSOR_K:
        n[:, heavy_channels(w)] *= np.float32(HEAVY_SCALE)
    return n


def kv_row(w: Workload, b: int, h: int, tensor: int, loop: int) -> np.ndarray:
    """bf16 bits [S, D] of loop ``loop``'s K (tensor=0) or V (tensor=1) for
    one (batch, kv_head) row. The final loop is the reference; loop l is the
    reference plus sigma_l times fresh noise, rounded to bf16."""
    ref = _ref_f32(w, b, h, tensor)
    if loop == w.n_loops - 1:
        return f32_to_bf16_bits(ref)
    x = ref + np.float32(w.sigma[loop]) * _noise_f32(w, b, h, tensor, loop)
    return f32_to_bf16_bits(x)


def kv_rows_all_loops(w: Workload, b: int, h: int, tensor: int) -> list:
    """All loops of one row, sharing one draw of the reference."""
    ref = _ref_f32(w, b, h, tensor)
    out = []
    for loop in range(w.n_loops):
        if loop == w.n_loops - 1:
            out.append(f32_to_bf16_bits(ref))
        else:
            out.append(f32_to_bf16_bits(ref + np.float32(w.sigma[loop]) * _noise_f32(w, b, h, tensor, loop)))
    return out


def q_row(w: Workload, b: int, hq: int, loop: int) -> np.ndarray:
    """bf16 bits [D] of the decode query of loop ``loop``, query head ``hq``."""
    rng = _rng(w, b, hq, TENSOR_Q, loop)
    return f32_to_bf16_bits(rng.standard_normal(w.head_dim, dtype=np.float32))


def q_tensor(w: Workload) -> np.ndarray:
    """bf16 bits [L, B, Hq, D]: one independent N(0,1) query per loop and head."""
    out = np.empty((w.n_loops, w.batch, w.n_q_heads, w.head_dim), dtype=np.uint16)
    for l in range(w.n_loops):
        for b in range(w.batch):
            for h in range(w.n_q_heads):
                out[l, b, h] = q_row(w, b, h, l)
    return out


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def kv_tensors(w: Workload, tensor: int) -> list:
    """All loops of K or V as bf16 bits, one array [B, Hkv, S, D] per loop."""
    outs = [np.empty((w.batch, w.n_kv_heads, w.seq_len, w.head_dim), dtype=np.uint16) for _ in range(w.n_loops)]

    def fill(bh):
        b, h = bh
        for loop, arr in enumerate(kv_rows_all_loops(w, b, h, tensor)):
            outs[loop][b, h] = arr

    rows = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, rows))
    return outs


# Scale range of a random packed group, relative to INT2's [0.01, 0.1]: the
# largest level of a b-bit grid is 2^(b-1) - 1/2, and these factors make it
# times the scale span the same range at every width (an encoder's step shrinks
# the same way with the width).
PACKED_SCALE_FACTOR = {2: 1.0, 3: 1.5 / 3.5, 4: 1.5 / 7.5, 8: 1.5 / 127.5}


def packed_row(w: Workload, b: int, h: int, tensor: int, loop: int):
    """Decode-only input for a residual loop: uniformly random code words
    [S, D*bits/32] (uint32) and fp16 scale bits [S, D/32] with values drawn
    uniformly from [0.01, 0.1] * PACKED_SCALE_FACTOR[bits]. Used where the bf16
    loop states would not fit (the peak-batch workload) and to exercise every
    code pattern."""
    bits = w.bits[loop]
    rng = _rng(w, b, h, TENSOR_PACKED_K + tensor, loop)
    words = rng.integers(0, 2**32, size=(w.seq_len, w.head_dim * bits // 32), dtype=np.uint64).astype(np.uint32)
    f = PACKED_SCALE_FACTOR[bits]
    scales = rng.uniform(0.01 * f, 0.1 * f, size=(w.seq_len, w.head_dim // GROUP)).astype(np.float16).view(np.uint16)
    return words, scales


def packed_tensors(w: Workload, tensor: int, loop: int):
    """packed_row over every row: words [B, Hkv, S, D*bits/32], scales [B, Hkv, S, D/32]."""
    bits = w.bits[loop]
    words = np.empty((w.batch, w.n_kv_heads, w.seq_len, w.head_dim * bits // 32), dtype=np.uint32)
    scales = np.empty((w.batch, w.n_kv_heads, w.seq_len, w.head_dim // GROUP), dtype=np.uint16)

    def fill(bh):
        b, h = bh
        words[b, h], scales[b, h] = packed_row(w, b, h, tensor, loop)

    rows = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, rows))
    return words, scales


def ref_tensor(w: Workload, tensor: int) -> np.ndarray:
    """Only the reference (final loop) of K or V, bf16 bits [B, Hkv, S, D]."""
    out = np.empty((w.batch, w.n_kv_heads, w.seq_len, w.head_dim), dtype=np.uint16)

    def fill(bh):
        b, h = bh
        out[b, h] = f32_to_bf16_bits(_ref_f32(w, b, h, tensor))

    rows = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, rows))
    return out


# ---------------------------------------------------------------------------
# the peak-batch sweep: the batch grows until the cache fills about 200 GB
# ---------------------------------------------------------------------------

PEAK_CACHE_BUDGET = 200 * 10**9
PEAK_TILE = 8  # batch entries drawn on the host; a larger batch repeats them in order


def cache_bytes_per_sequence(w: Workload, bits_per_loop, with_reference: bool = True) -> int:
    """K and V cache bytes of one sequence (every KV head and position): the
    bf16 reference plus, per residual loop of width b, D*b/8 bytes of codes and
    2*D/32 bytes of scales per vector. A bf16-KV cache passes its loops as
    zero widths and counts 2*D bytes per loop instead."""
    d = w.head_dim
    per = sum(d * b // 8 + 2 * d // GROUP for b in bits_per_loop if b)
    return 2 * w.n_kv_heads * w.seq_len * ((2 * d if with_reference else 0) + per)


def bf16_cache_bytes_per_sequence(w: Workload, n_loops: int) -> int:
    return 2 * w.n_kv_heads * w.seq_len * 2 * w.head_dim * n_loops


def encode_bytes_per_sequence(w: Workload) -> int:
    """Device bytes one sequence of an all-loop encode call holds: the bf16
    states of every loop of K and V (the final one is the reference) plus the
    packed codes and scales the call writes for the residual loops."""
    return bf16_cache_bytes_per_sequence(w, w.n_loops) + cache_bytes_per_sequence(w, w.bits, with_reference=False)


def peak_batch(bytes_per_sequence: int, budget: int = PEAK_CACHE_BUDGET, multiple: int = PEAK_TILE) -> int:
    """The largest batch, a multiple of ``multiple``, whose cache fits ``budget`` bytes."""
    return int(budget // bytes_per_sequence // multiple * multiple)


def tile_batch(src, batch: int):
    """A [batch, ...] copy of the tensor src [T, ...] on src's device whose
    entry b is src[b % T] (batch a multiple of T)."""
    t = src.shape[0]
    if batch % t:
        raise ValueError("batch must be a multiple of the tile")
    rest = tuple(src.shape[1:])
    out = src.new_empty((batch,) + rest)
    out.view((batch // t, t) + rest).copy_(src.unsqueeze(0).expand((batch // t, t) + rest))
    return out
