"""CPU oracle for the ResidualQuant hot path.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this module. The GPU product path never
calls it and shares no code with it.

It is plain NumPy in float64 and follows the method's steps in order:

* ResidualQuant (newx.sg page), Abstract: the final loop's K/V is kept as the
  reference, and every earlier loop is stored as a low-precision residual
  against it. The residual is rotated and given a least-squares scale, and a
  per-loop table sets each loop's precision (INT2, or INT4 for the loops it
  marks).
* ResidualQuant (newx.sg page), AI Summary: the rotation is orthogonal and the
  scale is a least-squares fit.
* ResidualQuant (paperaft JSON page), `summary`: a looped model's cache is
  stored in this custom residual format and decoded at attention time.

The pages give no equations, so the details below are readings of them:

* The rotation is the normalised Sylvester Walsh-Hadamard matrix H over
  head_dim. It is built densely here, not with butterflies. It is symmetric and
  its own inverse.
* Groups are 32 consecutive coordinates of the rotated residual y = H r.
* Codes are assigned in one pass at the absmax step s0 = max|y| / (2^(b-1) - 1/2):
  c = clip(floor(y / s0) + 2^(b-1), 0, 2^b - 1). The level is
  q = c - (2^(b-1) - 1/2), so the INT2 grid is {-1.5, -0.5, 0.5, 1.5}. A value
  exactly on a threshold goes to the level above it.
* Scale s = <y, q> / <q, q>, the least-squares fit for fixed codes, stored as
  IEEE fp16 (round to nearest even, saturated at 65504). An all-zero group gets
  codes 2^(b-1) and s = 0.
* Widths: INT2 and INT4 (Abstract), and INT3 and INT8 for a per-(layer, loop)
  table (the AI Summary calls the mixed precision layer-wise, the Abstract
  loop-wise; a table over both covers either reading).
* Packing for b in {2, 4, 8}: word w of a vector holds elements
  [(32/b) w, (32/b)(w+1)), element j of the word at bits [b j, b j + b).
  INT3 codes are stored as two bit planes: the low two bits of every code in
  the INT2 layout (D/16 words), then bit 2 of every code, one bit per
  coordinate (D/32 words; element j of word w at bit j). No code crosses a
  word boundary.
* Reconstruction is x_hat = x_ref + H (s16 * q), using the stored fp16 scale.
* Decode attention is exact softmax attention over all cached positions, with
  scale 1/sqrt(D). Query head h reads kv head floor(h / G).
"""
from __future__ import annotations

import numpy as np

GROUP = 32
FP16_MAX = 65504.0


# ----------------------------------------------------------------------------
# storage formats (bit patterns <-> float64)
# ----------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit patterns, rounded once to nearest (ties to even)
    straight from float64, so there is no double rounding. Finite normal
    inputs only; zero maps to +0."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(m * 256.0), e - 8)  # 8 significant bits, RNE via rint
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f16_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_f16(x) -> np.ndarray:
    """float64 -> IEEE fp16 bit patterns, round to nearest even, saturated."""
    x = np.clip(np.asarray(x, dtype=np.float64), -FP16_MAX, FP16_MAX)
    return x.astype(np.float16).view(np.uint16)


# ----------------------------------------------------------------------------
# rotation
# ----------------------------------------------------------------------------

def hadamard(d: int) -> np.ndarray:
    """Normalised Sylvester Walsh-Hadamard matrix of order d (a power of 2),
    natural order: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]], then / sqrt(d)."""
    if d < 1 or d & (d - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


# ----------------------------------------------------------------------------
# one group: code assignment and least-squares scale
# ----------------------------------------------------------------------------

WIDTHS = (2, 3, 4, 8)


def level_offset(bits: int) -> float:
    """q = c - level_offset(bits): 1.5 for INT2, 3.5 for INT3, 7.5 for INT4,
    127.5 for INT8."""
    return 2.0 ** (bits - 1) - 0.5


def assign_codes(y: np.ndarray, bits: int):
    """Codes of one group (last axis) at the absmax step.

    Returns (codes, s0). For an all-zero group, s0 is 0 and every code is
    2^(b-1), the level +1/2."""
    y = np.asarray(y, dtype=np.float64)
    m = np.max(np.abs(y), axis=-1, keepdims=True)
    top = 2 ** bits - 1
    half = 2 ** (bits - 1)
    s0 = m / level_offset(bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(m > 0, y / np.where(m > 0, s0, 1.0), 0.0)
    codes = np.clip(np.floor(u) + half, 0, top).astype(np.int64)
    codes = np.where(m > 0, codes, half)
    return codes, s0[..., 0]


def ls_scale(y: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Least-squares scale of a group for fixed levels q: argmin_s |y - s q|^2
    = <y, q> / <q, q>. Here |q| >= 1/2 in every element, so <q, q> > 0."""
    y = np.asarray(y, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    return np.sum(y * q, axis=-1) / np.sum(q * q, axis=-1)


def refit_codes(y: np.ndarray, s: np.ndarray, bits: int) -> np.ndarray:
    """Codes of one group (last axis) at a given step s: the nearest level
    (c - (2^(b-1) - 1/2)) s, by the same floor rule as the first assignment,
    clipped to the grid. A group with s = 0 keeps every code at 2^(b-1)."""
    y = np.asarray(y, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)[..., None]
    top = 2 ** bits - 1
    half = 2 ** (bits - 1)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s > 0, y / np.where(s > 0, s, 1.0), 0.0)
    codes = np.clip(np.floor(u) + half, 0, top).astype(np.int64)
    return np.where(s > 0, codes, half)


def quantize_groups(y: np.ndarray, bits: int, refits: int = 0, steps=None):
    """y[..., n_groups, group] -> (codes, s) with s the float64 LS scale
    (0 for all-zero groups).

    refits > 0 alternates the two steps the method names: codes for a fixed
    scale (nearest level), then the least-squares scale for fixed codes, that
    many more times after the first fit. Each half-step can only lower
    |y - s q|. If `steps` is a list, the step of every assignment (s0, then
    each refit's scale) is appended to it."""
    codes, s0 = assign_codes(y, bits)
    if steps is not None:
        steps.append(s0)
    q = codes - level_offset(bits)
    s = np.where(s0 > 0, ls_scale(y, q), 0.0)
    for _ in range(refits):
        if steps is not None:
            steps.append(s)
        codes = refit_codes(y, s, bits)
        q = codes - level_offset(bits)
        s = np.where(s0 > 0, ls_scale(y, q), 0.0)
    return codes, s


# ----------------------------------------------------------------------------
# bit packing
# ----------------------------------------------------------------------------

def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes[..., D] (ints in [0, 2^b)) -> uint32 words [..., D*b/32].
    b in {1, 2, 4, 8}: element j of word w is element (32/b)*w + j of the
    vector, at bits [b*j, b*j+b). b = 3: the INT2 words of the low two bits,
    then the one-bit words of bit 2."""
    if bits == 3:
        codes = np.asarray(codes, dtype=np.int64)
        return np.concatenate([pack_codes(codes & 3, 2), pack_codes(codes >> 2, 1)], axis=-1)
    codes = np.asarray(codes, dtype=np.uint64)
    per = 32 // bits
    d = codes.shape[-1]
    c = codes.reshape(codes.shape[:-1] + (d // per, per))
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    return np.sum(c << shifts, axis=-1).astype(np.uint32)


def unpack_codes(words: np.ndarray, bits: int) -> np.ndarray:
    if bits == 3:
        words = np.asarray(words, dtype=np.uint32)
        n2 = words.shape[-1] * 2 // 3  # INT2-plane words; the rest are bit-2 words
        return unpack_codes(words[..., :n2], 2) | (unpack_codes(words[..., n2:], 1) << 2)
    words = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    per = 32 // bits
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    c = (words[..., None] >> shifts) & np.uint64(2 ** bits - 1)
    return c.reshape(words.shape[:-1] + (words.shape[-1] * per,)).astype(np.int64)


# ----------------------------------------------------------------------------
# encode / reconstruct
# ----------------------------------------------------------------------------

def rotate(r: np.ndarray) -> np.ndarray:
    """y = H r for every vector on the last axis (H symmetric: r @ H == (H r)^T)."""
    d = r.shape[-1]
    return np.asarray(r, dtype=np.float64) @ hadamard(d)


def encode(x_bits, ref_bits, bits: int, group: int = GROUP, refits: int = 0):
    """Encode one loop of K or V against the reference.

    x_bits, ref_bits: bf16 patterns [..., D]. Returns (words uint32 [..., D*b/32],
    scale_bits uint16 (fp16) [..., D/group]). ``group`` is exposed only so the
    tests can quantize tiny groups; the storage format fixes 32. ``refits``
    adds that many code/scale alternations after the first fit.
    """
    if bits not in WIDTHS:
        raise ValueError("residual width must be 2, 3, 4 or 8")
    x = bf16_to_f64(x_bits)
    xr = bf16_to_f64(ref_bits)
    r = x - xr                                   # residual against the final loop
    y = rotate(r)                                # orthogonal rotation
    d = y.shape[-1]
    yg = y.reshape(y.shape[:-1] + (d // group, group))
    codes, s = quantize_groups(yg, bits, refits)  # per-group codes + LS scale
    s16 = f64_to_f16(s)                          # fp16 storage
    words = pack_codes(codes.reshape(y.shape), bits)
    return words, s16


def dequantize(words, scale_bits, bits: int, d: int, group: int = GROUP) -> np.ndarray:
    """Rotated-domain residual s16 * q for every vector: [..., D] float64."""
    codes = unpack_codes(words, bits)[..., :d]
    q = codes - level_offset(bits)
    s = f16_to_f64(scale_bits)
    qg = q.reshape(q.shape[:-1] + (d // group, group))
    return (qg * s[..., None]).reshape(q.shape)


def reconstruct(ref_bits, words, scale_bits, bits: int) -> np.ndarray:
    """x_hat = x_ref + H (s16 * q) in float64. bits == 0 means the loop is the
    reference itself."""
    xr = bf16_to_f64(ref_bits)
    if bits == 0:
        return xr
    d = xr.shape[-1]
    z = dequantize(words, scale_bits, bits, d)
    return xr + z @ hadamard(d)                  # H^T = H


def reconstruction_error(x_hat, x_bits, ref_bits) -> float:
    """|X_hat - X_l|_F / |X_l - X_ref|_F over a whole tensor."""
    x = bf16_to_f64(x_bits)
    xr = bf16_to_f64(ref_bits)
    return float(np.linalg.norm(x_hat - x) / np.linalg.norm(x - xr))


# ----------------------------------------------------------------------------
# decode attention
# ----------------------------------------------------------------------------

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Single-query softmax attention for each query row.

    q [R, D], k [S, D], v [S, D] float64 -> [R, D]."""
    z = (q @ k.T) * scale                        # [R, S]
    z = z - np.max(z, axis=-1, keepdims=True)
    p = np.exp(z)
    p = p / np.sum(p, axis=-1, keepdims=True)
    return p @ v


def decode_attn(q_bits, k_hat: list, v_hat: list, scale: float | None = None) -> np.ndarray:
    """Decode attention of every loop over its (reconstructed) cache.

    q_bits: bf16 [n_loops, B, Hq, D]; k_hat, v_hat: per loop float64 [B, Hkv, S, D].
    Query head h reads kv head h // (Hq / Hkv). Returns float64 [n_loops, B, Hq, D].
    """
    q = bf16_to_f64(q_bits)
    n_loops, batch, hq, d = q.shape
    hkv = k_hat[0].shape[1]
    g = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty_like(q)
    for l in range(n_loops):
        for b in range(batch):
            for kv in range(hkv):
                rows = slice(kv * g, (kv + 1) * g)
                out[l, b, rows] = attention(q[l, b, rows], k_hat[l][b, kv], v_hat[l][b, kv], scale)
    return out


def decode_attn_varlen(q_bits, k_hat: list, v_hat: list, seq_lens, tail_k_bits=None, tail_v_bits=None,
                       scale: float | None = None, present=None) -> np.ndarray:
    """Decode attention over a partly filled cache plus bf16 positions not
    yet encoded (the serving step around the hot path; paperaft JSON page,
    `summary`).

    q_bits: bf16 [n_loops, B, Hq, D]; k_hat, v_hat: per loop float64
    [B, Hkv, S_cap, D]; seq_lens: [B], the positions of sequence b are
    0 .. seq_lens[b]-1; tail_k_bits, tail_v_bits: per loop bf16 [B, Hkv, T, D]
    or None. present: bool [B, S_cap] or None (every position is there); a
    position with present[b, t] false is not part of sequence b's cache and
    takes no part in the softmax (a paged cache's missing block, see
    pages_present). Row (l, b, h) attends to its sequence's cached positions
    that are present, followed by its tail. A row with no position at all is
    zero.
    """
    q = bf16_to_f64(q_bits)
    n_loops, batch, hq, d = q.shape
    hkv = k_hat[0].shape[1]
    g = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros_like(q)
    for l in range(n_loops):
        for b in range(batch):
            n = int(seq_lens[b])
            keep = np.arange(n) if present is None else np.flatnonzero(np.asarray(present[b])[:n])
            for kv in range(hkv):
                k = k_hat[l][b, kv, keep]
                v = v_hat[l][b, kv, keep]
                if tail_k_bits is not None:
                    k = np.concatenate([k, bf16_to_f64(tail_k_bits[l][b, kv])], axis=0)
                    v = np.concatenate([v, bf16_to_f64(tail_v_bits[l][b, kv])], axis=0)
                if k.shape[0] == 0:
                    continue
                rows = slice(kv * g, (kv + 1) * g)
                out[l, b, rows] = attention(q[l, b, rows], k, v, scale)
    return out


# ----------------------------------------------------------------------------
# block-paged caches (the serving step around the hot path)
# ----------------------------------------------------------------------------

def gather_pages(pages, block_table, block_size: int, seq_len: int) -> np.ndarray:
    """The dense cache a block table describes (ResidualQuant, paperaft JSON
    page, `summary`: the cache lives in a serving stack, which pages it).

    pages: [n_blocks, Hkv, P, ...]; block_table: ints [B, max_blocks].
    Returns [B, Hkv, seq_len, ...] where position t of sequence b is
    pages[block_table[b, t // P], :, t % P]. A position whose table entry is
    not in [0, n_blocks) is filled with zeros (it is not part of the cache)."""
    pages = np.asarray(pages)
    table = np.asarray(block_table)
    n_blocks, hkv = pages.shape[0], pages.shape[1]
    out = np.zeros((table.shape[0], hkv, seq_len) + pages.shape[3:], dtype=pages.dtype)
    for b in range(table.shape[0]):
        for t in range(seq_len):
            blk = int(table[b, t // block_size])
            if 0 <= blk < n_blocks:
                out[b, :, t] = pages[blk, :, t % block_size]
    return out


def pages_present(block_table, block_size: int, n_blocks: int, seq_len: int) -> np.ndarray:
    """Which positions a block table maps to a block: bool [B, seq_len],
    true where the entry of position t of sequence b, block_table[b, t // P],
    lies in [0, n_blocks). Reading of a table entry that is not a block: the
    positions it covers are not part of the sequence's cache, so decode
    attention leaves them out of the softmax (decode_attn_varlen's `present`)
    rather than attending to a filler value."""
    table = np.asarray(block_table)
    t = np.arange(seq_len)
    blk = table[:, t // block_size]
    return (blk >= 0) & (blk < n_blocks)
