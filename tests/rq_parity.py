"""Helpers for comparing the GPU path with the CPU oracle.

Tolerances:
* packed codes are bit-exact, except for a coordinate whose rotated value y
  (fp64, normalised transform) lies within 1e-5 of a decision threshold
  k * s0. A group holding such a differing coordinate is also exempt from the
  scale check;
* fp16 scales agree within one fp16 ulp, because the GPU rounds fp32 -> fp16
  and the oracle rounds fp64 -> fp16;
* attention rows: max_i |o_gpu - o_ref| / max_i |o_ref| <= 2e-3 per
  (loop, batch, query head);
* reconstruction error e = |X_hat - X|_F / |X - X_ref|_F agrees within 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

BOUNDARY_EPS = 1e-5
ATTN_TOL = 2e-3
RECON_TOL = 1e-3


def to_dev(bits_u16: np.ndarray, dtype=torch.bfloat16, device="cuda") -> torch.Tensor:
    """uint16 bit patterns -> device tensor of a 16-bit dtype (bit copy)."""
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(device).view(dtype)


def words_to_dev(words: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(device)


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def to_host_words(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def unpack_words(words: np.ndarray, bits: int) -> np.ndarray:
    """Codes [..., D] of packed words, for words read back from the device, so
    that no oracle function takes the GPU's output. The layout is the library
    header's: for b in {2, 4, 8} word w holds coordinates [(32/b) w, (32/b)(w+1)),
    coordinate j of the word at bits [b j, b j + b); for b = 3 the INT2 words of
    the low two bits come first, then one word of bit 2 per 32 coordinates."""
    w = np.asarray(words).astype(np.uint32)
    if bits == 3:
        d = w.shape[-1] // 3 * 32
        lo = unpack_words(w[..., : d // 16], 2)
        hi = (w[..., d // 16:, None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)
        return lo | (hi.reshape(w.shape[:-1] + (d,)) << np.uint32(2))
    per = 32 // bits
    c = (w[..., :, None] >> (bits * np.arange(per, dtype=np.uint32))) & np.uint32((1 << bits) - 1)
    return c.reshape(w.shape[:-1] + (w.shape[-1] * per,))


def host_f64(bits_u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns read back from the device, as float64."""
    return workloads.bf16_bits_to_f32(bits_u16).astype(np.float64)


def recon_error(x_hat: np.ndarray, x_bits: np.ndarray, ref_bits: np.ndarray) -> float:
    """|X_hat - X|_F / |X - X_ref|_F of a reconstruction read back from the device."""
    x, xr = host_f64(x_bits), host_f64(ref_bits)
    return float(np.linalg.norm(x_hat - x) / np.linalg.norm(x - xr))


def exempt_mask(x_bits: np.ndarray, ref_bits: np.ndarray, bits: int) -> np.ndarray:
    """Coordinates within BOUNDARY_EPS of a code decision threshold (fp64)."""
    r = oracle.bf16_to_f64(x_bits) - oracle.bf16_to_f64(ref_bits)
    y = oracle.rotate(r)
    d = y.shape[-1]
    yg = y.reshape(y.shape[:-1] + (d // 32, 32))
    _, s0 = oracle.assign_codes(yg, bits)
    ks = np.arange(-(2 ** (bits - 1) - 1), 2 ** (bits - 1))  # -1..1 (INT2), -7..7 (INT4)
    dist = np.min(np.abs(yg[..., None] - s0[..., None, None] * ks), axis=-1)
    return (dist <= BOUNDARY_EPS).reshape(y.shape)


def compare_codes(gpu_words, gpu_scales, orc_words, orc_scales, x_bits, ref_bits, bits):
    """Assert parity of one encoded tensor (any leading shape, [..., D] coords).
    Returns the number of exempt coordinates that differed."""
    d = x_bits.shape[-1]
    cg = unpack_words(gpu_words, bits)
    co = unpack_words(orc_words, bits)
    diff = cg != co
    n_diff = int(diff.sum())
    bad_groups = np.zeros(gpu_scales.shape, dtype=bool)
    if n_diff:
        ex = exempt_mask(x_bits, ref_bits, bits)
        unexplained = diff & ~ex
        assert not unexplained.any(), f"{int(unexplained.sum())} code(s) differ away from a decision boundary"
        bad_groups = diff.reshape(diff.shape[:-1] + (d // 32, 32)).any(axis=-1)
    sg = gpu_scales.astype(np.int32)
    so = orc_scales.astype(np.int32)
    ulp = np.abs(sg - so)
    ok = (ulp <= 1) | bad_groups
    assert ok.all(), f"{int((~ok).sum())} scale(s) differ by more than one fp16 ulp (max {int(ulp.max())})"
    return n_diff


def row_rel_err(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row (last axis) max |gpu - ref| / max |ref|."""
    num = np.max(np.abs(gpu - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return num / den


def assert_attn_close(gpu: np.ndarray, ref: np.ndarray, tol: float = ATTN_TOL):
    e = row_rel_err(np.asarray(gpu, dtype=np.float64), ref)
    assert np.all(np.isfinite(gpu)), "non-finite attention output"
    assert e.max() <= tol, f"attention row error {e.max():.3e} > {tol} at row {np.unravel_index(e.argmax(), e.shape)}"
    return float(e.max())


def refit_exempt_groups(x_bits: np.ndarray, ref_bits: np.ndarray, bits: int, refits: int) -> np.ndarray:
    """Groups [..., D/32] holding a coordinate within BOUNDARY_EPS of a
    threshold of any assignment step (the first fit's s0 and every refit's
    scale). A decision taken differently at one step changes the next step's
    scale, so the whole group is exempt; elsewhere every step's decisions
    agree and the codes must be bit-exact."""
    r = oracle.bf16_to_f64(x_bits) - oracle.bf16_to_f64(ref_bits)
    y = oracle.rotate(r)
    d = y.shape[-1]
    yg = y.reshape(y.shape[:-1] + (d // 32, 32))
    steps = []
    oracle.quantize_groups(yg, bits, refits, steps=steps)
    ks = np.arange(-(2 ** (bits - 1) - 1), 2 ** (bits - 1))
    near = np.zeros(yg.shape[:-1], dtype=bool)
    for s in steps:
        dist = np.min(np.abs(yg[..., None] - s[..., None, None] * ks), axis=-1)
        near |= (dist <= BOUNDARY_EPS).any(axis=-1)
    return near


def compare_codes_refit(gpu_words, gpu_scales, orc_words, orc_scales, x_bits, ref_bits, bits, refits):
    """Parity of an encode with refits: codes and scales of every group that is
    not exempt (refit_exempt_groups) match the oracle (codes bit-exact, scales
    within one fp16 ulp). Returns the number of exempt groups that differ."""
    d = x_bits.shape[-1]
    cg = unpack_words(gpu_words, bits)
    co = unpack_words(orc_words, bits)
    gdiff = (cg != co).reshape(cg.shape[:-1] + (d // 32, 32)).any(axis=-1)
    ulp = np.abs(gpu_scales.astype(np.int32) - orc_scales.astype(np.int32))
    gdiff |= ulp > 1
    exempt = refit_exempt_groups(x_bits, ref_bits, bits, refits) if gdiff.any() else np.zeros_like(gdiff)
    bad = gdiff & ~exempt
    assert not bad.any(), f"{int(bad.sum())} group(s) differ away from every step's decision boundaries"
    return int((gdiff & exempt).sum())
