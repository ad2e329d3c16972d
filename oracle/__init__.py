"""CPU oracle for the ResidualQuant hot path (test infrastructure only).

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg may
import this package; the GPU path shares no code with it.
"""
from .rq_oracle import (  # noqa: F401
    GROUP,
    WIDTHS,
    assign_codes,
    attention,
    bf16_to_f64,
    decode_attn,
    decode_attn_varlen,
    dequantize,
    encode,
    f16_to_f64,
    f64_to_bf16,
    f64_to_f16,
    gather_pages,
    hadamard,
    level_offset,
    ls_scale,
    pack_codes,
    pages_present,
    quantize_groups,
    reconstruct,
    reconstruction_error,
    refit_codes,
    rotate,
    unpack_codes,
)
