"""CPU oracle (NumPy) for the int4 group-128 GEMV family, its export step and
the int8 output-head GEMV.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.
"""
from .q4g128 import (  # noqa: F401
    GROUP,
    dequantize,
    dequantize_fp16,
    gemm,
    gemm_fp16_weights,
    gemv,
    pack,
    term_magnitude,
    unpack,
)
from .quantize import quantize  # noqa: F401,E402
from .head_int8 import gemv_int8  # noqa: F401,E402
