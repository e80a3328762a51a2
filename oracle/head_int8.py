"""CPU oracle of the int8 output-head matrix-vector product.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module; the GPU library and its
Python binding never do, and it imports nothing from them.

What the pages fix (rumik-oss-1 int4 write-up, rtts.neoandmatrix.me, the
section on the remaining per-token time after the 36 layers, and "What I
would tell someone starting this"): int4 group-128 was too lossy for the
audio output head, which was moved to int8 with its own kernel.  The pages
give no int8 layout.  The reading taken here is the
plain per-row symmetric form:

    w[n][k] = q[n][k] * scale[n]      q int8 (all of -128..127 accepted),
                                      scale one fp16 value per output row,
    y[n]    = sum_k w[n][k] * x[k]    x fp16, computed here in fp64.

Pins: tests/test_oracle_head_int8_pins.py.
"""
from __future__ import annotations

import numpy as np


def gemv_int8(q: np.ndarray, scales: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y[n] = sum_k q[n][k] * scale[n] * x[k] in fp64 from int8 q [N][K], fp16 scales [N], fp16 x [K]."""
    q = np.asarray(q)
    if q.dtype != np.int8 or q.ndim != 2:
        raise ValueError("q must be int8 [N][K]")
    n, k = q.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    if s.shape != (n,):
        raise ValueError("scales must be fp16 [N]")
    xv = np.asarray(x, dtype=np.float16).astype(np.float64)
    if xv.shape != (k,):
        raise ValueError("x must be fp16 [K]")
    w = q.astype(np.float64) * s[:, None]
    return w @ xv
