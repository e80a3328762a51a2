"""CPU oracle of the export step: float weights -> int4 group-128 format.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module; the GPU library and its
Python binding never do, and it imports nothing from them.

What the pages fix (rumik-oss-1 int4 write-up, rtts.neoandmatrix.me,
section "Step 3: an int4 file and a first kernel on the laptop"): a short CPU
job quantised every projection in groups of 128 columns with one fp16 scale
and one fp16 minimum per group, two 4-bit codes per byte.  The pages print no
formula for the codes.  The reading taken here is the
plain min/max affine quantiser that matches the dequantisation
w = code * scale + min:

  1. per group, lo = min and hi = max of its 128 values;
  2. min   = fp16(lo), scale = fp16(fl32(hi - lo) / 15)   (15 = top code);
     a zero minimum is stored as +0.  The minimum of a group that holds
     -0 (with or without +0) is the number zero, but which signed zero a
     min-reduction returns depends on the order of its comparisons, so the
     stored form is fixed to the canonical +0 (lo + 0 in fp32 turns -0
     into +0);
  3. code  = clamp(round_half_even((w - min) / scale), 0, 15), computed
     against the STORED fp16 min and scale, so that the code is the nearest
     one under the dequantisation that will actually be applied;
  4. a group whose stored scale is 0 (all values equal, or a range too small
     for fp16) gets code 0 everywhere.

Precision.  The codes are integers decided by floating-point arithmetic, so
this oracle takes those decisions in the same precision as the GPU kernel:
every step above is one IEEE fp32 operation (subtraction, division by 15,
subtraction, division), each correctly rounded, and the fp16 conversions
round to nearest even.  Inputs must be finite with |w| <= 65504 so that the
fp16 minimum and scale are finite.

Pins of this module (tests/test_oracle_quantize_pins.py) check it against
exact rational arithmetic: exact round trips, the best code by brute force,
the reconstruction error bound, the degenerate groups, a step-by-step
emulation of the fp32 operations above (IEEE rounding written from its
definition on rationals) over values placed on the code boundaries, and the
signed-zero minimum.
"""
from __future__ import annotations

import numpy as np

GROUP = 128
TOP_CODE = 15


def quantize(W: np.ndarray):
    """float32 W [N][K] -> (codes uint8 [N][K], scales fp16 [N][K/128], mins fp16 [N][K/128]).

    Steps 1-4 of the module docstring, in fp32 as stated there.
    """
    W = np.asarray(W, dtype=np.float32)
    if W.ndim != 2:
        raise ValueError("W must be [N][K]")
    n, k = W.shape
    if k <= 0 or k % GROUP:
        raise ValueError(f"K={k} must be a positive multiple of {GROUP}")
    g = k // GROUP
    grp = W.reshape(n, g, GROUP)

    lo = grp.min(axis=2)                                   # step 1 (exact)
    hi = grp.max(axis=2)
    span = hi - lo                                         # fp32, rounded once
    scale32 = span / np.float32(TOP_CODE)                  # fp32, rounded once
    scales = scale32.astype(np.float16)                    # step 2: round to nearest even
    mins = (lo + np.float32(0)).astype(np.float16)         # -0 -> +0, then nearest even

    s = scales.astype(np.float32)[:, :, None]              # the stored values, exactly
    m = mins.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (grp - m) / s                                  # step 3: two fp32 roundings
    c = np.clip(np.rint(q), 0, TOP_CODE)                   # rint rounds half to even
    c = np.where(s == 0, 0, c)                             # step 4
    codes = c.astype(np.uint8).reshape(n, k)
    return codes, scales, mins
