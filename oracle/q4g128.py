"""CPU oracle for the int4 group-128 matrix-vector family.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct
statement of what the GPU library computes.  Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import it; the GPU library and its
Python binding never do, and it imports nothing from them.

Everything is computed in fp64 from the stored fp16/uint8 inputs.

The format (rumik-oss-1 int4 write-up, rtts.neoandmatrix.me, section
"Step 3: an int4 file and a first kernel on the laptop"): every projection
matrix W (N output rows x K input columns) is quantised in groups of 128
consecutive columns of a row; each group carries one fp16 scale and one fp16
minimum; two 4-bit codes share a byte.

Readings taken where the pages are silent:
  * the dequantised weight is  w = code * scale + min  (code 0 maps to the
    group minimum, code 15 to min + 15*scale);
  * within a byte the LOW nibble holds the EVEN column, the high nibble the
    odd column;
  * scales and minimums are two separate row-major [N][K/128] fp16 arrays;
  * activations are fp16, products and sums are exact here (fp64 of dyadic
    inputs), outputs are returned in fp64.

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def _check_k(k: int) -> int:
    if k <= 0 or k % GROUP:
        raise ValueError(f"K={k} must be a positive multiple of {GROUP}")
    return k // GROUP


def pack(codes: np.ndarray) -> np.ndarray:
    """uint8 codes [N][K] -> packed bytes [N][K/2].

    Byte j of a row holds column 2j in bits 0..3 and column 2j+1 in bits 4..7
    ("two 4-bit codes per byte", rumik write-up, Step 3).  Only the low four
    bits of each code are used.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    _check_k(k)
    even = codes[:, 0::2] & 0x0F
    odd = codes[:, 1::2] & 0x0F
    return (even | (odd << 4)).astype(np.uint8)


def unpack(packed: np.ndarray, k: int) -> np.ndarray:
    """packed bytes [N][K/2] -> uint8 codes [N][K] (inverse of `pack`)."""
    packed = np.asarray(packed, dtype=np.uint8)
    _check_k(k)
    n = packed.shape[0]
    if packed.shape != (n, k // 2):
        raise ValueError(f"packed shape {packed.shape} != ({n}, {k // 2})")
    codes = np.empty((n, k), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    return codes


def dequantize(packed: np.ndarray, scales: np.ndarray, mins: np.ndarray, k: int) -> np.ndarray:
    """Exact weights w[n][k] = code[n][k] * scale[n][k//128] + min[n][k//128] in fp64."""
    g = _check_k(k)
    codes = unpack(packed, k)
    n = codes.shape[0]
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    m = np.asarray(mins, dtype=np.float16).astype(np.float64)
    if s.shape != (n, g) or m.shape != (n, g):
        raise ValueError("scales/mins must be [N][K/128]")
    s_full = np.repeat(s, GROUP, axis=1)
    m_full = np.repeat(m, GROUP, axis=1)
    return codes.astype(np.float64) * s_full + m_full


def gemm(packed, scales, mins, X) -> np.ndarray:
    """Y[b][n] = sum_k w[n][k] * X[b][k] for every activation row b, in fp64.

    One activation vector per request (the continuous-batching passage of
    "Adding GPU backends to a pure-C TTS engine": each weight row is read once
    and used for all B requests; the result per request is the plain
    matrix-vector product).  The same contraction over M prompt tokens is the
    prompt-processing form (rumik write-up, "Step 8: a prefill that stays
    int4").
    """
    X = np.asarray(X, dtype=np.float16)
    if X.ndim != 2:
        raise ValueError("X must be [B][K]")
    k = X.shape[1]
    w = dequantize(packed, scales, mins, k)
    return X.astype(np.float64) @ w.T


def gemv(packed, scales, mins, x) -> np.ndarray:
    """y[n] = sum_k w[n][k] * x[k] in fp64 (the batch-1 decode product)."""
    x = np.asarray(x, dtype=np.float16).reshape(1, -1)
    return gemm(packed, scales, mins, x)[0]


def dequantize_fp16(packed, scales, mins, k: int) -> np.ndarray:
    """Weights first rounded to fp16 (round-to-nearest-even of the exact value).

    This is the operand of the prompt-processing design that dequantises each
    weight tile to fp16 on chip and then runs an fp16 matrix product.
    """
    return dequantize(packed, scales, mins, k).astype(np.float16)


def gemm_fp16_weights(packed, scales, mins, X) -> np.ndarray:
    """Y = X @ fp16(w).T in fp64: the exact result of the fp16-weight design."""
    X = np.asarray(X, dtype=np.float16)
    k = X.shape[1]
    w16 = dequantize_fp16(packed, scales, mins, k).astype(np.float64)
    return X.astype(np.float64) @ w16.T


def term_magnitude(packed, scales, mins, X) -> np.ndarray:
    """T[b][n] = sum_k (code*scale + |min|) * |X[b][k]|.

    Not part of the method: the magnitude of the terms a kernel adds up when
    it forms  scale*sum(code*x) + min*sum(x)  per group.  Floating-point
    summation error is bounded by a multiple of this quantity, so tests use
    it to state an error bound derived from the arithmetic.
    """
    X = np.asarray(X, dtype=np.float16).astype(np.float64)
    k = X.shape[1]
    codes = unpack(packed, k).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), GROUP, axis=1)
    m = np.repeat(np.abs(np.asarray(mins, dtype=np.float16).astype(np.float64)), GROUP, axis=1)
    return np.abs(X) @ (codes * s + m).T
