"""Shared plumbing for the GPU tests: device selection, uploads through the
library's own pack entry point, and the tolerances the parity tests assert.

Tolerances (stated once, used everywhere):
  * REL = 2e-3 relative per output element, with a floor of 2e-3 * rms of
    the reference over the same output vector:
        |y - y_ref| <= 2e-3 * (|y_ref| + rms(y_ref)).
    The floor is needed because a pure relative bound is undefined where the
    exact result crosses zero; its size (0.2% of the typical output) is far
    below the error of a dropped weight, group or doubled minimum.
  * For the exact-code kernels (GEMV and small batch) a tighter bound derived
    from the arithmetic: products code*x are exact in fp32 and every output
    passes through at most ~72 fp32 roundings (a 16-step dot chain, the
    per-chunk sum of x, two group updates per chunk and a 6-level lane
    tree), so  |y - y_ref| <= 128 * 2^-24 * T  with
    T = sum_k (code*scale + |min|) * |x_k|  (oracle.term_magnitude).
  * For the prompt-processing kernel, the same kind of bound against the
    fp16-weight oracle: |Y - Y16| <= 256 * 2^-24 * sum_k |fp16(w)*x|.
"""
import sys

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

REL = 2e-3
U32 = 2.0 ** -24


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def note(msg: str) -> None:
    """Write a progress line straight to the real stderr (bypasses capture)."""
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


def to_dev_f16(a: np.ndarray, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(dev)


def upload(w, dev, q4):
    """Upload synth.Weights; pack on the GPU with q4g128_pack."""
    codes = torch.from_numpy(np.ascontiguousarray(w.codes)).to(dev)
    packed = q4.q4g128_pack(codes)
    return packed, to_dev_f16(w.scales, dev), to_dev_f16(w.mins, dev)


def cpu(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rms_rows(y_ref: np.ndarray) -> np.ndarray:
    y2 = np.atleast_2d(y_ref)
    return np.sqrt(np.mean(y2 * y2, axis=1, keepdims=True))


def assert_rel(y_gpu, y_ref, what=""):
    yg = np.atleast_2d(np.asarray(y_gpu, dtype=np.float64))
    yr = np.atleast_2d(np.asarray(y_ref, dtype=np.float64))
    assert yg.shape == yr.shape, (yg.shape, yr.shape)
    bound = REL * (np.abs(yr) + rms_rows(yr))
    err = np.abs(yg - yr)
    bad = err > bound
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} of {bad.size} outputs outside 2e-3*(|y|+rms); "
        f"worst err {err.max():.3e} at {np.unravel_index(np.argmax(err - bound), err.shape)}")
    assert np.all(np.isfinite(yg))


def assert_bound(y_gpu, y_ref, T, c, what=""):
    yg = np.atleast_2d(np.asarray(y_gpu, dtype=np.float64))
    yr = np.atleast_2d(np.asarray(y_ref, dtype=np.float64))
    T = np.atleast_2d(T)
    err = np.abs(yg - yr)
    bound = c * U32 * T
    bad = err > bound
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} outputs above {c}*2^-24*T; worst ratio "
        f"{(err / np.maximum(bound, 1e-300)).max():.3f}")


def gemv_bound(packed_np, w, X):
    return oracle.term_magnitude(packed_np, w.scales, w.mins, X)


def prefill_bound_T(packed_np, w, X):
    k = X.shape[1]
    w16 = np.abs(oracle.dequantize_fp16(packed_np, w.scales, w.mins, k).astype(np.float64))
    return np.abs(np.asarray(X, dtype=np.float16).astype(np.float64)) @ w16.T
