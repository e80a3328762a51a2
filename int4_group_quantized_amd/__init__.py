"""Python binding of libq4g128 (int4 group-128 GEMV family for MI355X).

Argument marshalling only: every entry point checks tensor devices, dtypes,
shapes and contiguity, then passes raw device pointers, sizes and the
current HIP stream of the tensors' device to the C ABI of the same name
(include/q4g128.h).  All arithmetic runs in the library's HIP kernels; there
is no fallback path.  Importing this package fails loudly if the library is
not built.

PyTorch provides device memory and streams: fp16 arguments are torch.float16
tensors (the C ABI receives their bit patterns), codes/packed are torch.uint8,
outputs are torch.float32.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime before the library binds to it)

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libq4g128.so")

Q4_OK = 0
Q4_EINVAL = -1
Q4_ESHAPE = -2
Q4_EALIGN = -3
Q4_EDEVICE = -4
GROUP = 128
MAX_K = 32768
MAX_BATCH = 16
INT8_MAX_K = 8192
MAX_GROUPED = 65536


class GemvDesc(ctypes.Structure):
    """struct q4g128_gemv_desc of include/q4g128.h."""
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("mins", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64)]

EXPORTED = (
    "q4g128_pack",
    "q4g128_quantize",
    "q4g128_gemv",
    "q4g128_gemv_grouped",
    "q4g128_gemm_small_batch",
    "q4g128_gemm_prefill",
    "q4g128_gemm_prefill_epilogue",
    "q4g128_gemv_int8",
    "q4g128_status_string",
    "q4g128_last_hip_error",
)


class Q4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.q4g128_status_string(status).decode()
        if status == Q4_EDEVICE:
            msg += f" (hipError_t {_lib.q4g128_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python int4_group_quantized_amd/build.py` "
            "(or __graft_entry__.build()); there is no fallback implementation"
        )
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.q4g128_pack.argtypes = [vp, vp, i64, i64, vp]
    lib.q4g128_quantize.argtypes = [vp, vp, vp, vp, i64, i64, vp]
    lib.q4g128_gemv.argtypes = [vp, vp, vp, vp, vp, i64, i64, vp]
    lib.q4g128_gemv_grouped.argtypes = [ctypes.POINTER(GemvDesc), i64, vp]
    lib.q4g128_gemm_small_batch.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.q4g128_gemm_prefill.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.q4g128_gemv_int8.argtypes = [vp, vp, vp, vp, i64, i64, vp]
    lib.q4g128_gemm_prefill_epilogue.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
    for name in ("q4g128_pack", "q4g128_quantize", "q4g128_gemv", "q4g128_gemv_grouped", "q4g128_gemm_small_batch",
                 "q4g128_gemm_prefill",
                 "q4g128_gemv_int8", "q4g128_gemm_prefill_epilogue"):
        getattr(lib, name).restype = ctypes.c_int32
    lib.q4g128_status_string.argtypes = [ctypes.c_int32]
    lib.q4g128_status_string.restype = ctypes.c_char_p
    lib.q4g128_last_hip_error.argtypes = []
    lib.q4g128_last_hip_error.restype = ctypes.c_int32
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def _check(status: int, where: str) -> None:
    if status != Q4_OK:
        raise Q4Error(status, where)


def _dev_tensor(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
    return dev


def _stream(dev: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream


def _weights(packed, scales, mins):
    if packed.dim() != 2:
        raise ValueError("packed must be [N][K/2]")
    n, half_k = packed.shape
    k = 2 * half_k
    _dev_tensor(packed, "packed", torch.uint8, (n, half_k))
    _dev_tensor(scales, "scales", torch.float16, (n, k // GROUP))
    _dev_tensor(mins, "mins", torch.float16, (n, k // GROUP))
    return n, k


def q4g128_pack(codes: torch.Tensor, packed: torch.Tensor = None, stream=None) -> torch.Tensor:
    """codes uint8 [N][K] (low 4 bits used) -> packed uint8 [N][K/2]."""
    if codes.dim() != 2:
        raise ValueError("codes must be [N][K]")
    n, k = codes.shape
    _dev_tensor(codes, "codes", torch.uint8, (n, k))
    if packed is None:
        packed = torch.empty((n, k // 2), dtype=torch.uint8, device=codes.device)
    _dev_tensor(packed, "packed", torch.uint8, (n, k // 2))
    dev = _same_device(codes, packed)
    with torch.cuda.device(dev):
        _check(_lib.q4g128_pack(codes.data_ptr(), packed.data_ptr(), n, k, _stream(dev, stream)), "q4g128_pack")
    return packed


def q4g128_quantize(W: torch.Tensor, packed=None, scales=None, mins=None, stream=None):
    """float32 W [N][K] -> (packed uint8 [N][K/2], scales fp16 [N][K/128], mins fp16 [N][K/128])."""
    if W.dim() != 2:
        raise ValueError("W must be [N][K]")
    n, k = W.shape
    _dev_tensor(W, "W", torch.float32, (n, k))
    g = k // GROUP
    if packed is None:
        packed = torch.empty((n, k // 2), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty((n, g), dtype=torch.float16, device=W.device)
    if mins is None:
        mins = torch.empty((n, g), dtype=torch.float16, device=W.device)
    _dev_tensor(packed, "packed", torch.uint8, (n, k // 2))
    _dev_tensor(scales, "scales", torch.float16, (n, g))
    _dev_tensor(mins, "mins", torch.float16, (n, g))
    dev = _same_device(W, packed, scales, mins)
    with torch.cuda.device(dev):
        _check(_lib.q4g128_quantize(W.data_ptr(), packed.data_ptr(), scales.data_ptr(), mins.data_ptr(), n, k,
                                    _stream(dev, stream)), "q4g128_quantize")
    return packed, scales, mins


def q4g128_gemv(packed, scales, mins, x, y=None, stream=None) -> torch.Tensor:
    """y[N] fp32 = W x for fp16 x [K]."""
    n, k = _weights(packed, scales, mins)
    _dev_tensor(x, "x", torch.float16, (k,))
    if y is None:
        y = torch.empty((n,), dtype=torch.float32, device=packed.device)
    _dev_tensor(y, "y", torch.float32, (n,))
    dev = _same_device(packed, scales, mins, x, y)
    with torch.cuda.device(dev):
        _check(_lib.q4g128_gemv(packed.data_ptr(), scales.data_ptr(), mins.data_ptr(), x.data_ptr(),
                                y.data_ptr(), n, k, _stream(dev, stream)), "q4g128_gemv")
    return y


def gemv_descs(projections, ys):
    """ctypes array of q4g128_gemv_desc for [(packed, scales, mins, x)] and outputs ys (shapes checked)."""
    arr = (GemvDesc * len(projections))()
    for i, ((packed, scales, mins, x), y) in enumerate(zip(projections, ys)):
        n, k = _weights(packed, scales, mins)
        _dev_tensor(x, f"x[{i}]", torch.float16, (k,))
        _dev_tensor(y, f"y[{i}]", torch.float32, (n,))
        _same_device(projections[0][0], packed, scales, mins, x, y)
        arr[i] = GemvDesc(packed.data_ptr(), scales.data_ptr(), mins.data_ptr(), x.data_ptr(), y.data_ptr(), n, k)
    return arr


def q4g128_gemv_grouped(projections, ys=None, stream=None):
    """[y_i = W_i x_i] for independent projections [(packed, scales, mins, x)], in few launches.

    Each y_i is bit-identical to q4g128_gemv on projection i.  Returns the list of outputs.
    """
    projections = list(projections)
    if not projections:
        raise ValueError("projections must not be empty")
    if ys is None:
        ys = [torch.empty((p[0].shape[0],), dtype=torch.float32, device=p[0].device) for p in projections]
    if len(ys) != len(projections):
        raise ValueError("one output per projection")
    arr = gemv_descs(projections, ys)
    dev = projections[0][0].device
    with torch.cuda.device(dev):
        _check(_lib.q4g128_gemv_grouped(arr, len(projections), _stream(dev, stream)), "q4g128_gemv_grouped")
    return ys


def q4g128_gemm_small_batch(packed, scales, mins, X, Y=None, stream=None) -> torch.Tensor:
    """Y[B][N] fp32 = X W^T for fp16 X [B][K], 1 <= B <= 16; row b equals q4g128_gemv(X[b])."""
    n, k = _weights(packed, scales, mins)
    if X.dim() != 2:
        raise ValueError("X must be [B][K]")
    b = X.shape[0]
    _dev_tensor(X, "X", torch.float16, (b, k))
    if Y is None:
        Y = torch.empty((b, n), dtype=torch.float32, device=packed.device)
    _dev_tensor(Y, "Y", torch.float32, (b, n))
    dev = _same_device(packed, scales, mins, X, Y)
    with torch.cuda.device(dev):
        _check(_lib.q4g128_gemm_small_batch(packed.data_ptr(), scales.data_ptr(), mins.data_ptr(),
                                            X.data_ptr(), Y.data_ptr(), n, k, b, _stream(dev, stream)),
               "q4g128_gemm_small_batch")
    return Y


def q4g128_gemm_prefill(packed, scales, mins, X, Y=None, stream=None) -> torch.Tensor:
    """Y[M][N] fp32 = X fp16(W)^T for fp16 X [M][K] on the matrix cores."""
    n, k = _weights(packed, scales, mins)
    if X.dim() != 2:
        raise ValueError("X must be [M][K]")
    m = X.shape[0]
    _dev_tensor(X, "X", torch.float16, (m, k))
    if Y is None:
        Y = torch.empty((m, n), dtype=torch.float32, device=packed.device)
    _dev_tensor(Y, "Y", torch.float32, (m, n))
    dev = _same_device(packed, scales, mins, X, Y)
    with torch.cuda.device(dev):
        _check(_lib.q4g128_gemm_prefill(packed.data_ptr(), scales.data_ptr(), mins.data_ptr(),
                                        X.data_ptr(), Y.data_ptr(), n, k, m, _stream(dev, stream)),
               "q4g128_gemm_prefill")
    return Y


def q4g128_gemm_prefill_epilogue(packed, scales, mins, X, Y=None, stream=None) -> torch.Tensor:
    """Y[M][N] fp32 = X W^T for fp16 X [M][K]: exact codes on the matrix cores, scale and min per group on the result."""
    n, k = _weights(packed, scales, mins)
    if X.dim() != 2:
        raise ValueError("X must be [M][K]")
    m = X.shape[0]
    _dev_tensor(X, "X", torch.float16, (m, k))
    if Y is None:
        Y = torch.empty((m, n), dtype=torch.float32, device=packed.device)
    _dev_tensor(Y, "Y", torch.float32, (m, n))
    dev = _same_device(packed, scales, mins, X, Y)
    with torch.cuda.device(dev):
        _check(_lib.q4g128_gemm_prefill_epilogue(packed.data_ptr(), scales.data_ptr(), mins.data_ptr(),
                                                 X.data_ptr(), Y.data_ptr(), n, k, m, _stream(dev, stream)),
               "q4g128_gemm_prefill_epilogue")
    return Y


def q4g128_gemv_int8(q, scales, x, y=None, stream=None) -> torch.Tensor:
    """y[N] fp32 = scale[n] * (q x) for int8 q [N][K], fp16 scales [N], fp16 x [K]."""
    if q.dim() != 2:
        raise ValueError("q must be [N][K]")
    n, k = q.shape
    _dev_tensor(q, "q", torch.int8, (n, k))
    _dev_tensor(scales, "scales", torch.float16, (n,))
    _dev_tensor(x, "x", torch.float16, (k,))
    if y is None:
        y = torch.empty((n,), dtype=torch.float32, device=q.device)
    _dev_tensor(y, "y", torch.float32, (n,))
    dev = _same_device(q, scales, x, y)
    with torch.cuda.device(dev):
        _check(_lib.q4g128_gemv_int8(q.data_ptr(), scales.data_ptr(), x.data_ptr(), y.data_ptr(), n, k,
                                     _stream(dev, stream)), "q4g128_gemv_int8")
    return y


def q4g128_status_string(status: int) -> str:
    return _lib.q4g128_status_string(status).decode()
