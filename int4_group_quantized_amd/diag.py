"""ctypes binding of libq4g128_diag.so (include/q4g128_diag.h): benchmark
diagnostics of the batch-1 GEMV (read-only twin, streaming read, empty
launch).  Used by bench.py only; argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime before the library binds to it)

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
DIAG_PATH = os.path.join(_PKG_DIR, "libq4g128_diag.so")

EXPORTED = ("q4diag_out_words", "q4diag_gemv_read_twin", "q4diag_stream_read", "q4diag_empty")


def _load():
    if not os.path.exists(DIAG_PATH):
        raise ImportError(f"{DIAG_PATH} is missing: build it with `python int4_group_quantized_amd/build.py`")
    lib = ctypes.CDLL(DIAG_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.q4diag_out_words.argtypes = []
    lib.q4diag_gemv_read_twin.argtypes = [vp, vp, vp, vp, vp, i64, i64, vp]
    lib.q4diag_stream_read.argtypes = [vp, i64, vp, vp]
    lib.q4diag_empty.argtypes = [vp]
    for name in EXPORTED:
        getattr(lib, name).restype = ctypes.c_int32
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib
