"""C-ABI checks that run without a GPU.

The library must load, export every entry point that include/q4g128.h
declares, and reject every invalid argument combination with the documented
status code BEFORE any HIP call.  Pointer arguments here are fake addresses
that are never dereferenced: each call fails validation first.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4g128.h")

q4 = pytest.importorskip("int4_group_quantized_amd")

EINVAL, ESHAPE, EALIGN, OK = q4.Q4_EINVAL, q4.Q4_ESHAPE, q4.Q4_EALIGN, q4.Q4_OK

A = 0x7F0000000000  # 256-byte aligned fake device addresses, far apart
P, S, M, X, Y = (A + i * (1 << 36) for i in range(5))


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"Q4_API\s+[\w\s\*]+?\b(q4g128_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_symbols() == sorted(q4.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = q4.library()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    # the object file exports exactly these functions
    out = os.popen(f"nm -D --defined-only {q4.LIB_PATH}").read()
    funcs = sorted(line.split()[-1] for line in out.splitlines() if " T " in line)
    assert funcs == declared_symbols()


DIAG_HEADER = os.path.join(ROOT, "include", "q4g128_diag.h")


def test_diag_library_exports_its_header():
    from int4_group_quantized_amd import diag
    declared = sorted(set(re.findall(r"Q4DIAG_API\s+[\w\s\*]+?\b(q4diag_\w+)\s*\(", open(DIAG_HEADER).read())))
    assert declared == sorted(diag.EXPORTED)
    out = os.popen(f"nm -D --defined-only {diag.DIAG_PATH}").read()
    assert sorted(line.split()[-1] for line in out.splitlines() if " T " in line) == declared
    lib = diag.library()
    assert lib.q4diag_gemv_read_twin(None, S, M, X, Y, 64, 3072, None) == -1
    assert lib.q4diag_gemv_read_twin(P, S, M, X, Y, 64, 2048, None) == -2
    assert lib.q4diag_stream_read(P, 100, Y, None) == -1
    assert lib.q4diag_stream_read(P + 8, 1024, Y, None) == -1


def test_every_header_is_covered():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["q4g128.h", "q4g128_diag.h"]


def test_status_strings():
    for code in (OK, EINVAL, ESHAPE, EALIGN, q4.Q4_EDEVICE):
        s = q4.q4g128_status_string(code)
        assert s.startswith("Q4_"), s
    assert "unknown" in q4.q4g128_status_string(-99)
    assert q4.library().q4g128_last_hip_error() == 0


def gemv(p=P, s=S, m=M, x=X, y=Y, n=64, k=256):
    return q4.library().q4g128_gemv(p, s, m, x, y, n, k, None)


def batch(b, p=P, s=S, m=M, x=X, y=Y, n=64, k=256):
    return q4.library().q4g128_gemm_small_batch(p, s, m, x, y, n, k, b, None)


def prefill(mm, p=P, s=S, m=M, x=X, y=Y, n=64, k=256):
    return q4.library().q4g128_gemm_prefill(p, s, m, x, y, n, k, mm, None)


def prefill_epi(mm, p=P, s=S, m=M, x=X, y=Y, n=64, k=256):
    return q4.library().q4g128_gemm_prefill_epilogue(p, s, m, x, y, n, k, mm, None)


def pack(c=X, p=P, n=64, k=256):
    return q4.library().q4g128_pack(c, p, n, k, None)


def quantize(w=X, p=P, s=S, m=M, n=64, k=256):
    return q4.library().q4g128_quantize(w, p, s, m, n, k, None)


def head(qq=P, s=S, x=X, y=Y, n=64, k=256):
    return q4.library().q4g128_gemv_int8(qq, s, x, y, n, k, None)


@pytest.mark.parametrize("call", [
    lambda: gemv(p=None), lambda: gemv(s=None), lambda: gemv(m=None), lambda: gemv(x=None),
    lambda: gemv(y=None), lambda: gemv(n=0), lambda: gemv(n=-5),
    lambda: batch(0), lambda: batch(17), lambda: batch(-1), lambda: batch(4, x=None),
    lambda: prefill(0), lambda: prefill(-3), lambda: prefill(34, y=None),
    lambda: prefill_epi(0), lambda: prefill_epi(34, p=None), lambda: prefill_epi(34, y=M),
    lambda: pack(c=None), lambda: pack(p=None), lambda: pack(n=0),
    lambda: quantize(w=None), lambda: quantize(p=None), lambda: quantize(s=None), lambda: quantize(m=None),
    lambda: quantize(n=0), lambda: quantize(n=-2),
    lambda: head(qq=None), lambda: head(s=None), lambda: head(x=None), lambda: head(y=None), lambda: head(n=0),
])
def test_einval(call):
    assert call() == EINVAL


@pytest.mark.parametrize("k", [0, 64, 127, 130, 200, 32768 + 128, -128])
def test_eshape_k(k):
    expect = ESHAPE
    assert gemv(k=k) == expect
    assert batch(3, k=k) == expect
    assert prefill(5, k=k) == expect
    assert prefill_epi(5, k=k) == expect
    assert pack(k=k) == expect
    assert quantize(k=k) == expect
    assert head(k=k) == expect


def test_eshape_sizes():
    assert gemv(n=1 << 31) == ESHAPE
    assert prefill(1 << 31) == ESHAPE
    assert quantize(n=1 << 31) == ESHAPE
    # more groups than the export kernel's grid covers: N * K/128 > 2^36
    assert quantize(n=(1 << 31) - 256, k=32768) == ESHAPE


def test_head_int8_limits():
    assert head(k=8192 + 128) == ESHAPE  # int8 head rows are at most 8,192 codes
    assert head(n=1 << 31) == ESHAPE
    assert head(qq=P + 8) == EALIGN
    assert head(x=X + 2) == EALIGN
    assert head(s=S + 1) == EALIGN
    assert head(y=Y + 2) == EALIGN
    assert head(y=P + 64) == EINVAL   # y inside q
    assert head(y=X) == EINVAL        # y on x
    assert head(y=S + 4) == EINVAL    # y inside scales


@pytest.mark.parametrize("which", ["w", "p", "s", "m"])
def test_quantize_ealign(which):
    bad = {"w": X + 4, "p": P + 8, "s": S + 1, "m": M + 1}[which]
    assert quantize(**{which: bad}) == EALIGN
    assert quantize(s=S + 2, m=M + 2, n=0) == EINVAL  # 2-byte scales / mins pass alignment


def test_quantize_overlaps_rejected():
    assert quantize(p=X + 64) == EINVAL   # packed inside W
    assert quantize(s=X + 128) == EINVAL  # scales inside W
    assert quantize(m=P + 32) == EINVAL   # mins inside packed
    assert quantize(m=S + 64) == EINVAL   # mins inside scales


@pytest.mark.parametrize("which", ["p", "x", "s", "m", "y"])
def test_ealign(which):
    bad = {"p": P + 8, "x": X + 4, "s": S + 1, "m": M + 1, "y": Y + 2}[which]
    assert gemv(**{which: bad}) == EALIGN
    assert batch(2, **{which: bad}) == EALIGN
    assert prefill(20, **{which: bad}) == EALIGN
    assert prefill_epi(20, **{which: bad}) == EALIGN


def test_alignment_minimums_accepted_by_validation_order():
    # 2-byte aligned scales pass the alignment check and fail on something
    # else we planted (n = 0), proving the documented minimum is 2 bytes.
    assert gemv(s=S + 2, n=0) == EINVAL
    assert pack(c=X + 8) == EALIGN
    assert pack(p=P + 1) == EALIGN


def test_overlapping_output_rejected():
    # y inside the packed weights, inside x, inside scales
    assert gemv(y=P + 64) == EINVAL
    assert gemv(y=X) == EINVAL
    assert batch(4, y=S + 16) == EINVAL
    assert prefill(8, y=M) == EINVAL
    assert pack(p=X + 16) == EINVAL  # packed overlaps codes


def test_python_binding_rejects_cpu_tensors():
    import torch
    codes = torch.zeros((4, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):
        q4.q4g128_pack(codes)


def grouped(*descs, count=None):
    arr = (q4.GemvDesc * max(1, len(descs)))(*[q4.GemvDesc(*d) for d in descs])
    return q4.library().q4g128_gemv_grouped(arr if descs else None, len(descs) if count is None else count, None)


def desc(i, p=None, s=None, m=None, x=None, y=None, n=64, k=256):
    """Projection i of a fake group: its own 2^32-byte slot in each of the five regions."""
    off = i << 32
    return (P + off if p is None else p, S + off if s is None else s, M + off if m is None else m,
            X + off if x is None else x, Y + off if y is None else y, n, k)


def test_grouped_error_paths():
    assert grouped() == EINVAL                                  # NULL descs
    assert grouped(desc(0), count=0) == EINVAL
    assert grouped(desc(0), count=-1) == EINVAL
    assert grouped(desc(0), count=q4.MAX_GROUPED + 1) == EINVAL
    assert grouped(desc(0), desc(1, k=200)) == ESHAPE           # one bad K
    assert grouped(desc(0), desc(1, n=0)) == EINVAL
    assert grouped(desc(0), desc(1, p=P + 8)) == EALIGN
    assert grouped(desc(0), desc(1, y=Y + 2)) == EALIGN
    assert grouped(desc(0), desc(1, y=Y + 64)) == EINVAL        # two outputs overlap
    assert grouped(desc(0), desc(1, y=Y + 252)) == EINVAL       # overlap of one element (n = 64 floats)
    assert grouped(desc(0), desc(1, x=Y)) == EINVAL             # an output is another projection's input
    assert grouped(desc(0), desc(1, y=P + 128)) == EINVAL       # an output inside another's weights
    assert grouped(desc(0), desc(1, y=M + 64)) == EINVAL        # ... inside another's minimums
    assert grouped(desc(0), desc(1, y=X + 32)) == EINVAL        # ... over another's x


def test_grouped_shared_inputs_pass_validation():
    # x, weights and scales shared between projections are fine; n = 0 in the
    # last descriptor makes the call fail validation before any HIP call.
    assert grouped(desc(0), desc(1, x=X, p=P, s=S, m=M), desc(2, n=0)) == EINVAL
    # adjacent outputs (y_1 starts where y_0 ends) do not overlap
    assert grouped(desc(0), desc(1, y=Y + 256), desc(2, n=0)) == EINVAL
