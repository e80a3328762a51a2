"""GPU parity of the export step (q4g128_quantize) against oracle/quantize.py.

The codes, scales and minimums are decided by fp32 arithmetic that both sides
perform identically, so every comparison here is bit-exact: packed bytes,
fp16 scale bits and fp16 minimum bits.  Calls go through the C ABI.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import cpu, device, note
from test_oracle_quantize_pins import edge_groups

pytestmark = pytest.mark.gpu

q4 = pytest.importorskip("int4_group_quantized_amd")
torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _announce(request):
    note(f"[gpu-test] {request.node.nodeid}")
    yield


@pytest.fixture(scope="module")
def dev():
    return device()


def gpu_quantize(W: np.ndarray, dev):
    p, s, m = q4.q4g128_quantize(torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).to(dev))
    return cpu(p), cpu(s).view(np.uint16), cpu(m).view(np.uint16)


def assert_same(got, W, rows=None):
    p, s, m = got
    if rows is not None:
        p, s, m, W = p[rows], s[rows], m[rows], W[rows]
    codes, scales, mins = oracle.quantize(W)
    assert np.array_equal(s, scales.view(np.uint16)), "scales differ"
    assert np.array_equal(m, mins.view(np.uint16)), "minimums differ"
    assert np.array_equal(p, oracle.pack(codes)), "packed codes differ"


@pytest.mark.parametrize("n,k,seed", [(1, 128, 0), (3, 256, 1), (17, 384, 2), (33, 640, 3), (64, 1024, 4),
                                      (250, 3072, 5), (5, 32768, 6), (1000, 128, 7)])
def test_quantize_bit_exact(dev, n, k, seed):
    W = synth.float_weights(n, k, 500 + seed)
    assert_same(gpu_quantize(W, dev), W)


def test_quantize_edge_groups(dev):
    """Constant, two-valued, far-from-zero narrow, subnormal-scale, sub-fp16
    range and mixed-sign groups (clamping at both ends, scale 0)."""
    W = edge_groups(np.random.Generator(np.random.PCG64(41)), 40)
    W[3, :128] = np.abs(W[3, :128])
    W[3, 5], W[3, 6] = -0.0, 0.0  # a zero minimum of either sign is stored as +0
    assert_same(gpu_quantize(W, dev), W)


def test_quantize_exact_round_trip(dev):
    """Weights built as c*s + m with codes 0 and 15 in each group come back
    as exactly the codes, scales and minimums they were built from."""
    rng = np.random.Generator(np.random.PCG64(42))
    n, k = 24, 1024
    g = k // 128
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    codes[:, 0::128] = 0
    codes[:, 1::128] = 15
    scales = (2.0 ** -rng.integers(3, 11, (n, g))).astype(np.float16)
    mins = (-rng.integers(0, 257, (n, g)) / 128.0).astype(np.float16)
    W = (codes.astype(np.float64) * np.repeat(scales.astype(np.float64), 128, axis=1)
         + np.repeat(mins.astype(np.float64), 128, axis=1)).astype(np.float32)
    p, s, m = gpu_quantize(W, dev)
    assert np.array_equal(p, oracle.pack(codes))
    assert np.array_equal(s, scales.view(np.uint16))
    assert np.array_equal(m, mins.view(np.uint16))


def test_quantize_half_code_ties(dev):
    """Quotients on and next to the half-integers that separate codes.

    Dyadic rows (scale 2^-e, minimum a multiple of 2^-7): values m + (c + 1/2) s
    are exact ties, resolved to the even code, and their fp32 neighbours fall
    just either side.  Other rows take an arbitrary fp16 scale and minimum, so
    m + (c + 1/2) s rounds to fp32 within an ulp or so of a tie.  Every code
    must equal the oracle's, which divides with one correctly rounded fp32
    division; the kernel reaches its quotient through a reciprocal and must
    redo exactly these values."""
    rng = np.random.Generator(np.random.PCG64(43))
    n, k = 64, 1024
    g = k // 128
    c = rng.integers(0, 15, (n, k)).astype(np.float64) + 0.5  # half codes 0.5 .. 14.5
    s = np.where(np.arange(n)[:, None] < n // 2,
                 2.0 ** -rng.integers(3, 12, (n, g)),
                 rng.uniform(0.001, 0.05, (n, g)).astype(np.float16).astype(np.float64))
    m = np.where(np.arange(n)[:, None] < n // 2,
                 -rng.integers(0, 257, (n, g)) / 128.0,
                 -rng.uniform(0.0, 0.3, (n, g)).astype(np.float16).astype(np.float64))
    s_full = np.repeat(s, 128, axis=1)
    m_full = np.repeat(m, 128, axis=1)
    W = (m_full + c * s_full).astype(np.float32)
    nudge = rng.integers(-1, 2, (n, k))  # one fp32 ulp down, none, or up
    W = np.where(nudge < 0, np.nextafter(W, np.float32(-np.inf)),
                 np.where(nudge > 0, np.nextafter(W, np.float32(np.inf)), W)).astype(np.float32)
    # codes 0 and 15 in every group, so that the range is 15 s from m
    W[:, 0::128] = m_full[:, 0::128].astype(np.float32)
    W[:, 1::128] = (m_full[:, 1::128] + 15.0 * s_full[:, 1::128]).astype(np.float32)
    assert_same(gpu_quantize(W, dev), W)
    codes, _, _ = oracle.quantize(W)
    assert (codes % 2 == 0).sum() > 0 and (codes % 2 == 1).sum() > 0


def test_quantize_full_size(dev):
    """The fused 25,088 x 3,072 projection in the benchmark's launch: every
    row bit-exact against the oracle, every element within the reconstruction
    bound, and a repeated call bitwise identical."""
    n, k = synth.FUSED_N, synth.HIDDEN_K
    W = synth.float_weights(n, k, synth.SEEDS["float_weights"])
    Wd = torch.from_numpy(W).to(dev)
    p1, s1, m1 = (cpu(t) for t in q4.q4g128_quantize(Wd))
    assert_same((p1, s1.view(np.uint16), m1.view(np.uint16)), W)
    # reconstruction bound at full size (oracle-free property)
    codes = oracle.unpack(p1, k).astype(np.float64)
    S = np.repeat(s1.astype(np.float64), 128, axis=1)
    M = np.repeat(m1.astype(np.float64), 128, axis=1)
    grp = W.astype(np.float64).reshape(n, k // 128, 128)
    lo = np.repeat(grp.min(axis=2), 128, axis=1)
    hi = np.repeat(grp.max(axis=2), 128, axis=1)
    bound = S / 2 + 15 * np.abs(S - (hi - lo) / 15) + np.abs(lo - M)
    assert np.all(np.abs(W - (codes * S + M)) <= bound * (1 + 1e-9))
    p2, s2, m2 = (cpu(t) for t in q4.q4g128_quantize(Wd))
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2) and np.array_equal(m1, m2)
