"""GPU parity of the int8 output-head GEMV (q4g128_gemv_int8) against
oracle/head_int8.py, through the C ABI.

Products of codes and activations are exact on both sides and the GPU adds
them in fp32 along at most 33 steps per lane plus a 6-level lane tree and one
scale multiply, so besides the 2e-3 relative check every output must lie
within 128 * 2^-24 * scale * sum|q*x| of the fp64 oracle.  Dyadic inputs and
one-hot probes make every sum exact, and there the GPU must match bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import U32, assert_rel, cpu, device, note, to_dev_f16

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


def run(q, s, x, dev):
    qd = torch.from_numpy(np.ascontiguousarray(q)).to(dev)
    return cpu(q4.q4g128_gemv_int8(qd, to_dev_f16(s, dev), to_dev_f16(x, dev)))


def check(y, q, s, x, what):
    ref = oracle.gemv_int8(q, s, x)
    assert_rel(y, ref, what)
    T = np.abs(s.astype(np.float64)) * (np.abs(q.astype(np.float64)) @ np.abs(x.astype(np.float64)))
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= 128 * U32 * T + 1e-30), f"{what}: above 128*2^-24*T"


# K = 128 .. 8192; ragged rows where K/16 is not a multiple of 64
@pytest.mark.parametrize("n,k", [(1, 128), (3, 256), (65, 384), (300, 1024), (9, 1152), (1000, 2048), (129, 3072),
                                 (77, 4096), (33, 6016), (5, 8192), (2048, 2048)])
def test_head_int8_parity(dev, n, k):
    q, s, x = synth.head_int8_case(n, k, seed=7 * n + k)
    check(run(q, s, x, dev), q, s, x, f"head {n}x{k}")


def test_head_int8_full_size(dev):
    n, k = synth.HEAD_N, synth.HIDDEN_K
    q, s, x = synth.head_int8_case(n, k, synth.SEEDS["head_int8"])
    y1 = run(q, s, x, dev)
    check(y1, q, s, x, "head 16384x3072")
    assert np.array_equal(y1, run(q, s, x, dev)), "repeat call differs"


@pytest.mark.parametrize("k", [384, 3072, 8192])
def test_head_int8_dyadic_bit_exact(dev, k):
    rng = np.random.Generator(np.random.PCG64(60 + k))
    n = 200
    q = rng.integers(-128, 128, (n, k)).astype(np.int8)
    s = (2.0 ** -rng.integers(2, 9, n)).astype(np.float16)
    x = rng.integers(-3, 4, k).astype(np.float16)
    assert np.array_equal(run(q, s, x, dev).astype(np.float64), oracle.gemv_int8(q, s, x))


def test_head_int8_one_hot_every_code(dev):
    k = 256
    q = np.stack([np.arange(-128, 128, dtype=np.int16).astype(np.int8),
                  np.arange(127, -129, -1, dtype=np.int16).astype(np.int8)])
    s = np.array([0.0078125, 0.3], dtype=np.float16)
    for c in (0, 1, 2, 3, 5, 127, 128, 200, 255):
        x = np.zeros(k, dtype=np.float16)
        x[c] = 1
        y = run(q, s, x, dev)
        assert np.array_equal(y.astype(np.float64), oracle.gemv_int8(q, s, x)), c


def test_head_int8_row_permutation(dev):
    q, s, x = synth.head_int8_case(513, 3072, seed=77)
    perm = np.random.Generator(np.random.PCG64(78)).permutation(513)
    y = run(q, s, x, dev)
    yp = run(np.ascontiguousarray(q[perm]), np.ascontiguousarray(s[perm]), x, dev)
    assert np.array_equal(yp, y[perm])


@pytest.mark.parametrize("n_tall,n_short,k", [(16384, 4096, 3072), (8192, 2048, 4096)])
def test_head_int8_rows_do_not_depend_on_height(dev, n_tall, n_short, k):
    """The first n_short rows of a tall head matrix, given as a matrix of their
    own, give the same bits: the short matrix stages x before its first rows
    are requested (one row per wave), the tall 16,384 x 3,072 one after."""
    q, s, x = synth.head_int8_case(n_tall, k, seed=n_tall + k)
    y_tall = run(q, s, x, dev)
    y_short = run(q[:n_short].copy(), s[:n_short].copy(), x, dev)
    assert np.array_equal(y_short.view(np.uint32), y_tall[:n_short].view(np.uint32))
