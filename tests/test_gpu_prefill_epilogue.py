"""GPU parity of the prompt-processing form that applies scale and minimum
to the matrix-core result (q4g128_gemm_prefill_epilogue), against the fp64
oracle, through the C ABI.

No weight is rounded to fp16 in this form: codes are exact integers on the
matrix cores and only fp32 sums round.  Besides the 2e-3 relative check,
every output must lie within 512 * 2^-24 * T of the exact product, with
T = sum_k (code*scale + |min|) * |x| (oracle.term_magnitude): at most 127
roundings inside a group's 128-term contraction, 127 in its activation sum
and two per group in the epilogue, with margin.  Dyadic inputs make every
sum exact, and there the GPU must match bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_bound, assert_rel, cpu, device, note, to_dev_f16, upload
from test_oracle_pins import dyadic_case

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


def run(packed, s, m, X, dev):
    return cpu(q4.q4g128_gemm_prefill_epilogue(packed, s, m, to_dev_f16(X, dev)))


@pytest.mark.parametrize("mtok,n,k", [(1, 64, 128), (2, 70, 384), (15, 100, 512), (16, 128, 3072), (17, 65, 3072),
                                      (34, 300, 3072), (48, 129, 1152), (64, 129, 256), (65, 130, 640),
                                      (100, 257, 2048), (129, 300, 1536), (256, 96, 3072), (3, 33, 11008),
                                      (5, 40, 32768),
                                      # K split over the waves (up to 64 tokens): three rounds with padded
                                      # groups, two tiles per workgroup, waves with no group; four token
                                      # tiles (one group per wave and round): eleven rounds, partial tiles
                                      (48, 300, 8192), (20, 8000, 384), (33, 2500, 640),
                                      (56, 100, 640), (49, 70, 1152), (64, 300, 11008), (60, 2100, 3072),
                                      # blocks of 128 tokens per workgroup (above 64 tokens): eight row
                                      # tiles per workgroup, four blocks, a partial block
                                      (193, 32768, 256), (500, 700, 640), (200, 3000, 1024),
                                      # five blocks on 8,192 rows: 48 slices, a grid within the CUs
                                      (640, 8192, 256),
                                      # one block past a full wave on 24,000 rows: 256 tokens, then the
                                      # rest (one token, 44 tokens) routed on their own
                                      (257, 24000, 384), (300, 24000, 256),
                                      # one and two rows: most workgroups have an empty slice
                                      (7, 1, 128), (70, 2, 384),
                                      # more than 64 tokens in blocks of up to four token tiles (few
                                      # rows): uneven blocks, and a height at the rule's limit
                                      (193, 150, 384), (65, 16384, 256),
                                      # up to 96 tokens on many rows: two blocks (three and two, three
                                      # and three token tiles); one token more takes the one-launch kernel
                                      (80, 20000, 384), (96, 20000, 384), (97, 20000, 384),
                                      # large K with one and with two row tiles per wave
                                      (100, 100, 16384), (150, 100, 32768)])
def test_prefill_epilogue_parity(dev, mtok, n, k):
    w = synth.weights(n, k, seed=mtok * 1000 + n + 7)
    X = synth.activations(mtok, k, seed=mtok + 29)
    packed_np = oracle.pack(w.codes)
    packed, s, m = upload(w, dev, q4)
    Y = run(packed, s, m, X, dev)
    ref = oracle.gemm(packed_np, w.scales, w.mins, X)
    assert_rel(Y, ref, f"prefill epilogue M={mtok} {n}x{k}")
    assert_bound(Y, ref, oracle.term_magnitude(packed_np, w.scales, w.mins, X), 512, f"epilogue M={mtok}")


@pytest.mark.parametrize("mtok", [34, 256])
def test_prefill_epilogue_fused(dev, mtok):
    """The fused 25,088 x 3,072 projection: every output against the oracle
    (computed in blocks of 2,048 rows)."""
    w = synth.weights(synth.FUSED_N, synth.HIDDEN_K, synth.SEEDS["fused"])
    X = synth.prefill_activations(mtok)
    packed, s, m = upload(w, dev, q4)
    Y = run(packed, s, m, X, dev)
    packed_np = oracle.pack(w.codes)
    ref = np.empty(Y.shape, np.float64)
    T = np.empty(Y.shape, np.float64)
    for r0 in range(0, synth.FUSED_N, 2048):
        sl = slice(r0, min(synth.FUSED_N, r0 + 2048))
        ref[:, sl] = oracle.gemm(packed_np[sl], w.scales[sl], w.mins[sl], X)
        T[:, sl] = oracle.term_magnitude(packed_np[sl], w.scales[sl], w.mins[sl], X)
    assert_rel(Y, ref, f"epilogue fused M={mtok}")
    assert_bound(Y, ref, T, 512, f"epilogue fused M={mtok}")


@pytest.mark.parametrize("mtok", [1, 16, 34, 56, 70, 200])
def test_prefill_epilogue_dyadic_bit_exact(dev, mtok):
    n, k, codes, scales, mins, _x = dyadic_case(mtok, 96, 384)
    X = np.random.Generator(np.random.PCG64(300 + mtok)).integers(-3, 4, (mtok, k)).astype(np.float16)
    packed = q4.q4g128_pack(torch.from_numpy(codes).to(dev))
    Y = run(packed, to_dev_f16(scales, dev), to_dev_f16(mins, dev), X, dev)
    assert np.array_equal(Y.astype(np.float64), oracle.gemm(oracle.pack(codes), scales, mins, X))


def test_prefill_epilogue_deterministic_and_row_independent(dev):
    w = synth.weights(300, 1024, seed=91)
    X = synth.activations(40, 1024, seed=92)
    packed, s, m = upload(w, dev, q4)
    Y1 = run(packed, s, m, X, dev)
    assert np.array_equal(Y1, run(packed, s, m, X, dev))
    # a token's outputs do not depend on the other tokens of the call: the
    # same token at the same tile row of a call whose other tokens are zero
    X4 = np.zeros((4, 1024), dtype=np.float16)
    X4[3] = X[3]
    Y4 = run(packed, s, m, X4, dev)
    assert np.array_equal(Y4[3], Y1[3])
