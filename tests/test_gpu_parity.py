"""GPU parity: the HIP library against the fp64 CPU oracle.

Every call goes through the C ABI (via the thin ctypes binding).  Inputs are
seeded synthetic draws from synth/; expected values come from oracle/ or from
the hand-derived known answers in tests/golden/.
"""
import numpy as np
import pytest

import golden_cases
import oracle
import synth
from gpu_helpers import (assert_bound, assert_rel, cpu, device, gemv_bound, note, prefill_bound_T,
                         to_dev_f16, upload)
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


# --------------------------------------------------------------------------
# pack
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,k,seed", [(1, 128, 0), (3, 256, 1), (256, 512, 2), (77, 3072, 3), (5, 32768, 4)])
def test_pack_bit_exact(dev, n, k, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    codes = rng.integers(0, 256, (n, k), dtype=np.uint8)  # high bits must be ignored
    got = cpu(q4.q4g128_pack(torch.from_numpy(codes).to(dev)))
    assert np.array_equal(got, oracle.pack(codes))


def test_pack_full_size(dev):
    w = synth.weights(synth.FUSED_N, synth.HIDDEN_K, synth.SEEDS["fused"])
    got = cpu(q4.q4g128_pack(torch.from_numpy(w.codes).to(dev)))
    assert np.array_equal(got, oracle.pack(w.codes))


# --------------------------------------------------------------------------
# known answers and exact dyadic cases: bit-exact
# --------------------------------------------------------------------------

def _golden_on_gpu(case, dev):
    if case.packed is not None:
        packed = torch.from_numpy(case.packed).to(dev)
    else:
        packed = q4.q4g128_pack(torch.from_numpy(case.codes).to(dev))
    return packed, to_dev_f16(case.scales, dev), to_dev_f16(case.mins, dev), to_dev_f16(case.x, dev)


@pytest.mark.parametrize("case", golden_cases.load(), ids=lambda c: c.name)
def test_known_answers_exact(dev, case):
    packed, s, m, x = _golden_on_gpu(case, dev)
    assert float(cpu(q4.q4g128_gemv(packed, s, m, x))[0]) == case.expected
    X = x.reshape(1, -1).repeat(3, 1).contiguous()
    assert np.all(cpu(q4.q4g128_gemm_small_batch(packed, s, m, X)) == case.expected)
    assert np.all(cpu(q4.q4g128_gemm_prefill(packed, s, m, X)) == case.expected)


@pytest.mark.parametrize("n,k", [(4, 384), (37, 3072), (9, 8192), (130, 512), (3, 11008), (2, 32768)])
def test_dyadic_bit_exact(dev, n, k):
    for seed in range(2):
        _, _, codes, scales, mins, x = dyadic_case(seed, n, k)
        ref = oracle.gemv(oracle.pack(codes), scales, mins, x)
        w = synth.Weights(codes, scales, mins)
        packed, s, m = upload(w, dev, q4)
        xd = to_dev_f16(x, dev)
        assert np.array_equal(cpu(q4.q4g128_gemv(packed, s, m, xd)).astype(np.float64), ref)
        X = xd.reshape(1, -1).repeat(5, 1).contiguous()
        Yb = cpu(q4.q4g128_gemm_small_batch(packed, s, m, X)).astype(np.float64)
        assert np.array_equal(Yb, np.tile(ref, (5, 1)))
        Yp = cpu(q4.q4g128_gemm_prefill(packed, s, m, X)).astype(np.float64)
        assert np.array_equal(Yp, np.tile(ref, (5, 1)))
        for mtok in (70, 200):  # the wide prompt-processing kernel
            Xw = xd.reshape(1, -1).repeat(mtok, 1).contiguous()
            Yw = cpu(q4.q4g128_gemm_prefill(packed, s, m, Xw)).astype(np.float64)
            assert np.array_equal(Yw, np.tile(ref, (mtok, 1)))


# --------------------------------------------------------------------------
# random parity at tolerance (every lanes-per-row / chunks-per-lane variant)
# --------------------------------------------------------------------------

SHAPES = [
    (1, 128), (2, 256), (3, 384), (17, 512), (33, 640), (255, 768), (64, 1024), (5, 1152),
    (1000, 2048), (129, 3072), (31, 4096), (7, 6144), (300, 8192), (19, 11008), (3, 16384), (2, 32768),
    # ragged rows (K not a multiple of 512 and above 2,048): 64 lanes per row,
    # the last chunk column partial; 6 and 7 chunks per lane take the two paths
    (70, 2176), (40, 6400), (33, 12160), (20, 12416), (7, 32640), (2048, 11008),
]


@pytest.mark.parametrize("n,k", SHAPES)
def test_gemv_parity_shapes(dev, n, k):
    w, x = synth.gemv_case(n, k, seed=n * 7919 + k)
    packed_np = oracle.pack(w.codes)
    packed, s, m = upload(w, dev, q4)
    y = cpu(q4.q4g128_gemv(packed, s, m, to_dev_f16(x[0], dev)))
    ref = oracle.gemv(packed_np, w.scales, w.mins, x[0])
    assert_rel(y, ref, f"gemv {n}x{k}")
    assert_bound(y, ref, gemv_bound(packed_np, w, x)[0], 128, f"gemv {n}x{k}")


@pytest.mark.parametrize("name", ["tiny_256x512", "fused_25088x3072", "oproj_3072x3072", "down_3072x8192",
                                  "pages_fused_25088x2048", "pages_oproj_2048x2048", "pages_down_2048x11008"])
def test_gemv_parity_workloads(dev, name):
    w, x = synth.workload(name)
    packed_np = oracle.pack(w.codes)
    packed, s, m = upload(w, dev, q4)
    assert np.array_equal(cpu(packed), packed_np)
    y = cpu(q4.q4g128_gemv(packed, s, m, to_dev_f16(x[0], dev)))
    ref = oracle.gemv(packed_np, w.scales, w.mins, x[0])
    assert_rel(y, ref, name)
    assert_bound(y, ref, gemv_bound(packed_np, w, x)[0], 128, name)


def test_gemv_zero_and_scaling(dev):
    w, x = synth.gemv_case(96, 3072, seed=42)
    packed, s, m = upload(w, dev, q4)
    zero = torch.zeros(3072, dtype=torch.float16, device=dev)
    assert np.all(cpu(q4.q4g128_gemv(packed, s, m, zero)) == 0)
    y1 = cpu(q4.q4g128_gemv(packed, s, m, to_dev_f16(x[0], dev)))
    y4 = cpu(q4.q4g128_gemv(packed, s, m, to_dev_f16((x[0].astype(np.float64) * 4).astype(np.float16), dev)))
    assert np.array_equal(y4, y1 * 4)  # power-of-two scaling is exact in every rounding step


# --------------------------------------------------------------------------
# batch: bit-identity with the batch-1 call, and parity
# --------------------------------------------------------------------------

# Above the batch that fits in LDS (8 columns at K = 8,192, 4 at 11,008, 2 at
# 32,768) the rows are staged slot by slot; K = 5,120 / 7,168 and 5,632 take
# that path with 32 and 16 lanes per row, and more than 2,048 passes (3,072,
# 2,100 and 4,500 rows; 8,300 rows of 16 lanes) give each wave two of them.
@pytest.mark.parametrize("n,k", [(25088, 3072), (3072, 8192), (257, 512), (100, 11008), (33, 384), (9, 32768),
                                 (2048, 11008), (300, 2176), (64, 12160), (50, 12416),
                                 (130, 5120), (70, 5632), (33, 7168), (2100, 11008), (4500, 5120), (8300, 5632),
                                 (1, 11008), (5, 2048), (3, 1024),
                                 # more passes than one round of the grid, with every column in LDS:
                                 # the batched kernel (ragged rows at K = 2,176 and, for B <= 4,
                                 # 11,008; 64 lanes of three chunks at 6,144)
                                 (4200, 2176), (4500, 11008), (5000, 6144),
                                 # the column kernel at 32 lanes of two chunks (the pages' hidden
                                 # size) and odd row counts, whose last pass has one real row
                                 (25088, 2048), (8301, 2048), (9001, 3072)])
def test_small_batch_bit_identical_to_gemv(dev, n, k):
    w = synth.weights(n, k, seed=n + k)
    packed, s, m = upload(w, dev, q4)
    X = synth.activations(16, k, seed=4)
    Xd = to_dev_f16(X, dev)
    singles = np.stack([cpu(q4.q4g128_gemv(packed, s, m, Xd[b].contiguous())) for b in range(16)])
    for b in range(1, 17):
        Y = cpu(q4.q4g128_gemm_small_batch(packed, s, m, Xd[:b].contiguous()))
        assert np.array_equal(Y, singles[:b]), f"B={b}: batched rows differ from the batch-1 call"


@pytest.mark.parametrize("n,k", [(4200, 2176), (4500, 11008), (300, 2176)])
def test_small_batch_infinite_last_scale(dev, n, k):
    """Ragged rows whose last group has an infinite scale or minimum: every
    kernel feeds a ragged lane's missing chunk zero activations, so the
    result (NaN where inf * 0 occurs) is the batch-1 call's in every column."""
    w = synth.weights(n, k, seed=n + 3 * k)
    w.scales[::7, -1] = np.float16(np.inf)
    w.mins[3::11, -1] = np.float16(-np.inf)
    packed, s, m = upload(w, dev, q4)
    Xd = to_dev_f16(synth.activations(4, k, seed=5), dev)
    singles = np.stack([cpu(q4.q4g128_gemv(packed, s, m, Xd[b].contiguous())) for b in range(4)])
    for b in (2, 4):
        Y = cpu(q4.q4g128_gemm_small_batch(packed, s, m, Xd[:b].contiguous()))
        assert np.array_equal(Y.view(np.uint32), singles[:b].view(np.uint32)), f"B={b}"


@pytest.mark.parametrize("b", [2, 4, 8, 16])
def test_small_batch_parity_fused(dev, b):
    w = synth.weights(synth.FUSED_N, synth.HIDDEN_K, synth.SEEDS["fused"])
    X = synth.batch_activations(b)
    packed_np = oracle.pack(w.codes)
    packed, s, m = upload(w, dev, q4)
    Y = cpu(q4.q4g128_gemm_small_batch(packed, s, m, to_dev_f16(X, dev)))
    ref = oracle.gemm(packed_np, w.scales, w.mins, X)
    assert_rel(Y, ref, f"batch B={b}")
    assert_bound(Y, ref, oracle.term_magnitude(packed_np, w.scales, w.mins, X), 128, f"batch B={b}")


@pytest.mark.parametrize("b", [5, 16])
def test_small_batch_parity_pages_down(dev, b):
    # 2,048 x 11,008 (ragged rows): more columns than fit in LDS
    w = synth.weights(2048, 11008, seed=11)
    X = synth.activations(b, 11008, seed=12)
    packed_np = oracle.pack(w.codes)
    packed, s, m = upload(w, dev, q4)
    Y = cpu(q4.q4g128_gemm_small_batch(packed, s, m, to_dev_f16(X, dev)))
    ref = oracle.gemm(packed_np, w.scales, w.mins, X)
    assert_rel(Y, ref, f"pages' down B={b}")
    assert_bound(Y, ref, oracle.term_magnitude(packed_np, w.scales, w.mins, X), 128, f"pages' down B={b}")


def test_determinism_and_row_permutation(dev):
    w, x = synth.gemv_case(4099, 3072, seed=77)
    packed, s, m = upload(w, dev, q4)
    xd = to_dev_f16(x[0], dev)
    y0 = cpu(q4.q4g128_gemv(packed, s, m, xd))
    for _ in range(3):
        assert np.array_equal(cpu(q4.q4g128_gemv(packed, s, m, xd)), y0)
    perm = np.random.Generator(np.random.PCG64(3)).permutation(4099)
    wp = synth.Weights(w.codes[perm], w.scales[perm], w.mins[perm])
    pp, sp, mp = upload(wp, dev, q4)
    assert np.array_equal(cpu(q4.q4g128_gemv(pp, sp, mp, xd)), y0[perm])


@pytest.mark.parametrize("n_tall,n_short,k", [(25088, 3072, 3072), (25088, 2048, 2048), (16384, 4096, 4096),
                                               (6144, 2048, 8192), (8192, 2048, 11008)])
def test_gemv_rows_do_not_depend_on_height(dev, n_tall, n_short, k):
    """A row's result does not depend on the matrix it sits in: the first
    n_short rows of a tall matrix, given as a matrix of their own, give the
    same bits.  The short matrices run x-first (every wave has at most one or
    two passes, or the mapping runs one workgroup per CU) and the tall ones at
    K = 2,048 to 4,096 the default order, so this also holds the two launch
    orders of the batch-1 kernel to the same bits."""
    w = synth.weights(n_tall, k, seed=n_tall + k)
    x = synth.activations(1, k, seed=9)[0]
    xd = to_dev_f16(x, dev)
    packed, s, m = upload(w, dev, q4)
    y_tall = cpu(q4.q4g128_gemv(packed, s, m, xd))
    short = synth.Weights(w.codes[:n_short].copy(), w.scales[:n_short].copy(), w.mins[:n_short].copy())
    ps, ss, ms = upload(short, dev, q4)
    y_short = cpu(q4.q4g128_gemv(ps, ss, ms, xd))
    assert np.array_equal(y_short.view(np.uint32), y_tall[:n_short].view(np.uint32))


def test_non_default_stream(dev):
    w, x = synth.gemv_case(512, 1024, seed=5)
    packed, s, m = upload(w, dev, q4)
    xd = to_dev_f16(x[0], dev)
    ref = cpu(q4.q4g128_gemv(packed, s, m, xd))
    st = torch.cuda.Stream(dev)
    with torch.cuda.stream(st):
        y = q4.q4g128_gemv(packed, s, m, xd, stream=st)
    st.synchronize()
    assert np.array_equal(y.cpu().numpy(), ref)


# --------------------------------------------------------------------------
# prompt processing (matrix cores, fp16 weights)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mtok,n,k", [(1, 64, 128), (2, 70, 384), (15, 100, 512), (16, 128, 3072), (17, 65, 3072),
                                      (34, 200, 3072), (64, 129, 256), (65, 130, 640), (100, 33, 8192),
                                      (112, 128, 1024), (129, 300, 1536), (193, 45, 384), (300, 64, 2048),
                                      (5, 40, 32768),
                                      # K split over the waves of a workgroup (up to 64 tokens): three
                                      # rounds with padded groups, two tiles per workgroup, eight tiles
                                      # per workgroup, waves with no group; four token tiles (one group
                                      # per wave and round): eleven rounds, partial tiles
                                      (48, 300, 8192), (20, 8000, 384), (48, 32768, 256), (33, 2500, 640),
                                      (49, 70, 3072), (64, 300, 11008), (57, 2100, 1152),
                                      # blocks of 128 tokens paired per row slice (above 192 tokens):
                                      # 16 row tiles per workgroup, three and four blocks, a partial block
                                      (193, 32768, 256), (257, 4100, 256), (500, 700, 640), (200, 3000, 1024),
                                      # five blocks on 8,192 rows: 48 slices, a grid within the CUs
                                      (640, 8192, 256),
                                      # one block past a full wave on 24,000 rows: 256 tokens, then the
                                      # rest (one token, 44 tokens) routed on their own
                                      (257, 24000, 384), (300, 24000, 256),
                                      # one and three rows: most workgroups have an empty slice
                                      (5, 1, 256), (300, 3, 384),
                                      # more than 64 tokens in blocks of up to four token tiles (few
                                      # rows): uneven blocks, and a height at the rule's limit
                                      (193, 150, 384), (65, 16384, 256),
                                      # up to 96 tokens on many rows: two blocks (three and two, three
                                      # and three token tiles); one token more takes the one-launch kernel
                                      (80, 20000, 384), (96, 20000, 384), (97, 20000, 384),
                                      # the largest K with paired blocks
                                      (200, 100, 32768)])
def test_prefill_parity_shapes(dev, mtok, n, k):
    w = synth.weights(n, k, seed=mtok * 1000 + n)
    X = synth.activations(mtok, k, seed=mtok + 17)
    packed_np = oracle.pack(w.codes)
    packed, s, m = upload(w, dev, q4)
    Y = cpu(q4.q4g128_gemm_prefill(packed, s, m, to_dev_f16(X, dev)))
    assert_rel(Y, oracle.gemm(packed_np, w.scales, w.mins, X), f"prefill M={mtok} {n}x{k}")
    assert_bound(Y, oracle.gemm_fp16_weights(packed_np, w.scales, w.mins, X),
                 prefill_bound_T(packed_np, w, X), 256, f"prefill fp16-w M={mtok}")


@pytest.mark.parametrize("mtok", [34, 256])
def test_prefill_parity_fused(dev, mtok):
    w = synth.weights(synth.FUSED_N, synth.HIDDEN_K, synth.SEEDS["fused"])
    X = synth.prefill_activations(mtok)
    packed_np = oracle.pack(w.codes)
    packed, s, m = upload(w, dev, q4)
    Y = cpu(q4.q4g128_gemm_prefill(packed, s, m, to_dev_f16(X, dev)))
    assert_rel(Y, oracle.gemm(packed_np, w.scales, w.mins, X), f"prefill M={mtok}")
    assert_bound(Y, oracle.gemm_fp16_weights(packed_np, w.scales, w.mins, X),
                 prefill_bound_T(packed_np, w, X), 256, f"prefill fp16-w M={mtok}")


@pytest.mark.parametrize("mtok,n,k", [(40, 300, 1024),      # K split over the waves, three token tiles
                                      (60, 300, 1024),      # four token tiles, one group per wave and round
                                      (130, 300, 640),      # token blocks on few rows
                                      (100, 20000, 128),    # 65 to 192 tokens on many rows
                                      (200, 20000, 128)])   # blocks of 128 tokens paired per row slice
def test_prefill_deterministic(dev, mtok, n, k):
    """Two calls on the same inputs give the same bits on every prefill path
    (no atomics; every reduction runs in a fixed order)."""
    w = synth.weights(n, k, seed=mtok + n)
    X = to_dev_f16(synth.activations(mtok, k, seed=mtok + 3), dev)
    packed, s, m = upload(w, dev, q4)
    Y1 = cpu(q4.q4g128_gemm_prefill(packed, s, m, X))
    Y2 = cpu(q4.q4g128_gemm_prefill(packed, s, m, X))
    assert np.array_equal(Y1, Y2)
    E1 = cpu(q4.q4g128_gemm_prefill_epilogue(packed, s, m, X))
    E2 = cpu(q4.q4g128_gemm_prefill_epilogue(packed, s, m, X))
    assert np.array_equal(E1, E2)


def test_prefill_fp16_weights_short_k_bound(dev):
    """K = 128 (one group per row), 256 tokens x 32,768 rows: the short-K case
    where rounding each weight to fp16 is largest against the product.  Every
    output must be within 256 * 2^-24 * sum|fp16(w) x| of the exact product of
    the fp16 weights (the contract of q4g128_gemm_prefill).  Against the exact
    weights a few outputs may exceed 2e-3 * (|y| + rms): the count is
    reported, and the epilogue form, which keeps exact codes, must have none."""
    mtok, n, k = 256, 32768, 128
    w = synth.weights(n, k, seed=128256)
    X = synth.activations(mtok, k, seed=128257)
    packed_np = oracle.pack(w.codes)
    packed, s, m = upload(w, dev, q4)
    Xd = to_dev_f16(X, dev)
    Y = cpu(q4.q4g128_gemm_prefill(packed, s, m, Xd))
    assert_bound(Y, oracle.gemm_fp16_weights(packed_np, w.scales, w.mins, X),
                 prefill_bound_T(packed_np, w, X), 256, "prefill fp16-w K=128")
    ref = oracle.gemm(packed_np, w.scales, w.mins, X)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    over = int((np.abs(Y - ref) > 2e-3 * (np.abs(ref) + rms)).sum())
    note(f"[gpu-test]   fp16-weight prefill, K=128: {over} of {Y.size} outputs beyond 2e-3*(|y|+rms) "
         f"of the exact product (allowed by its contract)")
    Ye = cpu(q4.q4g128_gemm_prefill_epilogue(packed, s, m, Xd))
    assert_rel(Ye, ref, "epilogue K=128")


# --------------------------------------------------------------------------
# the 36-layer decode stack: sampled layers at full size, launched back to
# back on one stream as the benchmark does
# --------------------------------------------------------------------------

def test_stack_sampled_layers(dev):
    shapes = [(synth.FUSED_N, synth.HIDDEN_K), (synth.OPROJ_N, synth.OPROJ_K), (synth.DOWN_N, synth.DOWN_K)]
    for layer in (0, 35):
        mats = []
        for which, (n, k) in enumerate(shapes):
            w = synth.weights(n, k, synth.stack_seed(layer, which))
            mats.append((w, upload(w, dev, q4)))
        xs = [synth.activations(1, k, seed=90000 + layer * 3 + i)[0] for i, (_, k) in enumerate(shapes)]
        outs = [q4.q4g128_gemv(p, s, m, to_dev_f16(x, dev)) for (w, (p, s, m)), x in zip(mats, xs)]
        for (w, _), x, y in zip(mats, xs, outs):
            ref = oracle.gemv(oracle.pack(w.codes), w.scales, w.mins, x)
            assert_rel(cpu(y), ref, f"stack layer {layer} {w.n}x{w.k}")
