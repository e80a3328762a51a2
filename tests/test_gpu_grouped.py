"""GPU tests of q4g128_gemv_grouped: many independent projections per launch.

Every output must be bit-identical to q4g128_gemv on the same projection
(same lanes, chunk order and reductions per row), and within the GEMV's
tolerance of the fp64 oracle.  Calls go through the C ABI.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_bound, assert_rel, cpu, device, gemv_bound, note, to_dev_f16, upload

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


# One K per pass mapping of the batch-1 GEMV (lanes per row, chunks per lane,
# ragged or not), and two K that it runs on its batched kernel (launched one
# by one inside the grouped call).
KS = [128, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192,   # 4..64 lanes, 1..4 chunks
      2176, 4224, 6400, 8320, 11008,                                          # ragged, 2..6 chunks per lane
      16384, 12416]                                                           # batched-kernel shapes
NS = [1, 3, 5, 64, 1000, 4099]


def _singles(projs):
    return [cpu(q4.q4g128_gemv(p, s, m, x)) for p, s, m, x in projs]


def test_grouped_mixed_shapes_bit_identical(dev):
    rng = np.random.Generator(np.random.PCG64(2024))
    cases, projs = [], []
    for i, k in enumerate(KS):
        for n in (NS[i % len(NS)], NS[(i + 3) % len(NS)]):
            w, x = synth.gemv_case(n, k, seed=10 * k + n)
            p, s, m = upload(w, dev, q4)
            cases.append((w, x[0]))
            projs.append((p, s, m, to_dev_f16(x[0], dev)))
    order = rng.permutation(len(projs))  # variants interleaved in the call
    projs = [projs[i] for i in order]
    cases = [cases[i] for i in order]
    ys = q4.q4g128_gemv_grouped(projs)
    for (w, x), y, single in zip(cases, ys, _singles(projs)):
        got = cpu(y)
        assert np.array_equal(got, single), f"{w.n}x{w.k}: grouped output differs from q4g128_gemv"
        packed_np = oracle.pack(w.codes)
        ref = oracle.gemv(packed_np, w.scales, w.mins, x)
        assert_rel(got, ref, f"grouped {w.n}x{w.k}")
        assert_bound(got, ref, gemv_bound(packed_np, w, x.reshape(1, -1))[0], 128, f"grouped {w.n}x{w.k}")


def test_grouped_more_than_one_launch_per_variant(dev):
    """75 projections of one mapping (two launches of at most 64), rows
    from 1 to 700, and one shared weight set under several inputs."""
    projs, cases = [], []
    shared = None
    for i in range(75):
        n = 1 + (i * 37) % 700
        if i % 5 == 4 and shared is not None:
            w, (p, s, m) = shared
        else:
            w = synth.weights(n, 3072, seed=300 + i)
            p, s, m = upload(w, dev, q4)
            shared = (w, (p, s, m))
        x = synth.activations(1, 3072, seed=400 + i)[0]
        projs.append((p, s, m, to_dev_f16(x, dev)))
        cases.append((w, x))
    ys = q4.q4g128_gemv_grouped(projs)
    for (w, x), y, single in zip(cases, ys, _singles(projs)):
        got = cpu(y)
        assert np.array_equal(got, single)
        assert_rel(got, oracle.gemv(oracle.pack(w.codes), w.scales, w.mins, x), f"grouped {w.n}x3072")


def test_grouped_pages_step_shared_weights(dev):
    """The pages' 108-projection step (hidden 2,048) with one weight set per
    shape shared by all 36 layers and a fresh x per projection."""
    names = ["pages_fused_25088x2048", "pages_oproj_2048x2048", "pages_down_2048x11008"]
    base = []
    for name in names:
        w, _ = synth.workload(name)
        base.append((w, upload(w, dev, q4)))
    projs, xs = [], []
    for layer in range(36):
        for i, (w, (p, s, m)) in enumerate(base):
            x = synth.activations(1, w.k, seed=50000 + 3 * layer + i)[0]
            projs.append((p, s, m, to_dev_f16(x, dev)))
            xs.append(x)
    ys = q4.q4g128_gemv_grouped(projs)
    singles = _singles(projs)
    for y, single in zip(ys, singles):
        assert np.array_equal(cpu(y), single)
    for idx in (0, 1, 2, 105, 106, 107):
        w = base[idx % 3][0]
        assert_rel(cpu(ys[idx]), oracle.gemv(oracle.pack(w.codes), w.scales, w.mins, xs[idx]), f"pages step {idx}")


def test_grouped_decode_stack_full(dev):
    """The 36-layer decode step at full size (108 projections, fresh weights
    per layer, 2.14 GB), as the benchmark's grouped form calls it: every
    output bit-identical to its single call; layers 0 and 35 against the
    oracle."""
    shapes = [(synth.FUSED_N, synth.HIDDEN_K), (synth.OPROJ_N, synth.OPROJ_K), (synth.DOWN_N, synth.DOWN_K)]
    projs, host = [], {}
    for layer in range(synth.STACK_LAYERS):
        for which, (n, k) in enumerate(shapes):
            w = synth.weights(n, k, synth.stack_seed(layer, which))
            x = synth.activations(1, k, seed=90000 + 3 * layer + which)[0]
            projs.append(upload(w, dev, q4) + (to_dev_f16(x, dev),))
            if layer in (0, 35):
                host[(layer, which)] = (w, x)
        if layer % 6 == 5:
            note(f"[gpu-test]   stack layer {layer} uploaded")
    ys = q4.q4g128_gemv_grouped(projs)
    ys_again = [cpu(y).copy() for y in q4.q4g128_gemv_grouped(projs)]
    for idx, (y, single) in enumerate(zip(ys, _singles(projs))):
        got = cpu(y)
        assert np.array_equal(got, single), f"projection {idx}"
        assert np.array_equal(got, ys_again[idx]), f"projection {idx}: repeat differs"
    for (layer, which), (w, x) in host.items():
        got = cpu(ys[3 * layer + which])
        assert_rel(got, oracle.gemv(oracle.pack(w.codes), w.scales, w.mins, x), f"stack {layer}/{which}")


def test_grouped_graph_replays(dev):
    """The grouped call captured in a HIP graph: every replay, with eager
    work in between, rewrites the outputs with the eager result."""
    projs = []
    for i, (n, k) in enumerate([(4099, 3072), (3072, 8192), (700, 3072), (2048, 11008), (50, 16384)]):
        w, x = synth.gemv_case(n, k, seed=600 + i)
        projs.append(upload(w, dev, q4) + (to_dev_f16(x[0], dev),))
    ys = [torch.empty(p[0].shape[0], dtype=torch.float32, device=dev) for p in projs]
    st = torch.cuda.Stream(dev)
    with torch.cuda.stream(st):
        q4.q4g128_gemv_grouped(projs, ys, stream=st)
        eager = [y.clone() for y in ys]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            q4.q4g128_gemv_grouped(projs, ys, stream=st)
    st.synchronize()
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        with torch.cuda.stream(st):
            g.replay()
        st.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y, e), f"replay {rep}"
        _ = (torch.ones(1024, device=dev) * rep).sum().item()  # eager work between replays
