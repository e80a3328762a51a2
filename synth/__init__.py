"""Seeded synthetic inputs for the int4 group-128 weight format.

This module only draws random numbers.  It holds none of the method's
arithmetic (no packing, no dequantisation, no products): it returns the
unpacked 4-bit codes, the fp16 scales and minimums per 128-column group, and
fp16 activations.  Both the CPU oracle's tests and the GPU path's tests and
benchmark take their inputs from here, so the two sides see the same numbers
without sharing any code.

Value distributions follow the workload definition used throughout:
codes uniform on 0..15, scale uniform on [0.001, 0.02], minimum uniform on
[-0.15, 0], activations standard normal, each cast to fp16 with
round-to-nearest-even (the stored fp16 value is the truth).  The rumik-oss-1
write-up (rtts.neoandmatrix.me, "Step 3: an int4 file and a first kernel on
the laptop") fixes the format (two codes per byte, fp16 scale and minimum per
128-column group) but prints no weights, so these draws stand in for the
trained projection matrices.

Draw order per weight matrix, from one ``numpy.random.Generator(PCG64(seed))``:
codes (N, K) -> scales (N, G) -> mins (N, G) [-> activations (B, K) when the
same generator also supplies the activation vector].
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 128

SCALE_RANGE = (0.001, 0.02)
MIN_RANGE = (-0.15, 0.0)


@dataclass
class Weights:
    codes: np.ndarray   # uint8 [N][K], values 0..15
    scales: np.ndarray  # float16 [N][K/128]
    mins: np.ndarray    # float16 [N][K/128]

    @property
    def n(self) -> int:
        return self.codes.shape[0]

    @property
    def k(self) -> int:
        return self.codes.shape[1]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def draw_weights(rng: np.random.Generator, n: int, k: int) -> Weights:
    if k % GROUP:
        raise ValueError(f"k={k} is not a multiple of {GROUP}")
    g = k // GROUP
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    scales = rng.uniform(*SCALE_RANGE, (n, g)).astype(np.float16)
    mins = rng.uniform(*MIN_RANGE, (n, g)).astype(np.float16)
    return Weights(codes, scales, mins)


def draw_float_weights(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """float32 [N][K] stand-in for trained projection weights (input of the export step).

    Normal values with a per-row spread drawn uniformly on [0.005, 0.05]; the
    pages print no weights, so only the shape of the distribution matters.
    """
    spread = rng.uniform(0.005, 0.05, (n, 1))
    return (rng.standard_normal((n, k)) * spread).astype(np.float32)


def float_weights(n: int, k: int, seed: int) -> np.ndarray:
    """float32 weights of one matrix drawn from their own generator."""
    return draw_float_weights(_rng(seed), n, k)


def draw_head_int8(rng: np.random.Generator, n: int, k: int):
    """int8 output-head weights: codes uniform on -127..127 (the symmetric
    range), one fp16 scale per row uniform on [0.0005, 0.01]."""
    q = rng.integers(-127, 128, (n, k), dtype=np.int8)
    s = rng.uniform(0.0005, 0.01, n).astype(np.float16)
    return q, s


def head_int8_case(n: int, k: int, seed: int):
    """(q, scales, x) of one int8 head from one generator."""
    rng = _rng(seed)
    q, s = draw_head_int8(rng, n, k)
    x = draw_activations(rng, 1, k)[0]
    return q, s, x


def draw_activations(rng: np.random.Generator, b: int, k: int) -> np.ndarray:
    return rng.standard_normal((b, k)).astype(np.float16)


def weights(n: int, k: int, seed: int) -> Weights:
    """Weights of one matrix drawn from their own generator."""
    return draw_weights(_rng(seed), n, k)


def activations(b: int, k: int, seed: int) -> np.ndarray:
    """A [B][K] fp16 activation block drawn from its own generator."""
    return draw_activations(_rng(seed), b, k)


def gemv_case(n: int, k: int, seed: int, b: int = 1):
    """Weights then activations from ONE generator (the single-matrix cases)."""
    rng = _rng(seed)
    w = draw_weights(rng, n, k)
    x = draw_activations(rng, b, k)
    return w, x


# Named workloads.  Shapes: the fused q/k/v/gate/up projection has 25,088
# rows; the partner projections are 3,072 x 3,072 and 3,072 x 8,192.
FUSED_N, HIDDEN_K = 25088, 3072
OPROJ_N, OPROJ_K = 3072, 3072
DOWN_N, DOWN_K = 3072, 8192
STACK_LAYERS = 36
# The pages' own model (rumik-oss-1) appears to have hidden size 2,048: the
# fused projection keeps its 25,088 rows, o_proj is 2,048 x 2,048 and down is
# 2,048 x 11,008 (a reconstruction from the pages' per-token byte counts).
PAGES_HIDDEN = 2048
PAGES_FFN = 11008

SEEDS = {
    "tiny": 0,
    "fused": 1,
    "oproj": 2,
    "down": 3,
    "batch_x": 4,
    "prefill_x34": 5,
    "prefill_x256": 6,
    "float_weights": 21,
    "pages_fused": 11,
    "pages_oproj": 12,
    "pages_down": 13,
    "head_int8": 31,
}
# int8 output head: 16,384 rows (an assumed audio vocabulary of 8 codebooks x
# 2,048 entries; the pages give no head size) by the hidden size.
HEAD_N = 16384


def stack_seed(layer: int, which: int) -> int:
    """Seed of projection `which` (0 fused, 1 o_proj, 2 down) in layer `layer`."""
    return 1000 + 3 * layer + which


WORKLOADS = {
    # name: (N, K, seed)
    "tiny_256x512": (256, 512, SEEDS["tiny"]),
    "fused_25088x3072": (FUSED_N, HIDDEN_K, SEEDS["fused"]),
    "oproj_3072x3072": (OPROJ_N, OPROJ_K, SEEDS["oproj"]),
    "down_3072x8192": (DOWN_N, DOWN_K, SEEDS["down"]),
    "pages_fused_25088x2048": (FUSED_N, PAGES_HIDDEN, SEEDS["pages_fused"]),
    "pages_oproj_2048x2048": (PAGES_HIDDEN, PAGES_HIDDEN, SEEDS["pages_oproj"]),
    "pages_down_2048x11008": (PAGES_HIDDEN, PAGES_FFN, SEEDS["pages_down"]),
}


def workload(name: str, b: int = 1):
    n, k, seed = WORKLOADS[name]
    return gemv_case(n, k, seed, b)


def batch_activations(b: int, k: int = HIDDEN_K) -> np.ndarray:
    """First b rows of one 16-row draw, so every batch size shares its columns."""
    if not 1 <= b <= 16:
        raise ValueError("b must be in 1..16")
    return activations(16, k, SEEDS["batch_x"])[:b]


def prefill_activations(m: int, k: int = HIDDEN_K) -> np.ndarray:
    seed = {34: SEEDS["prefill_x34"], 256: SEEDS["prefill_x256"]}.get(m, 7000 + m)
    return activations(m, k, seed)
