"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each pin compares the oracle with something it does not compute the same
way: exact rational brute force, closed forms, hand-derived known answers
(tests/golden/known_answers.txt), pack/unpack round trips over every byte,
one-hot probes, exact dyadic cases and linearity.  The mutation tests at the
end plant plausible mistakes in a private copy of the oracle (nibble order,
min multiplicity, group index, sign, dropped term, transposed scales,
off-by-one codes) and check that at least one pin fails for each.
"""
import importlib.util
import os
from fractions import Fraction

import numpy as np
import pytest

import golden_cases
import oracle
import synth

ORACLE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "q4g128.py")


def fresh_oracle():
    """A private copy of the oracle module that a mutation test may patch."""
    spec = importlib.util.spec_from_file_location("oracle_copy", ORACLE_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


# --------------------------------------------------------------------------
# brute-force helpers: plain Python integers and Fractions, no NumPy math
# --------------------------------------------------------------------------

def bf_pack_row(codes_row):
    """Bytes of one row built as code_even + 16 * code_odd with Python ints."""
    out = []
    for j in range(0, len(codes_row), 2):
        out.append(int(codes_row[j]) + 16 * int(codes_row[j + 1]))
    return out


def bf_gemv(codes, scales, mins, x):
    """Exact y[n] = sum_k (c*s + m) * x as Fractions, read from unpacked codes."""
    n, k = codes.shape
    ys = []
    for r in range(n):
        acc = Fraction(0)
        for col in range(k):
            g = col // 128
            s = Fraction(float(scales[r, g]))
            m = Fraction(float(mins[r, g]))
            acc += (int(codes[r, col]) * s + m) * Fraction(float(x[col]))
        ys.append(acc)
    return ys


def bf_abs_terms(codes, scales, mins, x):
    n, k = codes.shape
    out = []
    for r in range(n):
        t = 0.0
        for col in range(k):
            g = col // 128
            t += abs((int(codes[r, col]) * float(scales[r, g]) + float(mins[r, g])) * float(x[col]))
        out.append(t)
    return out


# --------------------------------------------------------------------------
# pins, written against an oracle namespace so mutants can be fed through
# --------------------------------------------------------------------------

def pin_brute_force(orc, seed=11):
    """P1: random tiny matrices against exact rational sums."""
    rng = np.random.Generator(np.random.PCG64(seed))
    for n, k in [(1, 128), (3, 256), (5, 384), (8, 128), (3, 384)]:
        w = synth.draw_weights(rng, n, k)
        X = synth.draw_activations(rng, 2, k)
        Y = orc.gemm(orc.pack(w.codes), w.scales, w.mins, X)
        for b in range(2):
            exact = bf_gemv(w.codes, w.scales, w.mins, X[b])
            mag = bf_abs_terms(w.codes, w.scales, w.mins, X[b])
            for r in range(n):
                err = abs(Fraction(float(Y[b, r])) - exact[r])
                assert err <= Fraction(2) ** -40 * Fraction(mag[r] + 1e-300), (n, k, b, r, float(err))


def pin_closed_form_constant(orc):
    """P2: constant code c, scale s, min m, x = 1 gives y = K * (c*s + m)."""
    for c, s, m, k in [(15, 0.0625, -0.5, 128), (7, 0.01, -0.1, 1024), (0, 0.5, -0.125, 384), (9, 0.001, 0.0, 256)]:
        s16, m16 = np.float16(s), np.float16(m)
        n = 2
        codes = np.full((n, k), c, dtype=np.uint8)
        scales = np.full((n, k // 128), s16, dtype=np.float16)
        mins = np.full((n, k // 128), m16, dtype=np.float16)
        y = orc.gemv(orc.pack(codes), scales, mins, np.ones(k, dtype=np.float16))
        expect = k * (Fraction(c) * Fraction(float(s16)) + Fraction(float(m16)))
        assert all(Fraction(float(v)) == expect for v in y), (c, s, m, k, y, float(expect))


def pin_closed_form_groups(orc):
    """P2': per-group constants give y = sum_g 128 * (c_g*s_g + m_g)."""
    rng = np.random.Generator(np.random.PCG64(5))
    k, n = 640, 3
    g = k // 128
    cg = rng.integers(0, 16, (n, g))
    sg = rng.uniform(0.001, 0.02, (n, g)).astype(np.float16)
    mg = rng.uniform(-0.15, 0, (n, g)).astype(np.float16)
    codes = np.repeat(cg.astype(np.uint8), 128, axis=1)
    y = orc.gemv(orc.pack(codes), sg, mg, np.ones(k, dtype=np.float16))
    for r in range(n):
        expect = sum(128 * (int(cg[r, j]) * Fraction(float(sg[r, j])) + Fraction(float(mg[r, j]))) for j in range(g))
        assert abs(Fraction(float(y[r])) - expect) <= Fraction(2) ** -45, (r, float(y[r]), float(expect))


def pin_min_only(orc):
    """P3: all codes 0 gives y = sum_g m_g * sum_{k in g} x_k."""
    rng = np.random.Generator(np.random.PCG64(6))
    k, n = 512, 4
    g = k // 128
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.02, (n, g)).astype(np.float16)
    mins = rng.uniform(-0.15, 0, (n, g)).astype(np.float16)
    x = rng.integers(-4, 5, k).astype(np.float16)
    y = orc.gemv(orc.pack(codes), scales, mins, x)
    for r in range(n):
        expect = sum(Fraction(float(mins[r, j])) * sum(Fraction(float(v)) for v in x[j * 128:(j + 1) * 128]) for j in range(g))
        assert Fraction(float(y[r])) == expect


def pin_one_hot(orc):
    """P4: x = e_k returns column k of W; checks nibble order and group index."""
    rng = np.random.Generator(np.random.PCG64(7))
    n, k = 3, 384
    w = synth.draw_weights(rng, n, k)
    packed = orc.pack(w.codes)
    for col in [0, 1, 2, 3, 126, 127, 128, 129, 255, 256, 383]:
        x = np.zeros(k, dtype=np.float16)
        x[col] = 1
        y = orc.gemv(packed, w.scales, w.mins, x)
        g = col // 128
        for r in range(n):
            expect = int(w.codes[r, col]) * Fraction(float(w.scales[r, g])) + Fraction(float(w.mins[r, g]))
            assert Fraction(float(y[r])) == expect, (col, r)


def pin_dyadic_exact(orc):
    """P5: fp16-exact dyadic inputs make every sum exact, so y == exact."""
    for seed in range(3):
        n, k, codes, scales, mins, x = dyadic_case(seed, 4, 384)
        y = orc.gemv(orc.pack(codes), scales, mins, x)
        exact = bf_gemv(codes, scales, mins, x)
        assert [Fraction(float(v)) for v in y] == exact


def pin_pack(orc):
    """P6: pack matches code_even + 16*code_odd; all 256 bytes round-trip."""
    codes = np.array([[c1, c2] * 64 for c1 in range(16) for c2 in range(16)], dtype=np.uint8)
    packed = orc.pack(codes)
    for r in range(codes.shape[0]):
        assert list(packed[r]) == bf_pack_row(codes[r])
    assert orc.pack(np.array([[1, 2] * 64], dtype=np.uint8))[0, 0] == 0x21
    all_bytes = np.arange(256, dtype=np.uint8).reshape(2, 128)
    all_bytes = np.concatenate([all_bytes, all_bytes[:, ::-1]], axis=1)  # [2][256] -> K = 512
    assert np.array_equal(orc.pack(orc.unpack(all_bytes, 512)), all_bytes)
    rng = np.random.Generator(np.random.PCG64(8))
    c = rng.integers(0, 16, (5, 768), dtype=np.uint8)
    assert np.array_equal(orc.unpack(orc.pack(c), 768), c)


def pin_linearity(orc):
    """P7: x = 0 gives exact zeros; x * 2^j scales y by exactly 2^j."""
    rng = np.random.Generator(np.random.PCG64(9))
    w = synth.draw_weights(rng, 6, 256)
    packed = orc.pack(w.codes)
    assert np.all(orc.gemv(packed, w.scales, w.mins, np.zeros(256, dtype=np.float16)) == 0)
    x = synth.draw_activations(rng, 1, 256)[0]
    y = orc.gemv(packed, w.scales, w.mins, x)
    for j in (-3, 1, 4):
        y2 = orc.gemv(packed, w.scales, w.mins, (x.astype(np.float64) * 2.0 ** j).astype(np.float16))
        assert np.array_equal(y2, y * 2.0 ** j)


def pin_known_answers(orc):
    """Hand-derived known answers from tests/golden/known_answers.txt."""
    for case in golden_cases.load():
        packed = case.packed if case.packed is not None else orc.pack(case.codes)
        y = orc.gemv(packed, case.scales, case.mins, case.x)
        assert y.shape == (1,)
        assert float(y[0]) == case.expected, (case.name, float(y[0]), case.expected)


def pin_fp16_weights(orc):
    """The fp16-weight form equals the exact sum over fp16(c*s + m) weights."""
    rng = np.random.Generator(np.random.PCG64(12))
    n, k = 3, 256
    w = synth.draw_weights(rng, n, k)
    X = synth.draw_activations(rng, 2, k)
    Y = orc.gemm_fp16_weights(orc.pack(w.codes), w.scales, w.mins, X)
    for r in range(n):
        w16 = []
        for col in range(k):
            g = col // 128
            exact = int(w.codes[r, col]) * Fraction(float(w.scales[r, g])) + Fraction(float(w.mins[r, g]))
            w16.append(Fraction(float(np.float16(float(exact)))))  # exact -> fp64 is exact here, one rounding to fp16
        for b in range(2):
            exact_y = sum(w16[col] * Fraction(float(X[b, col])) for col in range(k))
            assert abs(Fraction(float(Y[b, r])) - exact_y) <= Fraction(2) ** -40


def pin_term_magnitude(orc, seed=13):
    """The error-bound magnitude T[b][n] = sum_k (code*scale + |min|) * |x_k|
    against exact rational sums on tiny matrices.

    Not a product of the method: it is the sum of the magnitudes of the terms
    a kernel adds when it forms scale*sum(code*x) + min*sum(x) per group, the
    quantity that the GPU tests scale by a multiple of 2^-24 to bound fp32
    summation error.  Negative minimums and mixed-sign x make every plausible
    slip visible (min without its absolute value, |w| instead of
    code*scale + |min|, a dropped min term).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    for n, k in [(1, 128), (3, 256), (4, 384)]:
        w = synth.draw_weights(rng, n, k)
        X = synth.draw_activations(rng, 2, k)
        T = orc.term_magnitude(orc.pack(w.codes), w.scales, w.mins, X)
        assert T.shape == (2, n)
        for b in range(2):
            for r in range(n):
                exact = Fraction(0)
                for col in range(k):
                    g = col // 128
                    exact += ((int(w.codes[r, col]) * Fraction(float(w.scales[r, g]))
                               + abs(Fraction(float(w.mins[r, g])))) * abs(Fraction(float(X[b, col]))))
                assert abs(Fraction(float(T[b, r])) - exact) <= Fraction(2) ** -40 * exact, (n, k, b, r)


PINS = [
    pin_brute_force,
    pin_closed_form_constant,
    pin_closed_form_groups,
    pin_min_only,
    pin_one_hot,
    pin_dyadic_exact,
    pin_pack,
    pin_linearity,
    pin_known_answers,
    pin_fp16_weights,
    pin_term_magnitude,
]


def dyadic_case(seed, n, k):
    """Inputs whose every partial sum is exact in fp32 (and fp64) in any order.

    scale in {2^-3, 2^-4, 2^-5}, min in {-j/32 : j = 0..16}, x in {-3..3}:
    each term c*s*x and m*x is a multiple of 2^-5 of magnitude below 2^7, so
    all sums over K <= 8192 stay multiples of 2^-5 below 2^20 < 2^(24-5).
    """
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    g = k // 128
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    scales = (2.0 ** -rng.integers(3, 6, (n, g))).astype(np.float16)
    mins = (-rng.integers(0, 17, (n, g)) / 32.0).astype(np.float16)
    x = rng.integers(-3, 4, k).astype(np.float16)
    return n, k, codes, scales, mins, x


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle)


# --------------------------------------------------------------------------
# planted mistakes: each mutant must be caught by at least one pin
# --------------------------------------------------------------------------

def _mutant_swapped_nibbles(mod):
    def unpack(packed, k):
        packed = np.asarray(packed, dtype=np.uint8)
        codes = np.empty((packed.shape[0], k), dtype=np.uint8)
        codes[:, 0::2] = packed >> 4
        codes[:, 1::2] = packed & 0x0F
        return codes
    mod.unpack = unpack


def _mutant_dequant(formula):
    def apply(mod):
        orig_unpack = mod.unpack

        def dequantize(packed, scales, mins, k):
            codes = orig_unpack(packed, k).astype(np.float64)
            s = np.repeat(np.asarray(scales, np.float16).astype(np.float64), 128, axis=1)
            m = np.repeat(np.asarray(mins, np.float16).astype(np.float64), 128, axis=1)
            return formula(codes, s, m, scales, mins)
        mod.dequantize = dequantize
    return apply


def _group64(codes, s, m, scales, mins):
    s64 = np.repeat(np.asarray(scales, np.float16).astype(np.float64), 64, axis=1)
    m64 = np.repeat(np.asarray(mins, np.float16).astype(np.float64), 64, axis=1)
    k = codes.shape[1]
    reps = -(-k // s64.shape[1])
    s64 = np.tile(s64, (1, reps))[:, :k]
    m64 = np.tile(m64, (1, reps))[:, :k]
    return codes * s64 + m64


def _transposed_scales(codes, s, m, scales, mins):
    sc = np.asarray(scales, np.float16).astype(np.float64)
    st = sc.T.reshape(sc.shape) if sc.shape[0] != sc.shape[1] else sc.T
    return codes * np.repeat(st, 128, axis=1) + m


def _mutant_dropped_last(mod):
    orig = mod.gemm

    def gemm(packed, scales, mins, X):
        X = np.array(X, dtype=np.float16)
        X[:, -1] = 0
        return orig(packed, scales, mins, X)
    mod.gemm = gemm


def _mutant_pack_order(mod):
    def pack(codes):
        codes = np.asarray(codes, dtype=np.uint8)
        return ((codes[:, 1::2] & 15) | ((codes[:, 0::2] & 15) << 4)).astype(np.uint8)
    mod.pack = pack


def _mutant_term_magnitude(formula):
    def apply(mod):
        orig_unpack = mod.unpack

        def term_magnitude(packed, scales, mins, X):
            X = np.asarray(X, dtype=np.float16).astype(np.float64)
            k = X.shape[1]
            c = orig_unpack(packed, k).astype(np.float64)
            s = np.repeat(np.asarray(scales, np.float16).astype(np.float64), 128, axis=1)
            m = np.repeat(np.asarray(mins, np.float16).astype(np.float64), 128, axis=1)
            return np.abs(X) @ formula(c, s, m).T
        mod.term_magnitude = term_magnitude
    return apply


MUTANTS = {
    "swapped_nibbles": _mutant_swapped_nibbles,
    "term_magnitude_drops_min": _mutant_term_magnitude(lambda c, s, m: c * s),
    "term_magnitude_signed_min": _mutant_term_magnitude(lambda c, s, m: c * s + m),
    "term_magnitude_abs_weight": _mutant_term_magnitude(lambda c, s, m: np.abs(c * s + m)),
    "min_counted_four_times": _mutant_dequant(lambda c, s, m, *_: c * s + 4 * m),
    "min_sign": _mutant_dequant(lambda c, s, m, *_: c * s - m),
    "code_plus_one": _mutant_dequant(lambda c, s, m, *_: (c + 1) * s + m),
    "zero_point_convention": _mutant_dequant(lambda c, s, m, *_: (c - 8) * s + m),
    "group_of_64": _mutant_dequant(_group64),
    "transposed_scales": _mutant_dequant(_transposed_scales),
    "dropped_last_column": _mutant_dropped_last,
    "pack_nibble_order": _mutant_pack_order,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    mod = fresh_oracle()
    MUTANTS[name](mod)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"


def test_fresh_copy_passes_all_pins():
    mod = fresh_oracle()
    for pin in PINS:
        pin(mod)
