"""Pins of the int8 output-head oracle (oracle/head_int8.py).

The oracle is checked against exact rational sums over Python integers and
Fractions, one-hot probes over every int8 value (sign handling), a closed
form, exact dyadic cases and linearity.  Planted mistakes (codes read as
unsigned, the scale taken per column, a dropped column, the sign flipped,
the scale applied twice) must each fail at least one pin.
"""
import importlib.util
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

ORACLE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "head_int8.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("head_copy", ORACLE_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def fr(v) -> Fraction:
    return Fraction(float(v))


def pin_brute_force(orc):
    """Random tiny heads against exact sums of int(q) * scale * x."""
    rng = np.random.Generator(np.random.PCG64(51))
    for n, k in [(1, 128), (3, 256), (5, 384), (2, 1024)]:
        q, s = synth.draw_head_int8(rng, n, k)
        x = synth.draw_activations(rng, 1, k)[0]
        y = orc.gemv_int8(q, s, x)
        for r in range(n):
            exact = fr(s[r]) * sum(int(q[r, c]) * fr(x[c]) for c in range(k))
            mag = float(s[r]) * sum(abs(int(q[r, c]) * float(x[c])) for c in range(k))
            assert abs(fr(y[r]) - exact) <= Fraction(2) ** -45 * Fraction(mag + 1e-300), (n, k, r)


def pin_one_hot_all_codes(orc):
    """x = e_c returns q[n][c] * scale[n] exactly, for every int8 value."""
    k = 256
    q = np.arange(-128, 128, dtype=np.int16).astype(np.int8).reshape(1, 256)
    q = np.concatenate([q, q[:, ::-1]], axis=0)
    s = np.array([0.0078125, 0.3], dtype=np.float16)
    for c in (0, 1, 2, 3, 127, 128, 129, 254, 255):
        x = np.zeros(k, dtype=np.float16)
        x[c] = 1
        y = orc.gemv_int8(q, s, x)
        for r in range(2):
            assert fr(y[r]) == int(q[r, c]) * fr(s[r]), (c, r, float(y[r]))


def pin_closed_form(orc):
    """Constant code v, x = 1: y = K * v * scale."""
    for v, sc, k in [(-128, 0.5, 128), (127, 0.001, 1024), (-3, 0.25, 384), (0, 1.0, 256)]:
        q = np.full((3, k), v, dtype=np.int8)
        s = np.full(3, sc, dtype=np.float16)
        y = orc.gemv_int8(q, s, np.ones(k, dtype=np.float16))
        assert all(fr(t) == k * v * fr(np.float16(sc)) for t in y), (v, sc, k)


def pin_dyadic_exact(orc):
    """Codes in -128..127, scales 2^-e, x in {-3..3}: every sum is exact."""
    rng = np.random.Generator(np.random.PCG64(52))
    n, k = 4, 512
    q = rng.integers(-128, 128, (n, k)).astype(np.int8)
    s = (2.0 ** -rng.integers(2, 9, n)).astype(np.float16)
    x = rng.integers(-3, 4, k).astype(np.float16)
    y = orc.gemv_int8(q, s, x)
    for r in range(n):
        assert fr(y[r]) == fr(s[r]) * sum(int(q[r, c]) * int(x[c]) for c in range(k))


def pin_linearity(orc):
    """x = 0 gives 0; x * 2^j scales y by exactly 2^j."""
    rng = np.random.Generator(np.random.PCG64(53))
    q, s = synth.draw_head_int8(rng, 6, 384)
    assert np.all(orc.gemv_int8(q, s, np.zeros(384, dtype=np.float16)) == 0)
    x = synth.draw_activations(rng, 1, 384)[0]
    y = orc.gemv_int8(q, s, x)
    for j in (-2, 3):
        y2 = orc.gemv_int8(q, s, (x.astype(np.float64) * 2.0 ** j).astype(np.float16))
        assert np.array_equal(y2, y * 2.0 ** j)


PINS = [pin_brute_force, pin_one_hot_all_codes, pin_closed_form, pin_dyadic_exact, pin_linearity]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_head_int8_pin(pin):
    pin(oracle)


def test_rejects_bad_arguments():
    q = np.zeros((2, 128), np.int8)
    with pytest.raises(ValueError):
        oracle.gemv_int8(q.astype(np.uint8), np.ones(2, np.float16), np.ones(128, np.float16))
    with pytest.raises(ValueError):
        oracle.gemv_int8(q, np.ones(3, np.float16), np.ones(128, np.float16))
    with pytest.raises(ValueError):
        oracle.gemv_int8(q, np.ones(2, np.float16), np.ones(64, np.float16))


def _replace(body):
    def apply(mod):
        def gemv_int8(q, scales, x):
            q = np.asarray(q)
            s = np.asarray(scales, dtype=np.float16).astype(np.float64)
            xv = np.asarray(x, dtype=np.float16).astype(np.float64)
            return body(q, s, xv)
        mod.gemv_int8 = gemv_int8
    return apply


MUTANTS = {
    "codes_unsigned": _replace(lambda q, s, x: (q.view(np.uint8).astype(np.float64) * s[:, None]) @ x),
    "scale_per_column": _replace(
        lambda q, s, x: (q.astype(np.float64) * np.resize(s, q.shape[1])[None, :]) @ x),
    "dropped_last_column": _replace(lambda q, s, x: (q[:, :-1].astype(np.float64) * s[:, None]) @ x[:-1]),
    "sign_flipped": _replace(lambda q, s, x: -(q.astype(np.float64) * s[:, None]) @ x),
    "scale_twice": _replace(lambda q, s, x: (q.astype(np.float64) * (s * s)[:, None]) @ x),
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
