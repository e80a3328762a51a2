"""Pins of the export-step oracle (oracle/quantize.py) against exact arithmetic.

Each pin checks the oracle with something it does not compute the same way:
exact round trips of weights built as code * scale + min, the best code per
element found by brute force over all 16 codes in rational arithmetic, the
reconstruction error bound that follows from the rounding of the stored
minimum and scale, nearest-even checks of the stored fp16 values against
their exact neighbours, and the degenerate groups.  The mutation tests at the
end plant plausible mistakes in a private copy of the oracle and check that
at least one pin fails for each.
"""
import importlib.util
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

ORACLE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "quantize.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("quantize_copy", ORACLE_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def fr(v) -> Fraction:
    return Fraction(float(v))


def fp16_neighbours(v: float):
    """The fp16 values just below and above the fp16 nearest to v."""
    h = np.float16(v)
    return np.nextafter(h, np.float16(-np.inf)), np.nextafter(h, np.float16(np.inf))


def assert_nearest_fp16(stored, exact: Fraction, what: str):
    """stored is an fp16 value at least as close to `exact` as its two neighbours."""
    d = abs(fr(stored) - exact)
    for nb in fp16_neighbours(float(stored)):
        if np.isfinite(nb):
            assert d <= abs(fr(nb) - exact), (what, float(stored), float(exact), float(nb))


def edge_groups(rng, n_rows: int) -> np.ndarray:
    """float32 [n_rows][128*8] of groups that exercise rounding of min and clamping.

    Per row: a constant group; two-valued group; a group far from zero with a
    narrow range (the fp16 minimum then differs from the true minimum by many
    scale steps, so codes clamp at 0 or 15); a group whose scale is an fp16
    subnormal; a group whose range is too small for any fp16 scale; a mixed
    sign group; and two ordinary normal groups.
    """
    rows = []
    for _ in range(n_rows):
        g = []
        g.append(np.full(128, rng.uniform(-2, 2), np.float32))
        two = np.where(rng.random(128) < 0.5, -1.0, 0.5).astype(np.float32)
        two[0], two[1] = -1.0, 0.5
        g.append(two)
        base = rng.choice([1000.2, 1000.3, -700.1, 513.77])
        g.append((base + rng.uniform(0, 0.15, 128)).astype(np.float32))
        g.append((rng.uniform(0, 1, 128) * 3e-5).astype(np.float32))
        one = np.float32(rng.uniform(0.5, 1.0))
        tiny = np.full(128, one, np.float32)
        tiny[rng.integers(0, 128, 5)] = np.nextafter(one, np.float32(2))
        g.append(tiny)
        g.append(rng.uniform(-3, 3, 128).astype(np.float32))
        g.append((rng.standard_normal(128) * 0.02).astype(np.float32))
        g.append((rng.standard_normal(128) * 0.003 + 0.01).astype(np.float32))
        rows.append(np.concatenate(g))
    return np.stack(rows)


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_exact_round_trip(orc):
    """Weights built exactly as c*s + m with codes 0 and 15 in every group
    come back as exactly (c, s, m): hi - lo = 15 s, so scale = s, min = m and
    every (w - m)/s is the integer c.
    """
    rng = np.random.Generator(np.random.PCG64(31))
    for n, k in [(3, 128), (4, 512), (2, 1152)]:
        g = k // 128
        codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
        for r in range(n):
            for j in range(g):
                pos = rng.choice(128, 2, replace=False) + 128 * j
                codes[r, pos[0]], codes[r, pos[1]] = 0, 15
        scales = (2.0 ** -rng.integers(3, 11, (n, g))).astype(np.float16)
        mins = (-rng.integers(0, 257, (n, g)) / 128.0).astype(np.float16)
        W = np.empty((n, k), np.float32)
        for r in range(n):
            for col in range(k):
                j = col // 128
                exact = int(codes[r, col]) * fr(scales[r, j]) + fr(mins[r, j])
                W[r, col] = float(exact)
                assert fr(W[r, col]) == exact  # representable in fp32
        c, s, m = orc.quantize(W)
        assert np.array_equal(c, codes)
        assert np.array_equal(s.view(np.uint16), scales.view(np.uint16))
        assert np.array_equal(m.view(np.uint16), mins.view(np.uint16))


def pin_best_code_brute_force(orc):
    """Every code is a nearest one under the stored fp16 scale and minimum:
    over all 16 codes, |w - (c*S + M)| computed exactly is minimal up to the
    fp32 rounding of the quotient (slack 2^-16 * S).  Also S and M are the
    nearest fp16 values to (hi - lo)/15 (within fp32's rounding of that
    quotient) and to the group minimum.
    """
    rng = np.random.Generator(np.random.PCG64(32))
    W = np.concatenate([synth.draw_float_weights(rng, 3, 256), edge_groups(rng, 3)[:, :256]], axis=0)
    W = np.concatenate([W, edge_groups(rng, 6)], axis=1)[:, :1024]
    c, s, m = orc.quantize(W)
    n, k = W.shape
    for r in range(n):
        for j in range(k // 128):
            vals = [fr(v) for v in W[r, 128 * j:128 * (j + 1)]]
            lo, hi = min(vals), max(vals)
            S, M = fr(s[r, j]), fr(m[r, j])
            assert_nearest_fp16(m[r, j], lo, "min")
            target = (hi - lo) / 15
            if S != 0 or target >= Fraction(2) ** -25:
                err_s = abs(S - target)
                for nb in fp16_neighbours(float(s[r, j])):
                    if np.isfinite(nb):
                        assert err_s <= abs(fr(nb) - target) + Fraction(2) ** -22 * target, (r, j)
            for t, w in enumerate(vals):
                code = int(c[r, 128 * j + t])
                assert 0 <= code <= 15
                if S == 0:
                    assert code == 0
                    continue
                errs = [abs(w - (cc * S + M)) for cc in range(16)]
                assert errs[code] <= min(errs) + Fraction(2) ** -16 * S, (r, j, t, code, errs.index(min(errs)))


def pin_reconstruction_bound(orc):
    """|w - (c*S + M)| <= S/2 + 15*|S - (hi-lo)/15| + |lo - M| for every element
    (the nearest-code error plus the clamping error at the two ends)."""
    rng = np.random.Generator(np.random.PCG64(33))
    W = np.concatenate([synth.draw_float_weights(rng, 48, 1024), edge_groups(rng, 8)], axis=0)
    c, s, m = orc.quantize(W)
    n, k = W.shape
    g = k // 128
    grp = W.astype(np.float64).reshape(n, g, 128)
    S = s.astype(np.float64)[:, :, None]
    M = m.astype(np.float64)[:, :, None]
    lo = grp.min(axis=2, keepdims=True)
    hi = grp.max(axis=2, keepdims=True)
    what = c.reshape(n, g, 128).astype(np.float64) * S + M
    bound = S / 2 + 15 * np.abs(S - (hi - lo) / 15) + np.abs(lo - M)
    assert np.all(np.abs(grp - what) <= bound * (1 + 1e-9) + 1e-30)


def pin_degenerate_groups(orc):
    """Constant group -> scale 0, codes 0, min = nearest fp16; two-valued group
    -1 / 0.5 -> codes 0 and 15; range below fp16's smallest scale -> scale 0."""
    W = np.zeros((1, 384), np.float32)
    W[0, :128] = 0.7
    W[0, 128:256] = np.where(np.arange(128) % 3 == 0, 0.5, -1.0)
    W[0, 256:] = 1.0
    W[0, 300] = np.nextafter(np.float32(1.0), np.float32(2))
    c, s, m = orc.quantize(W)
    assert float(s[0, 0]) == 0 and float(m[0, 0]) == float(np.float16(0.7)) and not c[0, :128].any()
    assert float(m[0, 1]) == -1.0 and float(s[0, 1]) == float(np.float16(0.1))
    assert list(c[0, 128:256]) == [15 if t % 3 == 0 else 0 for t in range(128)]
    assert float(s[0, 2]) == 0 and float(m[0, 2]) == 1.0 and not c[0, 256:].any()


def pin_export_bytes(orc):
    """The export of a ramp group packs to the known bytes 0x10, 0x32, ..., 0xFE
    (low nibble = even column), with scale 1/32 and min -1/4."""
    ramp = (-0.25 + (np.arange(128) % 16) / 32.0).astype(np.float32)
    c, s, m = orc.quantize(ramp.reshape(1, 128))
    assert float(s[0, 0]) == 1 / 32 and float(m[0, 0]) == -0.25
    packed = oracle.pack(c)
    assert list(packed[0, :8]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]


PINS = [
    pin_exact_round_trip,
    pin_best_code_brute_force,
    pin_reconstruction_bound,
    pin_degenerate_groups,
    pin_export_bytes,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_quantize_pin(pin):
    pin(oracle)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 100), np.float32))
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros(128, np.float32))


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------

def _replace_quantize(body):
    def apply(mod):
        def quantize(W):
            W = np.asarray(W, dtype=np.float32)
            n, k = W.shape
            grp = W.reshape(n, k // 128, 128)
            return body(grp, n, k)
        mod.quantize = quantize
    return apply


def _standard(grp, n, k, top=15, rnd=np.rint, group_of=128, use_stored=True, min_round=None, clamp=True):
    g_n = k // group_of
    grp = grp.reshape(n, g_n, group_of)
    lo, hi = grp.min(axis=2), grp.max(axis=2)
    s32 = (hi - lo) / np.float32(top)
    scales = s32.astype(np.float16)
    mins = lo.astype(np.float16) if min_round is None else min_round(lo)
    s = (scales.astype(np.float32) if use_stored else s32)[:, :, None]
    m = (mins.astype(np.float32) if use_stored else lo)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = rnd((grp - m) / s)
    if clamp:
        q = np.clip(q, 0, 15)
    q = np.where(s == 0, 0, q)
    codes = np.nan_to_num(q).astype(np.int64).astype(np.uint8).reshape(n, k)
    if group_of != 128:
        scales = scales.reshape(n, -1)[:, ::128 // group_of]
        mins = mins.reshape(n, -1)[:, ::128 // group_of]
    return codes, scales, mins


MUTANTS = {
    "divide_by_16": _replace_quantize(lambda grp, n, k: _standard(grp, n, k, top=16)),
    "floor_not_round": _replace_quantize(lambda grp, n, k: _standard(grp, n, k, rnd=np.floor)),
    "codes_against_unrounded_min_and_scale": _replace_quantize(lambda grp, n, k: _standard(grp, n, k, use_stored=False)),
    "min_truncated_toward_zero": _replace_quantize(
        lambda grp, n, k: _standard(grp, n, k, min_round=lambda lo: np.trunc(lo * 1024) / 1024)),
    "no_clamp": _replace_quantize(lambda grp, n, k: _standard(grp, n, k, clamp=False)),
    "group_of_64": _replace_quantize(lambda grp, n, k: _standard(grp, n, k, group_of=64)),
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
