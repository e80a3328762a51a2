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


# --------------------------------------------------------------------------
# IEEE rounding from its definition, on exact rationals (no NumPy arithmetic)
# --------------------------------------------------------------------------

def round_ieee(v: Fraction, p: int, emin: int, emax: int) -> Fraction:
    """The binary floating-point number nearest to v, ties to the even
    significand: p significand bits (the leading bit included), normal
    exponents emin..emax, subnormals below 2^emin with spacing 2^(emin-p+1).
    Overflow raises (the quantiser's inputs keep every step finite)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    r = a / ulp
    q = r.numerator // r.denominator
    rem = r - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    out = q * ulp
    if out >= Fraction(2) ** (emax + 1):
        raise OverflowError(float(v))
    return sign * out


def rn32(v: Fraction) -> Fraction:
    return round_ieee(v, 24, -126, 127)


def rn16(v: Fraction) -> Fraction:
    return round_ieee(v, 11, -14, 15)


def rne_int(v: Fraction) -> int:
    q = v.numerator // v.denominator
    rem = v - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return q


def emulate_group_fp32(vals):
    """One group through the quantiser's steps, each one correctly rounded
    IEEE operation on exact rationals: span = fl32(hi - lo), scale =
    fp16(fl32(span / 15)), min = fp16(lo) (a zero minimum of either sign is
    the rational 0, i.e. +0), code = clamp(rne(fl32(fl32(w - min) / scale))),
    code 0 where the stored scale is 0."""
    lo, hi = min(vals), max(vals)
    S = rn16(rn32(rn32(hi - lo) / 15))
    M = rn16(lo)
    if S == 0:
        return [0] * len(vals), S, M
    return [min(15, max(0, rne_int(rn32(rn32(w - M) / S)))) for w in vals], S, M


def emulate_group_exact(vals, S, M):
    """The same codes from the exact quotient (w - M) / S, no fp32 rounding."""
    return [min(15, max(0, rne_int((w - M) / S))) for w in vals]


def half_code_tie_rows(rng, n_rows: int) -> np.ndarray:
    """float32 [n_rows][1024]: groups whose values sit on and within two fp32
    ulps of the half-integers that separate codes.

    Each group gets an fp16 scale S (dyadic in some rows, arbitrary in the
    others) and an fp16 minimum M; values 0 and 1 are M and M + 15 S, so the
    stored scale and minimum are S and M; the other 126 are the fp32 numbers
    nearest to M + (c + 1/2) S for random c, moved by -2..2 ulps.  Here the
    rounding of w - M and of the quotient decides codes: exact arithmetic
    picks another code for some of them."""
    k = 1024
    W = np.empty((n_rows, k), np.float32)
    for r in range(n_rows):
        for j in range(k // 128):
            if r % 2 == 0:
                S = Fraction(2) ** -int(rng.integers(3, 12))
                M = Fraction(-int(rng.integers(0, 257)), 128)
            else:
                S = Fraction(float(np.float16(rng.uniform(0.001, 0.05))))
                M = -Fraction(float(np.float16(rng.uniform(0.0, 0.3))))
            vals = [M, M + 15 * S]
            for _ in range(126):
                c = int(rng.integers(0, 15))
                w = np.float32(float(rn32(M + (c + Fraction(1, 2)) * S)))
                for _ in range(abs(int(rng.integers(-2, 3)))):
                    w = np.nextafter(w, np.float32(np.inf) if rng.random() < 0.5 else np.float32(-np.inf))
                vals.append(Fraction(float(w)))
            for t, v in enumerate(vals):
                W[r, 128 * j + t] = float(v)
                assert Fraction(float(W[r, 128 * j + t])) == v
    return W


def pin_fp32_decision_steps(orc):
    """Codes, scales and minimums equal a step-by-step emulation of the
    stated fp32 operations in exact rational arithmetic, on groups built
    around the code boundaries.  The data must also separate fp32 decisions
    from exact ones (else it could not tell them apart): checked first."""
    rng = np.random.Generator(np.random.PCG64(34))
    W = half_code_tie_rows(rng, 6)
    c, s, m = orc.quantize(W)
    n, k = W.shape
    differ = 0
    for r in range(n):
        for j in range(k // 128):
            vals = [fr(v) for v in W[r, 128 * j:128 * (j + 1)]]
            codes, S, M = emulate_group_fp32(vals)
            differ += sum(a != b for a, b in zip(codes, emulate_group_exact(vals, S, M)))
            assert fr(s[r, j]) == S and fr(m[r, j]) == M, (r, j)
            assert list(c[r, 128 * j:128 * (j + 1)]) == codes, (r, j)
    assert differ > 0, "tie set does not separate fp32 from exact decisions"


def pin_signed_zero_minimum(orc):
    """The minimum of a group that holds -0 (and maybe +0) is the rational
    zero, whose sign depends on the order of comparisons: it is stored as +0
    (bits 0x0000) whatever the order."""
    W = np.zeros((1, 512), np.float32)
    pos = np.linspace(0.01, 0.5, 128).astype(np.float32)
    W[0, :128] = pos
    W[0, 0] = -0.0                              # -0 first, positives after
    W[0, 128:256] = pos
    W[0, 255] = -0.0                            # -0 last
    W[0, 256:384] = pos
    W[0, 256], W[0, 257] = -0.0, 0.0            # both signs
    W[0, 384:] = pos
    W[0, 384], W[0, 511] = 0.0, -0.0
    c, s, m = orc.quantize(W)
    assert list(m.view(np.uint16)[0]) == [0, 0, 0, 0]
    for j in range(4):
        vals = [fr(v) for v in W[0, 128 * j:128 * (j + 1)]]
        codes, S, _ = emulate_group_fp32(vals)
        assert fr(s[0, j]) == S and list(c[0, 128 * j:128 * (j + 1)]) == codes


PINS = [
    pin_exact_round_trip,
    pin_best_code_brute_force,
    pin_reconstruction_bound,
    pin_degenerate_groups,
    pin_export_bytes,
    pin_fp32_decision_steps,
    pin_signed_zero_minimum,
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


def _standard(grp, n, k, top=15, rnd=np.rint, group_of=128, use_stored=True, min_round=None, clamp=True,
              wide=np.float32):
    g_n = k // group_of
    grp = grp.reshape(n, g_n, group_of).astype(wide)
    lo, hi = grp.min(axis=2), grp.max(axis=2)
    s32 = (hi - lo) / wide(top)
    scales = s32.astype(np.float16)
    mins = (lo + wide(0)).astype(np.float16) if min_round is None else min_round(lo)
    s = (scales.astype(wide) if use_stored else s32)[:, :, None]
    m = (mins.astype(wide) if use_stored else lo)[:, :, None]
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
    "decisions_in_fp64": _replace_quantize(lambda grp, n, k: _standard(grp, n, k, wide=np.float64)),
    "min_keeps_sign_of_zero": _replace_quantize(
        lambda grp, n, k: _standard(grp, n, k, min_round=lambda lo: lo.astype(np.float16))),
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
