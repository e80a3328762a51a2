"""Loader for tests/golden/known_answers.txt (hand-derived known answers).

Produces, per case, either unpacked codes (specs "all" and "groups") or raw
packed bytes (spec "bytes"), plus fp16 scales/mins, the fp16 activation
vector and the expected output of the single row.  The loader does no
packing or dequantisation itself.
"""
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "known_answers.txt")


@dataclass
class Case:
    name: str
    k: int
    codes: Optional[np.ndarray]    # uint8 [1][K] or None
    packed: Optional[np.ndarray]   # uint8 [1][K/2] or None
    scales: np.ndarray             # float16 [1][G]
    mins: np.ndarray               # float16 [1][G]
    x: np.ndarray                  # float16 [K]
    expected: float


def _floats16(spec, g):
    vals = [float(v) for v in spec.split(",")]
    if len(vals) == 1:
        vals = vals * g
    arr = np.array(vals, dtype=np.float64)
    a16 = arr.astype(np.float16)
    assert np.array_equal(a16.astype(np.float64), arr), f"{spec} not fp16-exact"
    return a16.reshape(1, g)


def load():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, k, cspec, sspec, mspec, xspec, exp = [p.strip() for p in line.split("|")]
            k = int(k)
            g = k // 128
            codes = packed = None
            kind, _, body = cspec.partition(":")
            if kind == "all":
                codes = np.full((1, k), int(body), dtype=np.uint8)
            elif kind == "groups":
                cg = [int(v) for v in body.split(",")]
                assert len(cg) == g
                codes = np.repeat(np.array(cg, dtype=np.uint8), 128).reshape(1, k)
            elif kind == "bytes":
                packed = np.zeros((1, k // 2), dtype=np.uint8)
                bs = [int(v, 16) for v in body.split(",")]
                packed[0, : len(bs)] = bs
            else:
                raise ValueError(cspec)
            xkind, _, xbody = xspec.partition(":")
            if xkind == "all":
                x = np.full(k, float(xbody), dtype=np.float16)
            elif xkind == "onehot":
                x = np.zeros(k, dtype=np.float16)
                x[int(xbody)] = 1.0
            else:
                raise ValueError(xspec)
            cases.append(Case(name, k, codes, packed, _floats16(sspec, g), _floats16(mspec, g), x, float(exp)))
    return cases
