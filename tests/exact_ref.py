"""Independent exact references used to pin the oracle.

Everything here is brute force in exact rational arithmetic (fractions) over
value tables that come from the pages (tests/golden) or from a library decode
(torch's float8 types), never from the oracle or the HIP library.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_pairs(name: str):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out


def golden_kv(name: str) -> dict:
    return {p[0]: p[1:] for p in read_pairs(name)}


def e2m1_table():
    """code -> value from the pages' value set."""
    return {int(c): float(v) for c, v in read_pairs("e2m1_values.txt")}


def e4m3_lib_values():
    """all 256 E4M3 bit patterns decoded by torch (OCP e4m3fn)."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def e8m0_lib_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().numpy().astype(np.float64)


E2M1_POS = [(c, Fraction(v)) for c, v in sorted(e2m1_table().items()) if c < 8]


def exact_rtn(x: float, s: float, g: float) -> int:
    """Nearest E2M1 magnitude to |x|/(s g); tie -> even code (mantissa bit 0);
    saturate; zero magnitude -> +0; s == 0 -> 0.  Brute force over the table."""
    if s == 0:
        return 0
    y = abs(Fraction(x)) / (Fraction(s) * Fraction(g))
    best = None
    for c, v in E2M1_POS:
        d = abs(y - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    c = best[1]
    if c == 0:
        return 0
    return c | (8 if x < 0 else 0)


def exact_rtn_special(x: float, s: float, g: float, v: float) -> int:
    """Nearest of the 15 distinct standard values and v (code 8), by brute
    force over all 16.  If a standard value is among the nearest it wins (ties
    among standard values follow exact_rtn); otherwise v."""
    if s == 0:
        return 0
    y = Fraction(x) / (Fraction(s) * Fraction(g))
    dists = [abs(y - m) for _, m in E2M1_POS] + [abs(y + m) for _, m in E2M1_POS if m]
    dmin = min(dists)
    if abs(y - Fraction(v)) < dmin:
        return 8
    return exact_rtn(x, s, g)


def exact_nearest_scale(values: list, y: Fraction) -> int:
    """index of the nearest value (values sorted ascending, index = code);
    ties to the even code; past the last value saturates."""
    best = None
    for k, v in enumerate(values):
        d = abs(y - Fraction(v))
        if best is None or d < best[0] or (d == best[0] and k % 2 == 0):
            best = (d, k)
    return best[1]


def exact_sse(x, vals) -> Fraction:
    return sum((Fraction(float(a)) - Fraction(b)) ** 2 for a, b in zip(x, vals))
