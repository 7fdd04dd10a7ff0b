"""Pins of the oracle's rounding primitives: scale rounding against torch's
E4M3 cast and exact rational brute force; E2M1 round-to-nearest against
exact brute force over the pages' value set, exhaustively over bf16."""
from fractions import Fraction

import numpy as np
import torch

import oracle as O
from tests.exact_ref import exact_nearest_scale, exact_rtn, exact_rtn_special


def _e4m3_values():
    return [O.e4m3_value(k) for k in range(127)]


def test_round_scale_matches_torch_cast():
    # torch's fp32 -> float8_e4m3fn cast is round-to-nearest-even on [0, 448]
    rng = np.random.default_rng(0)
    vals = _e4m3_values()
    mids = [0.5 * (a + b) for a, b in zip(vals, vals[1:])]
    ys = np.concatenate([
        np.float32(vals), np.float32(mids), rng.uniform(0, 448, 4000).astype(np.float32),
        np.exp2(rng.uniform(-12, 8.8, 4000)).astype(np.float32)])
    ys = ys[ys <= 448]
    ref = torch.from_numpy(ys).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for y, r in zip(ys, ref):
        assert O.round_scale(O.SF_E4M3, float(y), 1.0, 1.0) == int(r), y


def test_round_scale_saturates():
    for y in (448.0, 449.0, 464.0, 480.0, 1e6, 3e38):
        assert O.round_scale(O.SF_E4M3, y, 1.0, 1.0) == 126
        assert O.round_scale(O.SF_E3M3, y, 1.0, 1.0) == (63 if y >= 30 else None)


def test_round_scale_exact_with_T_and_g():
    # a / (T g) decided exactly, including constructed ties
    rng = np.random.default_rng(1)
    for sf, valf, kmax in ((O.SF_E4M3, O.e4m3_value, 126), (O.SF_E3M3, O.e3m3_value, 63)):
        vals = [valf(k) for k in range(kmax + 1)]
        for _ in range(600):
            T = float(rng.choice([4.0, 6.0]))
            g = float(np.float32(np.exp2(rng.uniform(-20, 5)) * rng.uniform(1, 2)))
            if rng.random() < 0.3:  # tie: a = midpoint * T * g when exact in fp32
                k = int(rng.integers(0, kmax))
                a = 0.5 * (vals[k] + vals[k + 1]) * T * g
                if float(np.float32(a)) != a:
                    continue
            else:
                a = float(np.float32(vals[int(rng.integers(0, kmax + 1))] * T * g * rng.uniform(0.9, 1.1)))
            y = Fraction(a) / (Fraction(T) * Fraction(g))
            assert O.round_scale(sf, a, T, g) == exact_nearest_scale(vals, y), (sf, a, T, g)


def test_rtn_exhaustive_bf16_unit_scale():
    # every finite bf16 value (2^16 patterns minus NaN/Inf) at s = g = 1
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x)]
    # the decision only depends on |x| against 7 thresholds; brute force is slow
    # in Fractions, so check the distinct magnitudes and mirror the sign
    mags = np.unique(np.abs(x))
    for m in mags:
        r = exact_rtn(float(m), 1.0, 1.0)
        assert O.rtn(float(m), 1.0, 1.0) == r, m
        rn = exact_rtn(-float(m), 1.0, 1.0)
        assert O.rtn(-float(m), 1.0, 1.0) == rn, -m


def test_rtn_random_scales_and_ties():
    rng = np.random.default_rng(2)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for _ in range(3000):
        k = int(rng.integers(0, 127))
        s = O.e4m3_value(k)
        g = 1.0 if rng.random() < 0.5 else float(np.float32(rng.uniform(0.5, 2.0) * 2.0 ** rng.integers(-30, 10)))
        if rng.random() < 0.4:
            x = float(np.float32(rng.choice(mids) * s * g))
            x = -x if rng.random() < 0.5 else x
        else:
            x = float(np.float32(rng.standard_normal() * 4 * s * g))
        assert O.rtn(x, s, g) == exact_rtn(x, s, g), (x, s, g)


def test_rtn_zero_scale_and_signed_zero():
    assert O.rtn(3.0, 0.0, 1.0) == 0
    assert O.rtn(-0.0, 1.0, 1.0) == 0
    assert O.rtn(-0.1, 1.0, 1.0) == 0          # rounds to zero magnitude: +0
    assert O.rtn(-0.26, 1.0, 1.0) == 0x9


def test_rtn_special_brute_force():
    rng = np.random.default_rng(3)
    for v in (5.0, -5.0, 2.5, -2.5, 7.5, -3.5):
        for _ in range(800):
            s = O.e4m3_value(int(rng.integers(1, 127)))
            g = 1.0
            if rng.random() < 0.3:
                base = rng.choice([v, 4.0, 6.0, -4.0, -6.0, 2.0, 3.0])
                x = float(np.float32(0.5 * (base + v) * s))  # midpoints with v
            else:
                x = float(np.float32(rng.uniform(-8, 8) * s))
            assert O.rtn_special(x, s, g, v) == exact_rtn_special(x, s, g, v), (x, s, v)


def test_block_sse_exact_cases():
    # a block that is exactly representable has zero error
    s = O.e4m3_value(60)
    vals = np.array([6, 3, -1.5, 0.5, 0, 4, -6, 1] * 2, np.float64) * s
    x = vals.astype(np.float32)
    codes = [O.rtn(float(a), s, 1.0) for a in x]
    assert O.block_sse(x, codes, s, 1.0) == 0.0
    # binary32 sum of squares stays within the rounding bound of the exact value
    rng = np.random.default_rng(4)
    for _ in range(200):
        x = rng.standard_normal(16).astype(np.float32)
        k = O.round_scale(O.SF_E4M3, float(np.abs(x).max()), 6.0, 1.0)
        s = O.e4m3_value(k)
        codes = [O.rtn(float(a), s, 1.0) for a in x]
        exact = sum((Fraction(float(a)) - Fraction(O.e2m1_value(c)) * Fraction(s)) ** 2 for a, c in zip(x, codes))
        got = O.block_sse(x, codes, s, 1.0)
        assert abs(Fraction(got) - exact) <= exact * Fraction(16, 2 ** 23)
