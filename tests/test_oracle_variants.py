"""Pins of the oracle's scale-format variants: UE5M3 block scales and the
rules over them ("Finer is Better", findings and claims: the wide-exponent
UE5M3 against E4M3 + 4-over-6 + hierarchical scaling), the size-16
block-Hadamard, and the MXFP4 exponent-offset search by plain block error
(the MACaQ review, section 1, screens the standard exponent and offsets +1
and -1; here with a unit Hessian).  Each is checked against something other
than the oracle: numpy's half-precision decoder, scipy's Hadamard matrix,
exact rational arithmetic, constructed blocks."""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import datagen
import oracle as O
from tests.exact_ref import E2M1_POS, exact_nearest_scale


# ---------------------------------------------------------------- UE5M3
def test_ue5m3_values_match_half_precision_layout():
    # with bias 15 and subnormals, UE5M3 code k has the bits of the
    # half-precision number k << 7 (3 mantissa bits on top of 10); exponent
    # field 31 is Inf/NaN there and ordinary values here
    v = [O.ue5m3_value(k) for k in range(256)]
    for k in range(248):
        assert v[k] == float(np.array([k << 7], np.uint16).view(np.float16)[0]), k
    for m in range(8):
        assert v[248 + m] == (1 + m / 8) * 2.0 ** 16
    assert all(b > a for a, b in zip(v, v[1:]))
    assert v[255] == 122880.0 and v[1] == 2.0 ** -17
    # a far wider range than E4M3 (448 / 2^-9)
    assert v[255] / v[1] > 2 ** 33 > O.e4m3_value(126) / O.e4m3_value(1)


def test_ue5m3_round_scale_exact():
    vals = [O.ue5m3_value(k) for k in range(256)]
    rng = np.random.default_rng(11)
    ys = list(np.exp2(rng.uniform(-20, 18, 300)))
    ys += [0.5 * (vals[k] + vals[k + 1]) for k in range(0, 255, 7)]  # exact midpoints: ties to the even code
    ys += [vals[255] * 1.5, 0.0, 2.0 ** -19]
    for T in (6.0, 4.0):
        for y in ys:
            a = float(np.float32(y * T))
            k = O.round_scale(O.SF_UE5M3, a, T, 1.0)
            assert k == exact_nearest_scale(vals, Fraction(a) / Fraction(T)), (a, T)


def test_ue5m3_absmax_constructed_block_and_no_global_needed():
    s = O.ue5m3_value(201)
    x = (np.array([6, 3, -1.5, 0.5, 0, 4, -6, 1, 2, -3, 1.5, -0.5, 0, 6, -4, 2]) * s)[None].astype(np.float32)
    codes, scales, g = O.quantize(x, "ue5m3", 16, O.ABSMAX, O.G_NONE)
    assert scales[0, 0] == 201 and g == 1.0
    assert np.array_equal(O.dequantize(codes, scales, "ue5m3", 16), x)
    # a block far below E4M3's range without a global scale: abs-max E4M3
    # gives a zero scale (all codes 0), UE5M3 keeps the block
    tiny = (datagen.normal((1, 16), 12) * 2.0 ** -14).astype(np.float32)
    _, se, _ = O.quantize(tiny, "nvfp4", 16, O.ABSMAX, O.G_NONE)
    cu, su, _ = O.quantize(tiny, "ue5m3", 16, O.ABSMAX, O.G_NONE)
    assert se[0, 0] == 0 and su[0, 0] > 0 and np.any(cu != 0)


def _exact_sse(x, codes, s):
    return sum((Fraction(float(a)) - Fraction(O.e2m1_value(int(c))) * Fraction(s)) ** 2 for a, c in zip(x, codes))


def _codes(row, n):
    return [(int(row[j // 2]) >> (4 * (j & 1))) & 15 for j in range(n)]


def test_ue5m3_four_over_six_is_argmin_and_brute_is_global():
    rng = np.random.default_rng(12)
    x = (rng.standard_t(3, (24, 16)) * np.exp2(rng.uniform(-10, 10, (24, 1)))).astype(np.float32)
    c1, s1, _ = O.quantize(x, "ue5m3", 16, O.ABSMAX, O.G_NONE)
    c3, s3, _ = O.quantize(x, "ue5m3", 16, O.FOUR_OVER_SIX, O.G_NONE)
    for r in range(24):
        a = Fraction(float(np.abs(x[r]).max()))
        k6 = exact_nearest_scale([O.ue5m3_value(k) for k in range(256)], a / 6)
        k4 = exact_nearest_scale([O.ue5m3_value(k) for k in range(256)], a / 4)
        assert s1[r, 0] == k6
        e6 = _exact_sse(x[r], [O.rtn(float(v), O.ue5m3_value(k6), 1.0) for v in x[r]], O.ue5m3_value(k6))
        e4 = _exact_sse(x[r], [O.rtn(float(v), O.ue5m3_value(k4), 1.0) for v in x[r]], O.ue5m3_value(k4))
        if abs(e6 - e4) > Fraction(1, 10 ** 5) * max(e6, e4):   # clear of FP32 rounding
            assert s3[r, 0] == (k4 if e4 < e6 else k6)
    # brute force over all 255 positive scales on blocks of 4: the pick is the
    # exact minimum over every scale and every code tuple (separable per element)
    xb = (rng.standard_normal((12, 4)) * np.exp2(rng.uniform(-8, 8, (12, 1)))).astype(np.float32)
    cb, sb, _ = O.quantize(xb, "ue5m3", 4, O.BRUTE, O.G_NONE)
    for r in range(12):
        best = None
        for k in range(1, 256):
            s = Fraction(O.ue5m3_value(k))
            tot = sum(min((Fraction(float(v)) - sgn * m * s) ** 2 for _, m in E2M1_POS for sgn in (1, -1))
                      for v in xb[r])
            best = tot if best is None or tot < best else best
        got = _exact_sse(xb[r], _codes(cb[r], 4), O.ue5m3_value(int(sb[r, 0])))
        assert got <= best * (1 + Fraction(1, 10 ** 5))


# ---------------------------------------------------------------- Hadamard 16
def test_block_hadamard_16():
    H = scipy.linalg.hadamard(16).astype(np.float64)
    eye = np.eye(16, dtype=np.float32)
    Y = O.transform(eye, None, 16)
    assert np.array_equal(Y.astype(np.float64), H.T * 0.25)
    assert np.array_equal((4 * Y.astype(np.float64)) @ (4 * Y.astype(np.float64)).T, 16 * np.eye(16))
    rng = np.random.default_rng(13)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    y = O.transform(x, None, 16)
    ref = np.concatenate([x[:, g:g + 16].astype(np.float64) @ (H / 4) for g in range(0, 64, 16)], axis=1)
    assert np.max(np.abs(y - ref)) <= 1e-5 * np.max(np.abs(ref))
    n0 = np.linalg.norm(x.astype(np.float64).reshape(6, 4, 16), axis=2)
    n1 = np.linalg.norm(y.astype(np.float64).reshape(6, 4, 16), axis=2)
    assert np.max(np.abs(n1 / n0 - 1)) < 1e-6
    # the rotation cancels in the product when both operands take it
    w = rng.standard_normal((5, 64)).astype(np.float32)
    prod = O.transform(x, None, 16).astype(np.float64) @ O.transform(w, None, 16).astype(np.float64).T
    assert np.max(np.abs(prod - x.astype(np.float64) @ w.astype(np.float64).T)) < 1e-4


# ---------------------------------------------------------------- MXFP4 exponent search
def _mx_block(E, vals):
    return (np.asarray(vals, np.float64) * 2.0 ** E).astype(np.float32)[None]


def test_expsearch_constructed_picks():
    E = -3
    # one element at 4 * 2^E sets the standard exponent E; 31 elements at
    # 0.75 * 2^E sit on an E2M1 midpoint at E but are exact at E - 1, where
    # the maximum saturates (8 -> 6): E - 1 wins
    x = _mx_block(E, [4.0] + [0.75] * 31)
    _, s_std, _ = O.quantize(x, "mxfp4", 32, O.ABSMAX)
    _, s_srch, _ = O.quantize(x, "mxfp4", 32, O.EXPSEARCH)
    assert s_std[0, 0] == E + 127 and s_srch[0, 0] == E - 1 + 127
    # every element at 7.5 * 2^E saturates to 6 at E, and is 3.75 -> 4 at E + 1
    x = _mx_block(E, [7.5] * 32)
    _, s_std, _ = O.quantize(x, "mxfp4", 32, O.ABSMAX)
    _, s_srch, _ = O.quantize(x, "mxfp4", 32, O.EXPSEARCH)
    assert s_std[0, 0] == E + 127 and s_srch[0, 0] == E + 1 + 127
    # exactly representable at E: the standard exponent stays (zero error);
    # an all-zero block keeps the standard exponent -127
    x = _mx_block(E, [4, -6, 3, 0.5] * 8)
    _, s_srch, _ = O.quantize(x, "mxfp4", 32, O.EXPSEARCH)
    assert s_srch[0, 0] == E + 127
    _, s0, _ = O.quantize(np.zeros((1, 32), np.float32), "mxfp4", 32, O.EXPSEARCH)
    assert s0[0, 0] == 0


def test_expsearch_is_the_exact_argmin_and_never_worse():
    rng = np.random.default_rng(14)
    x = (rng.standard_t(3, (40, 64)) * np.exp2(rng.uniform(-6, 6, (40, 1)))).astype(np.float32)
    c1, s1, _ = O.quantize(x, "mxfp4", 32, O.ABSMAX)
    c2, s2, _ = O.quantize(x, "mxfp4", 32, O.EXPSEARCH)
    changed = 0
    for r in range(40):
        for b in range(2):
            xb = x[r, 32 * b:32 * b + 32]
            E0 = int(s1[r, b]) - 127
            exact = {}
            for E in (E0, E0 + 1, E0 - 1):
                codes = [O.rtn(float(v), 2.0 ** E, 1.0) for v in xb]
                exact[E] = _exact_sse(xb, codes, 2.0 ** E)
            Eg = int(s2[r, b]) - 127
            assert Eg in exact
            # the oracle's FP32 error of its pick is not above the standard one
            f_std = O.block_sse(xb, _codes(c1[r], 64)[32 * b:32 * b + 32], 2.0 ** E0, 1.0)
            f_got = O.block_sse(xb, _codes(c2[r], 64)[32 * b:32 * b + 32], 2.0 ** Eg, 1.0)
            assert f_got <= f_std
            ordered = sorted(exact.values())
            if ordered[1] - ordered[0] > Fraction(1, 10 ** 5) * ordered[1]:
                assert exact[Eg] == ordered[0]
            changed += Eg != E0
    assert changed > 0   # the search does move some exponents on heavy-tailed data
