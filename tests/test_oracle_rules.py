"""Pins of the oracle's scale-selection rules ("Finer is Better" Method 2,
RaZeR 2.1-2.2, MACaQ section 1) by constructed cases, exact brute force on
tiny blocks, and the invariants the pages state."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from tests.exact_ref import E2M1_POS, golden_kv

SPECIAL = (5.0, -5.0, 2.5, -2.5)


def _q(x, fmt="nvfp4", block=16, rule=O.ABSMAX, gmode=O.G_NONE, g=None, special=None):
    return O.quantize(np.ascontiguousarray(x, np.float32), fmt, block, rule, gmode, special=special, g=g)


def _exact_block_sse(x, codes, s, v=None):
    tot = Fraction(0)
    for a, c in zip(x, codes):
        val = Fraction(v) if (v is not None and c == 8) else Fraction(O.e2m1_value(int(c)))
        tot += (Fraction(float(a)) - val * Fraction(s)) ** 2
    return tot


def _codes(codes_row, n):
    return [(int(codes_row[j // 2]) >> (4 * (j & 1))) & 15 for j in range(n)]


def _block_sse_from(x, codes, scales, fmt, block, g=1.0, special=None):
    """per-block binary32 error of a quantized tensor, with g = 1"""
    rows, cols = x.shape
    out = np.empty((rows, cols // block), np.float32)
    for r in range(rows):
        cr = _codes(codes[r], cols)
        for b in range(cols // block):
            sb = int(scales[r, b])
            if fmt == "nvfp4":
                s, v = O.e4m3_value(sb), None
            elif fmt == "razer_a":
                s, v = O.e4m3_value(sb & 0x7F), (-5.0 if sb & 0x80 else 5.0)
            else:
                s, v = O.e3m3_value(sb & 0x3F), special[sb >> 6]
            out[r, b] = O.block_sse(x[r, b * block:(b + 1) * block], cr[b * block:(b + 1) * block], s, g, v)
    return out


# ---------------------------------------------------------------- R1 abs-max
def test_absmax_constructed_block_is_exact():
    # "Finer is Better" Method 2, abs-max: the block max lands on 6 * scale
    s = O.e4m3_value(83)
    x = (np.array([6, 3, -1.5, 0.5, 0, 4, -6, 1, 2, -3, 1.5, -0.5, 0, 6, -4, 2]) * s)[None].astype(np.float32)
    codes, scales, g = _q(x)
    assert scales[0, 0] == 83 and g == 1.0
    assert np.array_equal(O.dequantize(codes, scales, "nvfp4", 16), x)


def test_absmax_scale_is_nearest_e4m3_to_max_over_6():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((64, 64)) * np.exp2(rng.uniform(-12, 6, (64, 1)))).astype(np.float32)
    vals = [O.e4m3_value(k) for k in range(127)]
    _, scales, _ = _q(x)
    for r in range(64):
        for b in range(4):
            a = Fraction(float(np.abs(x[r, 16 * b:16 * b + 16]).max()))
            y = a / 6
            d = [abs(y - Fraction(v)) for v in vals]
            k = int(scales[r, b])
            assert d[k] == min(d)


# ---------------------------------------------------------------- R2 prevent-zero
def test_prevent_zero_removes_zero_scales_and_region_a():
    # "Finer is Better" Method 2 prevent-zero and region A: with g = 1, a block
    # whose max is in (0.25 * 2^-9, 6 * 2^-10] has scale 0 (all codes zero)
    # under abs-max and a nonzero code under prevent-zero.
    rng = np.random.default_rng(1)
    amax = np.exp2(rng.uniform(np.log2(0.26 * 2 ** -9), np.log2(6 * 2 ** -10), 200))
    x = rng.uniform(-1, 1, (200, 16)) * amax[:, None]
    x[np.arange(200), rng.integers(0, 16, 200)] = amax
    x = x.astype(np.float32)
    c1, s1, _ = _q(x)
    c2, s2, _ = _q(x, rule=O.ABSMAX | O.PREVENT_ZERO)
    assert np.all(s1 == 0) and np.all(c1 == 0)
    assert np.all(s2 == 1) and np.all(c2.reshape(200, -1).max(axis=1) > 0)
    e1 = _block_sse_from(x, c1, s1, "nvfp4", 16)
    e2 = _block_sse_from(x, c2, s2, "nvfp4", 16)
    assert np.all(e2 < e1)


def test_prevent_zero_never_worse_and_no_zero_codes():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 64)) * np.exp2(rng.uniform(-16, 2, (64, 1)))).astype(np.float32)
    for rule in (O.ABSMAX, O.FOUR_OVER_SIX):
        c1, s1, _ = _q(x, rule=rule)
        c2, s2, _ = _q(x, rule=rule | O.PREVENT_ZERO)
        assert np.all(s2 > 0)
        assert np.all(_block_sse_from(x, c2, s2, "nvfp4", 16) <= _block_sse_from(x, c1, s1, "nvfp4", 16))
    c, s, _ = _q(x, "razer_w", rule=O.ABSMAX | O.PREVENT_ZERO, special=SPECIAL)
    assert np.all((s & 0x3F) > 0)


# ---------------------------------------------------------------- R3 4-over-6
def test_four_over_six_constructed_pick():
    # a flat block {4,4,...}*s: mapping the max to 4 is exact, to 6 is not
    x = np.full((1, 16), 4.0, np.float32)
    codes, scales, _ = _q(x, rule=O.FOUR_OVER_SIX)
    assert O.e4m3_value(int(scales[0, 0])) == 1.0
    assert np.array_equal(O.dequantize(codes, scales, "nvfp4", 16), x)
    # a block with values on the 6-grid keeps 6
    s = O.e4m3_value(70)
    y = (np.array([6, 3, 1.5, 0.5] * 4) * s)[None].astype(np.float32)
    _, sc, _ = _q(y, rule=O.FOUR_OVER_SIX)
    assert sc[0, 0] == 70


def test_four_over_six_picks_the_lower_exact_error():
    # both candidates recomputed in exact arithmetic: the pick is never worse
    # than the other beyond binary32 rounding of the block sum
    rng = np.random.default_rng(3)
    x = rng.standard_normal((48, 64)).astype(np.float32)
    codes, scales, _ = _q(x, rule=O.FOUR_OVER_SIX)
    for r in range(48):
        cr = _codes(codes[r], 64)
        for b in range(4):
            xb = x[r, 16 * b:16 * b + 16]
            a = float(np.abs(xb).max())
            k6 = O.round_scale(O.SF_E4M3, a, 6.0, 1.0)
            k4 = O.round_scale(O.SF_E4M3, a, 4.0, 1.0)
            k = int(scales[r, b])
            assert k in (k6, k4)
            other = k4 if k == k6 else k6
            s_o = O.e4m3_value(other)
            e_pick = _exact_block_sse(xb, cr[16 * b:16 * b + 16], O.e4m3_value(k))
            e_other = _exact_block_sse(xb, [O.rtn(float(t), s_o, 1.0) for t in xb], s_o)
            assert e_pick <= e_other * (1 + Fraction(64, 2 ** 24))
    # never worse than abs-max per block (binary32, exact inequality)
    c1, s1, _ = _q(x)
    assert np.all(_block_sse_from(x, codes, scales, "nvfp4", 16) <= _block_sse_from(x, c1, s1, "nvfp4", 16))


# ---------------------------------------------------------------- R4 brute force
def test_brute_force_is_global_minimum_on_tiny_blocks():
    # "Finer is Better" Method 2 brute-force: for B = 4 enumerate every positive
    # E4M3 scale and every tuple of the 15 distinct values (exactly); the
    # oracle's pick must reach the exact minimum up to binary32 rounding.
    rng = np.random.default_rng(4)
    scales = [Fraction(O.e4m3_value(k)) for k in range(1, 127)]
    values = sorted({Fraction(m) for _, m in E2M1_POS} | {-Fraction(m) for _, m in E2M1_POS})
    assert len(values) == 15
    for trial in range(12):
        x = (rng.standard_normal(4) * 2.0 ** rng.integers(-6, 4)).astype(np.float32)
        xf = [Fraction(float(t)) for t in x]
        best = None
        for s in scales:
            # all 15^4 tuples: the sum separates, so the minimum over tuples is
            # the sum of per-element minima; enumerate tuples anyway on 1 scale
            tot = sum(min((xi - v * s) ** 2 for v in values) for xi in xf)
            best = tot if best is None else min(best, tot)
        codes, sc, _ = _q(x[None], block=4, rule=O.BRUTE)
        got = _exact_block_sse(x, _codes(codes[0], 4), O.e4m3_value(int(sc[0, 0])))
        assert got <= best * (1 + Fraction(8, 2 ** 24)), trial
    # literal enumeration of all 15^4 tuples for one scale confirms separability
    s = Fraction(O.e4m3_value(60))
    xf = [Fraction(float(t)) for t in (rng.standard_normal(4) * float(s) * 3).astype(np.float32)]
    brute = min(sum((xi - v * s) ** 2 for xi, v in zip(xf, tup)) for tup in itertools.product(values, repeat=4))
    assert brute == sum(min((xi - v * s) ** 2 for v in values) for xi in xf)


def test_brute_force_dominates_other_rules():
    rng = np.random.default_rng(5)
    x = (rng.standard_t(3, (32, 64))).astype(np.float32)
    cb, sb, _ = _q(x, rule=O.BRUTE)
    eb = _block_sse_from(x, cb, sb, "nvfp4", 16)
    for rule in (O.ABSMAX, O.ABSMAX | O.PREVENT_ZERO, O.FOUR_OVER_SIX, O.FOUR_OVER_SIX | O.PREVENT_ZERO):
        c, s, _ = _q(x, rule=rule)
        assert np.all(eb <= _block_sse_from(x, c, s, "nvfp4", 16)), rule


def test_brute_force_error_non_increasing_as_blocks_shrink():
    # "Finer is Better" findings: with the ideal scale the MSE improves as the
    # block shrinks.  For nested blocks (a 2B block splits into two B blocks)
    # the binary32 tree makes this an exact inequality per block; the tensor
    # MSE is then non-increasing for 32 -> 16 -> 8 -> 4 and strictly
    # decreasing on normal samples.
    rng = np.random.default_rng(6)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    errs = {}
    for B in (32, 16, 8, 4):
        c, s, _ = _q(x, block=B, rule=O.BRUTE)
        errs[B] = _block_sse_from(x, c, s, "nvfp4", B)
    for B in (32, 16, 8):
        child = errs[B // 2]
        pair = (child[:, 0::2] + child[:, 1::2]).astype(np.float32)
        assert np.all(errs[B] >= pair)
    mse = {B: float(np.sum(errs[B].astype(np.float64))) for B in errs}
    assert mse[32] > mse[16] > mse[8] > mse[4]


# ---------------------------------------------------------------- RaZeR
def test_razer_a_constructed_picks():
    # RaZeR 2.2: a block holding 5*s next to its max 6*s is exact with +5
    s = O.e4m3_value(72)
    base = np.array([6, 5, 1, -0.5, 0, 3, 2, 4, 1.5, 0.5, -1, -2, 5, 0, 0, 1]) * s
    x = base[None].astype(np.float32)
    codes, scales, _ = _q(x, "razer_a")
    assert scales[0, 0] == 72  # pick bit 0 -> +5
    assert np.array_equal(O.dequantize(codes, scales, "razer_a", 16), x)
    codes, scales, _ = _q(-x, "razer_a")
    assert scales[0, 0] == 0x80 | 72  # pick bit 1 -> -5
    assert np.array_equal(O.dequantize(codes, scales, "razer_a", 16), -x)
    pair = [float(v) for v in golden_kv("razer_special.txt")["activation_pair"]]
    assert pair == [5.0, -5.0]


def test_razer_never_worse_than_plain_at_same_scale():
    # the element set is a superset of the standard one, so each block's error
    # is at most the plain encoding's at the same scale
    rng = np.random.default_rng(7)
    x = rng.standard_t(4, (32, 64)).astype(np.float32)
    ca, sa, _ = _q(x, "razer_a")
    cn, sn, _ = _q(x, "nvfp4")
    assert np.array_equal(sa & 0x7F, sn)
    assert np.all(_block_sse_from(x, ca, sa, "razer_a", 16) <= _block_sse_from(x, cn, sn, "nvfp4", 16))
    cw, sw, _ = _q(x, "razer_w", special=SPECIAL)
    k = sw & 0x3F
    # the chosen pick is the argmin over the four special values
    for r in range(32):
        cr = _codes(cw[r], 64)
        for b in range(4):
            xb = x[r, 16 * b:16 * b + 16]
            s = O.e3m3_value(int(k[r, b]))
            errs = [O.block_sse(xb, [O.rtn_special(float(t), s, 1.0, v) for t in xb], s, 1.0, v) for v in SPECIAL]
            p = int(sw[r, b]) >> 6
            assert errs[p] == min(errs) and errs.index(min(errs)) == p
            assert cr[16 * b:16 * b + 16] == [O.rtn_special(float(t), s, 1.0, SPECIAL[p]) for t in xb]


def test_razer_special_values_are_half_multiples():
    gran = float(golden_kv("razer_special.txt")["granularity"][0])
    for v in SPECIAL:
        assert (v / gran) == int(v / gran)


# ---------------------------------------------------------------- MXFP4
def test_mxfp4_shared_exponent_and_saturation():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((32, 128)) * np.exp2(rng.uniform(-30, 30, (32, 1)))).astype(np.float32)
    codes, scales, _ = _q(x, "mxfp4", 32)
    for r in range(32):
        cr = _codes(codes[r], 128)
        for b in range(4):
            xb = x[r, 32 * b:32 * b + 32]
            a = Fraction(float(np.abs(xb).max()))
            E = int(scales[r, b]) - 127
            assert Fraction(4) <= a / Fraction(2) ** E < 8      # max lands in [4, 8)
            for t, c in zip(xb, cr[32 * b:32 * b + 32]):
                if abs(Fraction(float(t))) / Fraction(2) ** E > 6:
                    assert c & 7 == 7                              # saturates at 6
    z = np.zeros((1, 32), np.float32)
    c, s, _ = _q(z, "mxfp4", 32)
    assert s[0, 0] == 0 and np.all(c == 0)


# ---------------------------------------------------------------- global scale
@pytest.mark.parametrize("fmt,top", [("nvfp4", 126), ("razer_w", 63)])
def test_auto_global_scale(fmt, top):
    # "Finer is Better" Method 2 hierarchical: g * 6 * max-scale = tensor amax
    # (to binary32 rounding) and the block holding the max gets the top scale
    rng = np.random.default_rng(9)
    x = (rng.standard_t(3, (64, 64)) * 1e-3).astype(np.float32)
    special = SPECIAL if fmt == "razer_w" else None
    _, scales, g = _q(x, fmt, gmode=O.G_AUTO, special=special)
    amax = float(np.abs(x).max())
    denom = 2688.0 if fmt == "nvfp4" else 180.0
    assert abs(g * denom - amax) <= np.spacing(np.float32(amax)) * 1.0
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    k = int(scales[r, c // 16]) & (0x7F if fmt == "nvfp4" else 0x3F)
    assert k == top
    _, _, g0 = _q(np.zeros((2, 16), np.float32), fmt, gmode=O.G_AUTO, special=special)
    assert g0 == 1.0


def test_given_global_scale_equals_auto_when_same_value():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    c1, s1, g = _q(x, rule=O.FOUR_OVER_SIX, gmode=O.G_AUTO)
    c2, s2, g2 = _q(x, rule=O.FOUR_OVER_SIX, gmode=O.G_GIVEN, g=g)
    assert g2 == g and np.array_equal(c1, c2) and np.array_equal(s1, s2)
