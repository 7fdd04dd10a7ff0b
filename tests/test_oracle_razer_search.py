"""Pins of the oracle's RaZeR weight-only matmul and offline special-value
search (RaZeR summary, sections 2.2 and 2.3), against what the pages and the
mathematics fix:

* the weight-only product equals numpy's binary64 product of the widened bf16
  activations and the decoded weight, and a constructed all-special weight
  gives a closed form;
* the pairs are the 28 pairs a < b of the 8 candidate magnitudes (multiples
  of 0.5 up to 7.5 that are not E2M1 magnitudes), in lexicographic order;
* every pair's error is recomputed in exact rational arithmetic from a
  separate Python encoder of RaZeR-W quantization, and matches to FP32
  rounding; the pick is the exact minimum where the margin is clear;
* a pair's error equals the summed block error of the oracle's own RaZeR-W
  quantization under that table (two different oracle paths);
* constructed weights whose blocks need +-5.5 and +-2.5 pick (2.5, 5.5)."""
from fractions import Fraction

import numpy as np

import datagen
import oracle as O

MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
CAND = [2.5, 3.5, 4.5, 5.0, 5.5, 6.5, 7.0, 7.5]


# ---------------------------------------------------------------- weight-only matmul
def _weight(N, K, seed, fmt, special):
    w = datagen.student_t((N, K), seed, 4.0) * np.float32(0.03)
    codes, scales, g = O.quantize(w, fmt, 16, O.ABSMAX, O.G_AUTO, special=special)
    return codes, scales, g


def test_w4a16_is_the_binary64_product_of_the_decoded_operands():
    for fmt, sp in (("nvfp4", None), ("razer_w", datagen.RAZER_SPECIAL)):
        M, N, K = 7, 11, 96
        codes, scales, g = _weight(N, K, 8100, fmt, sp)
        a = datagen.to_bf16_bits(datagen.normal((M, K), 8101))
        got = O.gemm_w4a16_rows(a, fmt, codes, scales, g, sp, N)
        A = datagen.bf16_bits_to_f32(a).astype(np.float64)
        W = O.decode(codes, scales, fmt, 16, special=sp)
        ref = (np.float64(g) * (A @ W.T)).astype(np.float32)
        # both round a binary64 sum to FP32; the sums differ only in order
        assert np.all(np.abs(got.astype(np.float64) - ref) <= np.spacing(np.abs(ref).astype(np.float32)))
        # a row range is the same rows of the whole product
        part = O.gemm_w4a16_rows(a, fmt, codes, scales, g, sp, N, 2, 5)
        assert np.array_equal(part, got[2:5])


def test_w4a16_all_special_weight_closed_form():
    # every weight code 0x8 with table index 2 (value 2.5) and E3M3 code 24
    # (scale 1.0): W = 2.5 g everywhere, so C[m, n] = 2.5 g sum_k a[m, k]
    M, N, K = 3, 5, 64
    codes = np.full((N, K // 2), 0x88, np.uint8)
    scales = np.full((N, K // 16), (2 << 6) | 24, np.uint8)
    assert O.e3m3_value(24) == 1.0
    a_f = np.arange(M * K, dtype=np.float32).reshape(M, K) % 7 - 3
    a = datagen.to_bf16_bits(a_f)
    g = 0.75
    got = O.gemm_w4a16_rows(a, "razer_w", codes, scales, g, (5.0, -5.0, 2.5, -2.5), N)
    exp = 2.5 * g * a_f.astype(np.float64).sum(axis=1)
    assert np.array_equal(got, np.repeat(exp[:, None], N, axis=1).astype(np.float32))


# ---------------------------------------------------------------- pairs
def test_pairs_are_the_lexicographic_candidate_pairs():
    pairs = [O.razer_pair(p) for p in range(O.RAZER_NPAIRS)]
    expect = [(CAND[i], CAND[j]) for i in range(8) for j in range(i + 1, 8)]
    assert pairs == expect
    # the candidates: multiples of 0.5 in (0, 7.5] that E2M1 does not hold
    assert CAND == [v / 2 for v in range(1, 16) if v / 2 not in MAGS]


# ---------------------------------------------------------------- exact recomputation
def _nearest_mag(a, s):
    """nearest E2M1 magnitude to a / s (exact), ties to the even code"""
    q = Fraction(a) / s
    best = None
    for m, v in enumerate(MAGS):
        d = abs(q - Fraction(v))
        if best is None or d < best[0] or (d == best[0] and m % 2 == 0 and best[1] % 2 == 1):
            best = (d, m)
    return MAGS[best[1]]


def _block_err_exact(x, s, v):
    """exact squared error of RaZeR-W quantization of block x with scale s
    and special value v: an element of v's sign strictly inside the interval
    between the midpoints from |v| to its E2M1 neighbours takes v"""
    av = abs(v)
    below = max(m for m in MAGS if m < av)
    above = [m for m in MAGS if m > av]
    lo = Fraction(below + av) / 2
    hi = Fraction(above[0] + av) / 2 if above else None   # above 6: no upper bound
    err = Fraction(0)
    for e in x:
        f = Fraction(float(e))
        same_sign = (f > 0) if v > 0 else (f < 0)
        if s > 0 and same_sign and lo * s < abs(f) and (hi is None or abs(f) < hi * s):
            q = Fraction(v) * s
        elif s > 0:
            m = _nearest_mag(abs(f), s)
            q = Fraction(m) * s * (1 if f >= 0 else -1)
        else:
            q = Fraction(0)
        err += (f - q) ** 2
    return err


def test_pair_errors_match_exact_recomputation():
    x = (datagen.student_t((6, 64), 8200, 3.0) * np.float32(0.5)).astype(np.float32)
    sse, best = O.razer_table_search(x, 1.0)
    e3m3 = [O.e3m3_value(k) for k in range(64)]
    exact = [Fraction(0)] * 28
    for r in range(6):
        for b in range(4):
            xb = x[r, 16 * b:16 * b + 16]
            amax = Fraction(float(np.abs(xb).max()))
            # abs-max E3M3 scale: nearest to amax / 6, ties to the even code
            k = min(range(64), key=lambda j: (abs(Fraction(e3m3[j]) - amax / 6), j % 2))
            s = Fraction(e3m3[k])
            errs = {c: _block_err_exact(xb, s, c) for c in CAND + [-c for c in CAND]}
            p = 0
            for i in range(8):
                for j in range(i + 1, 8):
                    exact[p] += min(errs[CAND[i]], errs[-CAND[i]], errs[CAND[j]], errs[-CAND[j]])
                    p += 1
    for p in range(28):
        assert abs(Fraction(sse[p]) - exact[p]) <= Fraction(1, 10 ** 5) * exact[p], p
    ordered = sorted(exact)
    if ordered[1] - ordered[0] > Fraction(1, 10 ** 4) * ordered[1]:
        assert exact[best] == ordered[0]


def test_pair_error_is_the_quantized_block_error_under_that_table():
    w = datagen.student_t((9, 128), 8300, 4.0) * np.float32(0.02)
    g = O.auto_global(w, "razer_w")
    sse, best = O.razer_table_search(w, g)
    for p in (0, 5, best, 27):
        a, b = O.razer_pair(p)
        table = (a, -a, b, -b)
        codes, scales = O.quantize_rows(w, "razer_w", 16, O.ABSMAX, g, special=table)
        tot = 0.0
        for r in range(w.shape[0]):
            row = 0.0
            for blk in range(w.shape[1] // 16):
                sb = int(scales[r, blk])
                k, pick = sb & 63, sb >> 6
                c = [(int(codes[r, (16 * blk + i) // 2]) >> (4 * (i & 1))) & 15 for i in range(16)]
                row = row + O.block_sse(w[r, 16 * blk:16 * blk + 16], c, O.e3m3_value(k), g, table[pick])
            tot = tot + row
        assert tot == sse[p], p
    assert best == int(np.argmin(sse))


def test_constructed_blocks_pick_two_and_a_half_and_five_and_a_half():
    # scale 1.0 (amax 6); half the blocks hold many +5.5 (exact only with
    # special +5.5), the other half many -2.5 (exact only with -2.5)
    rows = []
    for r in range(8):
        blk = np.zeros(16, np.float32)
        blk[0] = 6.0
        if r % 2 == 0:
            blk[1:12] = 5.5
        else:
            blk[1:12] = -2.5
        rows.append(np.tile(blk, 2))
    x = np.stack(rows)
    sse, best = O.razer_table_search(x, 1.0)
    assert O.razer_pair(best) == (2.5, 5.5)
    assert sse[best] == 0.0
    # the default pair (5, 2.5) is not exact here
    assert sse[[i for i in range(28) if O.razer_pair(i) == (2.5, 5.0)][0]] > 0


def test_all_zero_weight_keeps_the_first_pair():
    sse, best = O.razer_table_search(np.zeros((3, 32), np.float32), 1.0)
    assert best == 0 and np.all(sse == 0)
