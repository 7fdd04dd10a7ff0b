"""Pins of the oracle's MACaQ weight calibration (MACaQ review, sections 1 and
3): Hessian-weighted exponent screening over the standard exponent and
offsets +1 / -1, then Flip-Refinement, against what the page states and the
mathematics fixes:

* the objective is the layer-output reconstruction error ||X W^T - X W^^T||_F^2
  (checked with numpy on the dequantized weights);
* with a diagonal Hessian the objective separates per element, round to
  nearest is already optimal and the refinement makes no move;
* the screening picks the exact (rational) argmin of e^T H_bb e;
* the refinement never increases the objective and stops at a point where no
  single one-level move gains (checked independently in binary64);
* a move cap of zero leaves the screened round-to-nearest codes."""
from fractions import Fraction

import numpy as np

import datagen
import oracle as O


def calib(N=12, K=256, T=768, seed=0, corr=True):
    g = datagen.rng(seed)
    X = g.standard_normal((T, K))
    if corr:  # correlated channels and a few outlier channels, as activations have
        X = X + 0.7 * X[:, [0]] + 0.4 * np.roll(X, 1, axis=1)
        X[:, g.choice(K, 4, replace=False)] *= 15.0
    W = (g.standard_t(4, (N, K)) * 0.02).astype(np.float32)
    return X, W, X.T @ X


def _dequant(codes, scales):
    return O.dequantize(codes, scales, "mxfp4", 32).astype(np.float64)


def test_objective_is_layer_output_error():
    X, W, H = calib()
    codes, scales, moves, obj = O.macaq_quantize(W, H)
    Wq = _dequant(codes, scales)
    err = np.sum((X @ (W.astype(np.float64) - Wq).T) ** 2, axis=0)
    assert np.allclose(obj[:, 1], err, rtol=1e-9, atol=0)
    assert np.all(moves > 0) and np.all(obj[:, 1] < obj[:, 0])


def test_diagonal_hessian_needs_no_move():
    X, W, H = calib(seed=1)
    for Hd in (np.eye(H.shape[0]), np.diag(np.diag(H))):
        codes, scales, moves, _ = O.macaq_quantize(W, Hd)
        assert np.all(moves == 0)
        # the codes are round to nearest at the screened exponents
        for r in range(W.shape[0]):
            for b in range(W.shape[1] // 32):
                E = int(scales[r, b]) - 127
                for i in range(32):
                    k = 32 * b + i
                    c = (int(codes[r, k // 2]) >> (4 * (k & 1))) & 15
                    assert c == O.rtn(float(W[r, k]), 2.0 ** E, 1.0)


def test_screening_is_the_exact_weighted_argmin():
    X, W, H = calib(N=6, K=128, seed=2)
    _, scales, _, _ = O.macaq_quantize(W, H, max_moves=0)
    checked = 0
    for r in range(W.shape[0]):
        for b in range(W.shape[1] // 32):
            w = W[r, 32 * b:32 * b + 32]
            hb = H[32 * b:32 * b + 32, 32 * b:32 * b + 32]
            a = float(np.abs(w).max())
            E0 = int(np.floor(np.log2(a))) - 2
            cost = {}
            for E in (E0, E0 + 1, E0 - 1):
                e = [Fraction(float(v)) - Fraction(O.e2m1_value(O.rtn(float(v), 2.0 ** E, 1.0))) * Fraction(2) ** E
                     for v in w]
                cost[E] = sum(e[i] * Fraction(float(hb[i, j])) * e[j] for i in range(32) for j in range(32))
            vals = sorted(cost.values())
            if vals[1] - vals[0] > Fraction(1, 10 ** 9) * vals[1]:
                assert int(scales[r, b]) - 127 == min(cost, key=cost.get)
                checked += 1
    assert checked > 10


def test_refinement_is_monotone_and_stops_at_a_local_minimum():
    levels = np.array([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    X, W, H = calib(N=5, K=256, seed=3)
    codes0, scales0, _, obj0 = O.macaq_quantize(W, H, max_moves=0)
    codes, scales, moves, obj = O.macaq_quantize(W, H)
    assert np.array_equal(scales, scales0)       # exponents are fixed by the screening
    assert np.all(obj[:, 1] <= obj0[:, 1])
    Wq = _dequant(codes, scales)
    for r in range(W.shape[0]):
        d = Wq[r] - W[r].astype(np.float64)
        f = d @ H @ d
        assert abs(f - obj[r, 1]) <= 1e-9 * f
        grad = H @ d
        sc = 2.0 ** (np.repeat(scales[r].astype(np.int64), 32) - 127)
        q = Wq[r] / sc
        for k in range(W.shape[1]):
            lv = int(np.where(levels == q[k])[0][0])
            for nl in (lv + 1, lv - 1):
                if 0 <= nl < 15:
                    delta = (levels[nl] - levels[lv]) * sc[k]
                    assert 2 * delta * grad[k] + delta * delta * H[k, k] >= -1e-9 * f


def test_move_cap_zero_keeps_round_to_nearest():
    X, W, H = calib(N=3, K=64, seed=4)
    codes, scales, moves, obj = O.macaq_quantize(W, H, max_moves=0)
    assert np.all(moves == 0) and np.array_equal(obj[:, 0], obj[:, 1])
