"""Pins of the oracle's pre-transforms (MACaQ sections 1 and 3), dequantize
and W4A4 matmul: against scipy's Hadamard matrix, numpy binary64 BLAS, closed
forms and the identity X D B (W D^-1 B)^T = X W^T stated on the MACaQ page."""
from fractions import Fraction

import numpy as np
import scipy.linalg
import torch

import oracle as O
from tests.exact_ref import e2m1_table, e4m3_lib_values, e8m0_lib_values, golden_kv

C32 = np.uint32(0x3E3504F3).view(np.float32)


def test_fwht_is_sylvester_hadamard():
    H = scipy.linalg.hadamard(32).astype(np.float64)
    eye = np.eye(32, dtype=np.float32)
    Y = O.transform(eye, None, 32)          # row i = transform of unit vector e_i
    assert np.array_equal(Y.astype(np.float64), (H * float(C32)).T.astype(np.float32).astype(np.float64))
    # H H^T = 32 I and c = RN32(2^-2.5) makes the rotation orthonormal
    Hr = Y.astype(np.float64) / float(C32)
    assert np.array_equal(Hr @ Hr.T, 32 * np.eye(32))
    assert float(C32) == np.float32(2.0 ** -2.5)
    assert int(golden_kv("formats.txt")["hadamard_size"][0]) == 32


def test_block_hadamard_acts_per_group_and_preserves_norm():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    y = O.transform(x, None, 32)
    H = scipy.linalg.hadamard(32) / np.sqrt(32.0)
    ref = np.concatenate([x[:, g:g + 32].astype(np.float64) @ H for g in range(0, 128, 32)], axis=1)
    assert np.max(np.abs(y - ref)) <= 1e-5 * np.max(np.abs(ref))
    n0 = np.linalg.norm(x.astype(np.float64).reshape(8, 4, 32), axis=2)
    n1 = np.linalg.norm(y.astype(np.float64).reshape(8, 4, 32), axis=2)
    assert np.max(np.abs(n1 / n0 - 1)) < 1e-6


def test_scale_and_rotation_cancel_in_the_product():
    # MACaQ section 1: activations take x D B online, the weights absorb
    # W D^-1 B offline, so the layer output X W^T is unchanged
    rng = np.random.default_rng(1)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    w = (rng.standard_normal((24, 64)) * 0.02).astype(np.float32)
    t, r = O.channel_scale(x, w, 0.75)
    xa = O.transform(x, t, 32).astype(np.float64)
    wa = O.transform(w, r, 32).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.max(np.abs(xa @ wa.T - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_channel_scale_balances_channels():
    # MACaQ section 3: t_j ~ (sigma_j^W / rms_j^x)^alpha, alpha = 0.75.
    # After scaling, log rms(x_j t_j) = (1-alpha) log rms_x + alpha log sigma_W
    alpha = float(golden_kv("formats.txt")["alpha"][0])
    assert alpha == 0.75
    rng = np.random.default_rng(2)
    cols = 32
    sx = np.exp2(rng.uniform(-3, 6, cols))
    sw = np.exp2(rng.uniform(-8, -2, cols))
    x = (rng.standard_normal((512, cols)) * sx).astype(np.float32)
    w = (rng.standard_normal((256, cols)) * sw).astype(np.float32)
    t, r = O.channel_scale(x, w, alpha)
    rx = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=0))
    rw = np.sqrt(np.mean(w.astype(np.float64) ** 2, axis=0))
    lhs = np.log(rx * t)
    rhs = (1 - alpha) * np.log(rx) + alpha * np.log(rw)
    assert np.max(np.abs(lhs - rhs)) < 1e-6
    # outlier channels get the smaller scale; scaling X by c scales t by c^-alpha
    t2, _ = O.channel_scale((x * 8).astype(np.float32), w, alpha)
    assert np.max(np.abs(t2 / t - 8.0 ** -alpha)) < 1e-6
    assert np.array_equal(r, (np.float32(1) / t).astype(np.float32))
    # a zero column gets t = 1
    x[:, 3] = 0
    t3, _ = O.channel_scale(x, w, alpha)
    assert t3[3] == 1.0


def test_dequantize_values_independent_decode():
    # decode through the pages' E2M1 table and torch's E4M3/E8M0 decoders
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    e2 = e2m1_table()
    e4 = e4m3_lib_values()
    e8 = e8m0_lib_values()
    for fmt, B in (("nvfp4", 16), ("mxfp4", 32)):
        gmode = O.G_AUTO if fmt == "nvfp4" else O.G_NONE
        codes, scales, g = O.quantize(x, fmt, B, O.ABSMAX, gmode)
        deq = O.dequantize(codes, scales, fmt, B, g)
        for r in range(8):
            for j in range(64):
                c = (codes[r, j // 2] >> (4 * (j & 1))) & 15
                s = e4[scales[r, j // B]] if fmt == "nvfp4" else e8[scales[r, j // B]]
                ref = np.float32(Fraction(e2[c]) * Fraction(s) * Fraction(float(g)))
                assert deq[r, j] == ref


def _quant(x, fmt, B, rule=O.ABSMAX, gmode=O.G_NONE, special=None):
    return O.quantize(np.ascontiguousarray(x, np.float32), fmt, B, rule, gmode, special=special)


def test_gemm_exact_regime_matches_binary64_blas_bitwise():
    # every scale in [1, 2), g = 1, K <= 256: all partial sums are exact in
    # binary32, so any summation order gives the same bits
    rng = np.random.default_rng(4)
    M, N, K = 16, 24, 256
    a = rng.choice([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], (M, K)).astype(np.float32)
    w = rng.choice([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], (N, K)).astype(np.float32)
    a[:, ::16] = 6.0  # every block max is 6 -> scale 1
    w[:, ::16] = -6.0
    ca, sa, _ = _quant(a, "nvfp4", 16)
    cw, sw, _ = _quant(w, "nvfp4", 16)
    assert np.all(sa == 56) and np.all(sw == 56)  # E4M3 code of 1.0
    c = O.gemm_rows("nvfp4", ca, sa, 1.0, "nvfp4", cw, sw, 1.0, None, M, N, K)
    ref = (a.astype(np.float64) @ w.astype(np.float64).T).astype(np.float32)
    assert np.array_equal(c, ref)


def test_gemm_matches_blas_on_decoded_operands():
    rng = np.random.default_rng(5)
    M, N, K = 12, 20, 96
    a = rng.standard_t(4, (M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    for fa, fw, B, special in (("nvfp4", "nvfp4", 16, None), ("razer_a", "razer_w", 16, (5.0, -5.0, 2.5, -2.5)),
                               ("mxfp4", "mxfp4", 32, None)):
        gm = O.G_NONE if fa == "mxfp4" else O.G_AUTO
        ca, sa, ga = _quant(a, fa, B, gmode=gm)
        cw, sw, gw = _quant(w, fw, B, gmode=gm, special=special)
        da = O.decode(ca, sa, fa, B)
        dw = O.decode(cw, sw, fw, B, special)
        ref = (da @ dw.T) * float(np.float32(ga * gw))
        c = O.gemm_rows(fa, ca, sa, ga, fw, cw, sw, gw, special, M, N, K)
        assert np.max(np.abs(c - ref)) <= 1e-6 * np.max(np.abs(ref))
        # the decoded operands reproduce the dequantized tensors
        assert np.array_equal((da * float(ga)).astype(np.float32), O.dequantize(ca, sa, fa, B, ga))
        # entries API agrees with the row API
        ms = rng.integers(0, M, 30)
        ns = rng.integers(0, N, 30)
        e = O.gemm_entries(fa, ca, sa, ga, fw, cw, sw, gw, special, M, N, K, ms, ns)
        assert np.array_equal(e, c[ms, ns])


def test_gemm_one_hot_weight_selects_columns():
    rng = np.random.default_rng(6)
    M, N, K = 8, 16, 64
    a = rng.standard_normal((M, K)).astype(np.float32)
    ca, sa, _ = _quant(a, "nvfp4", 16)
    w = np.zeros((N, K), np.float32)
    cols = rng.integers(0, K, N)
    w[np.arange(N), cols] = 6.0   # block max 6 -> scale 1, the element decodes to 6 exactly
    cw, sw, _ = _quant(w, "nvfp4", 16)
    c = O.gemm_rows("nvfp4", ca, sa, 1.0, "nvfp4", cw, sw, 1.0, None, M, N, K)
    deq = O.dequantize(ca, sa, "nvfp4", 16)
    assert np.array_equal(c, 6 * deq[:, cols])
