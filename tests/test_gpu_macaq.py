"""GPU parity of fp4q_macaq_quantize (MACaQ exponent screening and
Flip-Refinement) against the oracle: codes, exponents and the number of moves
per row must match exactly (both sides do the same binary64 operations in the
same order).  The Hessian is an input, formed here from seeded activations
with numpy; neither side computes it."""
import numpy as np
import pytest

import datagen
import oracle as O
from tests.gpu_util import case, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp4_e4m3_amd as B
    return B


def calib(N, K, T, seed, wscale=0.02):
    g = datagen.rng(seed)
    X = g.standard_normal((T, K))
    X = X + 0.7 * X[:, [0]] + 0.4 * np.roll(X, 1, axis=1)
    X[:, g.choice(K, 4, replace=False)] *= 15.0
    W = (g.standard_t(4, (N, K)) * wscale).astype(np.float32)
    return W, X.T @ X


def run(B, W, H, max_moves=None, workspace_rows=None):
    import torch
    N, K = W.shape
    mm = 2 * K if max_moves is None else max_moves
    oc, os_, om, _ = O.macaq_quantize(W, H, mm)
    case(f"macaq {N}x{K} max_moves={mm} workspace rows={workspace_rows}")
    wsb = None if workspace_rows is None else 8 * K * workspace_rows
    codes, scales, moves = B.macaq_quantize(dev(W), dev(H), mm, wsb)
    torch.cuda.synchronize()
    assert np.array_equal(host(scales), os_), "exponents differ"
    assert np.array_equal(host(moves), om), "move counts differ"
    assert np.array_equal(host(codes), oc), "codes differ"
    return om


@pytest.mark.parametrize("N,K", [(24, 256), (9, 96), (5, 512), (3, 2048)])
def test_macaq_small(B, N, K):
    W, H = calib(N, K, 3 * K, 7000 + K)
    moves = run(B, W, H)
    assert moves.sum() > 0


def test_macaq_passes_caps_and_extremes(B):
    W, H = calib(40, 512, 1024, 7100)
    run(B, W, H, workspace_rows=7)           # six passes over the rows, the last one short
    run(B, W, H, max_moves=0)
    run(B, W, H, max_moves=5)
    # weights near the bottom of the FP32 range: exponents below -126 (the
    # exact round-to-nearest path) in the screening
    Wt = (W * np.float32(2.0 ** -128)).astype(np.float32)
    run(B, Wt, H * 2.0 ** 200)


def test_macaq_linear_workload_sampled_rows(B):
    # the MXFP4 linear workload's weight (14336 x 4096) with the Hessian of its
    # activations (4096 x 4096, bf16 values): the whole weight on the GPU, the
    # oracle on sampled rows
    import torch
    d = datagen.mxfp4_linear()
    X = datagen.bf16_bits_to_f32(d["X_bf16"]).astype(np.float64)
    H = X.T @ X
    W = d["W"]
    case("macaq full weight 14336 x 4096")
    codes, scales, moves = B.macaq_quantize(dev(W), dev(H))
    torch.cuda.synchronize()
    rows = np.sort(datagen.rng(7200).choice(W.shape[0], 6, replace=False))
    oc, os_, om, obj = O.macaq_quantize(W[rows], H)
    assert np.array_equal(host(scales)[rows], os_)
    assert np.array_equal(host(moves)[rows], om)
    assert np.array_equal(host(codes)[rows], oc)
    assert np.all(obj[:, 1] < obj[:, 0])
