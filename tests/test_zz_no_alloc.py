"""The matmul entry point that allocates nothing, fp4q_gemm_w4a4_noalloc,
against fp4q_gemm_w4a4 on the same operands: the same bytes.  Three calls in a
row, each smaller than the one before, all of which split K (so all use the
library's own array): the RaZeR decode workload at M = 128, a decode shape at
M = 16, and a two-tile shape of the tile kernel.  Outputs start as NaN, so an
entry that was not written shows."""
import numpy as np
import pytest

import datagen
from tests.gpu_util import case, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp4_e4m3_amd as B
    return B


def _run(B, entry, fa, ac, as_, ag, fw, wc, ws, wg, sp, M, N, K):
    import torch
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    entry(fa, ac, as_, ag, fw, wc, ws, wg, sp, M, N, K, out, B.FP4Q_F32, N)
    torch.cuda.synchronize()
    return host(out).view(np.uint32).copy()


def test_noalloc_matches_allocating_entry(B):
    cases = [("razer_a", "razer_w", 128, 17408, 5120), ("nvfp4", "nvfp4", 16, 4096, 2048),
             ("nvfp4", "nvfp4", 200, 300, 1024)]
    for fa, fw, M, N, K in cases:
        a = datagen.student_t((M, K), 990 + M, 4.0)
        w = datagen.normal((N, K), 991, 0.02)
        sp = datagen.RAZER_SPECIAL if fw == "razer_w" else None
        case(f"no-alloc gemm {fa}x{fw} {M}x{N}x{K}: operands")
        ac, as_, ag = B.quantize(dev(a), fa, 16, "absmax", "auto")
        wc, ws, wg = B.quantize(dev(w), fw, 16, "absmax", "auto", special=sp or (0.0,) * 4)
        case(f"no-alloc gemm {fa}x{fw} {M}x{N}x{K}: allocating entry")
        ref = _run(B, B.fp4q_gemm_w4a4, fa, ac, as_, ag, fw, wc, ws, wg, sp, M, N, K)
        case(f"no-alloc gemm {fa}x{fw} {M}x{N}x{K}: non-allocating entry")
        got = _run(B, B.fp4q_gemm_w4a4_noalloc, fa, ac, as_, ag, fw, wc, ws, wg, sp, M, N, K)
        assert np.all(np.isfinite(ref.view(np.float32)))
        assert np.array_equal(got, ref)
