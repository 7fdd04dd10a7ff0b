"""GPU parity of the RaZeR weight-only matmul (bf16 activations, NVFP4 or
RaZeR-W weights) and of the offline special-value search against the oracle.

The matmul is checked entry by entry against the oracle's binary64 product
with the FP32-accumulation error bound 2 (K + 8) 2^-24 g sum_k |a_k w_k| plus
one unit in the last place of the output type (the bf16 products are exact in
FP32, so only the additions round), and bit for bit where every partial sum
is exact in FP32.  The search is bit-exact: the same FP32 block errors summed
in binary64 in the same order, and the same pick.  Weight operands come from
the oracle quantizer; at full size the sampled rows of a HIP-quantized
weight are overwritten with the oracle's."""
import numpy as np
import pytest

import datagen
import oracle as O
from tests.gpu_util import case, dev, host, scalar_dev

pytestmark = pytest.mark.gpu

SPECIAL = datagen.RAZER_SPECIAL


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp4_e4m3_amd as B
    return B


def err_bound(a_bits, w_dec, g, K):
    A = np.abs(datagen.bf16_bits_to_f32(a_bits).astype(np.float64))
    return 2.0 * (K + 8) * 2.0 ** -24 * abs(g) * (A @ np.abs(w_dec).T)


def assert_within(got, ref, bound, out_dtype):
    ref = ref.astype(np.float64)
    if out_dtype == "bf16":
        # RNE of the FP32 result: one bf16 unit on top of the accumulation bound
        ulp = np.abs(ref) * 2.0 ** -7 + 2.0 ** -133
    else:
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= bound + ulp)


def gpu_w4a16(B, a_bits, fmt, codes, scales, g, sp, out_dtype="f32", lda_pad=0, ldc_pad=0):
    import torch
    M, K = a_bits.shape
    N = codes.shape[0]
    a_full = np.zeros((M, K + lda_pad), np.uint16)
    a_full[:, :K] = a_bits
    a = dev(a_full, bf16=True)[:, :K]
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    per16 = 4 if out_dtype == "f32" else 8
    ld = -(-(N + ldc_pad) // per16) * per16
    out = torch.full((M, ld), float("nan"), dtype=dt, device="cuda")
    c = out[:, :N]
    case(f"w4a16 {fmt} {M}x{N}x{K} {out_dtype} lda+{lda_pad} ldc {ld}")
    B.gemm_w4a16(a, fmt, dev(codes), dev(scales), scalar_dev(g), sp, out=c)
    torch.cuda.synchronize()
    r = host(c)
    if out_dtype != "f32":
        r = datagen.bf16_bits_to_f32(r)
    return r


@pytest.mark.parametrize("fmt", ["nvfp4", "razer_w"])
@pytest.mark.parametrize("M", [1, 16, 37, 128, 200])
@pytest.mark.parametrize("N,K", [(96, 512), (300, 1024)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_w4a16_small(B, fmt, M, N, K, out_dtype):
    sp = SPECIAL if fmt == "razer_w" else None
    w = datagen.normal((N, K), 7000 + N, 0.02)
    codes, scales, g = O.quantize(w, fmt, 16, O.ABSMAX, O.G_AUTO, special=sp)
    a = datagen.to_bf16_bits(datagen.student_t((M, K), 7100 + M, 4.0))
    ref = O.gemm_w4a16_rows(a, fmt, codes, scales, g, sp, N)
    if out_dtype == "bf16":
        ref = datagen.bf16_bits_to_f32(datagen.to_bf16_bits(ref))
    got = gpu_w4a16(B, a, fmt, codes, scales, g, sp, out_dtype, lda_pad=8 * (M % 3), ldc_pad=8)
    assert_within(got, ref, err_bound(a, O.decode(codes, scales, fmt, 16, special=sp), g, K), out_dtype)


@pytest.mark.parametrize("fmt", ["nvfp4", "razer_w"])
def test_w4a16_exact_regime_bitwise(B, fmt):
    # unit block scales, small integer activations: every partial sum is a
    # multiple of 0.5 below 2^14, exact in FP32 in any order
    M, N, K = 40, 130, 1024
    g = datagen.rng(7200)
    codes = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    if fmt == "razer_w":
        scales = ((g.integers(0, 4, (N, K // 16)) << 6) | 24).astype(np.uint8)   # E3M3 1.0, any table entry
    else:
        scales = np.full((N, K // 16), 56, np.uint8)   # E4M3 1.0
    sp = SPECIAL if fmt == "razer_w" else None
    a = datagen.to_bf16_bits(g.integers(-3, 4, (M, K)).astype(np.float32))
    ref = O.gemm_w4a16_rows(a, fmt, codes, scales, 1.0, sp, N)
    got = gpu_w4a16(B, a, fmt, codes, scales, 1.0, sp)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def rows_of(n, k, seed):
    idx = datagen.rng(seed).choice(n, size=min(k, n), replace=False)
    return np.sort(np.concatenate([idx, [0, n - 1]])).astype(np.int64)


@pytest.mark.parametrize("M", [1, 16, 128])
def test_w4a16_razer_decode_workload(B, M):
    # the decode workload (K 5120, N 17408) with a RaZeR-W weight: the full
    # weight quantized on the GPU under the oracle's global scale, its sampled
    # rows replaced by the oracle's codes, then the entries at (sampled
    # activation rows x sampled weight rows)
    import torch
    d = datagen.razer_decode(M)
    a, w = d["A_bf16"], d["W"]
    N, K = w.shape
    g = O.auto_global(w, "razer_w")
    wr = rows_of(N, 192, 7300)
    case(f"w4a16 decode workload M={M}: weight quantize")
    codes, scales, _ = B.quantize(dev(w), "razer_w", 16, "absmax", "given", special=SPECIAL, global_=scalar_dev(g))
    oc, os_ = O.quantize_rows(w[wr], "razer_w", 16, O.ABSMAX, g, SPECIAL)
    idx = torch.as_tensor(wr, device="cuda")
    codes.index_copy_(0, idx, dev(oc))
    scales.index_copy_(0, idx, dev(os_))
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    case(f"w4a16 decode workload M={M}: matmul")
    B.gemm_w4a16(dev(a, bf16=True), "razer_w", codes, scales, scalar_dev(g), SPECIAL, out=out)
    torch.cuda.synchronize()
    ar = np.arange(M) if M <= 16 else rows_of(M, 14, 7301)
    got = host(out.index_select(0, torch.as_tensor(ar, device="cuda")).index_select(1, idx))
    ref = O.gemm_w4a16_rows(a[ar], "razer_w", oc, os_, g, SPECIAL, len(wr))
    assert_within(got, ref, err_bound(a[ar], O.decode(oc, os_, "razer_w", 16, special=SPECIAL), g, K), "f32")


def test_w4a16_split_k_is_deterministic(B):
    import torch
    M, N, K = 16, 17408, 5120
    w = datagen.normal((N, K), 7400, 0.02)
    a = dev(datagen.to_bf16_bits(datagen.student_t((M, K), 7401, 4.0)), bf16=True)
    case("w4a16 determinism: operands")
    codes, scales, g = B.quantize(dev(w), "razer_w", 16, "absmax", "auto", special=SPECIAL)
    outs = []
    for i in range(3):
        case(f"w4a16 determinism: launch {i}")
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        B.gemm_w4a16(a, "razer_w", codes, scales, g, SPECIAL, out=out)
        torch.cuda.synchronize()
        outs.append(host(out).view(np.uint32).copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    assert np.all(np.isfinite(outs[0].view(np.float32)))


# ---------------------------------------------------------------- special-value search
def search_pair(B, w_np, w_gpu, gmode, g_given=None):
    import torch
    rows, cols = w_np.shape
    if gmode == "auto":
        g = O.auto_global(w_np if w_np.dtype == np.float32 else datagen.bf16_bits_to_f32(w_np), "razer_w")
    elif gmode == "given":
        g = g_given
    else:
        g = 1.0
    case(f"razer table search {tuple(w_gpu.shape)} {w_gpu.dtype} g={gmode}")
    table, sse, gbuf = B.razer_table_search(w_gpu, gmode, global_=scalar_dev(g_given if gmode == "given" else 1.0))
    torch.cuda.synchronize()
    osse, best = O.razer_table_search(w_np, g)
    if gmode == "auto":
        assert host(gbuf)[0] == np.float32(g)
    assert np.array_equal(host(sse).view(np.uint64), osse.view(np.uint64))
    a, b = O.razer_pair(best)
    assert np.array_equal(host(table), np.array([a, -a, b, -b], np.float32))
    return best


@pytest.mark.parametrize("rows,cols", [(1, 16), (5, 64), (67, 272), (300, 128)])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("gmode", ["none", "auto", "given"])
def test_search_small(B, rows, cols, bf16, gmode):
    w = datagen.student_t((rows, cols), 7500 + rows, 4.0) * np.float32(0.03)
    if bf16:
        wn = datagen.to_bf16_bits(w)
        wg = dev(wn, bf16=True)
    else:
        wn, wg = w, dev(w)
    search_pair(B, wn, wg, gmode, g_given=2.0e-3)


def test_search_strided_rows_and_constructed_pick(B):
    wide = (datagen.normal((33, 96), 7600, 0.05)).astype(np.float32)
    search_pair(B, np.ascontiguousarray(wide[:, :64]), dev(wide)[:, :64], "auto")
    rows = []
    for r in range(8):
        blk = np.zeros(16, np.float32)
        blk[0] = 6.0
        blk[1:12] = 5.5 if r % 2 == 0 else -2.5
        rows.append(np.tile(blk, 2))
    x = np.stack(rows)
    best = search_pair(B, x, dev(x), "none")
    assert O.razer_pair(best) == (2.5, 5.5)


def test_search_zero_rows_writes_first_pair(B):
    import torch
    w = torch.zeros((1, 32), dtype=torch.float32, device="cuda")[:0]  # no rows, a valid address
    case("razer table search, no rows")
    table, sse, _ = B.razer_table_search(w, "none")
    torch.cuda.synchronize()
    assert np.all(host(sse) == 0)
    assert np.array_equal(host(table), np.array([2.5, -2.5, 3.5, -3.5], np.float32))


def test_search_decode_weight(B):
    # the decode workload's weight (17408 x 5120) searched whole under the
    # automatic global scale; the oracle checks the global scale and a
    # contiguous 384-row slice searched by the same kernel
    import torch
    w = datagen.razer_decode(1)["W"]
    wg = dev(w)
    case("razer table search: decode weight, whole")
    table, sse, gbuf = B.razer_table_search(wg, "auto")
    torch.cuda.synchronize()
    g = O.auto_global(w, "razer_w")
    assert host(gbuf)[0] == np.float32(g)
    s = host(sse)
    assert np.all(np.isfinite(s)) and np.all(s > 0)
    best = int(np.argmin(s))
    a, b = O.razer_pair(best)
    assert np.array_equal(host(table), np.array([a, -a, b, -b], np.float32))
    r0 = 9001
    sl = np.ascontiguousarray(w[r0:r0 + 384])
    case("razer table search: decode weight, slice")
    table2, sse2, _ = B.razer_table_search(wg[r0:r0 + 384], "given", global_=scalar_dev(g))
    torch.cuda.synchronize()
    osse, obest = O.razer_table_search(sl, g)
    assert np.array_equal(host(sse2).view(np.uint64), osse.view(np.uint64))
