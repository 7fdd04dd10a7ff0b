"""GPU parity of fp4q_gemm_w4a4 against the CPU oracle (binary64
accumulation): relative Frobenius error <= 1e-3 (the W4A4 tolerance), and
bit-equality in the regime where every partial sum is exact in FP32.

The GEMM inputs are produced by the oracle quantizer (never by the HIP
quantizer).  At full workload sizes the GPU GEMM consumes a buffer whose
sampled rows come from the oracle; only entries that depend on those rows
alone are compared."""
import numpy as np
import pytest

import datagen
import oracle as O
from tests.gpu_util import case, dev, host, rel_fro, scalar_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3
SPECIAL = datagen.RAZER_SPECIAL


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp4_e4m3_amd as B
    return B


def check(got, ref, out_dtype):
    """FP32 output against the oracle's FP32 C; bf16 output against the
    oracle's C rounded to bf16 (nearest even), both at the W4A4 tolerance"""
    if out_dtype != "f32":
        ref = datagen.bf16_bits_to_f32(datagen.to_bf16_bits(ref))
    assert rel_fro(got, ref) <= TOL


def oquant(x, fmt, rule=O.ABSMAX, gmode=O.G_AUTO, special=None):
    block = 32 if fmt == "mxfp4" else 16
    if fmt == "mxfp4":
        gmode = O.G_NONE
    return O.quantize(x, fmt, block, rule, gmode, special=special)


def gpu_gemm(B, fa, ca, sa, ga, fw, cw, sw, gw, special, out_dtype="f32", ldc_pad=0):
    import torch
    M, N = ca.shape[0], cw.shape[0]
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    per16 = 4 if out_dtype == "f32" else 8  # row pitch must be a multiple of 16 bytes
    ld = -(-(N + ldc_pad) // per16) * per16
    out = torch.empty((M, ld), dtype=dt, device="cuda")
    c = out[:, :N]
    B.gemm(fa, dev(ca), dev(sa), scalar_dev(ga), fw, dev(cw), dev(sw), scalar_dev(gw), special, out=c)
    torch.cuda.synchronize()
    r = host(c)
    if out_dtype != "f32":
        r = datagen.bf16_bits_to_f32(r)
    return r


@pytest.mark.parametrize("fa,fw", [("nvfp4", "nvfp4"), ("razer_a", "razer_w"), ("razer_a", "nvfp4"),
                                   ("nvfp4", "razer_w"), ("nvfp4", "razer_a"), ("mxfp4", "mxfp4")])
@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (100, 130, 96), (1, 17, 160), (133, 67, 32), (7, 300, 544)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_small(B, fa, fw, M, N, K, out_dtype):
    if fa == "mxfp4" and K % 32:
        pytest.skip("MXFP4 needs K % 32 == 0")
    a = datagen.student_t((M, K), 500 + M, 4.0)
    w = datagen.normal((N, K), 600 + N, 0.02)
    sp = SPECIAL if fw == "razer_w" else None
    ca, sa, ga = oquant(a, fa)
    cw, sw, gw = oquant(w, fw, special=sp)
    ref = O.gemm_rows(fa, ca, sa, ga, fw, cw, sw, gw, sp, M, N, K)
    case(f"gemm {fa}x{fw} {M}x{N}x{K} {out_dtype}")
    got = gpu_gemm(B, fa, ca, sa, ga, fw, cw, sw, gw, sp, out_dtype, ldc_pad=8)
    check(got, ref, out_dtype)


# decode shapes (M <= 128, in one, two or four row blocks of 32): several K
# splits and A windows (K a multiple of 512, or of 256 for four blocks), the
# smallest K, waves past N, and K the small-M kernel does not take (the tile
# kernel's)
@pytest.mark.parametrize("fa,fw", [("nvfp4", "nvfp4"), ("razer_a", "razer_w"), ("nvfp4", "razer_a")])
@pytest.mark.parametrize("M,N,K", [(5, 200, 2560), (32, 129, 4096), (1, 384, 4096), (2, 70, 512), (3, 64, 1040),
                                   (9, 150, 2080), (40, 200, 2560), (64, 300, 1536), (70, 100, 2304),
                                   (128, 64, 1024), (100, 129, 2048)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_decode_shapes(B, fa, fw, M, N, K, out_dtype):
    a = datagen.student_t((M, K), 700 + M, 4.0)
    w = datagen.normal((N, K), 800 + N, 0.02)
    sp = SPECIAL if fw == "razer_w" else None
    ca, sa, ga = oquant(a, fa)
    cw, sw, gw = oquant(w, fw, special=sp)
    ref = O.gemm_rows(fa, ca, sa, ga, fw, cw, sw, gw, sp, M, N, K)
    case(f"gemm decode {fa}x{fw} {M}x{N}x{K} {out_dtype}")
    got = gpu_gemm(B, fa, ca, sa, ga, fw, cw, sw, gw, sp, out_dtype)
    check(got, ref, out_dtype)


# MXFP4 shapes with K % 512 == 0 (the LDS-DMA staging path, scales loaded per
# group of four 128-element stages): ragged M and N, one group (K = 512),
# FP32 output with few tiles (K splits rounded to whole groups, some splits
# left empty) and bf16 output
@pytest.mark.parametrize("M,N,K", [(300, 260, 1024), (64, 96, 2048), (257, 129, 512), (33, 300, 1536),
                                   (1, 1, 512), (2, 40, 1024), (1, 300, 2560)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_mxfp4_group_staging(B, M, N, K, out_dtype):
    a = datagen.student_t((M, K), 920 + M, 4.0)
    w = datagen.normal((N, K), 921 + N, 0.02)
    ca, sa, ga = oquant(a, "mxfp4")
    cw, sw, gw = oquant(w, "mxfp4")
    ref = O.gemm_rows("mxfp4", ca, sa, ga, "mxfp4", cw, sw, gw, None, M, N, K)
    case(f"gemm mxfp4 group staging {M}x{N}x{K} {out_dtype}")
    got = gpu_gemm(B, "mxfp4", ca, sa, ga, "mxfp4", cw, sw, gw, None, out_dtype)
    check(got, ref, out_dtype)


# NVFP4-family shapes with K % 256 == 0 and M > 128 (the tile kernel's
# LDS-DMA staging in pairs of stages): 2, 3, 5 and 7 pairs cover the tail
# variants (one to three pairs after the four-stage main loop, with and
# without a load in the tail); FP32 output on two tiles also splits K into
# pair-aligned ranges
@pytest.mark.parametrize("fa,fw", [("nvfp4", "nvfp4"), ("razer_a", "razer_w")])
@pytest.mark.parametrize("K", [512, 768, 1280, 1792])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_nvfp4_pair_staging(B, fa, fw, K, out_dtype):
    M, N = 200, 300
    a = datagen.student_t((M, K), 960 + K, 4.0)
    w = datagen.normal((N, K), 961 + K, 0.02)
    sp = SPECIAL if fw == "razer_w" else None
    ca, sa, ga = oquant(a, fa)
    cw, sw, gw = oquant(w, fw, special=sp)
    ref = O.gemm_rows(fa, ca, sa, ga, fw, cw, sw, gw, sp, M, N, K)
    case(f"gemm pair staging {fa}x{fw} {M}x{N}x{K} {out_dtype}")
    got = gpu_gemm(B, fa, ca, sa, ga, fw, cw, sw, gw, sp, out_dtype)
    check(got, ref, out_dtype)


# scale rows at any byte alignment (only codes and C must be 16-byte aligned):
# 16-byte aligned scales take the MXFP4 LDS-DMA path when K % 512 == 0, word
# aligned ones the register path with word loads, others byte loads
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("off", [0, 1, 4, 8])
def test_gemm_scale_alignment(B, fmt, off):
    import torch
    M, N, K = 200, 300, 1024
    a = datagen.student_t((M, K), 930 + off, 4.0)
    w = datagen.normal((N, K), 931 + off, 0.02)
    ca, sa, ga = oquant(a, fmt)
    cw, sw, gw = oquant(w, fmt)
    ref = O.gemm_rows(fmt, ca, sa, ga, fmt, cw, sw, gw, None, M, N, K)

    def shifted(arr):
        buf = torch.zeros(arr.size + 32, dtype=torch.uint8, device="cuda")
        v = buf[off:off + arr.size].view(arr.shape)
        v.copy_(dev(arr))
        return buf, v
    bufa, sa_d = shifted(sa)
    bufw, sw_d = shifted(sw)
    assert sa_d.data_ptr() % 16 == off and sw_d.data_ptr() % 16 == off
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    case(f"gemm {fmt} {M}x{N}x{K} scales at byte offset {off}")
    B.gemm(fmt, dev(ca), sa_d, scalar_dev(ga), fmt, dev(cw), sw_d, scalar_dev(gw), None, out=out)
    torch.cuda.synchronize()
    assert rel_fro(host(out), ref) <= TOL


def _high_low_word_offset(lo, nbytes):
    """Byte offset (a multiple of 256) from an address whose low 32 bits are
    `lo` to the first one whose low 32 bits lie in [2^31, 2^32 - nbytes]."""
    if 2**31 <= lo and lo + nbytes <= 2**32:
        return 0
    return ((2**32 + 2**31 - lo) % 2**32 + 255) & ~255


def test_high_low_word_offset():
    for lo in (0, 256, 2**31 - 512, 2**31, 2**32 - 4096, 2**32 - 256):
        off = _high_low_word_offset(lo, 4096)
        assert off % 256 == 0 and off <= 2**31 + 4096
        assert 2**31 <= (lo + off) % 2**32 <= 2**32 - 4096


# C where the low 32 bits of every tile's address have bit 31 set: the
# epilogue forms 64-bit addresses from two 32-bit halves.  K = 128 is one
# stage, so FP32 output runs without K splits; 300 x 260 has whole wave tiles
# and ragged ones.
@pytest.mark.parametrize("fa,fw", [("nvfp4", "nvfp4"), ("mxfp4", "mxfp4")])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_output_address_low_word_above_2g(B, fa, fw, out_dtype):
    import torch
    M, N, K = 300, 260, 128
    a = datagen.student_t((M, K), 910, 4.0)
    w = datagen.normal((N, K), 911, 0.02)
    ca, sa, ga = oquant(a, fa)
    cw, sw, gw = oquant(w, fw)
    ref = O.gemm_rows(fa, ca, sa, ga, fw, cw, sw, gw, None, M, N, K)
    dt, es = (torch.float32, 4) if out_dtype == "f32" else (torch.bfloat16, 2)
    ld = -(-N // (16 // es)) * (16 // es)
    nbytes = M * ld * es
    big = torch.empty(2**31 + 2**22, dtype=torch.uint8, device="cuda")
    off = _high_low_word_offset(big.data_ptr() % 2**32, nbytes)
    assert off + nbytes <= big.numel() and (big.data_ptr() + off) % 2**32 >= 2**31
    out = big[off:off + nbytes].view(dt).view(M, ld)
    c = out[:, :N]
    case(f"gemm {fa}x{fw} {M}x{N}x{K} {out_dtype} at low word {(big.data_ptr() + off) % 2**32:#x}")
    B.gemm(fa, dev(ca), dev(sa), scalar_dev(ga), fw, dev(cw), dev(sw), scalar_dev(gw), None, out=c)
    torch.cuda.synchronize()
    got = host(c)
    if out_dtype != "f32":
        got = datagen.bf16_bits_to_f32(got)
    del out, c, big
    check(got, ref, out_dtype)


@pytest.mark.parametrize("fa,fw", [("nvfp4", "nvfp4"), ("mxfp4", "mxfp4"), ("razer_a", "razer_w")])
def test_gemm_exact_regime_bitwise(B, fa, fw):
    # g = 1, every block scale 1 (E4M3 code 56, E8M0 127, E3M3 code 24), K <= 256:
    # every partial sum is a multiple of 2^-2 below 2^14, exact in FP32, so the
    # result does not depend on the summation order
    M, N, K = 48, 80, 256
    g = datagen.rng(7)
    grid = np.array([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    a = g.choice(grid, (M, K)).astype(np.float32)
    w = g.choice(grid, (N, K)).astype(np.float32)
    bs = 32 if fa == "mxfp4" else 16
    a[:, ::bs] = 6.0
    w[:, ::bs] = -6.0
    sp = SPECIAL if fw == "razer_w" else None
    if fa == "mxfp4":
        a[:, ::bs] = 4.0  # max in [4, 8) gives E = 0
        w[:, ::bs] = -4.0
    ca, sa, ga = O.quantize(a, fa, bs, O.ABSMAX, O.G_NONE)
    cw, sw, gw = O.quantize(w, fw, bs, O.ABSMAX, O.G_NONE, special=sp)
    ref = O.gemm_rows(fa, ca, sa, ga, fw, cw, sw, gw, sp, M, N, K)
    case(f"gemm exact {fa}x{fw}")
    got = gpu_gemm(B, fa, ca, sa, ga, fw, cw, sw, gw, sp)
    assert np.array_equal(got, ref)


def test_gemm_razer_special_codes_decode(B):
    # a weight made of special values only: every W element is code 0x8
    M, N, K = 32, 40, 64
    a = datagen.normal((M, K), 800)
    ca, sa, ga = oquant(a, "nvfp4")
    sp = (2.5, -7.5, 5.0, -3.5)
    w = np.tile(np.array([2.5, -7.5, 5.0, -3.5] * (K // 4), np.float32), (N, 1))
    cw, sw, gw = O.quantize(w, "razer_w", 16, O.ABSMAX, O.G_NONE, special=sp)
    ref = O.gemm_rows("nvfp4", ca, sa, ga, "razer_w", cw, sw, gw, sp, M, N, K)
    case("gemm razer special-only weight")
    got = gpu_gemm(B, "nvfp4", ca, sa, ga, "razer_w", cw, sw, gw, sp)
    assert rel_fro(got, ref) <= TOL


# ------------------------------------------------------------------ full-size workloads
def spliced_gemm(B, fa, fw, a_src, w_src, a_rows, w_rows, a_fmt_args, w_fmt_args, special=None, out_bf16=False):
    """GPU-quantize the full operands (fast), overwrite the sampled rows with the
    oracle's quantization of those rows (oracle global scales used for both),
    run the GPU GEMM and compare the entries (a_rows x w_rows) with the oracle."""
    import torch
    block = 32 if fa == "mxfp4" else 16

    def prep(x_np, x_gpu, fmt, args, rows, sp):
        rule, gmode, t, had = args
        if gmode == "auto":
            g = O.auto_global(O.transform(x_np, t, had), fmt)
        else:
            g = 1.0
        gbuf = scalar_dev(g)
        mode = "given" if gmode == "auto" else gmode
        case(f"gemm operand quantize {fmt} {tuple(x_gpu.shape)}")
        codes, scales, _ = B.quantize(x_gpu, fmt, block, rule, mode, chan_scale=dev(t) if t is not None else None,
                                      hadamard=had, special=sp or (0.0,) * 4, global_=gbuf)
        orule = {"absmax": O.ABSMAX, "4over6": O.FOUR_OVER_SIX}[rule]
        oc, os_ = O.quantize_rows(O.transform(x_np[rows], t, had), fmt, block, orule, g, sp)
        idx = torch.as_tensor(rows, device="cuda")
        codes.index_copy_(0, idx, dev(oc))
        scales.index_copy_(0, idx, dev(os_))
        return codes, scales, g, oc, os_

    ac, as_, ga, oac, oas = prep(*a_src, fa, a_fmt_args, a_rows, None)
    wc, ws, gw, owc, ows = prep(*w_src, fw, w_fmt_args, w_rows, special)
    M, N, K = ac.shape[0], wc.shape[0], 2 * ac.shape[1]
    case(f"gemm full {fa}x{fw} {M}x{N}x{K}")
    out = torch.empty((M, N), dtype=torch.bfloat16 if out_bf16 else torch.float32, device="cuda")
    B.gemm(fa, ac, as_, scalar_dev(ga), fw, wc, ws, scalar_dev(gw), special, out=out)
    torch.cuda.synchronize()
    sub = out.index_select(0, torch.as_tensor(a_rows, device="cuda")).index_select(1, torch.as_tensor(w_rows, device="cuda"))
    got = host(sub)
    if out_bf16:
        got = datagen.bf16_bits_to_f32(got)
    ref = O.gemm_rows(fa, oac, oas, ga, fw, owc, ows, gw, special, len(a_rows), len(w_rows), K)
    return got, ref


def rows_of(n, k, seed):
    idx = datagen.rng(seed).choice(n, size=min(k, n), replace=False)
    return np.sort(np.concatenate([idx, [0, n - 1]])).astype(np.int64)


def test_tiny_workload_full(B):
    d = datagen.tiny()
    ca, sa, _ = O.quantize(d["A"], "nvfp4", 16, O.ABSMAX, O.G_NONE)
    for rule in (O.ABSMAX, O.FOUR_OVER_SIX, O.BRUTE):
        cw, sw, _ = O.quantize(d["W"], "nvfp4", 16, rule, O.G_NONE)
        ref = O.gemm_rows("nvfp4", ca, sa, 1.0, "nvfp4", cw, sw, 1.0, None, 64, 256, 256)
        case(f"gemm tiny workload rule {rule}")
        got = gpu_gemm(B, "nvfp4", ca, sa, 1.0, "nvfp4", cw, sw, 1.0, None)
        assert rel_fro(got, ref) <= TOL


def test_mxfp4_linear_workload(B):
    d = datagen.mxfp4_linear()
    t, r = O.channel_scale(d["X_bf16"], d["W"], 0.75)
    got, ref = spliced_gemm(B, "mxfp4", "mxfp4", (d["X_bf16"], dev(d["X_bf16"], bf16=True)), (d["W"], dev(d["W"])),
                            rows_of(4096, 24, 50), rows_of(14336, 96, 51),
                            ("absmax", "none", t, 32), ("absmax", "none", r, 32))
    assert rel_fro(got, ref) <= TOL


@pytest.mark.parametrize("M", [1, 16, 128])
def test_razer_decode_workload(B, M):
    d = datagen.razer_decode(M)
    a = d["A_bf16"]
    got, ref = spliced_gemm(B, "razer_a", "razer_w", (a, dev(a, bf16=True)), (d["W"], dev(d["W"])),
                            np.arange(M, dtype=np.int64) if M <= 16 else rows_of(M, 16, 60), rows_of(17408, 256, 61),
                            ("absmax", "auto", None, 0), ("absmax", "auto", None, 0), special=SPECIAL)
    assert rel_fro(got, ref) <= TOL


@pytest.mark.parametrize("N", datagen.PREFILL_N)
def test_prefill_workload(B, N):
    a = datagen.prefill_act()
    w = datagen.prefill_weight(N)
    got, ref = spliced_gemm(B, "nvfp4", "nvfp4", (a, dev(a, bf16=True)), (w, dev(w)),
                            rows_of(32768, 12, 70), rows_of(N, 64, 71),
                            ("4over6", "auto", None, 0), ("4over6", "auto", None, 0), out_bf16=(N == 17408))
    check(got, ref, "bf16" if N == 17408 else "f32")


# Launches with few output tiles split K; the splits' partial results are
# added by a separate pass in split order, so repeated launches give the same
# bytes: the decode workload at M = 16 and 128 (small-M kernel) and two-tile
# shapes of the tile kernel, both formats.  Parity at these shapes is the
# business of the workload and staging tests.
@pytest.mark.parametrize("fa,fw,M,N,K", [("razer_a", "razer_w", 128, 17408, 5120), ("nvfp4", "nvfp4", 200, 300, 1024),
                                         ("mxfp4", "mxfp4", 200, 300, 2048), ("nvfp4", "nvfp4", 16, 17408, 5120)])
def test_gemm_fp32_split_k_is_deterministic(B, fa, fw, M, N, K):
    import torch
    a = datagen.student_t((M, K), 980 + M, 4.0)
    w = datagen.normal((N, K), 981, 0.02)
    sp = SPECIAL if fw == "razer_w" else None
    block = 32 if fa == "mxfp4" else 16
    gm = "none" if fa == "mxfp4" else "auto"
    case(f"gemm determinism {fa}x{fw} {M}x{N}x{K}: operands")
    ac, as_, ag = B.quantize(dev(a), fa, block, "absmax", gm)
    wc, ws, wg = B.quantize(dev(w), fw, block, "absmax", gm, special=sp or (0.0,) * 4)
    outs = []
    for i in range(3):
        case(f"gemm determinism {fa}x{fw} {M}x{N}x{K}: launch {i}")
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        B.gemm(fa, ac, as_, ag, fw, wc, ws, wg, sp, out=out)
        torch.cuda.synchronize()
        outs.append(host(out).view(np.uint32).copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    assert np.all(np.isfinite(outs[0].view(np.float32)))  # every entry written


# M = 1 (the matrix-vector kernel): K from one block to 8192 (1, 2, 3, 5 and 8
# blocks per lane, ragged block counts that leave lanes past the row end), N
# from one row to more rows than the launch has waves, every format pair of
# the NVFP4 family, both output types; and K past the kernel's limit
@pytest.mark.parametrize("fa,fw", [("nvfp4", "nvfp4"), ("razer_a", "razer_w"), ("razer_a", "nvfp4"),
                                   ("nvfp4", "razer_a")])
@pytest.mark.parametrize("N,K", [(1, 16), (33, 272), (300, 1040), (129, 2064), (70, 3072), (5000, 5120),
                                 (64, 8192), (40, 8208)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_single_row(B, fa, fw, N, K, out_dtype):
    a = datagen.student_t((1, K), 900 + K, 4.0)
    w = datagen.normal((N, K), 910 + N, 0.02)
    sp = SPECIAL if fw == "razer_w" else None
    ca, sa, ga = oquant(a, fa)
    cw, sw, gw = oquant(w, fw, special=sp)
    ref = O.gemm_rows(fa, ca, sa, ga, fw, cw, sw, gw, sp, 1, N, K)
    case(f"gemm single row {fa}x{fw} 1x{N}x{K} {out_dtype}")
    got = gpu_gemm(B, fa, ca, sa, ga, fw, cw, sw, gw, sp, out_dtype)
    check(got, ref, out_dtype)


@pytest.mark.parametrize("fa,fw", [("nvfp4", "nvfp4"), ("razer_a", "razer_w")])
def test_gemm_single_row_exact_regime_bitwise(B, fa, fw):
    # unit scales and g = 1, K = 1024: every partial sum is a multiple of 2^-2
    # below 2^14, exact in FP32 in any order, so the row equals the oracle's
    N, K = 200, 1024
    g = datagen.rng(17)
    grid = np.array([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    a = g.choice(grid, (1, K)).astype(np.float32)
    w = g.choice(grid, (N, K)).astype(np.float32)
    a[:, ::16] = 6.0
    w[:, ::16] = -6.0
    sp = SPECIAL if fw == "razer_w" else None
    ca, sa, ga = O.quantize(a, fa, 16, O.ABSMAX, O.G_NONE)
    cw, sw, gw = O.quantize(w, fw, 16, O.ABSMAX, O.G_NONE, special=sp)
    ref = O.gemm_rows(fa, ca, sa, ga, fw, cw, sw, gw, sp, 1, N, K)
    case(f"gemm single row exact {fa}x{fw}")
    got = gpu_gemm(B, fa, ca, sa, ga, fw, cw, sw, gw, sp)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("special", [(7.5, -3.5, 4.5, -6.5), (-7.5, 7.5, 3.5, -2.5)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_single_row_wide_specials(B, special, out_dtype):
    # RaZeR-W tables with four-significant-bit specials (7.5, 6.5, 4.5): their
    # f16 patterns need the low byte; the row sums stay exact
    N, K = 700, 5120
    a = datagen.student_t((1, K), 950, 4.0)
    w = datagen.normal((N, K), 951, 0.02)
    ca, sa, ga = oquant(a, "razer_a")
    cw, sw, gw = oquant(w, "razer_w", special=special)
    ref = O.gemm_rows("razer_a", ca, sa, ga, "razer_w", cw, sw, gw, special, 1, N, K)
    case(f"gemm single row wide specials {special} {out_dtype}")
    got = gpu_gemm(B, "razer_a", ca, sa, ga, "razer_w", cw, sw, gw, special, out_dtype)
    check(got, ref, out_dtype)
    # the same weight in the exact regime: unit scales, g = 1, K = 1024
    M1, K1 = 1, 1024
    g = datagen.rng(952)
    grid = np.array([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    a1 = g.choice(grid, (M1, K1)).astype(np.float32)
    w1 = np.concatenate([g.choice(grid, (64, K1)), g.choice(np.array(special, np.float32), (64, K1))]).astype(np.float32)
    a1[:, ::16] = 6.0
    w1[:, ::16] = -6.0
    ca1, sa1, ga1 = O.quantize(a1, "nvfp4", 16, O.ABSMAX, O.G_NONE)
    cw1, sw1, gw1 = O.quantize(w1, "razer_w", 16, O.ABSMAX, O.G_NONE, special=special)
    ref1 = O.gemm_rows("nvfp4", ca1, sa1, ga1, "razer_w", cw1, sw1, gw1, special, M1, 128, K1)
    got1 = gpu_gemm(B, "nvfp4", ca1, sa1, ga1, "razer_w", cw1, sw1, gw1, special)
    assert np.array_equal(got1, ref1)
