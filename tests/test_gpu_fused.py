"""GPU parity of the matmul that quantizes bf16 activations as it loads them
and of the per-segment weight global scales of fused projections.

* Activations quantized on load: the codes and scales it can hand back are
  the oracle quantizer's, byte for byte (NVFP4, block 16, abs-max or
  4-over-6, GIVEN or no global scale); C is the oracle's matmul of those
  codes within the W4A4 tolerance, and bit for bit where every partial sum is
  exact in FP32.
* Segments: each segment's columns against the oracle's matmul of that
  segment alone with its own global scale; equal segment scales give the
  unsegmented launch's bytes; power-of-two ratios between segment scales
  scale those bytes exactly."""
import numpy as np
import pytest

import datagen
import oracle as O
from tests.gpu_util import case, dev, host, rel_fro, scalar_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3
SPECIAL = datagen.RAZER_SPECIAL
ORULE = {"absmax": O.ABSMAX, "4over6": O.FOUR_OVER_SIX}


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp4_e4m3_amd as B
    return B


def oweight(N, K, seed, fw):
    w = datagen.normal((N, K), seed, 0.02)
    sp = SPECIAL if fw == "razer_w" else None
    codes, scales, g = O.quantize(w, fw, 16, O.ABSMAX, O.G_AUTO, special=sp)
    return codes, scales, g, sp


def run_act(B, a_bits, rule, g_a, fw, cw, sw, gw, sp, out_dtype="f32", seg_rows=None):
    import torch
    M, K = a_bits.shape
    N = cw.shape[0]
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    per16 = 4 if out_dtype == "f32" else 8
    ld = -(-(N + 8) // per16) * per16
    out = torch.full((M, ld), float("nan"), dtype=dt, device="cuda")
    c = out[:, :N]
    wg = dev(np.asarray(gw, np.float32).reshape(-1)) if gw is not None else None
    case(f"act-quantized matmul {rule} x {fw} {M}x{N}x{K} {out_dtype} g_a={g_a} seg={seg_rows}")
    _, codes, scales = B.gemm_act_bf16(dev(a_bits, bf16=True), rule, scalar_dev(g_a) if g_a is not None else None, fw,
                                       dev(cw), dev(sw), wg, seg_rows, sp, out=c, keep_codes=True)
    torch.cuda.synchronize()
    r = host(c)
    if out_dtype != "f32":
        r = datagen.bf16_bits_to_f32(r)
    return r, host(codes), host(scales)


def oracle_act(a_bits, rule, g_a, fw, cw, sw, gw, sp):
    gm = O.G_GIVEN if g_a is not None else O.G_NONE
    oc, os_, g = O.quantize(a_bits, "nvfp4", 16, ORULE[rule], gm, g=g_a)
    M, K = a_bits.shape
    ref = O.gemm_rows("nvfp4", oc, os_, g, fw, cw, sw, gw, sp, M, cw.shape[0], K)
    return oc, os_, ref


@pytest.mark.parametrize("rule", ["absmax", "4over6"])
@pytest.mark.parametrize("fw", ["nvfp4", "razer_a", "razer_w"])
@pytest.mark.parametrize("M", [1, 7, 32, 33, 100, 128, 130])
@pytest.mark.parametrize("N,K", [(96, 512), (300, 1024)])
def test_act_bf16_small(B, rule, fw, M, N, K):
    cw, sw, gw, sp = oweight(N, K, 9000 + N, fw)
    a = datagen.to_bf16_bits(datagen.student_t((M, K), 9100 + M, 4.0))
    g_a = None if M % 2 else 0.75 * O.auto_global(datagen.bf16_bits_to_f32(a), "nvfp4")
    out_dtype = "bf16" if M == 33 else "f32"
    got, codes, scales = run_act(B, a, rule, g_a, fw, cw, sw, gw, sp, out_dtype)
    oc, os_, ref = oracle_act(a, rule, g_a, fw, cw, sw, gw, sp)
    assert np.array_equal(scales, os_), "scales differ"
    assert np.array_equal(codes, oc), "codes differ"
    if out_dtype == "bf16":
        ref = datagen.bf16_bits_to_f32(datagen.to_bf16_bits(ref))
    assert rel_fro(got, ref) <= TOL


@pytest.mark.parametrize("rule", ["absmax", "4over6"])
@pytest.mark.parametrize("M", [5, 64, 128])
def test_act_bf16_exact_regime_bitwise(B, rule, M):
    # every activation block holds a +-6 and E2M1 values (scale 1 at g = 1,
    # codes exact); weight scales 1: each product is a multiple of 0.25 below
    # 37 and every partial sum is exact in FP32 in any order
    N, K = 130, 1024
    g = datagen.rng(9200 + M)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    a = vals[g.integers(0, 8, (M, K))] * np.where(g.random((M, K)) < 0.5, -1, 1).astype(np.float32)
    a[:, ::16] = 6.0
    a_bits = datagen.to_bf16_bits(a.astype(np.float32))
    cw = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sw = np.full((N, K // 16), 56, np.uint8)  # E4M3 1.0
    got, codes, scales = run_act(B, a_bits, rule, None, "nvfp4", cw, sw, 1.0, None)
    oc, os_, ref = oracle_act(a_bits, rule, None, "nvfp4", cw, sw, 1.0, None)
    assert np.array_equal(codes, oc) and np.array_equal(scales, os_)
    assert np.all(scales == 56)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def rows_of(n, k, seed):
    idx = datagen.rng(seed).choice(n, size=min(k, n), replace=False)
    return np.sort(np.concatenate([idx, [0, n - 1]])).astype(np.int64)


@pytest.mark.parametrize("M", [1, 16, 128])
def test_act_bf16_decode_workload(B, M):
    # decode-sized activations (K 5120) quantized on load with 4-over-6 under
    # a GIVEN global scale against the 17408 x 5120 RaZeR-W weight: every
    # activation code and scale, and C at sampled weight rows
    import torch
    d = datagen.razer_decode(M)
    a, w = d["A_bf16"], d["W"]
    N, K = w.shape
    g_w = O.auto_global(w, "razer_w")
    g_a = O.auto_global(datagen.bf16_bits_to_f32(a), "nvfp4")
    wr = rows_of(N, 192, 9300)
    case(f"act-quantized decode M={M}: weight quantize")
    cw, sw, _ = B.quantize(dev(w), "razer_w", 16, "absmax", "given", special=SPECIAL, global_=scalar_dev(g_w))
    ocw, osw = O.quantize_rows(w[wr], "razer_w", 16, O.ABSMAX, g_w, SPECIAL)
    idx = torch.as_tensor(wr, device="cuda")
    cw.index_copy_(0, idx, dev(ocw))
    sw.index_copy_(0, idx, dev(osw))
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    case(f"act-quantized decode M={M}: matmul")
    _, codes, scales = B.gemm_act_bf16(dev(a, bf16=True), "4over6", scalar_dev(g_a), "razer_w", cw, sw,
                                       scalar_dev(g_w), None, SPECIAL, out=out, keep_codes=True)
    torch.cuda.synchronize()
    oc, os_, _ = O.quantize(a, "nvfp4", 16, O.FOUR_OVER_SIX, O.G_GIVEN, g=g_a)
    assert np.array_equal(host(scales), os_) and np.array_equal(host(codes), oc)
    got = host(out.index_select(1, idx))
    ref = O.gemm_rows("nvfp4", oc, os_, g_a, "razer_w", ocw, osw, g_w, SPECIAL, M, len(wr), K)
    assert rel_fro(got, ref) <= TOL


# ---------------------------------------------------------------- segments
def concat_weights(fw, segs, K, seed):
    parts = [oweight(n, K, seed + i, fw) for i, n in enumerate(segs)]
    cw = np.concatenate([p[0] for p in parts])
    sw = np.concatenate([p[1] for p in parts])
    gs = np.array([p[2] for p in parts], np.float32)
    return cw, sw, gs, parts[0][3], parts


@pytest.mark.parametrize("fa,fw", [("nvfp4", "nvfp4"), ("razer_a", "razer_w"), ("mxfp4", "mxfp4")])
@pytest.mark.parametrize("M,K", [(1, 512), (64, 256), (300, 1024)])
@pytest.mark.parametrize("segs", [(96, 32, 40), (256, 256, 512, 64), (130,)])
def test_segmented_matches_each_segment(B, fa, fw, M, K, segs):
    import torch
    block = 32 if fa == "mxfp4" else 16
    N = sum(segs)
    a = datagen.student_t((M, K), 9400 + M, 4.0)
    gm = O.G_NONE if fa == "mxfp4" else O.G_AUTO
    ca, sa, ga = O.quantize(a, fa, block, O.ABSMAX, gm)
    if fa == "mxfp4":
        ws = [datagen.normal((n, K), 9500 + i, 0.02 * (i + 1)) for i, n in enumerate(segs)]
        parts = [O.quantize(w, "mxfp4", 32, O.ABSMAX, O.G_NONE) for w in ws]
        cw = np.concatenate([p[0] for p in parts])
        sw = np.concatenate([p[1] for p in parts])
        gs = np.array([0.5 * (i + 1) for i in range(len(segs))], np.float32)  # any per-segment factor
        sp = None
    else:
        cw, sw, gs, sp, parts = concat_weights(fw, segs, K, 9500)
    out = torch.full((M, -(-N // 4) * 4), float("nan"), dtype=torch.float32, device="cuda")[:, :N]
    case(f"segmented {fa}x{fw} M={M} K={K} segs={segs}")
    B.gemm_segmented(fa, dev(ca), dev(sa), scalar_dev(ga), fw, dev(cw), dev(sw), dev(gs), list(segs), sp, out=out)
    torch.cuda.synchronize()
    got = host(out)
    n0 = 0
    for i, n in enumerate(segs):
        ref = O.gemm_rows(fa, ca, sa, ga, fw, cw[n0:n0 + n], sw[n0:n0 + n], float(gs[i]), sp, M, n, K)
        assert rel_fro(got[:, n0:n0 + n], ref) <= TOL, i
        n0 += n


@pytest.mark.parametrize("M,N,K", [(16, 17408, 5120), (300, 700, 1024), (1, 4096, 512)])
def test_segmented_scale_identities(B, M, N, K):
    # equal segment scales give the unsegmented launch's bytes; segment
    # scales g 2^e_i give those bytes times 2^e_i exactly
    import torch
    a = datagen.student_t((M, K), 9600 + M, 4.0)
    w = datagen.normal((N, K), 9601, 0.02)
    case(f"segment identities {M}x{N}x{K}: operands")
    ca, sa, ga = B.quantize(dev(a), "nvfp4", 16, "absmax", "auto")
    cw, sw, gw = B.quantize(dev(w), "nvfp4", 16, "absmax", "auto")
    segs = [N // 2, N // 4, N - N // 2 - N // 4]
    base = torch.empty((M, N), dtype=torch.float32, device="cuda")
    B.gemm("nvfp4", ca, sa, ga, "nvfp4", cw, sw, gw, None, out=base)
    same = torch.empty_like(base)
    B.gemm_segmented("nvfp4", ca, sa, ga, "nvfp4", cw, sw, gw.repeat(3), segs, None, out=same)
    shifts = torch.tensor([1.0, 4.0, 0.125], dtype=torch.float32, device="cuda")
    scaled = torch.empty_like(base)
    B.gemm_segmented("nvfp4", ca, sa, ga, "nvfp4", cw, sw, gw.repeat(3) * shifts, segs, None, out=scaled)
    torch.cuda.synchronize()
    hb, hs, hx = host(base), host(same), host(scaled)
    assert np.array_equal(hb.view(np.uint32), hs.view(np.uint32))
    ref = np.concatenate([hb[:, :segs[0]], hb[:, segs[0]:segs[0] + segs[1]] * np.float32(4.0),
                          hb[:, segs[0] + segs[1]:] * np.float32(0.125)], axis=1)
    assert np.array_equal(hx.view(np.uint32), ref.view(np.uint32))


def test_act_bf16_fused_projection_segments(B):
    # a decode-sized fused projection: three weights (4096, 1024 and 1024
    # rows, K 5120), each under its own global scale, against activations
    # quantized on load; each segment against the oracle alone
    segs = (4096, 1024, 1024)
    K, M = 5120, 4
    cw, sw, gs, _, _ = concat_weights("nvfp4", segs, K, 9700)
    a = datagen.to_bf16_bits(datagen.student_t((M, K), 9701, 4.0))
    g_a = O.auto_global(datagen.bf16_bits_to_f32(a), "nvfp4")
    got, codes, scales = run_act(B, a, "4over6", g_a, "nvfp4", cw, sw, gs, None, seg_rows=list(segs))
    oc, os_, _ = O.quantize(a, "nvfp4", 16, O.FOUR_OVER_SIX, O.G_GIVEN, g=g_a)
    assert np.array_equal(codes, oc) and np.array_equal(scales, os_)
    n0 = 0
    for i, n in enumerate(segs):
        ref = O.gemm_rows("nvfp4", oc, os_, g_a, "nvfp4", cw[n0:n0 + n], sw[n0:n0 + n], float(gs[i]), None, M, n, K)
        assert rel_fro(got[:, n0:n0 + n], ref) <= TOL, i
        n0 += n
