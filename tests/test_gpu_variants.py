"""GPU parity of the scale-format variants against the oracle, byte for byte:
UE5M3 block scales under every rule, the size-16 block-Hadamard in every
kernel that applies a rotation (with the automatic global scale on both of
its launch paths), and the MXFP4 exponent-offset search, on ragged tensors,
strided rows, extreme magnitudes and sampled rows of full-size workloads."""
import numpy as np
import pytest

import datagen
import oracle as O
from tests.gpu_util import case, dev, host, scalar_dev
from tests.test_gpu_quantize import mixed_tensor, run_pair, sample_rows, sampled_parity, to_input

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp4_e4m3_amd as B
    return B


def run_pair_rule(B, x_np, x_gpu, fmt, block, rule_name, orule, gmode, g_given=None, t=None, had=0):
    """run_pair for rules the shared helper does not name (the exponent search)"""
    import torch
    ogm = {"none": O.G_NONE, "given": O.G_GIVEN}[gmode]
    oc, os_, _ = O.quantize(x_np, fmt, block, orule, ogm, chan_scale=t, hadamard=had, g=g_given)
    case(f"quantize {fmt} B={block} {rule_name} g={gmode} {tuple(x_gpu.shape)} had={had} chan={t is not None}")
    codes, scales, _ = B.quantize(x_gpu, fmt, block, rule_name, gmode, chan_scale=dev(t) if t is not None else None,
                                  hadamard=had, global_=scalar_dev(g_given if g_given else 1.0))
    torch.cuda.synchronize()
    assert np.array_equal(host(scales), os_), "scales differ"
    assert np.array_equal(host(codes), oc), "codes differ"


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("block", [4, 8, 16, 32])
@pytest.mark.parametrize("rule", ["absmax", "absmax+pz", "4over6", "4over6+pz", "brute"])
@pytest.mark.parametrize("gmode", ["none", "given"])
def test_ue5m3_small(B, bf16, block, rule, gmode):
    x = mixed_tensor(37, 256, seed=5000 + block)
    xn, xg = to_input(x, bf16)
    run_pair(B, xn, xg, "ue5m3", block, rule, gmode, g_given=3.0e-3 if gmode == "given" else None)


def test_ue5m3_strided_and_extremes(B):
    # a row pitch past the row (the generic kernel), and magnitudes at both
    # ends of UE5M3's range with no global scale
    wide = mixed_tensor(23, 320, seed=5100)
    run_pair(B, np.ascontiguousarray(wide[:, :256]), dev(wide)[:, :256], "ue5m3", 16, "4over6", "none")
    g = datagen.rng(5101)
    x = (g.standard_normal((16, 128)) * np.exp2(g.uniform(-22, 22, (16, 1)))).astype(np.float32)
    for rule in ("absmax", "4over6", "absmax+pz"):
        run_pair(B, x, dev(x), "ue5m3", 16, rule, "none")
        run_pair(B, x, dev(x), "ue5m3", 32, rule, "none")


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("fmt,block,rule", [("nvfp4", 16, "4over6"), ("nvfp4", 32, "absmax"), ("nvfp4", 4, "4over6"),
                                            ("nvfp4", 8, "brute"), ("razer_a", 16, "absmax"),
                                            ("razer_w", 16, "absmax"), ("ue5m3", 16, "4over6")])
@pytest.mark.parametrize("chan", [False, True])
def test_hadamard16(B, bf16, fmt, block, rule, chan):
    x = mixed_tensor(21, 192, seed=5200 + block)
    xn, xg = to_input(x, bf16)
    t = None
    if chan:
        w = datagen.normal((40, 192), 5201, 0.02)
        t, _ = O.channel_scale(xn, w, 0.75)
    gmode = "none" if fmt == "ue5m3" else "auto"
    sp = datagen.RAZER_SPECIAL if fmt == "razer_w" else None
    run_pair(B, xn, xg, fmt, block, rule, gmode, t=t, had=16, special=sp)


@pytest.mark.parametrize("rows,cols", [(1, 4096), (3, 4096), (300, 1024)])
def test_hadamard16_auto_global_paths(B, rows, cols):
    # automatic g in the quantize launch itself (up to 8192 elements) and by
    # the separate abs-max pass
    x = datagen.student_t((rows, cols), 5300 + rows, 3.0)
    for bf16 in (False, True):
        xn, xg = to_input(x, bf16)
        run_pair(B, xn, xg, "nvfp4", 16, "4over6", "auto", had=16)
        run_pair(B, xn, xg, "nvfp4", 16, "absmax", "auto", had=16, t=(datagen.rng(5301).random(cols) + 0.5)
                 .astype(np.float32))


def extreme_rows(rows, cols, seed):
    """mixed rows plus rows near the bottom of the FP32 range, where the
    exponent search's lowest candidate is subnormal"""
    x = mixed_tensor(rows, cols, seed)
    g = datagen.rng(seed + 1)
    for r in range(0, rows, 5):
        x[r] = (g.standard_normal(cols) * 2.0 ** -124).astype(np.float32)
    return x


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("chan,had", [(False, 0), (True, 32), (False, 16), (True, 0)])
def test_mxfp4_expsearch(B, bf16, chan, had):
    x = extreme_rows(41, 256, 5400) if not bf16 else mixed_tensor(41, 256, 5400)
    xn, xg = to_input(x, bf16)
    t = None
    if chan:
        w = datagen.normal((64, 256), 5401, 0.02)
        t, _ = O.channel_scale(xn, w, 0.75)
    run_pair_rule(B, xn, xg, "mxfp4", 32, "expsearch", O.EXPSEARCH, "none", t=t, had=had)
    # and the standard exponent with the size-16 rotation
    if had == 16:
        run_pair(B, xn, xg, "mxfp4", 32, "absmax", "none", t=t, had=16)


def test_mxfp4_expsearch_linear_workload(B):
    # the MXFP4 linear workload's activations (bf16, 8 outlier channels) with
    # the channel scale and the size-32 rotation, and its weights, under the
    # exponent search: sampled rows at full size
    import torch
    d = datagen.mxfp4_linear()
    t, r = O.channel_scale(d["X_bf16"], d["W"], 0.75)
    for name, x_np, x_gpu, tt, rows in (("X", d["X_bf16"], dev(d["X_bf16"], bf16=True), t, sample_rows(4096, 48, 24)),
                                        ("W", d["W"], dev(d["W"]), r, sample_rows(14336, 48, 25))):
        case(f"mxfp4 expsearch full {name}")
        codes, scales, _ = B.quantize(x_gpu, "mxfp4", 32, "expsearch", "none", chan_scale=dev(tt), hadamard=32)
        torch.cuda.synchronize()
        idx = torch.as_tensor(rows, device="cuda")
        oc, os_ = O.quantize_rows(O.transform(x_np[rows], tt, 32), "mxfp4", 32, O.EXPSEARCH, 1.0)
        assert np.array_equal(host(scales.index_select(0, idx)), os_)
        assert np.array_equal(host(codes.index_select(0, idx)), oc)


def test_ue5m3_sweep_workload(B):
    x = datagen.sweep("student_t3")
    xg = dev(x)
    for block in (4, 8, 16, 32):
        for rule in ("absmax", "4over6"):
            sampled_parity(B, x, xg, "ue5m3", block, rule, "none", sample_rows(4096, 32, 60 + block))


@pytest.mark.parametrize("block", [4, 16, 32])
def test_ue5m3_dequantize_bitexact(B, block):
    import torch
    x = datagen.student_t((33, 128), 5500 + block, 3.0) * np.float32(2.0 ** -9)
    codes, scales, _ = O.quantize(x, "ue5m3", block, O.FOUR_OVER_SIX, O.G_NONE)
    ref = O.dequantize(codes, scales, "ue5m3", block)
    for out in ("f32", "bf16"):
        case(f"dequantize ue5m3 B={block} -> {out}")
        got = B.dequantize(dev(codes), dev(scales), "ue5m3", block, None,
                           out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
        torch.cuda.synchronize()
        got = host(got)
        if out == "f32":
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
        else:
            assert np.array_equal(got, datagen.to_bf16_bits(ref))
