"""GPU parity of fp4q_dequantize (bit-exact) and fp4q_channel_scale (within
binary64-sum rounding) against the oracle."""
import numpy as np
import pytest

import datagen
import oracle as O
from tests.gpu_util import case, dev, host, scalar_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp4_e4m3_amd as B
    return B


@pytest.mark.parametrize("fmt,block", [("nvfp4", 4), ("nvfp4", 8), ("nvfp4", 16), ("nvfp4", 32), ("mxfp4", 32),
                                       ("razer_a", 16), ("razer_w", 16), ("razer_w", 4)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_bitexact(B, fmt, block, out):
    import torch
    x = datagen.student_t((45, 192), 900 + block, 3.0)
    sp = datagen.RAZER_SPECIAL if fmt == "razer_w" else None
    gm = O.G_NONE if fmt == "mxfp4" else O.G_AUTO
    codes, scales, g = O.quantize(x, fmt, block, O.ABSMAX, gm, special=sp)
    ref = O.dequantize(codes, scales, fmt, block, g, sp)
    case(f"dequantize {fmt} B={block} -> {out}")
    got = B.dequantize(dev(codes), dev(scales), fmt, block, scalar_dev(g) if gm != O.G_NONE else None,
                       special=sp or (0.0,) * 4, out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    got = host(got)
    if out == "f32":
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    else:
        assert np.array_equal(got, datagen.to_bf16_bits(ref))


def test_dequantize_odd_width_and_pitch(B):
    import torch
    x = datagen.normal((7, 12), 950)
    codes, scales, g = O.quantize(x, "nvfp4", 4, O.FOUR_OVER_SIX, O.G_AUTO)
    ref = O.dequantize(codes, scales, "nvfp4", 4, g)
    out = torch.zeros((7, 16), dtype=torch.float32, device="cuda")
    case("dequantize 7x12 pitch 16")
    desc = B.make_desc("nvfp4", 4)
    B.fp4q_dequantize(desc, dev(codes), dev(scales), scalar_dev(g), 7, 12, out, B.FP4Q_F32, 16)
    torch.cuda.synchronize()
    got = host(out)
    assert np.array_equal(got[:, :12], ref) and np.all(got[:, 12:] == 0)


@pytest.mark.parametrize("xbf16", [False, True])
def test_channel_scale(B, xbf16):
    import torch
    x = datagen.with_outlier_channels(datagen.normal((300, 256), 960), 961)[0]
    w = datagen.normal((500, 256), 962, 0.02)
    xn = datagen.to_bf16_bits(x) if xbf16 else x
    t_ref, r_ref = O.channel_scale(xn, w, 0.75)
    case(f"channel_scale bf16={xbf16}")
    t, r = B.channel_scale(dev(xn, bf16=xbf16), dev(w), 0.75)
    torch.cuda.synchronize()
    t, r = host(t), host(r)
    # binary64 sums in a different order: at most one fp32 ulp apart
    assert np.max(np.abs(t.view(np.int32).astype(np.int64) - t_ref.view(np.int32))) <= 1
    assert np.max(np.abs(r.view(np.int32).astype(np.int64) - r_ref.view(np.int32))) <= 2
    assert np.array_equal(r, (np.float32(1.0) / t).astype(np.float32))
