"""Pins of two oracle parts that every bf16 workload and the RaZeR weight side
rest on, each against something other than the oracle itself:

* the bf16 -> fp32 widening of the input (every finite bf16 bit pattern,
  against torch's bfloat16 decoder), through the transform, the channel
  scale and the quantizer;
* the RaZeR decode (RaZeR summary, sections 2.1 and 2.2): the scale byte's
  free bits pick the block's special value, which code 0x8 (the redundant
  zero) then stands for.  Checked in exact rational arithmetic from the
  pages' E2M1 value set, an E3M3 table enumerated here from its definition
  (6 bits, 3 exponent and 3 mantissa bits, bias 3, subnormals) and torch's
  E4M3 decoder.
"""
from fractions import Fraction

import numpy as np
import torch

import datagen
import oracle as O
from tests.exact_ref import e2m1_table, e4m3_lib_values


def all_finite_bf16() -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits.astype(np.uint32) >> 7) & 0xFF) != 0xFF
    return bits[finite]


def torch_widen(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.float().numpy()


def test_bf16_widening_every_finite_pattern():
    bits = all_finite_bf16()
    assert bits.size == 65536 - 256
    x = bits.reshape(-1, 32)            # 2040 rows of 32
    got = O.transform(x)                # widen only: no channel scale, no rotation
    ref = torch_widen(x)
    # bit for bit, so that -0, subnormals and the extremes are covered too
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_input_equals_its_widened_fp32_everywhere():
    # the bf16 branch of every oracle entry point must see exactly the fp32
    # values torch decodes: transform with channel scale and rotation, the
    # channel scale itself, and the full quantizer of every format
    g = datagen.rng(77)
    x32 = (g.standard_t(3, (48, 256)) * 2.0 ** g.integers(-20, 20, (48, 1))).astype(np.float32)
    xb = datagen.to_bf16_bits(x32)
    xw = torch_widen(xb)
    w = datagen.normal((64, 256), 78, 0.02)
    t, r = O.channel_scale(xb, w, 0.75)
    t2, r2 = O.channel_scale(xw, w, 0.75)
    assert np.array_equal(t, t2) and np.array_equal(r, r2)
    assert np.array_equal(O.transform(xb, t, 32).view(np.uint32), O.transform(xw, t, 32).view(np.uint32))
    wb = datagen.to_bf16_bits(w)
    tw, _ = O.channel_scale(xw, wb, 0.75)
    tw2, _ = O.channel_scale(xw, torch_widen(wb), 0.75)
    assert np.array_equal(tw, tw2)
    for fmt, block, rule, gmode, sp in (("nvfp4", 16, O.FOUR_OVER_SIX, O.G_AUTO, None),
                                        ("nvfp4", 4, O.ABSMAX | O.PREVENT_ZERO, O.G_AUTO, None),
                                        ("razer_a", 16, O.ABSMAX, O.G_AUTO, None),
                                        ("razer_w", 16, O.ABSMAX, O.G_AUTO, datagen.RAZER_SPECIAL),
                                        ("mxfp4", 32, O.ABSMAX, O.G_NONE, None)):
        a = O.quantize(xb, fmt, block, rule, gmode, chan_scale=t, hadamard=32, special=sp)
        b = O.quantize(xw, fmt, block, rule, gmode, chan_scale=t, hadamard=32, special=sp)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2], fmt


def e3m3_table():
    """the 64 E3M3 values in code order: code = 8 e + m; e = 0 subnormal
    m/8 * 2^(1-3), else (1 + m/8) * 2^(e-3)"""
    vals = []
    for e in range(8):
        for m in range(8):
            if e == 0:
                vals.append(Fraction(m, 8) * Fraction(1, 4))
            else:
                vals.append((1 + Fraction(m, 8)) * Fraction(2) ** (e - 3))
    return vals


def special_rich_tensor(rows: int, special, seed: int) -> np.ndarray:
    """blocks whose elements sit at multiples of the block scale, with the
    special values and the standard grid mixed, so that every pick occurs"""
    g = datagen.rng(seed)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -2, -4, -6], np.float64)
    x = np.empty((rows, 64), np.float64)
    for r in range(rows):
        v = float(special[r % len(special)])
        for b in range(4):
            blk = g.choice(grid, 16)
            blk[g.integers(0, 16, 3)] = v      # the wanted special value, several times
            blk[0] = 6.0 if v > -6.0 else 4.0  # a block max of 6 keeps the scale at 1/6 of it
            x[r, 16 * b:16 * b + 16] = blk * 2.0 ** g.integers(-3, 4)
    return x.astype(np.float32)


def test_razer_w_decode_independent():
    e2 = e2m1_table()
    e3 = e3m3_table()
    assert len(set(e3)) == 64 and e3[63] == 30 and e3[1] == Fraction(1, 32)
    # the second table has values past 6, which a block can pick only when its
    # scale rounded down far enough; its in-range values 4.5 and -3.5 are picked
    for special, want in ((datagen.RAZER_SPECIAL, {0, 1, 2, 3}), ((7.5, -3.5, 4.5, -6.5), {1, 2})):
        x = special_rich_tensor(24, special, 90)
        codes, scales, g = O.quantize(x, "razer_w", 16, O.ABSMAX, O.G_AUTO, special=special)
        dec = O.decode(codes, scales, "razer_w", 16, special)
        deq = O.dequantize(codes, scales, "razer_w", 16, g, special)
        picks_seen = set()
        for r in range(x.shape[0]):
            for j in range(64):
                c = int((codes[r, j // 2] >> (4 * (j & 1))) & 15)
                sb = int(scales[r, j // 16])
                s = e3[sb & 0x3F]
                if c == 8:
                    v = Fraction(float(special[sb >> 6]))
                    picks_seen.add(sb >> 6)
                else:
                    v = Fraction(e2[c])
                assert Fraction(float(dec[r, j])) == v * s, (r, j)
                assert deq[r, j] == np.float32(float(v * s * Fraction(float(g)))), (r, j)
        # the decode read every one of the four picks from the scale byte
        assert picks_seen >= want, picks_seen


def test_razer_a_decode_independent():
    e2 = e2m1_table()
    e4 = e4m3_lib_values()
    x = special_rich_tensor(16, (5.0, -5.0), 91)
    codes, scales, g = O.quantize(x, "razer_a", 16, O.ABSMAX, O.G_AUTO)
    dec = O.decode(codes, scales, "razer_a", 16)
    deq = O.dequantize(codes, scales, "razer_a", 16, g)
    signs = set()
    for r in range(x.shape[0]):
        for j in range(64):
            c = int((codes[r, j // 2] >> (4 * (j & 1))) & 15)
            sb = int(scales[r, j // 16])
            s = Fraction(float(e4[sb & 0x7F]))
            if c == 8:
                v = Fraction(-5 if sb & 0x80 else 5)   # the freed sign bit picks -5
                signs.add(int(v))
            else:
                v = Fraction(e2[c])
            assert Fraction(float(dec[r, j])) == v * s, (r, j)
            assert deq[r, j] == np.float32(float(v * s * Fraction(float(g)))), (r, j)
    assert signs == {5, -5}
