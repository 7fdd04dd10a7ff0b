"""Pins of the oracle's number formats and containers against the pages and
against torch's float8 decoders (an independent library)."""
import math

import numpy as np
import pytest

import oracle as O
from tests.exact_ref import e2m1_table, e4m3_lib_values, e8m0_lib_values, golden_kv


def test_e2m1_value_set_matches_pages():
    # RaZeR summary, section 1: the FP4 set {+-0, +-0.5, ..., +-6}
    gold = e2m1_table()
    assert sorted(gold) == list(range(16))
    for c, v in gold.items():
        got = O.e2m1_value(c)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), c
    # exactly two zeros (the redundancy RaZeR remaps) and 15 distinct values
    vals = [O.e2m1_value(c) for c in range(16)]
    assert sum(v == 0 for v in vals) == 2
    assert len(set(vals)) == 15


def test_e4m3_decode_matches_torch():
    lib = e4m3_lib_values()
    for k in range(127):
        assert O.e4m3_value(k) == lib[k], k
    pos = [O.e4m3_value(k) for k in range(1, 127)]
    assert len(pos) == 126 and all(b > a for a, b in zip(pos, pos[1:]))
    assert O.e4m3_value(126) == float(golden_kv("formats.txt")["e4m3_max"][0]) == 448.0
    assert O.e4m3_value(1) == 2.0 ** -9
    assert np.isnan(lib[127])  # code 127 is NaN in OCP E4M3: never produced


def test_e8m0_decode_matches_torch():
    lib = e8m0_lib_values()
    for k in range(255):
        assert O.e8m0_value(k) == lib[k], k


def test_e3m3_six_bit_format():
    # RaZeR summary 2.1: a 6-bit scale for weights (64 codes).  Bias 3 with
    # subnormals is the reading taken here: 64 distinct non-negative values,
    # strictly increasing, 8 per binade with uniform spacing, max 30, min 2^-5.
    v = [O.e3m3_value(k) for k in range(64)]
    assert v[0] == 0 and all(b > a for a, b in zip(v, v[1:]))
    assert v[63] == 30.0 and v[1] == 2.0 ** -5
    for e in range(1, 8):
        binade = v[8 * e: 8 * e + 8]
        steps = {b - a for a, b in zip(binade, binade[1:])}
        assert len(steps) == 1 and binade[0] == 2.0 ** (e - 3)
    assert int(golden_kv("formats.txt")["razer_w_scale_bits"][0]) == 6 == int(math.log2(64))


@pytest.mark.parametrize("fmt,block,bits_key", [
    ("nvfp4", 16, "nvfp4_bits"), ("mxfp4", 32, "mxfp4_bits"),
    ("razer_a", 16, "nvfp4_bits"), ("razer_w", 16, "nvfp4_bits")])
def test_bits_per_element(fmt, block, bits_key):
    # MACaQ review sections 1 and 3: NVFP4 4.50 bits, MXFP4 4.25 bits; RaZeR
    # summary section 3: the same memory footprint as NVFP4.
    x = np.random.default_rng(0).standard_normal((8, 256)).astype(np.float32)
    special = (5.0, -5.0, 2.5, -2.5) if fmt == "razer_w" else None
    codes, scales, _ = O.quantize(x, fmt, block, O.ABSMAX, O.G_NONE, special=special)
    bits = 8.0 * (codes.nbytes + scales.nbytes) / x.size
    assert bits == float(golden_kv("formats.txt")[bits_key][0])


def test_block_sizes_from_pages():
    kv = golden_kv("formats.txt")
    assert int(kv["nvfp4_block"][0]) == 16 and int(kv["mxfp4_block"][0]) == 32
    x = np.random.default_rng(1).standard_normal((2, 64)).astype(np.float32)
    for b in map(int, kv["sweep_blocks"]):
        _, scales, _ = O.quantize(x, "nvfp4", b)
        assert scales.shape == (2, 64 // b)


def test_code_packing_low_nibble_even():
    # element j of a row lives in byte j/2, the even element in the low nibble
    x = np.array([[0.5, -1.0, 2.0, 6.0] + [0.0] * 12], np.float32)
    codes, scales, _ = O.quantize(x, "nvfp4", 16)
    s = O.e4m3_value(int(scales[0, 0]))
    assert s == 1.0
    assert codes[0, 0] == (0x1 | (0xA << 4)) and codes[0, 1] == (0x4 | (0x7 << 4))
