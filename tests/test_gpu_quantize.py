"""GPU parity of fp4q_quantize against the CPU oracle: codes, scales, special
picks and the global scale must match byte for byte.

Small ragged tensors exercise every format x rule x block x dtype x global
mode (and the transforms); the five workloads are checked at full size on
sampled rows (the oracle computes those rows one by one)."""
import numpy as np
import pytest

import datagen
import oracle as O
from tests.gpu_util import case, dev, host, scalar_dev

pytestmark = pytest.mark.gpu

SPECIAL = datagen.RAZER_SPECIAL
SPECIAL2 = (7.5, -3.5, 4.5, -6.5)


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp4_e4m3_amd as B
    return B


def mixed_tensor(rows: int, cols: int, seed: int) -> np.ndarray:
    """rows of different character: normal, heavy tails, tiny and large
    magnitudes, zeros, values on the E2M1 grid (ties), outlier columns"""
    g = datagen.rng(seed)
    x = np.empty((rows, cols), np.float32)
    for r in range(rows):
        kind = r % 7
        if kind == 0:
            v = g.standard_normal(cols)
        elif kind == 1:
            v = g.standard_t(3, cols)
        elif kind == 2:
            v = g.standard_normal(cols) * 2.0 ** -14
        elif kind == 3:
            v = g.standard_normal(cols) * 2.0 ** 12
        elif kind == 4:
            v = np.zeros(cols)
            v[g.integers(0, cols, 3)] = g.standard_normal(3)
        elif kind == 5:  # grid points and midpoints times a power of two
            grid = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6])
            v = g.choice(grid, cols) * g.choice([-1, 1], cols) * 2.0 ** g.integers(-3, 3)
        else:
            v = g.standard_normal(cols)
            v[g.integers(0, cols, 2)] *= 60
        x[r] = v
    return x


def to_input(x: np.ndarray, bf16: bool):
    if bf16:
        b = datagen.to_bf16_bits(x)
        return b, dev(b, bf16=True)
    return x, dev(x)


def run_pair(B, x_np, x_gpu, fmt, block, rule, gmode, g_given=None, t=None, had=0, special=None):
    """GPU quantize and oracle quantize of the same tensor; assert equality"""
    import torch
    rows, cols = x_np.shape
    ogm = {"none": O.G_NONE, "auto": O.G_AUTO, "given": O.G_GIVEN}[gmode]
    orule = {"absmax": O.ABSMAX, "4over6": O.FOUR_OVER_SIX, "brute": O.BRUTE}[rule.split("+")[0]]
    if "+pz" in rule:
        orule |= O.PREVENT_ZERO
    sp = special if special is not None else (0.0, 0.0, 0.0, 0.0)
    oc, os_, og = O.quantize(x_np, fmt, block, orule, ogm, chan_scale=t, hadamard=had,
                             special=special, g=g_given)
    gbuf = scalar_dev(g_given if g_given is not None else 1.0)
    tg = dev(t) if t is not None else None
    case(f"quantize {fmt} B={block} {rule} g={gmode} {x_gpu.dtype} {rows}x{cols} had={had} chan={t is not None}")
    codes, scales, gg = B.quantize(x_gpu, fmt, block, rule, gmode, chan_scale=tg, hadamard=had,
                                   special=sp, global_=gbuf)
    torch.cuda.synchronize()
    assert np.array_equal(host(scales), os_), "scales differ"
    assert np.array_equal(host(codes), oc), "codes differ"
    if gmode != "none":
        assert host(gg)[0] == np.float32(og), (host(gg)[0], og)


NV_RULES = ["absmax", "absmax+pz", "4over6", "4over6+pz", "brute"]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("block", [4, 8, 16, 32])
@pytest.mark.parametrize("rule", NV_RULES)
@pytest.mark.parametrize("gmode", ["none", "auto", "given"])
def test_nvfp4_small(B, bf16, block, rule, gmode):
    x = mixed_tensor(37, 256, seed=1000 + block)
    xn, xg = to_input(x, bf16)
    run_pair(B, xn, xg, "nvfp4", block, rule, gmode, g_given=0.0123 if gmode == "given" else None)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("block", [4, 8, 16, 32])
@pytest.mark.parametrize("fmt,rule,special", [
    ("razer_a", "absmax", None), ("razer_a", "absmax+pz", None),
    ("razer_w", "absmax", SPECIAL), ("razer_w", "absmax+pz", SPECIAL2)])
@pytest.mark.parametrize("gmode", ["none", "auto", "given"])
def test_razer_small(B, bf16, block, fmt, rule, special, gmode):
    x = mixed_tensor(29, 256, seed=2000 + block)
    xn, xg = to_input(x, bf16)
    run_pair(B, xn, xg, fmt, block, rule, gmode, g_given=0.0377 if gmode == "given" else None, special=special)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("chan,had", [(False, 0), (True, 0), (False, 32), (True, 32)])
def test_mxfp4_small(B, bf16, chan, had):
    x = mixed_tensor(41, 256, seed=3000)
    xn, xg = to_input(x, bf16)
    t = None
    if chan:
        w = datagen.normal((64, 256), 3001, 0.02)
        t, _ = O.channel_scale(xn, w, 0.75)
    run_pair(B, xn, xg, "mxfp4", 32, "absmax", "none", t=t, had=had)


@pytest.mark.parametrize("fmt,rule", [("nvfp4", "4over6"), ("nvfp4", "brute"), ("razer_a", "absmax"),
                                      ("razer_w", "absmax")])
def test_transforms_with_nvfp4_family(B, fmt, rule):
    x = mixed_tensor(19, 128, seed=3100)
    xn, xg = to_input(x, True)
    w = datagen.normal((48, 128), 3101, 0.02)
    t, _ = O.channel_scale(xn, w, 0.75)
    run_pair(B, xn, xg, fmt, 16, rule, "auto", t=t, had=32, special=SPECIAL if fmt == "razer_w" else None)


def test_edge_shapes(B):
    # one block per row, blocks of 4 with cols % 8 == 4 (4-element lanes),
    # a single row, a row pitch larger than the row, an all-zero tensor
    x = mixed_tensor(5, 4, seed=4000)
    run_pair(B, x, dev(x), "nvfp4", 4, "4over6", "auto")
    x = mixed_tensor(9, 12, seed=4001)
    for rule in ("absmax", "brute"):
        run_pair(B, x, dev(x), "nvfp4", 4, rule, "auto")
    run_pair(B, x, dev(x), "razer_w", 4, "absmax", "auto", special=SPECIAL)
    x = mixed_tensor(1, 32, seed=4002)
    run_pair(B, x, dev(x), "nvfp4", 32, "4over6", "given", g_given=3.5e-4)
    wide = mixed_tensor(23, 320, seed=4003)
    xg = dev(wide)[:, :256]  # pitch 320 elements
    run_pair(B, np.ascontiguousarray(wide[:, :256]), xg, "nvfp4", 16, "4over6", "auto")
    z = np.zeros((8, 64), np.float32)
    run_pair(B, z, dev(z), "nvfp4", 16, "4over6", "auto")
    run_pair(B, z, dev(z), "razer_a", 16, "absmax+pz", "auto")
    run_pair(B, z, dev(z), "mxfp4", 32, "absmax", "none")


def test_extreme_global_scales(B):
    # GIVEN scales far from the data: scales saturate at 448 or underflow to 0
    x = mixed_tensor(14, 128, seed=4100)
    for g in (1e-30, 2.0 ** -140, 1e25, 7.0):
        run_pair(B, x, dev(x), "nvfp4", 16, "4over6+pz", "given", g_given=g)
        run_pair(B, x, dev(x), "razer_a", 16, "absmax", "given", g_given=g)


def test_repeatable(B):
    import torch
    x = mixed_tensor(64, 512, seed=4200)
    xg = dev(datagen.to_bf16_bits(x), bf16=True)
    case("repeatability nvfp4 4over6 auto")
    outs = [B.quantize(xg, "nvfp4", 16, "4over6", "auto") for _ in range(3)]
    torch.cuda.synchronize()
    for c, s, g in outs[1:]:
        assert torch.equal(c, outs[0][0]) and torch.equal(s, outs[0][1]) and torch.equal(g, outs[0][2])


# ------------------------------------------------------------------ full-size workloads, sampled rows
def sampled_parity(B, x_np, x_gpu, fmt, block, rule, gmode, rows_idx, t=None, had=0, special=None,
                   g_given=None):
    """GPU quantizes the whole tensor; the oracle recomputes the sampled rows with
    the oracle's own global scale (computed over the whole transformed tensor)."""
    import torch
    orule = {"absmax": O.ABSMAX, "4over6": O.FOUR_OVER_SIX, "brute": O.BRUTE}[rule.split("+")[0]]
    if "+pz" in rule:
        orule |= O.PREVENT_ZERO
    if gmode == "auto":
        g_or = O.auto_global(O.transform(x_np, t, had), fmt)
    elif gmode == "given":
        g_or = g_given
    else:
        g_or = 1.0
    gbuf = scalar_dev(g_or)
    case(f"quantize full {fmt} B={block} {rule} g={gmode} {tuple(x_gpu.shape)}")
    codes, scales, gg = B.quantize(x_gpu, fmt, block, rule, gmode, chan_scale=dev(t) if t is not None else None,
                                   hadamard=had, special=special or (0.0,) * 4, global_=gbuf)
    torch.cuda.synchronize()
    if gmode == "auto":
        assert host(gg)[0] == np.float32(g_or)
    idx = torch.as_tensor(rows_idx, device="cuda")
    gc = host(codes.index_select(0, idx))
    gs = host(scales.index_select(0, idx))
    xt = O.transform(x_np[rows_idx], t, had)
    oc, os_ = O.quantize_rows(xt, fmt, block, orule, g_or, special)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


def sample_rows(n_rows: int, k: int, seed: int) -> np.ndarray:
    idx = datagen.rng(seed).choice(n_rows, size=min(k, n_rows), replace=False)
    return np.sort(np.concatenate([idx, [0, n_rows - 1]])).astype(np.int64)


@pytest.mark.parametrize("dist", ["normal", "student_t3"])
def test_sweep_workload_4096(B, dist):
    x = datagen.sweep(dist)
    xg = dev(x)
    for block in (4, 8, 16, 32):
        for rule in ("absmax", "absmax+pz", "4over6", "brute"):
            k = 12 if rule == "brute" else 48
            sampled_parity(B, x, xg, "nvfp4", block, rule, "auto", sample_rows(4096, k, 10 + block))


def test_mxfp4_linear_workload(B):
    d = datagen.mxfp4_linear()
    xb = d["X_bf16"]
    w = d["W"]
    t, r = O.channel_scale(xb, w, 0.75)
    sampled_parity(B, xb, dev(xb, bf16=True), "mxfp4", 32, "absmax", "none", sample_rows(4096, 64, 20), t=t, had=32)
    sampled_parity(B, w, dev(w), "mxfp4", 32, "absmax", "none", sample_rows(14336, 64, 21), t=r, had=32)


# automatic g on both sides of the single-launch threshold (8192 elements):
# 1 x 8192 finds g inside the quantize launch, 2 x 4608 with the separate
# abs-max and finalize launches; codes, scales and g must match the oracle
@pytest.mark.parametrize("rows,cols", [(1, 8192), (2, 4608), (1, 5120)])
def test_auto_global_launch_paths(B, rows, cols):
    x = datagen.student_t((rows, cols), 950 + rows, 3.0)
    xg = dev(x)
    t = (datagen.rng(951).random(cols) + 0.5).astype(np.float32)
    run_pair(B, x, xg, "nvfp4", 16, "4over6", "auto", t=t, had=32)
    run_pair(B, x, xg, "razer_w", 16, "absmax", "auto", special=SPECIAL)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("rows,cols", [(61, 512), (2100, 1024)])
def test_auto_global_contiguous_hadamard(B, bf16, rows, cols):
    # the separate abs-max pass on contiguous rows with the block-Hadamard
    # applied (no channel scale); at 2100 x 1024 the second chunk a thread
    # loads per iteration is live for part of the grid
    x = datagen.student_t((rows, cols), 970 + rows, 3.0)
    xn, xg = to_input(x, bf16)
    run_pair(B, xn, xg, "nvfp4", 16, "absmax", "auto", had=32)
    run_pair(B, xn, xg, "razer_w", 16, "absmax", "auto", had=32, special=SPECIAL)


def test_razer_decode_workload(B):
    w = datagen.razer_decode(1)["W"]
    sampled_parity(B, w, dev(w), "razer_w", 16, "absmax", "auto", sample_rows(17408, 64, 30), special=SPECIAL)
    for M in (1, 16, 128):
        a = datagen.razer_decode(M, with_weight=False)["A_bf16"]
        run_pair(B, a, dev(a, bf16=True), "razer_a", 16, "absmax", "auto")


def test_prefill_workload(B):
    a = datagen.prefill_act()
    g = O.auto_global(O.transform(a[:4096]), "nvfp4")  # a calibrated, fixed global scale
    sampled_parity(B, a, dev(a, bf16=True), "nvfp4", 16, "4over6", "given", sample_rows(32768, 64, 40), g_given=g)
    w = datagen.prefill_weight(5120)
    sampled_parity(B, w, dev(w), "nvfp4", 16, "4over6", "auto", sample_rows(5120, 64, 41))


def test_tiny_workload_quantize_and_gemm(B):
    # the tiny NVFP4 workload on its own tensors: W 256 x 256 under abs-max,
    # 4-over-6 and brute force, A 64 x 256 under abs-max (block 16, E4M3, no
    # global scale), all through the HIP quantizer byte for byte; then the
    # W4A4 matmul of the HIP-produced codes against the oracle's matmul of the
    # oracle's codes
    import torch
    from tests.gpu_util import rel_fro
    d = datagen.tiny()
    ag = dev(d["A"])
    wg = dev(d["W"])
    run_pair(B, d["A"], ag, "nvfp4", 16, "absmax", "none")
    case("tiny workload: activation quantize")
    ac, as_, _ = B.quantize(ag, "nvfp4", 16, "absmax", "none")
    oac, oas, _ = O.quantize(d["A"], "nvfp4", 16, O.ABSMAX, O.G_NONE)
    for rule, orule in (("absmax", O.ABSMAX), ("4over6", O.FOUR_OVER_SIX), ("brute", O.BRUTE)):
        run_pair(B, d["W"], wg, "nvfp4", 16, rule, "none")
        case(f"tiny workload: weight quantize {rule} and GEMM 64x256x256")
        wc, ws, _ = B.quantize(wg, "nvfp4", 16, rule, "none")
        c = B.gemm("nvfp4", ac, as_, None, "nvfp4", wc, ws, None)
        torch.cuda.synchronize()
        owc, ows, _ = O.quantize(d["W"], "nvfp4", 16, orule, O.G_NONE)
        ref = O.gemm_rows("nvfp4", oac, oas, 1.0, "nvfp4", owc, ows, 1.0, None, 64, 256, 256)
        assert rel_fro(host(c), ref) <= 1e-3


def test_mxfp4_linear_device_channel_scale(B):
    # the MXFP4 linear workload as the benchmark runs it: t and r from the
    # device's channel-scale kernel (within one fp32 ulp of the oracle's; the
    # binary64 column sums add in another order), then the quantizer at full
    # size with those t and r; sampled rows against the oracle given the same
    # t and r, byte for byte
    import torch
    d = datagen.mxfp4_linear()
    xb, w = d["X_bf16"], d["W"]
    t_or, r_or = O.channel_scale(xb, w, 0.75)
    case("channel scale 4096 x 4096 bf16 with 14336 x 4096 fp32")
    tg, rg = B.channel_scale(dev(xb, bf16=True), dev(w), 0.75)
    torch.cuda.synchronize()
    t, r = host(tg), host(rg)
    assert np.max(np.abs(t.view(np.int32).astype(np.int64) - t_or.view(np.int32))) <= 1
    assert np.max(np.abs(r.view(np.int32).astype(np.int64) - r_or.view(np.int32))) <= 2
    sampled_parity(B, xb, dev(xb, bf16=True), "mxfp4", 32, "absmax", "none", sample_rows(4096, 64, 22), t=t, had=32)
    sampled_parity(B, w, dev(w), "mxfp4", 32, "absmax", "none", sample_rows(14336, 64, 23), t=r, had=32)


def near_tie_blocks(n_want: int, seed: int, bf16: bool, g: float) -> np.ndarray:
    """16-element blocks whose two 4-over-6 candidates have nearly equal block
    errors (a quarter exact ties, the rest the smallest gaps), from a large seeded
    sample: the region where the rule is hardest to decide.  The gap is only
    estimated here (float64, nearest E4M3 scale, nearest E2M1 value), which
    is enough to aim the sample; the test compares with the oracle."""
    rg = datagen.rng(seed)
    parts = [rg.standard_normal((100000, 16)), rg.standard_t(3, (100000, 16)),
             rg.uniform(-1, 1, (100000, 16)),
             rg.choice(np.array([0, 0.5, 1, 1.5, 2, 2.5, 3, 3.5, 4, 5, 6]), (100000, 16)) * rg.choice([-1, 1], (100000, 16))]
    x = np.concatenate(parts).astype(np.float32) * np.float32(2.0) ** rg.integers(-3, 4, (400000, 1)).astype(np.float32)
    if bf16:
        x = datagen.bf16_bits_to_f32(datagen.to_bf16_bits(x))
    xd = x.astype(np.float64)
    k = np.arange(127)
    e4m3 = np.where(k >> 3 == 0, (k & 7) * 2.0 ** -9, (8 + (k & 7)) * 2.0 ** ((k >> 3) - 10))
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    a = np.abs(xd).max(1)

    def err(T):
        r = a / (T * g)
        s = e4m3[np.clip(np.searchsorted((e4m3[:-1] + e4m3[1:]) / 2, r), 0, 126)]
        t = np.abs(xd) / np.maximum(s * g, 1e-300)[:, None]
        v = grid[np.abs(t[..., None] - grid).argmin(-1)]
        return ((t - v) ** 2).sum(1) * (s * g) ** 2

    e6, e4 = err(6.0), err(4.0)
    gap = np.abs(e4 - e6) / np.maximum(e4 + e6, 1e-300)
    ties = np.flatnonzero(gap == 0)[: n_want // 4]
    near = np.flatnonzero(gap > 0)
    near = near[np.argsort(gap[near])[: n_want - len(ties)]]
    return x[np.concatenate([ties, near])]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("gmode", ["given", "auto"])
def test_four6_near_ties(B, bf16, gmode):
    # 4096 blocks as 256 rows of 16 blocks, the contiguous 4-over-6 path
    g = 0.0123
    blocks = near_tie_blocks(4096, 7000 + 2 * bf16 + (gmode == "auto"), bf16, g)
    x = blocks.reshape(256, 256)
    xn, xg = to_input(x, bf16)
    run_pair(B, xn, xg, "nvfp4", 16, "4over6", gmode, g_given=g if gmode == "given" else None)
    run_pair(B, xn, xg, "nvfp4", 16, "4over6+pz", gmode, g_given=g if gmode == "given" else None)
