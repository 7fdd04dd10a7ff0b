"""The 4-over-6 rule decided from estimates: the decision bound, checked on
the CPU.

The GPU quantizer for NVFP4 4-over-6 (blocks of 16) encodes each candidate
scale once, at y = x * rlo with rlo just below 1/(s g), estimates its block
error in units of s g as S = sum (y - v(y))^2, and keeps the scale whose
estimate wins by more than a margin M (otherwise it runs the exact rule).
Here that decision is emulated in float32 on the host -- the reciprocal of
s g moved by up to one ulp either way, as the hardware's reciprocal is only
that accurate -- over seeded blocks of several distributions and over
blocks whose two exact errors are nearly or exactly equal.  Wherever the
emulated estimate decides, the oracle's 4-over-6 must have chosen the same
scale code.  This pins the margin's constants to the rule, independently of
the device.  (A kernel that decided differently would also fail the GPU
parity tests; this test fails on the CPU if the bound itself is too
narrow.)
"""
import numpy as np

import datagen
import oracle as O

F32 = np.float32
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def e4m3_values() -> np.ndarray:
    k = np.arange(127)
    return np.where(k >> 3 == 0, (k & 7) * 2.0 ** -9, (8 + (k & 7)) * 2.0 ** ((k >> 3) - 10))


def nearest_code(a: np.ndarray, T: float, g: float) -> np.ndarray:
    """E4M3 code nearest to a / (T g) (ties to even), saturating at 126,
    decided exactly: each midpoint times T g is exact in binary64"""
    v = e4m3_values()
    thr = (v[:-1] + v[1:]) / 2 * T * float(g)
    k = np.searchsorted(thr, a, side="left")  # a <= thr[k] -> k
    tie = (k < 126) & (a == thr[np.minimum(k, 125)])
    k = np.where(tie & (k % 2 == 1), k + 1, k)
    return np.minimum(k, 126)


def e2m1_rne(y: np.ndarray) -> np.ndarray:
    """value of the nearest E2M1 code to y (ties to the even code), saturating at 6"""
    ay = np.abs(y.astype(np.float64))
    mids = (E2M1[:-1] + E2M1[1:]) / 2
    k = np.searchsorted(mids, ay, side="left")
    tie = (k < 7) & (ay == mids[np.minimum(k, 6)])
    k = np.where(tie & (k % 2 == 1), k + 1, k)
    return np.sign(y) * E2M1[np.minimum(k, 7)]


def f32_ulp_nudge(v: np.ndarray, rng) -> np.ndarray:
    """v moved by -1, 0 or +1 ulp (the reciprocal's accuracy)"""
    step = rng.integers(-1, 2, v.shape).astype(np.int64)
    return (v.view(np.int32).astype(np.int64) + step).astype(np.int32).view(np.float32)


def estimate(x: np.ndarray, g: np.float32, k: np.ndarray, rng):
    """(S, s) of one candidate for each block: the kernel's float32 steps"""
    s = e4m3_values()[k].astype(F32)
    sg = (s * g).astype(F32)
    r = f32_ulp_nudge((F32(1) / sg).astype(F32), rng)
    rl = (r * F32(1.0 - 2.0 ** -20)).astype(F32)
    y = (x * rl[:, None]).astype(F32)
    d = (y - e2m1_rne(y).astype(F32)).astype(F32)
    # two float32 FMA chains over elements 0-7 and 8-15, then their sum
    sa = np.zeros(len(x), F32)
    sb = np.zeros(len(x), F32)
    for i in range(8):
        sa = (sa.astype(np.float64) + d[:, i].astype(np.float64) ** 2).astype(F32)
        sb = (sb.astype(np.float64) + d[:, 8 + i].astype(np.float64) ** 2).astype(F32)
    return (sa + sb).astype(F32), s, rl


def decide(x: np.ndarray, g: float, rng):
    """pick4, pick6 and the two scale codes of the emulated estimate"""
    g = F32(g)
    a = np.abs(x).max(1).astype(np.float64)
    k6 = nearest_code(a, 6.0, g)
    k4 = nearest_code(a, 4.0, g)
    S6, s6, rl6 = estimate(x, g, k6, rng)
    S4, s4, rl4 = estimate(x, g, k4, rng)
    af = a.astype(F32)
    ag = (f32_ulp_nudge(np.full(len(x), F32(1) / g, F32), rng) * F32(1.0 + 2.0 ** -20)).astype(F32)
    P6 = ((s6 * s6).astype(F32) * S6).astype(F32)
    P4 = ((s4 * s4).astype(F32) * S4).astype(F32)
    A = (af * ag).astype(F32)
    M = (F32(1.5625 * 2.0 ** -17) * A * (np.sqrt(P4) + np.sqrt(P6)).astype(F32) + F32(2.0 ** -31) * (A * A)
         + F32(2.0 ** -17) * (P4 + P6)).astype(F32)
    sg6, sg4 = (s6 * g).astype(F32), (s4 * g).astype(F32)
    valid = (k6 > 0) & (sg6 >= 2.0 ** -50) & (sg4 <= 2.0 ** 50) & ((af * rl6) < 64) & ((P4 + P6) < 2.0 ** 100)
    pick4 = valid & (k4 != k6) & ((P4 + M).astype(F32) < P6)
    pick6 = valid & ((k4 == k6) | (P4 > (P6 + M).astype(F32)))
    return pick4, pick6, k4, k6


def blocks(seed: int) -> np.ndarray:
    rg = datagen.rng(seed)
    n = 40000
    parts = [rg.standard_normal((n, 16)), rg.standard_t(3, (n, 16)), rg.uniform(-1, 1, (n, 16)),
             rg.standard_normal((n, 16)) * (rg.random((n, 16)) < 0.3),
             rg.choice(np.array([0, 0.5, 1, 1.5, 2, 2.5, 3, 3.5, 4, 5, 6]), (n, 16)) * rg.choice([-1, 1], (n, 16))]
    x = np.concatenate(parts) * 2.0 ** rg.integers(-6, 7, (5 * n, 1))
    return x.astype(F32)


def check(x: np.ndarray, g: float, seed: int):
    rng = np.random.default_rng(seed)
    pick4, pick6, k4, k6 = decide(x, g, rng)
    _, sc, _ = O.quantize(x, "nvfp4", 16, O.FOUR_OVER_SIX, O.G_GIVEN, g=g)
    chosen = sc[:, 0].astype(np.int64)
    assert np.all(chosen[pick4] == k4[pick4]), "estimate picked 4 where the rule keeps 6"
    assert np.all(chosen[pick6] == k6[pick6]), "estimate kept 6 where the rule picks 4"
    return pick4.sum() + pick6.sum(), len(x)


def test_estimate_decisions_agree_with_the_rule():
    decided = total = 0
    for i, g in enumerate((0.0123, 1.0, 3.1e-3, 0.77)):
        d, t = check(blocks(9100 + i), g, 9200 + i)
        decided += d
        total += t
    assert decided > 0.95 * total  # the exact path stays rare


def test_estimate_near_ties():
    # blocks whose two exact errors are closest (from 1.6M seeded blocks):
    # the region where an under-sized margin would flip the decision
    x = np.concatenate([blocks(9300 + i) for i in range(8)])
    g = 0.0123
    xd = x.astype(np.float64)
    a = np.abs(xd).max(1)
    gap = np.empty(len(x))
    e = []
    for T in (6.0, 4.0):
        s = e4m3_values()[nearest_code(a, T, g)]
        t = np.abs(xd) / (s * g)[:, None]
        e.append(((t - np.abs(e2m1_rne(t))) ** 2).sum(1) * (s * g) ** 2)
    gap = np.abs(e[1] - e[0]) / np.maximum(e[0] + e[1], 1e-300)
    idx = np.argsort(gap)[:20000]
    check(x[idx], g, 9400)
