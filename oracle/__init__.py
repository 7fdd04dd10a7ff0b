"""CPU oracle for block-scaled FP4 quantization and the W4A4 matmul.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (the ``block_scaled_fp4_e4m3_amd`` package and its HIP library) never
touches it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, one IEEE operation per step,
built with ``-ffp-contract=off``); this module only marshals numpy arrays
through ctypes.  Each C function cites the passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

# formats, rules, global modes (the oracle's own numbering)
NVFP4, MXFP4, RAZER_A, RAZER_W, UE5M3 = 0, 1, 2, 3, 4
ABSMAX, FOUR_OVER_SIX, BRUTE, EXPSEARCH = 0, 1, 2, 3
PREVENT_ZERO = 0x100
G_NONE, G_AUTO, G_GIVEN = 0, 1, 2
SF_E4M3, SF_E3M3, SF_UE5M3 = 0, 1, 2
F32, BF16 = 0, 1

FORMATS = {"nvfp4": NVFP4, "mxfp4": MXFP4, "razer_a": RAZER_A, "razer_w": RAZER_W, "ue5m3": UE5M3}


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C11, no contraction, no fast-math)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "oracle.h"))
    ):
        tmp = _SO + ".tmp"
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
             "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        d, i, f, l, vp = ctypes.c_double, ctypes.c_int, ctypes.c_float, ctypes.c_long, ctypes.c_void_p
        sig = {
            "or_e2m1_value": (d, [i]), "or_e4m3_value": (d, [i]),
            "or_e3m3_value": (d, [i]), "or_e8m0_value": (d, [i]), "or_ue5m3_value": (d, [i]),
            "or_round_scale": (i, [i, d, d, d]),
            "or_rtn": (i, [f, d, d]),
            "or_rtn_special": (i, [f, d, d, d]),
            "or_block_sse": (f, [vp, vp, i, d, f, i, d]),
            "or_transform": (None, [vp, i, l, l, l, vp, i, vp]),
            "or_auto_global": (f, [vp, l, l, i]),
            "or_quantize_rows": (i, [i, i, i, vp, vp, l, l, f, vp, vp]),
            "or_quantize": (i, [i, i, i, i, vp, i, vp, vp, i, l, l, l, vp, vp, vp]),
            "or_dequantize": (i, [i, i, vp, vp, vp, f, l, l, vp]),
            "or_decode_row": (i, [i, i, vp, vp, vp, l, vp]),
            "or_gemm_rows": (i, [i, vp, vp, f, i, vp, vp, f, vp, l, l, l, l, l, vp]),
            "or_gemm_entries": (i, [i, vp, vp, f, i, vp, vp, f, vp, l, l, l, vp, vp, l, vp]),
            "or_channel_scale": (None, [vp, i, l, l, vp, i, l, l, l, d, vp, vp]),
            "or_macaq_quantize": (i, [vp, l, l, l, vp, l, l, vp, vp, vp, vp]),
            "or_gemm_w4a16_rows": (i, [vp, l, i, vp, vp, f, vp, l, l, l, l, l, vp]),
            "or_razer_table_search": (i, [vp, i, l, l, l, f, vp]),
            "or_razer_pair": (None, [i, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _fmt(f) -> int:
    return FORMATS[f] if isinstance(f, str) else int(f)


def _x_and_dtype(x: np.ndarray):
    """fp32 arrays pass as F32; uint16 arrays are bf16 bit patterns."""
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), F32
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), BF16
    raise TypeError("oracle input must be float32 or uint16 (bf16 bits)")


def _special(special):
    if special is None:
        return None
    return np.ascontiguousarray(np.asarray(special, dtype=np.float32).reshape(4))


# -- primitives ---------------------------------------------------------------
def e2m1_value(c: int) -> float: return lib().or_e2m1_value(c)
def e4m3_value(k: int) -> float: return lib().or_e4m3_value(k)
def e3m3_value(k: int) -> float: return lib().or_e3m3_value(k)
def e8m0_value(k: int) -> float: return lib().or_e8m0_value(k)
def ue5m3_value(k: int) -> float: return lib().or_ue5m3_value(k)
def round_scale(sf: int, a: float, T: float, g: float) -> int: return lib().or_round_scale(sf, a, T, g)
def rtn(x: float, s: float, g: float) -> int: return lib().or_rtn(x, s, g)
def rtn_special(x: float, s: float, g: float, v: float) -> int: return lib().or_rtn_special(x, s, g, v)


def block_sse(x: np.ndarray, codes, s: float, g: float, special: float | None = None) -> float:
    x = np.ascontiguousarray(x, dtype=np.float32)
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.int32))
    assert x.size == c.size and x.size in (1, 2, 4, 8, 16, 32)
    return lib().or_block_sse(_p(x), _p(c), x.size, s, g, 0 if special is None else 1,
                              0.0 if special is None else special)


# -- tensors ------------------------------------------------------------------
def transform(x: np.ndarray, t: np.ndarray | None = None, hadamard: int = 0) -> np.ndarray:
    x, dt = _x_and_dtype(x)
    rows, cols = x.shape
    out = np.empty((rows, cols), np.float32)
    tt = None if t is None else np.ascontiguousarray(t, dtype=np.float32)
    lib().or_transform(_p(x), dt, rows, cols, cols, _p(tt), hadamard, _p(out))
    return out


def auto_global(xt: np.ndarray, fmt) -> float:
    xt = np.ascontiguousarray(xt, dtype=np.float32)
    return lib().or_auto_global(_p(xt), xt.shape[0], xt.shape[1], _fmt(fmt))


def quantize_rows(xt: np.ndarray, fmt, block: int, rule: int, g: float = 1.0, special=None):
    xt = np.ascontiguousarray(xt, dtype=np.float32)
    rows, cols = xt.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // block), np.uint8)
    sp = _special(special)
    rc = lib().or_quantize_rows(_fmt(fmt), block, rule, _p(sp), _p(xt), rows, cols, g, _p(codes), _p(scales))
    if rc:
        raise ValueError(f"or_quantize_rows rejected the arguments ({rc})")
    return codes, scales


def quantize(x: np.ndarray, fmt, block: int, rule: int = ABSMAX, gmode: int = G_NONE,
             chan_scale: np.ndarray | None = None, hadamard: int = 0, special=None,
             g: float | None = None):
    """Full quantize: widen, channel scale, block-Hadamard, global scale, encode.
    Returns (codes, scales, g)."""
    x, dt = _x_and_dtype(x)
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, max(cols // block, 0)), np.uint8)
    gbuf = np.array([1.0 if g is None else g], np.float32)
    t = None if chan_scale is None else np.ascontiguousarray(chan_scale, dtype=np.float32)
    sp = _special(special)
    rc = lib().or_quantize(_fmt(fmt), block, rule, gmode, _p(t), hadamard, _p(sp), _p(x), dt,
                           rows, cols, cols, _p(codes), _p(scales), _p(gbuf))
    if rc:
        raise ValueError(f"or_quantize rejected the arguments ({rc})")
    return codes, scales, float(gbuf[0])


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt, block: int, g: float = 1.0,
               special=None) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    cols = 2 * half
    out = np.empty((rows, cols), np.float32)
    sp = _special(special)
    rc = lib().or_dequantize(_fmt(fmt), block, _p(sp), _p(codes), _p(scales), g, rows, cols, _p(out))
    if rc:
        raise ValueError("or_dequantize rejected the arguments")
    return out


def decode(codes: np.ndarray, scales: np.ndarray, fmt, block: int, special=None) -> np.ndarray:
    """value * block scale for every element, binary64, rows x cols."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    cols = 2 * half
    out = np.empty((rows, cols), np.float64)
    sp = _special(special)
    for r in range(rows):
        lib().or_decode_row(_fmt(fmt), block, _p(sp), _p(codes[r]), _p(scales[r]), cols, _p(out[r]))
    return out


def gemm_rows(fa, a_codes, a_scales, g_a, fw, w_codes, w_scales, g_w, w_special, M, N, K,
              m0: int = 0, m1: int | None = None) -> np.ndarray:
    m1 = M if m1 is None else m1
    out = np.empty((m1 - m0, N), np.float32)
    a_codes, a_scales = np.ascontiguousarray(a_codes), np.ascontiguousarray(a_scales)
    w_codes, w_scales = np.ascontiguousarray(w_codes), np.ascontiguousarray(w_scales)
    sp = _special(w_special)
    rc = lib().or_gemm_rows(_fmt(fa), _p(a_codes), _p(a_scales), g_a, _fmt(fw), _p(w_codes), _p(w_scales),
                            g_w, _p(sp), M, N, K, m0, m1, _p(out))
    if rc:
        raise ValueError("or_gemm_rows rejected the arguments")
    return out


def gemm_entries(fa, a_codes, a_scales, g_a, fw, w_codes, w_scales, g_w, w_special, M, N, K,
                 ms, ns) -> np.ndarray:
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.size, np.float32)
    a_codes, a_scales = np.ascontiguousarray(a_codes), np.ascontiguousarray(a_scales)
    w_codes, w_scales = np.ascontiguousarray(w_codes), np.ascontiguousarray(w_scales)
    sp = _special(w_special)
    rc = lib().or_gemm_entries(_fmt(fa), _p(a_codes), _p(a_scales), g_a, _fmt(fw), _p(w_codes),
                               _p(w_scales), g_w, _p(sp), M, N, K, _p(ms), _p(ns), ms.size, _p(out))
    if rc:
        raise ValueError("or_gemm_entries rejected the arguments")
    return out


def channel_scale(x: np.ndarray, w: np.ndarray, alpha: float = 0.75):
    """t_j = (rms_j(W) / rms_j(X))^alpha rounded to fp32, and r_j = 1/t_j."""
    x, dx = _x_and_dtype(x)
    w, dw = _x_and_dtype(w)
    cols = x.shape[1]
    assert w.shape[1] == cols
    t = np.empty(cols, np.float32)
    r = np.empty(cols, np.float32)
    lib().or_channel_scale(_p(x), dx, x.shape[0], cols, _p(w), dw, w.shape[0], cols, cols, alpha, _p(t), _p(r))
    return t, r


def macaq_quantize(w: np.ndarray, h: np.ndarray, max_moves: int | None = None):
    """MACaQ weight calibration of W (N x K fp32) with the Hessian H (K x K
    binary64): screened exponents and Flip-Refinement.  Returns (codes,
    scales, moves per row, objective before/after per row)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    h = np.ascontiguousarray(h, dtype=np.float64)
    N, K = w.shape
    assert h.shape == (K, K)
    codes = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, K // 32), np.uint8)
    moves = np.empty(N, np.int32)
    obj = np.empty((N, 2), np.float64)
    mm = 2 * K if max_moves is None else max_moves
    rc = lib().or_macaq_quantize(_p(w), N, K, K, _p(h), K, mm, _p(codes), _p(scales), _p(moves), _p(obj))
    if rc:
        raise ValueError("or_macaq_quantize rejected the arguments")
    return codes, scales, moves, obj


def gemm_w4a16_rows(a_bf16: np.ndarray, fw, w_codes, w_scales, g_w, w_special, N, m0=0, m1=None) -> np.ndarray:
    """C = g_w A W^^T for A in bf16 bits (M x K) and W as codes/scales (block 16)."""
    a = np.ascontiguousarray(a_bf16, dtype=np.uint16)
    M, K = a.shape
    m1 = M if m1 is None else m1
    out = np.empty((m1 - m0, N), np.float32)
    w_codes, w_scales = np.ascontiguousarray(w_codes), np.ascontiguousarray(w_scales)
    sp = _special(w_special)
    rc = lib().or_gemm_w4a16_rows(_p(a), K, _fmt(fw), _p(w_codes), _p(w_scales), g_w, _p(sp), M, N, K, m0, m1,
                                  _p(out))
    if rc:
        raise ValueError("or_gemm_w4a16_rows rejected the arguments")
    return out


RAZER_NPAIRS = 28


def razer_pair(p: int):
    a, b = ctypes.c_float(), ctypes.c_float()
    lib().or_razer_pair(p, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def razer_table_search(x: np.ndarray, g: float):
    """Tensor error of every special-value pair and the index of the best."""
    x, dt = _x_and_dtype(x)
    rows, cols = x.shape
    sse = np.empty(RAZER_NPAIRS, np.float64)
    best = lib().or_razer_table_search(_p(x), dt, rows, cols, cols, g, _p(sse))
    if best < 0:
        raise ValueError("or_razer_table_search rejected the arguments")
    return sse, best
