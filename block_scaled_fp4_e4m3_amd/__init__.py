"""block_scaled_fp4_e4m3_amd -- Python binding of libfp4q (include/fp4q.h).

Argument marshalling only: every step of quantization and the W4A4 matmul
runs in the HIP kernels of libfp4q.so.  PyTorch supplies device memory and
the current HIP stream.  There is no fallback: if the library is missing,
importing this package raises.

The functions named like the C entry points (fp4q_quantize, ...) take torch
tensors, or plain integers for raw device addresses, and raise FP4QError on a
non-OK status.  quantize()/dequantize()/gemm() are conveniences that allocate
their outputs with torch and call those.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp4q.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python block_scaled_fp4_e4m3_amd/build.py` "
        "(or __graft_entry__.build()); there is no fallback implementation")

_lib = ctypes.CDLL(LIB_PATH)

# ---- constants (fp4q.h) -------------------------------------------------------
FP4Q_OK, FP4Q_ERR_NULL, FP4Q_ERR_SHAPE, FP4Q_ERR_ALIGN = 0, 1, 2, 3
FP4Q_ERR_FORMAT, FP4Q_ERR_ARG, FP4Q_ERR_UNSUPPORTED, FP4Q_ERR_DEVICE = 4, 5, 6, 7
FP4Q_NVFP4, FP4Q_MXFP4, FP4Q_NVFP4_RAZER_A, FP4Q_NVFP4_RAZER_W, FP4Q_UE5M3 = 0, 1, 2, 3, 4
FP4Q_F32, FP4Q_BF16 = 0, 1
FP4Q_RULE_ABSMAX, FP4Q_RULE_4OVER6, FP4Q_RULE_BRUTE, FP4Q_RULE_EXPSEARCH = 0, 1, 2, 3
FP4Q_FLAG_PREVENT_ZERO = 0x100
FP4Q_GLOBAL_NONE, FP4Q_GLOBAL_AUTO, FP4Q_GLOBAL_GIVEN = 0, 1, 2

FORMATS = {"nvfp4": FP4Q_NVFP4, "mxfp4": FP4Q_MXFP4, "razer_a": FP4Q_NVFP4_RAZER_A,
           "razer_w": FP4Q_NVFP4_RAZER_W, "ue5m3": FP4Q_UE5M3}
RULES = {"absmax": FP4Q_RULE_ABSMAX, "4over6": FP4Q_RULE_4OVER6, "brute": FP4Q_RULE_BRUTE,
         "expsearch": FP4Q_RULE_EXPSEARCH}
GLOBAL_MODES = {"none": FP4Q_GLOBAL_NONE, "auto": FP4Q_GLOBAL_AUTO, "given": FP4Q_GLOBAL_GIVEN}


class fp4q_quant_desc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("format", ctypes.c_int),
        ("block", ctypes.c_int32),
        ("rule", ctypes.c_uint32),
        ("global_mode", ctypes.c_int),
        ("chan_scale", ctypes.c_void_p),
        ("hadamard", ctypes.c_int32),
        ("special", ctypes.c_float * 4),
    ]


_vp, _i64, _int, _u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
_SIGS = {
    "fp4q_quantize": (_int, [ctypes.POINTER(fp4q_quant_desc), _vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "fp4q_dequantize": (_int, [ctypes.POINTER(fp4q_quant_desc), _vp, _vp, _vp, _i64, _i64, _vp, _int, _i64, _vp]),
    "fp4q_gemm_w4a4": (_int, [_int, _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _i64, _vp]),
    "fp4q_gemm_w4a4_noalloc": (_int, [_int, _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int,
                                      _i64, _vp]),
    "fp4q_channel_scale": (_int, [_vp, _int, _i64, _i64, _vp, _int, _i64, _i64, _i64, ctypes.c_double, _vp, _vp, _vp]),
    "fp4q_macaq_quantize": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "fp4q_gemm_w4a4_segmented": (_int, [_int, _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _int, _vp, _i64, _i64, _i64,
                                        _vp, _int, _i64, _vp]),
    "fp4q_gemm_w4a4_act_bf16": (_int, [_vp, _i64, _u32, _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _int, _vp, _i64,
                                       _i64, _i64, _vp, _int, _i64, _vp]),
    "fp4q_gemm_w4a16": (_int, [_vp, _i64, _int, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _i64, _vp]),
    "fp4q_razer_table_search": (_int, [_vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                       _vp]),
    "fp4q_status_string": (ctypes.c_char_p, [_int]),
    "fp4q_abi_version": (_u32, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class FP4QError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fp4q_status_string(status)} (status {status})")


def fp4q_status_string(status: int) -> str:
    return _lib.fp4q_status_string(status).decode()


def fp4q_abi_version() -> int:
    return int(_lib.fp4q_abi_version())


# ---- marshalling helpers --------------------------------------------------------
def _ptr(t) -> int | None:
    """device address of a tensor, an int address, or None"""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FP4Q_F32
    if t.dtype == torch.bfloat16:
        return FP4Q_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: fp32 or bf16 expected")


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _fmt(f) -> int:
    return FORMATS[f] if isinstance(f, str) else int(f)


def _rule(r) -> int:
    if isinstance(r, str):
        parts = r.split("+")
        v = RULES[parts[0]]
        if "pz" in parts[1:]:
            v |= FP4Q_FLAG_PREVENT_ZERO
        return v
    return int(r)


def _gmode(g) -> int:
    return GLOBAL_MODES[g] if isinstance(g, str) else int(g)


def _check(status: int, where: str):
    if status != FP4Q_OK:
        raise FP4QError(status, where)


def make_desc(fmt="nvfp4", block=16, rule="absmax", global_mode="none", chan_scale=None,
              hadamard=0, special=(0.0, 0.0, 0.0, 0.0)) -> fp4q_quant_desc:
    d = fp4q_quant_desc()
    d.struct_size = ctypes.sizeof(fp4q_quant_desc)
    d.format = _fmt(fmt)
    d.block = int(block)
    d.rule = _rule(rule)
    d.global_mode = _gmode(global_mode)
    d.chan_scale = _ptr(chan_scale)
    d.hadamard = int(hadamard)
    for i in range(4):
        d.special[i] = float(special[i])
    return d


# ---- the C entry points, same names -----------------------------------------------
def fp4q_quantize(desc: fp4q_quant_desc, x, x_dtype: int, rows: int, cols: int, ld_x: int,
                  codes, scales, global_, stream=None) -> None:
    _check(_lib.fp4q_quantize(ctypes.byref(desc), _ptr(x), x_dtype, rows, cols, ld_x, _ptr(codes),
                              _ptr(scales), _ptr(global_), _stream(stream)), "fp4q_quantize")


def fp4q_dequantize(desc: fp4q_quant_desc, codes, scales, global_, rows: int, cols: int, out,
                    out_dtype: int, ld_out: int, stream=None) -> None:
    _check(_lib.fp4q_dequantize(ctypes.byref(desc), _ptr(codes), _ptr(scales), _ptr(global_), rows, cols,
                                _ptr(out), out_dtype, ld_out, _stream(stream)), "fp4q_dequantize")


def fp4q_gemm_w4a4(fa, a_codes, a_scales, a_global, fw, w_codes, w_scales, w_global, w_special,
                   M: int, N: int, K: int, c, c_dtype: int, ldc: int, stream=None) -> None:
    sp = None
    if w_special is not None:
        sp = (ctypes.c_float * 4)(*[float(v) for v in w_special])
    _check(_lib.fp4q_gemm_w4a4(_fmt(fa), _ptr(a_codes), _ptr(a_scales), _ptr(a_global), _fmt(fw),
                               _ptr(w_codes), _ptr(w_scales), _ptr(w_global),
                               ctypes.cast(sp, ctypes.c_void_p) if sp is not None else None,
                               M, N, K, _ptr(c), c_dtype, ldc, _stream(stream)), "fp4q_gemm_w4a4")


def fp4q_gemm_w4a4_noalloc(fa, a_codes, a_scales, a_global, fw, w_codes, w_scales, w_global, w_special,
                           M: int, N: int, K: int, c, c_dtype: int, ldc: int, stream=None) -> None:
    sp = None
    if w_special is not None:
        sp = (ctypes.c_float * 4)(*[float(v) for v in w_special])
    _check(_lib.fp4q_gemm_w4a4_noalloc(_fmt(fa), _ptr(a_codes), _ptr(a_scales), _ptr(a_global), _fmt(fw),
                                       _ptr(w_codes), _ptr(w_scales), _ptr(w_global),
                                       ctypes.cast(sp, ctypes.c_void_p) if sp is not None else None,
                                       M, N, K, _ptr(c), c_dtype, ldc, _stream(stream)), "fp4q_gemm_w4a4_noalloc")


def fp4q_macaq_quantize(w, N: int, K: int, ldw: int, h, ldh: int, max_moves: int, codes, scales, moves,
                        workspace, workspace_bytes: int, stream=None) -> None:
    _check(_lib.fp4q_macaq_quantize(_ptr(w), N, K, ldw, _ptr(h), ldh, max_moves, _ptr(codes), _ptr(scales),
                                    _ptr(moves), _ptr(workspace), workspace_bytes, _stream(stream)),
           "fp4q_macaq_quantize")


def _seg(seg_rows):
    if seg_rows is None or len(seg_rows) == 0:
        return None, 0
    arr = (ctypes.c_int64 * len(seg_rows))(*[int(v) for v in seg_rows])
    return arr, len(seg_rows)


def _special_arr(w_special):
    return None if w_special is None else (ctypes.c_float * 4)(*[float(v) for v in w_special])


def fp4q_gemm_w4a4_segmented(fa, a_codes, a_scales, a_global, fw, w_codes, w_scales, w_global, seg_rows,
                             w_special, M: int, N: int, K: int, c, c_dtype: int, ldc: int, stream=None) -> None:
    seg, nseg = _seg(seg_rows)
    sp = _special_arr(w_special)
    _check(_lib.fp4q_gemm_w4a4_segmented(_fmt(fa), _ptr(a_codes), _ptr(a_scales), _ptr(a_global), _fmt(fw),
                                         _ptr(w_codes), _ptr(w_scales), _ptr(w_global),
                                         ctypes.cast(seg, ctypes.c_void_p) if seg is not None else None, nseg,
                                         ctypes.cast(sp, ctypes.c_void_p) if sp is not None else None,
                                         M, N, K, _ptr(c), c_dtype, ldc, _stream(stream)), "fp4q_gemm_w4a4_segmented")


def fp4q_gemm_w4a4_act_bf16(a, lda: int, a_rule, a_global, a_codes_out, a_scales_out, fw, w_codes, w_scales,
                            w_global, seg_rows, w_special, M: int, N: int, K: int, c, c_dtype: int, ldc: int,
                            stream=None) -> None:
    seg, nseg = _seg(seg_rows)
    sp = _special_arr(w_special)
    _check(_lib.fp4q_gemm_w4a4_act_bf16(_ptr(a), lda, _rule(a_rule), _ptr(a_global), _ptr(a_codes_out),
                                        _ptr(a_scales_out), _fmt(fw), _ptr(w_codes), _ptr(w_scales), _ptr(w_global),
                                        ctypes.cast(seg, ctypes.c_void_p) if seg is not None else None, nseg,
                                        ctypes.cast(sp, ctypes.c_void_p) if sp is not None else None,
                                        M, N, K, _ptr(c), c_dtype, ldc, _stream(stream)), "fp4q_gemm_w4a4_act_bf16")


def fp4q_gemm_w4a16(a, lda: int, fw, w_codes, w_scales, w_global, w_special, M: int, N: int, K: int, c,
                    c_dtype: int, ldc: int, stream=None) -> None:
    sp = None
    if w_special is not None:
        sp = (ctypes.c_float * 4)(*[float(v) for v in w_special])
    _check(_lib.fp4q_gemm_w4a16(_ptr(a), lda, _fmt(fw), _ptr(w_codes), _ptr(w_scales), _ptr(w_global),
                                ctypes.cast(sp, ctypes.c_void_p) if sp is not None else None,
                                M, N, K, _ptr(c), c_dtype, ldc, _stream(stream)), "fp4q_gemm_w4a16")


def fp4q_razer_table_search(w, w_dtype: int, rows: int, cols: int, ld_w: int, global_mode, global_, pair_sse,
                            table, workspace, workspace_bytes: int, stream=None) -> None:
    _check(_lib.fp4q_razer_table_search(_ptr(w), w_dtype, rows, cols, ld_w, _gmode(global_mode), _ptr(global_),
                                        _ptr(pair_sse), _ptr(table), _ptr(workspace), workspace_bytes,
                                        _stream(stream)), "fp4q_razer_table_search")


def fp4q_channel_scale(x, x_dtype: int, rows_x: int, ldx: int, w, w_dtype: int, rows_w: int, ldw: int,
                       cols: int, alpha: float, t, r, stream=None) -> None:
    _check(_lib.fp4q_channel_scale(_ptr(x), x_dtype, rows_x, ldx, _ptr(w), w_dtype, rows_w, ldw, cols,
                                   float(alpha), _ptr(t), _ptr(r), _stream(stream)), "fp4q_channel_scale")


# ---- conveniences (torch allocates the outputs) ------------------------------------
def quantize(x, fmt="nvfp4", block=16, rule="absmax", global_mode="none", chan_scale=None,
             hadamard=0, special=(0.0, 0.0, 0.0, 0.0), global_=None, codes=None, scales=None,
             stream=None):
    """Quantize a 2-D CUDA tensor (fp32/bf16; row pitch = stride(0)).  Returns
    (codes uint8 [rows, cols/2], scales uint8 [rows, cols/block], global fp32 [1])."""
    import torch
    rows, cols = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along its last dimension")
    dev = x.device
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // block), dtype=torch.uint8, device=dev)
    if global_ is None:
        global_ = torch.ones(1, dtype=torch.float32, device=dev)
    desc = make_desc(fmt, block, rule, global_mode, chan_scale, hadamard, special)
    fp4q_quantize(desc, x, _dtype_code(x), rows, cols, x.stride(0), codes, scales, global_, stream)
    return codes, scales, global_


def dequantize(codes, scales, fmt="nvfp4", block=16, global_=None, special=(0.0, 0.0, 0.0, 0.0),
               out_dtype=None, stream=None):
    import torch
    out_dtype = out_dtype or torch.float32
    rows, half = codes.shape
    out = torch.empty((rows, 2 * half), dtype=out_dtype, device=codes.device)
    desc = make_desc(fmt, block, special=special)
    fp4q_dequantize(desc, codes, scales, global_, rows, 2 * half, out, _dtype_code(out), out.stride(0), stream)
    return out


def gemm(fa, a_codes, a_scales, a_global, fw, w_codes, w_scales, w_global, w_special=None,
         out_dtype=None, out=None, stream=None):
    """C = (g_a g_w) A^ W^T from codes/scales of A [M, K/2] and W [N, K/2]."""
    import torch
    M, N, K = a_codes.shape[0], w_codes.shape[0], 2 * a_codes.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a_codes.device)
    fp4q_gemm_w4a4(fa, a_codes, a_scales, a_global, fw, w_codes, w_scales, w_global, w_special,
                   M, N, K, out, _dtype_code(out), out.stride(0), stream)
    return out


def channel_scale(x, w, alpha=0.75, stream=None):
    import torch
    cols = x.shape[1]
    t = torch.empty(cols, dtype=torch.float32, device=x.device)
    r = torch.empty(cols, dtype=torch.float32, device=x.device)
    fp4q_channel_scale(x, _dtype_code(x), x.shape[0], x.stride(0), w, _dtype_code(w), w.shape[0], w.stride(0),
                       cols, alpha, t, r, stream)
    return t, r


def macaq_quantize(w, h, max_moves=None, workspace_bytes=None, stream=None):
    """MACaQ calibration of an fp32 CUDA weight (N x K) with a binary64 Hessian
    (K x K).  Returns (codes, scales, moves per row)."""
    import torch
    N, K = w.shape
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, K // 32), dtype=torch.uint8, device=w.device)
    moves = torch.empty(N, dtype=torch.int32, device=w.device)
    wsb = workspace_bytes or max(8 * K, min(N, 4096) * 8 * K)
    ws = torch.empty(wsb // 8, dtype=torch.float64, device=w.device)
    fp4q_macaq_quantize(w, N, K, w.stride(0), h, h.stride(0), 2 * K if max_moves is None else max_moves,
                        codes, scales, moves, ws, wsb, stream)
    return codes, scales, moves


def gemm_w4a16(a, fw, w_codes, w_scales, w_global=None, w_special=None, out_dtype=None, out=None, stream=None):
    """C = g_w A W^^T for bf16 activations A [M, K] and a block-16 NVFP4 or
    RaZeR-W weight W^ [N, K/2]."""
    import torch
    if a.dtype != torch.bfloat16 or a.stride(1) != 1:
        raise ValueError("a must be bf16 with unit stride along its last dimension")
    M, K = a.shape
    N = w_codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a.device)
    fp4q_gemm_w4a16(a, a.stride(0), fw, w_codes, w_scales, w_global, w_special, M, N, K, out, _dtype_code(out),
                    out.stride(0), stream)
    return out


def razer_table_search(w, global_mode="auto", global_=None, stream=None):
    """RaZeR-W special-value search over a CUDA weight (fp32/bf16, rows x
    cols).  Returns (table fp32 [4], errors of the 28 pairs fp64 [28], global
    fp32 [1])."""
    import torch
    rows, cols = w.shape
    dev = w.device
    if global_ is None:
        global_ = torch.ones(1, dtype=torch.float32, device=dev)
    pair_sse = torch.empty(28, dtype=torch.float64, device=dev)
    table = torch.empty(4, dtype=torch.float32, device=dev)
    ws = torch.empty(max(rows, 1) * 28, dtype=torch.float64, device=dev)
    fp4q_razer_table_search(w, _dtype_code(w), rows, cols, w.stride(0), global_mode, global_, pair_sse, table, ws,
                            ws.numel() * 8, stream)
    return table, pair_sse, global_


def gemm_segmented(fa, a_codes, a_scales, a_global, fw, w_codes, w_scales, w_globals, seg_rows, w_special=None,
                   out_dtype=None, out=None, stream=None):
    """C = A^ W^T with W^ the concatenation of len(seg_rows) weights, segment
    i taking the global scale w_globals[i] (device fp32 [nseg])."""
    import torch
    M, N, K = a_codes.shape[0], w_codes.shape[0], 2 * a_codes.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a_codes.device)
    fp4q_gemm_w4a4_segmented(fa, a_codes, a_scales, a_global, fw, w_codes, w_scales, w_globals, seg_rows, w_special,
                             M, N, K, out, _dtype_code(out), out.stride(0), stream)
    return out


def gemm_act_bf16(a, rule, a_global, fw, w_codes, w_scales, w_global=None, seg_rows=None, w_special=None,
                  out_dtype=None, out=None, keep_codes=False, stream=None):
    """W4A4 matmul of bf16 activations A [M, K] quantized on load (NVFP4,
    block 16, rule "absmax" or "4over6", global a_global or 1).  Returns C, or
    (C, codes, scales) with keep_codes."""
    import torch
    if a.dtype != torch.bfloat16 or a.stride(1) != 1:
        raise ValueError("a must be bf16 with unit stride along its last dimension")
    M, K = a.shape
    N = w_codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a.device)
    codes = scales = None
    if keep_codes:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=a.device)
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=a.device)
    fp4q_gemm_w4a4_act_bf16(a, a.stride(0), rule, a_global, codes, scales, fw, w_codes, w_scales, w_global, seg_rows,
                            w_special, M, N, K, out, _dtype_code(out), out.stride(0), stream)
    return (out, codes, scales) if keep_codes else out
