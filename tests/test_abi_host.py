"""Host-side checks of libfp4q's C ABI, no GPU needed: the library loads,
exports every function include/fp4q.h declares, and reports each documented
argument error before touching the HIP runtime.

The argument-error calls run in a child process with no visible GPU, so that
a validation bug that let a call through could not launch a kernel on fake
pointers: such a call would return FP4Q_ERR_DEVICE and fail the test."""
import ctypes
import os
import re
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4q.h")
LIB = os.path.join(ROOT, "block_scaled_fp4_e4m3_amd", "libfp4q.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4q_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libfp4q.so is not built; run __graft_entry__.build()")
    return ctypes.CDLL(LIB)


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"fp4q_quantize", "fp4q_dequantize", "fp4q_gemm_w4a4", "fp4q_channel_scale",
            "fp4q_status_string", "fp4q_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    lib.fp4q_abi_version.restype = ctypes.c_uint32
    assert lib.fp4q_abi_version() == 1
    lib.fp4q_status_string.restype = ctypes.c_char_p
    lib.fp4q_status_string.argtypes = [ctypes.c_int]
    seen = set()
    for s in range(8):
        txt = lib.fp4q_status_string(s)
        assert txt and txt not in seen
        seen.add(txt)
    assert lib.fp4q_status_string(99) == b"unknown status"


def test_binding_names_match_header():
    # the Python binding exposes the same entry points (import needs only the .so)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    code = "import block_scaled_fp4_e4m3_amd as B; print(' '.join(sorted(B.EXPORTED)))"
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == declared_functions()


CHILD = textwrap.dedent(r'''
import ctypes, json, sys
sys.path.insert(0, ROOT)
L = ctypes.CDLL(LIB)

class Desc(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("format", ctypes.c_int), ("block", ctypes.c_int32),
                ("rule", ctypes.c_uint32), ("global_mode", ctypes.c_int), ("chan_scale", ctypes.c_void_p),
                ("hadamard", ctypes.c_int32), ("special", ctypes.c_float * 4)]

vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
L.fp4q_quantize.argtypes = [ctypes.POINTER(Desc), vp, ci, i64, i64, i64, vp, vp, vp, vp]
L.fp4q_dequantize.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, i64, i64, vp, ci, i64, vp]
L.fp4q_gemm_w4a4.argtypes = [ci, vp, vp, vp, ci, vp, vp, vp, vp, i64, i64, i64, vp, ci, i64, vp]
L.fp4q_gemm_w4a4_noalloc.argtypes = L.fp4q_gemm_w4a4.argtypes
L.fp4q_channel_scale.argtypes = [vp, ci, i64, i64, vp, ci, i64, i64, i64, ctypes.c_double, vp, vp, vp]
L.fp4q_macaq_quantize.argtypes = [vp, i64, i64, i64, vp, i64, i64, vp, vp, vp, vp, ctypes.c_size_t, vp]
L.fp4q_gemm_w4a4_segmented.argtypes = [ci, vp, vp, vp, ci, vp, vp, vp, vp, ci, vp, i64, i64, i64, vp, ci, i64, vp]
L.fp4q_gemm_w4a4_act_bf16.argtypes = [vp, i64, ctypes.c_uint32, vp, vp, vp, ci, vp, vp, vp, vp, ci, vp, i64, i64, i64,
                                      vp, ci, i64, vp]
L.fp4q_gemm_w4a16.argtypes = [vp, i64, ci, vp, vp, vp, vp, i64, i64, i64, vp, ci, i64, vp]
L.fp4q_razer_table_search.argtypes = [vp, ci, i64, i64, i64, ci, vp, vp, vp, vp, ctypes.c_size_t, vp]
P = 0x100000  # aligned fake device address; never dereferenced on any error path

def desc(**kw):
    d = Desc(); d.struct_size = ctypes.sizeof(Desc); d.format = 0; d.block = 16; d.rule = 0
    d.global_mode = 0; d.chan_scale = None; d.hadamard = 0
    for i, v in enumerate((5.0, -5.0, 2.5, -2.5)): d.special[i] = v
    for k, v in kw.items():
        if k == "special":
            for i, s in enumerate(v): d.special[i] = s
        else:
            setattr(d, k, v)
    return d

def q(d=None, x=P, xt=0, rows=4, cols=64, ld=64, codes=P, scales=P, g=P):
    d = desc() if d is None else d
    return L.fp4q_quantize(None if d == "null" else ctypes.byref(d), x, xt, rows, cols, ld, codes, scales, g, None)

def dq(d=None, codes=P, scales=P, g=None, rows=4, cols=64, out=P, ot=0, ld=64):
    d = desc() if d is None else d
    return L.fp4q_dequantize(ctypes.byref(d), codes, scales, g, rows, cols, out, ot, ld, None)

SP = (ctypes.c_float * 4)(5.0, -5.0, 2.5, -2.5)
def gm(fa=0, fw=0, a=P, sa=P, w=P, sw=P, sp=None, M=8, N=8, K=64, c=P, ct=0, ldc=8):
    return L.fp4q_gemm_w4a4(fa, a, sa, None, fw, w, sw, None, sp, M, N, K, c, ct, ldc, None)

def gn(fa=0, fw=0, a=P, sa=P, w=P, sw=P, sp=None, M=8, N=8, K=64, c=P, ct=0, ldc=8):
    return L.fp4q_gemm_w4a4_noalloc(fa, a, sa, None, fw, w, sw, None, sp, M, N, K, c, ct, ldc, None)

def mq(w=P, N=4, K=64, ldw=64, h=P, ldh=64, mm=10, codes=P, scales=P, moves=None, ws=P, wsb=1 << 20):
    return L.fp4q_macaq_quantize(w, N, K, ldw, h, ldh, mm, codes, scales, moves, ws, wsb, None)

SEG = (ctypes.c_int64 * 3)(4, 2, 2)
def sg(fa=0, fw=0, g=P, seg=ctypes.cast(SEG, vp), nseg=3, M=8, N=8, K=64, c=P, ldc=8):
    return L.fp4q_gemm_w4a4_segmented(fa, P, P, None, fw, P, P, g, seg, nseg, None, M, N, K, c, 0, ldc, None)

def ab(a=P, lda=512, rule=1, co=None, so=None, fw=0, g=P, seg=None, nseg=0, sp=None, M=8, N=8, K=512, c=P, ldc=8):
    return L.fp4q_gemm_w4a4_act_bf16(a, lda, rule, None, co, so, fw, P, P, g, seg, nseg, sp, M, N, K, c, 0, ldc, None)

def wa(a=P, lda=512, fw=0, w=P, sw=P, g=None, sp=None, M=8, N=8, K=512, c=P, ct=0, ldc=8):
    return L.fp4q_gemm_w4a16(a, lda, fw, w, sw, g, sp, M, N, K, c, ct, ldc, None)

def ts(w=P, wt=0, rows=4, cols=64, ld=64, gmode=1, g=P, sse=P, table=P, ws=P, wsb=1 << 20):
    return L.fp4q_razer_table_search(w, wt, rows, cols, ld, gmode, g, sse, table, ws, wsb, None)

def cs(x=P, rows_x=4, ldx=8, w=P, rows_w=4, ldw=8, cols=8, alpha=0.75, t=P, r=P):
    return L.fp4q_channel_scale(x, 0, rows_x, ldx, w, 0, rows_w, ldw, cols, alpha, t, r, None)

res = {
 # quantize: NULL
 "q_null_desc": q(d="null"), "q_null_x": q(x=None), "q_null_codes": q(codes=None),
 "q_null_scales": q(scales=None), "q_null_global_auto": q(d=desc(global_mode=1), g=None),
 "q_null_global_given": q(d=desc(global_mode=2), g=None),
 # quantize: SHAPE
 "q_rows_neg": q(rows=-1), "q_cols_zero": q(cols=0), "q_cols_block": q(cols=40),
 "q_ld_small": q(ld=32), "q_had_cols": q(d=desc(hadamard=32, block=16), cols=48, ld=48),
 # quantize: ALIGN
 "q_x_align": q(x=P + 4), "q_ld_align": q(ld=66), "q_codes_align": q(codes=P + 2),
 "q_chan_align": q(d=desc(chan_scale=P + 4)), "q_ld_align_bf16": q(xt=1, ld=68),
 # quantize: FORMAT / ARG
 "q_bad_format": q(d=desc(format=7)), "q_bad_struct": q(d=desc(struct_size=8)),
 "q_bad_block": q(d=desc(block=12)), "q_mx_block": q(d=desc(format=1, block=16)),
 "q_bad_rule": q(d=desc(rule=3)), "q_bad_flag": q(d=desc(rule=0x200)),
 "q_razer_rule": q(d=desc(format=2, rule=1)), "q_mx_rule": q(d=desc(format=1, block=32, rule=1)),
 "q_mx_pz": q(d=desc(format=1, block=32, rule=0x100)), "q_mx_global": q(d=desc(format=1, block=32, global_mode=1)),
 "q_bad_mode": q(d=desc(global_mode=3)), "q_bad_had": q(d=desc(hadamard=8)),
 "q_had16_cols": q(d=desc(hadamard=16, block=4), cols=40, ld=40),
 "q_ue5m3_auto": q(d=desc(format=4, global_mode=1)), "q_ue5m3_rule": q(d=desc(format=4, rule=3)),
 "q_nv_expsearch": q(d=desc(rule=3)), "q_bad_format5": q(d=desc(format=5)),
 "q_bad_dtype": q(xt=2),
 "q_special_grid": q(d=desc(format=3, special=(5.0, -5.0, 2.5, 4.0))),
 "q_special_half": q(d=desc(format=3, special=(5.0, -5.0, 2.25, -2.5))),
 "q_special_big": q(d=desc(format=3, special=(5.0, -5.0, 8.0, -2.5))),
 "q_special_zero": q(d=desc(format=3, special=(5.0, -5.0, 0.0, -2.5))),
 "q_special_nan": q(d=desc(format=3, special=(5.0, float("nan"), 2.5, -2.5))),
 # dequantize
 "dq_null_out": dq(out=None), "dq_null_codes": dq(codes=None), "dq_shape": dq(cols=40),
 "dq_ld": dq(ld=32), "dq_align": dq(out=P + 8), "dq_ld_align": dq(ld=66), "dq_dtype": dq(ot=5),
 "dq_format": dq(d=desc(format=9)), "dq_block": dq(d=desc(block=64)),
 # gemm
 "g_null_a": gm(a=None), "g_null_c": gm(c=None), "g_null_special": gm(fw=3, sp=None),
 "g_mixed": gm(fa=1, fw=0, K=64), "g_razer_w_a": gm(fa=3, fw=3, sp=ctypes.cast(SP, vp)),
 "g_bad_format": gm(fa=5), "g_ue5m3": gm(fa=4, fw=4), "g_ue5m3_w": gm(fa=0, fw=4), "g_K_block": gm(K=24), "g_K_mx": gm(fa=1, fw=1, K=48),
 "g_K_zero": gm(K=0), "g_M_neg": gm(M=-1), "g_ldc": gm(ldc=4), "g_align": gm(a=P + 4),
 "g_ldc_align": gm(ldc=9), "g_dtype": gm(ct=3), "g_K_big": gm(K=(1 << 24) + 16),
 "g_tiles": gm(M=1 << 40, N=1 << 40, ldc=1 << 40),
 "g_bad_special": gm(fw=3, sp=ctypes.cast((ctypes.c_float * 4)(5.0, -5.0, 3.0, -2.5), vp)),
 # the non-allocating matmul: the same checks
 "gn_null_a": gn(a=None), "gn_mixed": gn(fa=1, fw=0), "gn_K_block": gn(K=24), "gn_align": gn(c=P + 4),
 "gn_dtype": gn(ct=3),
 # MACaQ calibration
 "m_null_w": mq(w=None), "m_null_ws": mq(ws=None), "m_K": mq(K=48, ldw=64), "m_K_big": mq(K=5152, ldw=5152, ldh=5152),
 "m_ldh": mq(ldh=32), "m_N": mq(N=-1), "m_moves": mq(mm=-1), "m_ws": mq(wsb=8 * 64 - 8), "m_align": mq(h=P + 4),
 # weight-only matmul
 "w_null_a": wa(a=None), "w_null_sp": wa(fw=3), "w_format_mx": wa(fw=1), "w_format_ra": wa(fw=2),
 "w_K": wa(K=256, lda=256), "w_lda": wa(lda=256), "w_lda_big": wa(lda=(1 << 24) + 8), "w_ldc": wa(ldc=4),
 "w_M": wa(M=-1), "w_align_a": wa(a=P + 8), "w_align_lda": wa(lda=516), "w_align_sw": wa(sw=P + 4),
 "w_dtype": wa(ct=2), "w_special": wa(fw=3, sp=ctypes.cast((ctypes.c_float * 4)(5.0, -5.0, 4.0, -2.5), vp)),
 # segmented matmul
 "s_nseg": sg(nseg=9), "s_nseg_neg": sg(nseg=-1), "s_null_seg": sg(seg=None), "s_null_g": sg(g=None),
 "s_sum": sg(N=9, ldc=12), "s_neg": sg(seg=ctypes.cast((ctypes.c_int64 * 3)(4, -2, 6), vp)),
 "s_align": sg(g=P + 2), "s_mixed": sg(fa=1), "s_K": sg(K=24),
 # matmul quantizing bf16 activations on load
 "a_null_a": ab(a=None), "a_one_out": ab(co=P), "a_rule": ab(rule=2), "a_rule_flag": ab(rule=0x101),
 "a_fw_mx": ab(fw=1), "a_K": ab(K=256, lda=256), "a_lda": ab(lda=256), "a_align": ab(co=P + 4, so=P),
 "a_lda_align": ab(lda=516), "a_seg": ab(seg=ctypes.cast(SEG, vp), nseg=3, N=7), "a_sp": ab(fw=3),
 # special-value search
 "t_null_w": ts(w=None), "t_null_w0": ts(w=None, rows=0, ws=None, gmode=5), "t_null_table": ts(table=None), "t_null_g": ts(g=None), "t_null_ws": ts(ws=None),
 "t_cols": ts(cols=40, ld=40), "t_ld": ts(ld=32), "t_rows": ts(rows=-1), "t_ws": ts(wsb=4 * 28 * 8 - 8),
 "t_mode": ts(gmode=3), "t_dtype": ts(wt=4), "t_align": ts(sse=P + 4), "t_align_w": ts(ld=66),
 # channel scale
 "c_null": cs(t=None), "c_rows": cs(rows_x=0), "c_ld": cs(ldx=4), "c_alpha": cs(alpha=float("inf")),
}
print(json.dumps(res))
''')

EXPECTED = {
    "q_null_desc": 1, "q_null_x": 1, "q_null_codes": 1, "q_null_scales": 1, "q_null_global_auto": 1,
    "q_null_global_given": 1,
    "q_rows_neg": 2, "q_cols_zero": 2, "q_cols_block": 2, "q_ld_small": 2, "q_had_cols": 2,
    "q_x_align": 3, "q_ld_align": 3, "q_codes_align": 3, "q_chan_align": 3, "q_ld_align_bf16": 3,
    "q_bad_format": 4, "q_bad_struct": 5, "q_bad_block": 5, "q_mx_block": 5, "q_bad_rule": 5, "q_bad_flag": 5,
    "q_razer_rule": 5, "q_mx_rule": 5, "q_mx_pz": 5, "q_mx_global": 5, "q_bad_mode": 5, "q_bad_had": 5,
    "q_had16_cols": 2, "q_ue5m3_auto": 5, "q_ue5m3_rule": 5, "q_nv_expsearch": 5, "q_bad_format5": 4,
    "q_bad_dtype": 5, "q_special_grid": 5, "q_special_half": 5, "q_special_big": 5, "q_special_zero": 5,
    "q_special_nan": 5,
    "dq_null_out": 1, "dq_null_codes": 1, "dq_shape": 2, "dq_ld": 2, "dq_align": 3, "dq_ld_align": 3,
    "dq_dtype": 5, "dq_format": 4, "dq_block": 5,
    "g_null_a": 1, "g_null_c": 1, "g_null_special": 1, "g_mixed": 4, "g_razer_w_a": 4, "g_bad_format": 4,
    "g_ue5m3": 4, "g_ue5m3_w": 4,
    "g_K_block": 2, "g_K_mx": 2, "g_K_zero": 2, "g_M_neg": 2, "g_ldc": 2, "g_align": 3, "g_ldc_align": 3,
    "g_dtype": 5, "g_bad_special": 5, "g_K_big": 2, "g_tiles": 2,
    "gn_null_a": 1, "gn_mixed": 4, "gn_K_block": 2, "gn_align": 3, "gn_dtype": 5,
    "m_null_w": 1, "m_null_ws": 1, "m_K": 2, "m_K_big": 2, "m_ldh": 2, "m_N": 2, "m_moves": 5, "m_ws": 5,
    "m_align": 3,
    "w_null_a": 1, "w_null_sp": 1, "w_format_mx": 4, "w_format_ra": 4, "w_K": 2, "w_lda": 2, "w_lda_big": 2,
    "w_ldc": 2, "w_M": 2, "w_align_a": 3, "w_align_lda": 3, "w_align_sw": 3, "w_dtype": 5, "w_special": 5,
    "s_nseg": 5, "s_nseg_neg": 5, "s_null_seg": 1, "s_null_g": 1, "s_sum": 2, "s_neg": 2, "s_align": 3,
    "s_mixed": 4, "s_K": 2,
    "a_null_a": 1, "a_one_out": 1, "a_rule": 5, "a_rule_flag": 5, "a_fw_mx": 4, "a_K": 2, "a_lda": 2, "a_align": 3,
    "a_lda_align": 3, "a_seg": 2, "a_sp": 1,
    "t_null_w": 1, "t_null_w0": 5, "t_null_table": 1, "t_null_g": 1, "t_null_ws": 1, "t_cols": 2, "t_ld": 2, "t_rows": 2,
    "t_ws": 5, "t_mode": 5, "t_dtype": 5, "t_align": 3, "t_align_w": 3,
    "c_null": 1, "c_rows": 2, "c_ld": 2, "c_alpha": 5,
}


def test_argument_errors_are_reported_before_any_launch():
    import json
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    code = f"ROOT = {ROOT!r}\nLIB = {LIB!r}\n" + CHILD
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    got = json.loads(out.stdout.strip().splitlines()[-1])
    assert got == EXPECTED


def test_zero_rows_and_empty_gemm_enqueue_nothing():
    # rows == 0 / M == 0 are valid and return OK without any HIP call, even
    # with no visible device
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    code = f"ROOT = {ROOT!r}\nLIB = {LIB!r}\n" + CHILD.split("res = {")[0] + textwrap.dedent('''
print(q(rows=0), dq(rows=0), gm(M=0), gm(N=0), q(d=desc(global_mode=1), rows=0), gn(M=0), mq(N=0), wa(M=0),
      wa(N=0), sg(M=0), ab(M=0))
''')
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["0"] * 11
