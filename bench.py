#!/usr/bin/env python3
"""Benchmark of the FP4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]

A step is one pass of the whole path over one batch of synthetic input:

  prefill (default)  32768 x 5120 bf16 activations (Student-t, nu=4):
                     online NVFP4 4-over-6 quantization with a calibrated
                     (given) global scale, then the three projection W4A4
                     GEMMs N = 10240, 17408, 5120 (K = 5120) against weights
                     quantized offline (NVFP4, 4-over-6, auto global scale),
                     bf16 output.
  mxfp4_linear       4096 x 4096 bf16 activations with 8 outlier channels:
                     channel scale + block-Hadamard + MXFP4 quantization, then
                     the 4096 x 14336 x 4096 MXFP4 GEMM, fp32 output.
  razer_decode       RaZeR-A quantization of M x 5120 activations (M = 128),
                     then the GEMM against RaZeR-W weights 17408 x 5120;
                     also reported at M = 1 and 16 (graph-timed).

Inputs are resident in HBM before the timed region.  Prints one JSON line.
Kernel times come from HIP events recorded on the stream the kernels run on
(torch's current stream, which the library is handed).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "fp4": 10100.0}   # dense, published
METRIC = "FP4 quantize GB/s (% HBM peak); W4A4 GEMM TFLOP/s (% MFMA peak)"


def log(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


# ---------------------------------------------------------------- workloads
class Prefill:
    name = "prefill_hybrid_layer"
    M, K, NS = 32768, 5120, (10240, 17408, 5120)
    compute_dtype = "f16"
    gemm_kernel = "gemm_tile_kernel"
    quant_kernel = "nv16_four6_kernel"

    def __init__(self, B):
        import torch
        import datagen
        self.B = B
        log("[bench] generating prefill activations and weights")
        a = datagen.prefill_act(self.M, self.K)
        self.x = dev_bf16(a)
        # calibrated global scale for the online quantizer: the auto scale of a
        # calibration slice (rows 0..4095), computed by the library itself
        _, _, g = B.quantize(self.x[:4096], "nvfp4", 16, "4over6", "auto")
        self.g_act = g
        self.codes = torch.empty((self.M, self.K // 2), dtype=torch.uint8, device="cuda")
        self.scales = torch.empty((self.M, self.K // 16), dtype=torch.uint8, device="cuda")
        self.w = []
        for n in self.NS:
            w = torch.from_numpy(datagen.prefill_weight(n, self.K)).cuda()
            wc, ws, wg = B.quantize(w, "nvfp4", 16, "4over6", "auto")  # offline
            del w
            out = torch.empty((self.M, n), dtype=torch.bfloat16, device="cuda")
            self.w.append((wc, ws, wg, out))
        torch.cuda.synchronize()
        self.gemm_flops = [2.0 * self.M * n * self.K for n in self.NS]
        self.quant_bytes = self.M * self.K * 2 + self.M * self.K // 2 + self.M * self.K // 16

    def config(self):
        return {"workload": f"{self.name}_M{self.M}_K{self.K}_N{'-'.join(map(str, self.NS))}",
                "quant": "nvfp4 block16 e4m3 4over6 given-global bf16-in", "gemm": "nvfp4 x nvfp4 -> bf16",
                "M": self.M, "K": self.K, "N": list(self.NS)}

    def quantize_call(self):
        self.B.quantize(self.x, "nvfp4", 16, "4over6", "given", global_=self.g_act, codes=self.codes,
                        scales=self.scales)

    def gemm_calls(self, ev=None):
        for i, (wc, ws, wg, out) in enumerate(self.w):
            if ev: ev.mark(f"g{i}s")
            self.B.gemm("nvfp4", self.codes, self.scales, self.g_act, "nvfp4", wc, ws, wg, out=out)
            if ev: ev.mark(f"g{i}")

    def step(self, ev=None):
        if ev: ev.mark("q0")
        self.quantize_call()
        if ev: ev.mark("q1")
        self.gemm_calls(ev)


class MxLinear:
    name = "mxfp4_linear"
    M, K, N = 4096, 4096, 14336
    compute_dtype = "fp4"
    gemm_kernel = "gemm_tile_kernel"
    quant_kernel = "mx32_kernel"

    def __init__(self, B):
        import torch
        import datagen
        self.B = B
        d = datagen.mxfp4_linear(self.M, self.K, self.N)
        self.x = dev_bf16(d["X_bf16"])
        w = torch.from_numpy(d["W"]).cuda()
        self.t, r = B.channel_scale(self.x, w, 0.75)  # calibration
        self.wc, self.ws, _ = B.quantize(w, "mxfp4", 32, "absmax", "none", chan_scale=r, hadamard=32)
        del w
        self.codes = torch.empty((self.M, self.K // 2), dtype=torch.uint8, device="cuda")
        self.scales = torch.empty((self.M, self.K // 32), dtype=torch.uint8, device="cuda")
        self.out = torch.empty((self.M, self.N), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        self.NS = (self.N,)
        self.gemm_flops = [2.0 * self.M * self.N * self.K]
        self.quant_bytes = self.M * self.K * 2 + self.M * self.K // 2 + self.M * self.K // 32

    def config(self):
        return {"workload": f"{self.name}_M{self.M}_K{self.K}_N{self.N}",
                "quant": "mxfp4 + channel scale + block-Hadamard 32, bf16-in", "gemm": "mxfp4 x mxfp4 -> f32",
                "M": self.M, "K": self.K, "N": [self.N]}

    def quantize_call(self):
        self.B.quantize(self.x, "mxfp4", 32, "absmax", "none", chan_scale=self.t, hadamard=32,
                        codes=self.codes, scales=self.scales)

    def gemm_calls(self, ev=None):
        if ev: ev.mark("g0s")
        self.B.gemm("mxfp4", self.codes, self.scales, None, "mxfp4", self.wc, self.ws, None, out=self.out)
        if ev: ev.mark("g0")

    def step(self, ev=None):
        if ev: ev.mark("q0")
        self.quantize_call()
        if ev: ev.mark("q1")
        self.gemm_calls(ev)


class RazerDecode:
    name = "razer_decode"
    M, K, N = 128, 5120, 17408
    compute_dtype = "f16"
    gemm_kernel = "gemm_small_m_kernel"
    quant_kernel = "quantize_kernel"

    def __init__(self, B, M=128):
        import torch
        import datagen
        self.B = B
        self.M = M
        d = datagen.razer_decode(M, self.N, self.K)
        self.x = dev_bf16(d["A_bf16"])
        w = torch.from_numpy(d["W"]).cuda()
        self.sp = datagen.RAZER_SPECIAL
        self.wc, self.ws, self.wg = B.quantize(w, "razer_w", 16, "absmax", "auto", special=self.sp)
        del w
        self.codes = torch.empty((M, self.K // 2), dtype=torch.uint8, device="cuda")
        self.scales = torch.empty((M, self.K // 16), dtype=torch.uint8, device="cuda")
        self.g = torch.ones(1, dtype=torch.float32, device="cuda")
        self.out = torch.empty((M, self.N), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        self.NS = (self.N,)
        self.gemm_flops = [2.0 * M * self.N * self.K]
        self.quant_bytes = M * self.K * 2 + M * self.K // 2 + M * self.K // 16

    def config(self):
        return {"workload": f"{self.name}_M{self.M}_K{self.K}_N{self.N}",
                "quant": "razer_a block16 auto-global bf16-in", "gemm": "razer_a x razer_w -> f32",
                "M": self.M, "K": self.K, "N": [self.N]}

    def small_m(self, ms=(1, 16)):
        """The same step at decode batch sizes: RaZeR-A quantize of the first M
        activation rows and the GEMM against the same weights, each timed over
        20 launches captured in one HIP graph (these kernels run for tens of
        microseconds, less than a launch from Python).  The GEMM streams the
        weights once: % HBM is on those bytes."""
        import torch
        B = self.B
        w_bytes = self.N * self.K // 2 + self.N * self.K // 16
        res = []
        for M in ms:
            x = self.x[:M]
            codes = torch.empty((M, self.K // 2), dtype=torch.uint8, device="cuda")
            scales = torch.empty((M, self.K // 16), dtype=torch.uint8, device="cuda")
            g = torch.ones(1, dtype=torch.float32, device="cuda")
            out = torch.empty((M, self.N), dtype=torch.float32, device="cuda")
            t_q = graph_us(lambda: B.quantize(x, "razer_a", 16, "absmax", "auto", global_=g, codes=codes,
                                              scales=scales))
            # the same rows under NVFP4 abs-max, the plain rule the RaZeR-A time compares with
            t_r1 = graph_us(lambda: B.quantize(x, "nvfp4", 16, "absmax", "auto", global_=g, codes=codes,
                                               scales=scales))
            B.quantize(x, "razer_a", 16, "absmax", "auto", global_=g, codes=codes, scales=scales)
            t_g = graph_us(lambda: B.gemm("razer_a", codes, scales, g, "razer_w", self.wc, self.ws, self.wg,
                                          self.sp, out=out))
            gbs = w_bytes / (t_g * 1e-6) / 1e9
            res.append({"M": M, "quantize_us": round(t_q, 2), "quantize_absmax_nvfp4_us": round(t_r1, 2),
                        "gemm_us": round(t_g, 2),
                        "gemm_weight_bytes": w_bytes, "gemm_GB/s": round(gbs, 1),
                        "gemm_frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                        "gemm_hbm_floor_us": round(w_bytes / (HBM_PEAK_GBS * 1e3), 2)})
        return res

    def quantize_call(self):
        self.B.quantize(self.x, "razer_a", 16, "absmax", "auto", global_=self.g, codes=self.codes,
                        scales=self.scales)

    def gemm_calls(self, ev=None):
        if ev: ev.mark("g0s")
        self.B.gemm("razer_a", self.codes, self.scales, self.g, "razer_w", self.wc, self.ws, self.wg, self.sp,
                    out=self.out)
        if ev: ev.mark("g0")

    def step(self, ev=None):
        if ev: ev.mark("q0")
        self.quantize_call()
        if ev: ev.mark("q1")
        self.gemm_calls(ev)


WORKLOADS = {"prefill": Prefill, "mxfp4_linear": MxLinear, "razer_decode": RazerDecode}


def graph_us(fn, launches: int = 20, replays: int = 5) -> float:
    """microseconds per call of fn, from `launches` calls captured in one HIP
    graph and replayed, timed with HIP events on the replaying stream"""
    import torch
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(launches):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (launches * replays)


class Marks:
    """HIP events on the current stream, named by position in the step"""

    def __init__(self):
        self.rec = []

    def mark(self, name):
        import torch
        e = torch.cuda.Event(enable_timing=True)
        e.record(torch.cuda.current_stream())
        self.rec.append((name, e))

    def durations(self):
        """ms between a mark and the next: quantize = q0 -> q1, gemm i = g{i}s -> g{i}
        (the start mark sits right before the launch, so a wait for the host
        to enqueue the GEMM after a short quantize is not counted)"""
        out = {}
        for (n0, e0), (n1, e1) in zip(self.rec, self.rec[1:]):
            if (n0, n1) == ("q0", "q1") or (n0.endswith("s") and n1 == n0[:-1]):
                out.setdefault(n1, []).append(e0.elapsed_time(e1))
        return out


# ---------------------------------------------------------------- the other rows, measured beside the step
def event_ms(fn, reps: int = 3) -> float:
    """milliseconds per call of a long-running fn (HIP events on the current stream)"""
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def rate(nbytes=None, flops=None, us=None, peak_tf=None):
    out = {"us": round(us, 2)}
    if nbytes is not None:
        gbs = nbytes / (us * 1e-6) / 1e9
        out.update({"bytes": int(nbytes), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
    if flops is not None:
        tf = flops / (us * 1e-6) / 1e12
        out.update({"flops": flops, "TFLOP/s": round(tf, 1)})
        if peak_tf:
            out["frac_mfma"] = round(tf / peak_tf, 4)
    return out


def measure_mxfp4_linear(B) -> dict:
    """4096 x 4096 bf16 activations with 8 outlier channels: channel scale +
    block-Hadamard 32 + MXFP4 quantize (standard exponent, and the
    exponent-offset search), then the 4096 x 14336 x 4096 MXFP4 GEMM, fp32 out"""
    import torch
    wl = MxLinear(B)
    qb = wl.quant_bytes
    t_q = graph_us(wl.quantize_call)
    t_qs = graph_us(lambda: B.quantize(wl.x, "mxfp4", 32, "expsearch", "none", chan_scale=wl.t, hadamard=32,
                                       codes=wl.codes, scales=wl.scales))
    wl.quantize_call()
    t_g = event_ms(lambda: wl.gemm_calls(), reps=10) * 1e3
    res = {"workload": wl.config()["workload"], "quantize": {"kernel": "mx32_kernel", **rate(qb, us=t_q)},
           "quantize_expsearch": rate(qb, us=t_qs),
           "gemm": {"kernel": "gemm_tile_kernel", **rate(flops=wl.gemm_flops[0], us=t_g,
                                                         peak_tf=MFMA_PEAK_TFLOPS["fp4"])}}
    del wl
    torch.cuda.empty_cache()
    return res


def measure_decode(B) -> dict:
    """The RaZeR decode layer (K 5120, N 17408) at M = 1, 16, 128: RaZeR-A
    quantize + RaZeR-A x RaZeR-W GEMM; the weight-only matmul on bf16
    activations; the NVFP4 4-over-6 activation quantize fused into the
    matmul against the same weight, beside the two launches it replaces; a
    fused three-way projection (segments 4096/1024/1024 rows of 5120, each
    under its own global scale) beside the plain matmul of the same shape.
    Graph-timed.  The weight stream (codes + scales, read once per launch)
    sets each matmul's HBM floor."""
    import torch
    wl = RazerDecode(B, 128)
    res = {"workload": "razer_decode_K5120_N17408", "weight_bytes": wl.N * wl.K // 2 + wl.N * wl.K // 16,
           "cases": wl.small_m((1, 16, 128))}
    w_bytes = res["weight_bytes"]
    _, _, g_a = B.quantize(wl.x, "nvfp4", 16, "4over6", "auto")
    for c in res["cases"]:
        M = c["M"]
        x = wl.x[:M]
        out = torch.empty((M, wl.N), dtype=torch.float32, device="cuda")
        codes = torch.empty((M, wl.K // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((M, wl.K // 16), dtype=torch.uint8, device="cuda")
        t_w16 = graph_us(lambda: B.gemm_w4a16(x, "razer_w", wl.wc, wl.ws, wl.wg, wl.sp, out=out))
        t_fused = graph_us(lambda: B.gemm_act_bf16(x, "4over6", g_a, "razer_w", wl.wc, wl.ws, wl.wg, None, wl.sp,
                                                   out=out))
        t_q = graph_us(lambda: B.quantize(x, "nvfp4", 16, "4over6", "given", global_=g_a, codes=codes,
                                          scales=scales))
        B.quantize(x, "nvfp4", 16, "4over6", "given", global_=g_a, codes=codes, scales=scales)
        t_g = graph_us(lambda: B.gemm("nvfp4", codes, scales, g_a, "razer_w", wl.wc, wl.ws, wl.wg, wl.sp, out=out))
        c["w4a16"] = {"kernel": "gemm_small_m_kernel (bf16 A)", **rate(w_bytes + M * wl.K * 2, us=t_w16)}
        c["act_quantized_on_load"] = {"kernel": "gemm_small_m_kernel (A quantized on load)",
                                      **rate(w_bytes + M * wl.K * 2, us=t_fused),
                                      "separate_quantize_us": round(t_q, 2), "separate_gemm_us": round(t_g, 2)}
    # fused projection with per-segment global scales (M = 16), nvfp4 weights
    M, segs = 16, [4096, 1024, 1024]
    N = sum(segs)
    w = torch.randn((N, wl.K), device="cuda") * 0.02
    wc, ws, wg = B.quantize(w, "nvfp4", 16, "absmax", "auto")
    del w
    gs = torch.stack([wg[0], wg[0] * 2, wg[0] * 0.5])
    ca, sa, ga = B.quantize(wl.x[:M], "nvfp4", 16, "absmax", "auto")
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    t_seg = graph_us(lambda: B.gemm_segmented("nvfp4", ca, sa, ga, "nvfp4", wc, ws, gs, segs, None, out=out))
    t_one = graph_us(lambda: B.gemm("nvfp4", ca, sa, ga, "nvfp4", wc, ws, wg, None, out=out))
    res["segmented_projection"] = {"M": M, "segments": segs, "K": wl.K, "segmented_us": round(t_seg, 2),
                                   "single_scale_us": round(t_one, 2)}
    # offline special-value search over the same 17408 x 5120 weight (fp32)
    wf = torch.from_numpy(__import__("datagen").razer_decode(1)["W"]).cuda()
    t_s = event_ms(lambda: B.razer_table_search(wf, "auto"), reps=3) * 1e3
    table, _, _ = B.razer_table_search(wf, "auto")
    res["table_search"] = {"kernel": "razer_search_rows_kernel", "shape": list(wf.shape),
                           **rate(wf.numel() * 4, us=t_s), "table": [float(v) for v in table.cpu()]}
    del wf, wl
    torch.cuda.empty_cache()
    return res


def measure_variants(B) -> dict:
    """The scale-format variants on 4096 x 4096 FP32 normal samples (block
    16 unless stated): UE5M3 scales (4-over-6, no global), NVFP4 4-over-6
    after a size-16 block-Hadamard (given global), MXFP4 exponent-offset
    search (block 32); graph-timed, algorithmic bytes = input + codes + scales"""
    import torch
    import datagen
    x = torch.from_numpy(datagen.sweep("normal")).cuda()
    R, C = x.shape
    codes = torch.empty((R, C // 2), dtype=torch.uint8, device="cuda")
    s16 = torch.empty((R, C // 16), dtype=torch.uint8, device="cuda")
    s32 = torch.empty((R, C // 32), dtype=torch.uint8, device="cuda")
    g = torch.full((1,), float(x.abs().max()) / 2688.0, device="cuda")
    b16, b32 = R * C * 4 + R * C // 2 + R * C // 16, R * C * 4 + R * C // 2 + R * C // 32
    out = {"workload": "scale_variants_4096x4096_f32"}
    out["ue5m3_4over6"] = rate(b16, us=graph_us(lambda: B.quantize(x, "ue5m3", 16, "4over6", "none", codes=codes,
                                                                     scales=s16)))
    out["nvfp4_had16_4over6"] = rate(b16, us=graph_us(lambda: B.quantize(x, "nvfp4", 16, "4over6", "given",
                                                                           hadamard=16, global_=g, codes=codes,
                                                                           scales=s16)))
    out["nvfp4_4over6"] = rate(b16, us=graph_us(lambda: B.quantize(x, "nvfp4", 16, "4over6", "given", global_=g,
                                                                     codes=codes, scales=s16)))
    out["mxfp4_expsearch"] = rate(b32, us=graph_us(lambda: B.quantize(x, "mxfp4", 32, "expsearch", "none",
                                                                        codes=codes, scales=s32)))
    out["mxfp4_absmax"] = rate(b32, us=graph_us(lambda: B.quantize(x, "mxfp4", 32, "absmax", "none", codes=codes,
                                                                     scales=s32)))
    del x
    torch.cuda.empty_cache()
    return out


def measure_macaq(B) -> dict:
    """MACaQ calibration of a 1024 x 4096 slice of the MXFP4 linear weight
    (N(0, 0.02)) with the binary64 Hessian X^T X of 4096 synthetic
    activation rows (the MXFP4 linear recipe: normal with 8 outlier
    channels), move cap 2K per row; one call timed with HIP events"""
    import torch
    import datagen
    d = datagen.mxfp4_linear(4096, 4096, 1024)
    X = torch.from_numpy(datagen.bf16_bits_to_f32(d["X_bf16"])).cuda().double()
    H = X.T @ X
    W = torch.from_numpy(d["W"]).cuda()
    del X
    t = event_ms(lambda: B.macaq_quantize(W, H), reps=1)
    _, _, moves = B.macaq_quantize(W, H)
    torch.cuda.synchronize()
    res = {"workload": "macaq_N1024_K4096", "ms": round(t, 2), "rows_per_s": round(1024 / (t * 1e-3), 1),
           "mean_moves_per_row": round(float(moves.double().mean()), 1)}
    del W, H
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- CPU baseline
def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n


def cpu_baseline_parallel(wl, threads: int, budget_s: float = 10.0):
    """The same oracle calls on `threads` threads at once, each on its own
    rows (the oracle's C functions run without the interpreter lock): the
    quantize of 32 rows per thread and one activation row against 512
    replicated weight rows per thread, repeated for the budget; per-element
    and per-MAC times from the aggregate, extrapolated to one whole step."""
    import concurrent.futures as cf
    import datagen
    import oracle as O
    K = wl.K
    a = datagen.prefill_act(32 * threads, K)
    g = float(wl.g_act.item())
    codes, scales = O.quantize_rows(O.transform(a[:2]), "nvfp4", 16, O.FOUR_OVER_SIX, g)
    wsamp = [O.quantize_rows(datagen.normal((1, K), 12 + i, 0.02), "nvfp4", 16, O.FOUR_OVER_SIX, 1e-4)
             for i in range(len(wl.NS))]
    xt = O.transform(a)

    def q_job(i):
        O.quantize_rows(xt[32 * i:32 * i + 32], "nvfp4", 16, O.FOUR_OVER_SIX, g)

    with cf.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(q_job, range(threads)))
        tq = (time.perf_counter() - t0) / (32 * threads * K)

        per_mac = []
        for (wc1, ws1) in wsamp:
            wc = np.repeat(wc1, 512, axis=0)
            ws = np.repeat(ws1, 512, axis=0)

            def g_job(_):
                n, t1 = 0, time.perf_counter()
                while time.perf_counter() - t1 < budget_s / (2 * len(wl.NS)):
                    O.gemm_rows("nvfp4", codes, scales, 1.0, "nvfp4", wc, ws, 1.0, None, 2, 512, K, 0, 1)
                    n += 512 * K
                return n

            t0 = time.perf_counter()
            done = sum(ex.map(g_job, range(threads)))
            per_mac.append((time.perf_counter() - t0) / done)
    return tq * wl.M * K + sum(tm * wl.M * n * K for tm, n in zip(per_mac, wl.NS))


def cpu_baseline(wl, budget_s: float = 20.0):
    """The oracle, as it is, on a bounded sample of the same workload, single
    thread; extrapolated linearly to one whole step.  For the prefill step
    also on the host's cores at once (at most 16 threads)."""
    import datagen
    import oracle as O
    O.build()
    K = wl.K
    if isinstance(wl, Prefill):
        rows = 256
        a = datagen.prefill_act(rows, K)  # same distribution; a slice of the recipe
        g = float(wl.g_act.item())
        t0 = time.perf_counter()
        O.quantize_rows(O.transform(a), "nvfp4", 16, O.FOUR_OVER_SIX, g)
        tq = (time.perf_counter() - t0) / (rows * K)  # s per element
        codes, scales = O.quantize_rows(O.transform(a[:2]), "nvfp4", 16, O.FOUR_OVER_SIX, g)
        fa = fw = "nvfp4"
        wsamp = [O.quantize_rows(datagen.normal((1, K), 12 + i, 0.02), "nvfp4", 16, O.FOUR_OVER_SIX, 1e-4)
                 for i in range(len(wl.NS))]
        sp = None
    elif isinstance(wl, MxLinear):
        rows = 256
        a = datagen.mxfp4_linear(wl.M, wl.K, 16)["X_bf16"][:rows]
        t = wl.t.cpu().numpy()
        t0 = time.perf_counter()
        O.quantize(a, "mxfp4", 32, O.ABSMAX, O.G_NONE, chan_scale=t, hadamard=32)
        tq = (time.perf_counter() - t0) / (rows * K)
        codes, scales, _ = O.quantize(a[:2], "mxfp4", 32, O.ABSMAX, O.G_NONE, chan_scale=t, hadamard=32)
        fa = fw = "mxfp4"
        wsamp = [O.quantize_rows(datagen.normal((1, K), 6, 0.02), "mxfp4", 32, O.ABSMAX, 1.0)]
        sp = None
    else:
        rows = min(wl.M, 128)
        a = datagen.razer_decode(wl.M, with_weight=False)["A_bf16"][:rows]
        t0 = time.perf_counter()
        O.quantize(a, "razer_a", 16, O.ABSMAX, O.G_AUTO)
        tq = (time.perf_counter() - t0) / (rows * K)
        codes, scales, _ = O.quantize(a[:2], "razer_a", 16, O.ABSMAX, O.G_AUTO)
        fa, fw = "razer_a", "razer_w"
        sp = datagen.RAZER_SPECIAL
        wsamp = [O.quantize_rows(datagen.normal((1, K), 7, 0.02), "razer_w", 16, O.ABSMAX, 1e-4, sp)]
    # GEMM: time one A row against a replicated sample of W rows until the budget is used
    t_gemm_per_mac = []
    for (wc1, ws1), n in zip(wsamp, wl.NS):
        reps = 2048
        wc = np.repeat(wc1, reps, axis=0)
        ws = np.repeat(ws1, reps, axis=0)
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < budget_s / (2 * len(wl.NS)):
            O.gemm_rows(fa, codes, scales, 1.0, fw, wc, ws, 1.0, sp, 2, reps, K, 0, 1)
            done += reps * K
        t_gemm_per_mac.append((time.perf_counter() - t0) / done)
    t_step = tq * wl.M * K + sum(tm * wl.M * n * K for tm, n in zip(t_gemm_per_mac, wl.NS))
    flops = sum(wl.gemm_flops)
    model, ncpu = cpu_info()
    out = {
        "value": flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"single-thread oracle: quantize of {rows} x {K} rows, GEMM of 1 activation row against "
                   f"2048 weight rows per projection repeated for ~{budget_s / 2:.0f} s; per-element and per-MAC "
                   f"times extrapolated linearly to the full step"),
        "step_s_extrapolated": t_step,
        "cpu_model": model,
        "host_cpus": ncpu,
    }
    if isinstance(wl, Prefill) and ncpu > 1:
        threads = min(ncpu, 16)
        t_par = cpu_baseline_parallel(wl, threads)
        out.update({"value": flops / t_par / 1e12, "cores": threads, "step_s_extrapolated": t_par,
                    "single_thread_value": flops / t_step / 1e12,
                    "sample": out["sample"] + f"; value: the same oracle on {threads} threads at once, "
                              f"each on its own rows (32 quantized rows and 1 x 512 GEMM rows per thread, "
                              f"~{10:.0f} s)"})
    return out


# ---------------------------------------------------------------- per-workload table
def oracle_times(jobs, threads: int):
    """seconds per job (zero-argument oracle calls of equal size, on disjoint
    rows or repeated), run one after another, then the wall time of all of
    them at once on `threads` threads (the oracle's C functions run without
    the interpreter lock) divided by their number: the time per job's worth
    of work on that many cores"""
    import concurrent.futures as cf
    t0 = time.perf_counter()
    for j in jobs:
        j()
    single = (time.perf_counter() - t0) / len(jobs)
    with cf.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda j: j(), jobs))
        par = time.perf_counter() - t0
    return single, par / len(jobs)


def config_table(B) -> dict:
    """GPU time and oracle time for each workload's quantize and GEMM: the GPU
    graph- or event-timed at full size; the oracle on row samples (stated
    per entry), single thread and on up to 16 host threads at once,
    extrapolated linearly to the full size"""
    import torch
    import datagen
    import oracle as O
    O.build()
    model, ncpu = cpu_info()
    threads = max(1, min(16, ncpu))
    out = {"cpu_model": model, "host_cpus": ncpu, "threads": threads, "rows": []}

    def add(cfg, op, gpu_us, work, unit, sample, jobs, scale):
        """jobs: `threads` oracle calls of equal size; scale: full work / one call's work"""
        one, par = oracle_times(jobs, threads)
        rate = lambda sec: work / sec / (1e9 if unit == "GB/s" else 1e12)
        out["rows"].append({"config": cfg, "op": op, "gpu_us": round(gpu_us, 2),
                            f"gpu_{unit}": round(rate(gpu_us * 1e-6), 2),
                            "oracle_1t_s": round(one * scale, 3), f"oracle_1t_{unit}": rate(one * scale),
                            f"oracle_{threads}t_s": round(par * scale, 3),
                            f"oracle_{threads}t_{unit}": rate(par * scale), "oracle_sample": sample})
        log(f"[table] {cfg} {op}: gpu {gpu_us:.1f} us, oracle {one * scale:.2f} s (1 thread)")

    # C1: tiny
    d = datagen.tiny()
    W, A = torch.from_numpy(d["W"]).cuda(), torch.from_numpy(d["A"]).cuda()
    for rule, orule in (("absmax", O.ABSMAX), ("4over6", O.FOUR_OVER_SIX), ("brute", O.BRUTE)):
        t = graph_us(lambda: B.quantize(W, "nvfp4", 16, rule, "none"))
        nb = 256 * 256 * 4 + 256 * 128 + 256 * 16
        add("tiny", f"quantize W 256x256 nvfp4 {rule}", t, nb, "GB/s", "whole tensor",
            [lambda: O.quantize(d["W"], "nvfp4", 16, orule, O.G_NONE)] * threads, 1.0)
    ca, sa, _ = B.quantize(A, "nvfp4", 16, "absmax", "none")
    cw, sw, _ = B.quantize(W, "nvfp4", 16, "absmax", "none")
    o = torch.empty((64, 256), device="cuda")
    t = graph_us(lambda: B.gemm("nvfp4", ca, sa, None, "nvfp4", cw, sw, None, out=o))
    oca, osa, _ = O.quantize(d["A"], "nvfp4", 16, O.ABSMAX, O.G_NONE)
    ocw, osw, _ = O.quantize(d["W"], "nvfp4", 16, O.ABSMAX, O.G_NONE)
    add("tiny", "gemm 64x256x256", t, 2.0 * 64 * 256 * 256, "TFLOP/s", "whole product",
        [lambda: O.gemm_rows("nvfp4", oca, osa, 1.0, "nvfp4", ocw, osw, 1.0, None, 64, 256, 256)] * threads, 1.0)
    # C2: sweep (B = 16; the other blocks and rules: --quant-sweep)
    x_np = datagen.sweep("normal")
    x = torch.from_numpy(x_np).cuda()
    g = torch.full((1,), float(np.abs(x_np).max()) / 2688.0, device="cuda")
    for rule, orule in (("absmax", O.ABSMAX), ("4over6", O.FOUR_OVER_SIX)):
        t = graph_us(lambda: B.quantize(x, "nvfp4", 16, rule, "given", global_=g))
        nb = 4096 * 4096 * 4 + 4096 * 2048 + 4096 * 256
        add("sweep", f"quantize 4096x4096 f32 nvfp4 B16 {rule} given g", t, nb, "GB/s", "64 rows per call",
            [(lambda i=i: O.quantize_rows(x_np[64 * i:64 * i + 64], "nvfp4", 16, orule, float(g.item())))
             for i in range(threads)], 4096 / 64)
    del x
    # C3: MXFP4 linear
    wl = MxLinear(B)
    t = graph_us(wl.quantize_call)
    dm = datagen.mxfp4_linear(4096, 4096, 16)
    tt = wl.t.cpu().numpy()
    add("mxfp4_linear", "act quantize 4096x4096 bf16 mxfp4 D+B", t, wl.quant_bytes, "GB/s", "64 rows per call",
        [(lambda i=i: O.quantize(dm["X_bf16"][64 * i:64 * i + 64], "mxfp4", 32, O.ABSMAX, O.G_NONE, chan_scale=tt,
                                 hadamard=32)) for i in range(threads)], 4096 / 64)
    wl.quantize_call()
    t = event_ms(lambda: wl.gemm_calls(), reps=10) * 1e3
    oc, os_, _ = O.quantize(dm["X_bf16"][:2], "mxfp4", 32, O.ABSMAX, O.G_NONE, chan_scale=tt, hadamard=32)
    w1 = O.quantize_rows(datagen.normal((1, 4096), 6, 0.02), "mxfp4", 32, O.ABSMAX, 1.0)
    wc, ws = np.repeat(w1[0], 1024, axis=0), np.repeat(w1[1], 1024, axis=0)
    add("mxfp4_linear", "gemm 4096x14336x4096 f32 out", t, wl.gemm_flops[0], "TFLOP/s",
        "1 activation row x 1024 weight rows per call",
        [lambda: O.gemm_rows("mxfp4", oc, os_, 1.0, "mxfp4", wc, ws, 1.0, None, 2, 1024, 4096, 0, 1)] * threads,
        4096 * 14336 / 1024)
    del wl
    torch.cuda.empty_cache()
    # C4: RaZeR decode
    dec = RazerDecode(B, 128)
    for M in (1, 16, 128):
        xm = dec.x[:M]
        codes = torch.empty((M, 2560), dtype=torch.uint8, device="cuda")
        scales = torch.empty((M, 320), dtype=torch.uint8, device="cuda")
        gq = torch.ones(1, device="cuda")
        out_m = torch.empty((M, 17408), device="cuda")
        tq = graph_us(lambda: B.quantize(xm, "razer_a", 16, "absmax", "auto", global_=gq, codes=codes,
                                         scales=scales))
        B.quantize(xm, "razer_a", 16, "absmax", "auto", global_=gq, codes=codes, scales=scales)
        tg = graph_us(lambda: B.gemm("razer_a", codes, scales, gq, "razer_w", dec.wc, dec.ws, dec.wg, dec.sp,
                                     out=out_m))
        am = datagen.razer_decode(M, with_weight=False)["A_bf16"]
        add("razer_decode", f"razer_a quantize {M}x5120 auto g", tq, M * 5120 * 2 + M * 2560 + M * 320, "GB/s",
            "whole tensor", [lambda: O.quantize(am, "razer_a", 16, O.ABSMAX, O.G_AUTO)] * threads, 1.0)
        oc, os_, og = O.quantize(am[:1], "razer_a", 16, O.ABSMAX, O.G_AUTO)
        w1 = O.quantize_rows(datagen.normal((1, 5120), 7, 0.02), "razer_w", 16, O.ABSMAX, 1e-4, dec.sp)
        wc, ws = np.repeat(w1[0], 1024, axis=0), np.repeat(w1[1], 1024, axis=0)
        add("razer_decode", f"gemm {M}x17408x5120", tg, 2.0 * M * 17408 * 5120, "TFLOP/s",
            "1 activation row x 1024 weight rows per call",
            [lambda: O.gemm_rows("razer_a", oc, os_, og, "razer_w", wc, ws, 1.0, dec.sp, 1, 1024, 5120, 0, 1)]
            * threads, M * 17408 / 1024)
    del dec
    torch.cuda.empty_cache()
    # C5: prefill
    pf = Prefill(B)
    tq = graph_us(pf.quantize_call)
    ap = datagen.prefill_act(64 * threads, 5120)
    gp = float(pf.g_act.item())
    add("prefill", "act quantize 32768x5120 bf16 nvfp4 4over6 given g", tq, pf.quant_bytes, "GB/s",
        "64 rows per call", [(lambda i=i: O.quantize(ap[64 * i:64 * i + 64], "nvfp4", 16, O.FOUR_OVER_SIX, O.G_GIVEN,
                                                     g=gp)) for i in range(threads)], 32768 / 64)
    pf.quantize_call()
    oc, os_, _ = O.quantize(ap[:1], "nvfp4", 16, O.FOUR_OVER_SIX, O.G_GIVEN, g=gp)
    for i, (n, (wc_, ws_, wg_, o_)) in enumerate(zip(pf.NS, pf.w)):
        t = event_ms(lambda: pf.B.gemm("nvfp4", pf.codes, pf.scales, pf.g_act, "nvfp4", wc_, ws_, wg_, out=o_),
                     reps=5) * 1e3
        w1 = O.quantize_rows(datagen.normal((1, 5120), 12 + i, 0.02), "nvfp4", 16, O.FOUR_OVER_SIX, 1e-4)
        wc, ws = np.repeat(w1[0], 1024, axis=0), np.repeat(w1[1], 1024, axis=0)
        add("prefill", f"gemm 32768x{n}x5120 bf16 out", t, pf.gemm_flops[i], "TFLOP/s",
            "1 activation row x 1024 weight rows per call",
            [lambda: O.gemm_rows("nvfp4", oc, os_, gp, "nvfp4", wc, ws, 1.0, None, 1, 1024, 5120, 0, 1)] * threads,
            32768 * n / 1024)
    return out


# ---------------------------------------------------------------- traffic from PMC runs
def source_sha(kernel_source: str) -> str:
    """SHA-256 of a kernel source and the headers it includes"""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp4_e4m3_amd", "csrc")
    for name in (kernel_source, "nv_encode.hpp", "fp4q_internal.hpp"):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def traffic_record(kernel_source: str, name: str = "traffic.json"):
    """a committed record from rocprofv3 --pmc runs (HBM bytes, MFMA busy),
    only if it was taken from the current kernel source"""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_sha(kernel_source):
        return None
    return rec


# ---------------------------------------------------------------- profile helpers
COPY_PROBE_BYTES = 1 << 30


def copy_probe():
    """A plain elementwise kernel of known traffic (reads and writes 1 GiB of
    FP32 per launch), for scaling the HBM counters of rocprofv3 --pmc runs"""
    import torch
    n = COPY_PROBE_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log("[bench] copy probe done")


def quant_sweep() -> dict:
    """NVFP4 quantizer over 4096 x 4096 FP32 tensors (normal samples, and a
    heavy-tailed Student-t with 3 degrees of freedom), for abs-max,
    prevent-zero, 4-over-6 and the brute-force search at block sizes 4, 8, 16
    and 32 ([Finer] Method 2).  Each case is timed by graph replay, once with
    a given global scale (one pass over the input) and once with the automatic
    one (abs-max pass, finalize and zeroing launches added).  Algorithmic bytes
    per launch: the FP32 input, half a byte of codes and 1/B byte of scale per
    element."""
    import torch
    import datagen
    import block_scaled_fp4_e4m3_amd as B
    out = {"workload": "nvfp4_quantize_sweep_4096x4096_f32", "timing": "graph replay",
           "peak_GB/s": 8000.0, "cases": []}
    for dist in ("normal", "student_t3"):
        x_np = datagen.sweep(dist)
        R, C = x_np.shape
        x = torch.from_numpy(x_np).to("cuda")
        g = torch.full((1,), float(np.abs(x_np).max()) / 2688.0, device="cuda")
        ga = torch.empty(1, device="cuda")
        codes = torch.empty((R, C // 2), dtype=torch.uint8, device="cuda")
        for rule in ("absmax", "absmax+pz", "4over6", "brute"):
            for blk in (4, 8, 16, 32):
                scales = torch.empty((R, C // blk), dtype=torch.uint8, device="cuda")
                t = graph_us(lambda: B.quantize(x, "nvfp4", blk, rule, "given", global_=g, codes=codes,
                                                scales=scales))
                ta = graph_us(lambda: B.quantize(x, "nvfp4", blk, rule, "auto", global_=ga, codes=codes,
                                                 scales=scales))
                nbytes = R * C * 4 + R * C // 2 + R * C // blk
                out["cases"].append({"dist": dist, "rule": rule, "block": blk, "given_us": round(t, 2),
                                     "bytes": nbytes, "GB/s": round(nbytes / t / 1e3, 1),
                                     "frac_hbm": round(nbytes / t / 1e3 / 8000.0, 4), "auto_us": round(ta, 2)})
                log(f"[sweep] {dist} {rule} B={blk}: {t:.1f} us given, {ta:.1f} us auto")
        del x, codes
    return out


def summarize_stats(stats_csv: str, out_md: str, title: str, command: str) -> None:
    """rocprofv3 kernel_stats.csv -> short markdown table"""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    with open(out_md, "w") as f:
        f.write(f"# {title}\n\nCommand (from the repository root, on an MI355X):\n\n```\n{command}\n```\n\n")
        f.write("| kernel | calls | average (us) | min (us) | max (us) | share (%) |\n|---|---|---|---|---|---|\n")
        for r in rows:
            name = r["Name"].replace("fp4q::(anonymous namespace)::", "").replace("void ", "")
            name = name.split("(")[0] if "at::native" not in name else name[:60]
            f.write(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                    f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |\n")


def _counter_means(csv_path: str, counter: str, name_part: str, largest_grid: bool = False):
    """mean value of a counter over the dispatches of kernels matching
    name_part (with largest_grid: only those with the largest grid, the
    workload's own launches)"""
    import csv
    rows = [r for r in csv.DictReader(open(csv_path)) if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]]
    if largest_grid and rows:
        g = max(int(r["Grid_Size"]) for r in rows)
        rows = [r for r in rows if int(r["Grid_Size"]) == g]
    vals = [float(r["Counter_Value"]) for r in rows]
    if not vals:
        raise SystemExit(f"no {counter} samples for kernels matching {name_part!r} in {csv_path}")
    return float(np.mean(vals)), len(vals)


def mfma_from_pmc(workload: str, csv_path: str, out_json: str, kernel: str = "gemm_tile_kernel",
                  xcds: int = 8, simds: int = 1024) -> dict:
    """MFMA busy fraction and shader clock of `kernel` from one rocprofv3 run
    of SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and
    SQ_INSTS_VALU_MFMA_MOPS_F16 (the profiler's MfmaUtil: busy cycles summed
    over the SIMDs over GUI-active cycles times the SIMD count; the reported
    GRBM_GUI_ACTIVE is the sum over the XCDs)"""
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if kernel not in r["Kernel_Name"]:
            continue
        d = per.setdefault(r["Dispatch_Id"], {"dur_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatches of {kernel!r} in {csv_path}")
    busy = [d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / xcds * simds) for d in per.values()]
    clk = [d["GRBM_GUI_ACTIVE"] / xcds / d["dur_ns"] for d in per.values()]
    flops = [d.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) * 512 for d in per.values()]
    rec = {"workload": workload, "kernel": kernel, "source_sha256": source_sha("gemm.hip"),
           "dispatches": len(per), "mfma_busy": float(np.mean(busy)), "sclk_GHz": float(np.mean(clk)),
           "mfma_flops_per_launch": float(np.mean(flops))}
    json.dump(rec, open(out_json, "w"), indent=1)
    return rec


def traffic_from_pmc(workload: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str,
                     out_json: str, kernel: str = "gemm_tile_kernel", source: str = "gemm.hip",
                     largest_grid: bool = False) -> dict:
    """HBM bytes per launch of `kernel` from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the copy probe"""
    fk, nf = _counter_means(fetch_csv, "FETCH_SIZE", kernel, largest_grid)
    wk, nw = _counter_means(write_csv, "WRITE_SIZE", kernel, largest_grid)
    cf, _ = _counter_means(copy_fetch_csv, "FETCH_SIZE", "neg")
    cw, _ = _counter_means(copy_write_csv, "WRITE_SIZE", "neg")
    f_scale = cf * 1024.0 / COPY_PROBE_BYTES   # counter KiB per true KiB
    w_scale = cw * 1024.0 / COPY_PROBE_BYTES
    fetch_b = fk * 1024.0 / f_scale
    write_b = wk * 1024.0 / w_scale
    rec = {"workload": workload, "kernel": kernel, "source_sha256": source_sha(source),
           "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
           "bytes_per_launch": fetch_b + write_b, "dispatches": {"fetch": nf, "write": nw},
           "copy_probe_scale": {"fetch": f_scale, "write": w_scale}}
    json.dump(rec, open(out_json, "w"), indent=1)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other rows (MXFP4 linear, decode batch sizes, variants, MACaQ, search)")
    ap.add_argument("--copy-probe", action="store_true", help="run the counter-scaling copy kernel and exit")
    ap.add_argument("--config-table", action="store_true",
                    help="GPU and oracle (1 thread and all host threads) times of every workload's quantize and "
                         "GEMM, one JSON line, exit")
    ap.add_argument("--quant-sweep", action="store_true",
                    help="time the NVFP4 quantizer over rules x block sizes on 4096 x 4096 FP32, print one JSON line, exit")
    ap.add_argument("--only", choices=["quantize", "gemm"],
                    help="run 20 launches of the workload's quantize (or its GEMMs) and exit: a short program "
                         "for rocprofv3 counter runs")
    ap.add_argument("--summarize-stats", nargs=4, metavar=("STATS_CSV", "OUT_MD", "TITLE", "COMMAND"),
                    help="write a markdown summary of a rocprofv3 kernel_stats.csv and exit")
    ap.add_argument("--mfma-record", nargs=2, metavar=("PMC_CSV", "OUT_JSON"),
                    help="MFMA busy fraction and clock of the GEMM of --workload from a rocprofv3 --pmc CSV, then exit")
    ap.add_argument("--quant-traffic-record", nargs=5,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "OUT_JSON"),
                    help="HBM bytes per quantize launch of --workload from rocprofv3 --pmc CSVs, then exit")
    ap.add_argument("--traffic-record", nargs=5,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "OUT_JSON"),
                    help="HBM bytes per GEMM launch of --workload from rocprofv3 --pmc CSVs, then exit")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    wl_name = {"prefill": "prefill_hybrid_layer_M32768_K5120_N10240-17408-5120",
               "mxfp4_linear": "mxfp4_linear_M4096_K4096_N14336",
               "razer_decode": "razer_decode_M128_K5120_N17408"}[args.workload]
    if args.traffic_record:
        print(json.dumps(traffic_from_pmc(wl_name, *args.traffic_record)))
        return
    if args.quant_traffic_record:
        print(json.dumps(traffic_from_pmc(wl_name, *args.quant_traffic_record,
                                          kernel=WORKLOADS[args.workload].quant_kernel, source="quantize.hip",
                                          largest_grid=True)))
        return
    if args.mfma_record:
        print(json.dumps(mfma_from_pmc(wl_name, *args.mfma_record, kernel=WORKLOADS[args.workload].gemm_kernel)))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: libfp4q has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_fp4_e4m3_amd as B
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe()
        return
    if args.quant_sweep:
        print(json.dumps(quant_sweep()))
        return
    if args.config_table:
        print(json.dumps(config_table(B)))
        return

    wl = WORKLOADS[args.workload](B)
    if args.only:
        for i in range(20):
            if args.only == "quantize":
                wl.quantize_call()
            else:
                wl.gemm_calls()
        torch.cuda.synchronize()
        log(f"[bench] 20 {args.only} launches of {wl.config()['workload']} done")
        return
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()

    # timed region: whole steps, synchronised on both sides
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        wl.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps

    # per-kernel durations over the same number of steps, events between launches
    marks = Marks()
    for _ in range(args.steps):
        wl.step(marks)
    torch.cuda.synchronize()
    d = marks.durations()
    q_interval_ms = float(np.mean(d["q1"]))
    # the quantize launch alone, replayed in a HIP graph: GPU time per launch
    # without the host launch gaps that the step interval includes (it is
    # short enough for them to matter)
    q_ms = graph_us(wl.quantize_call) * 1e-3
    g_ms = [float(np.mean(d[f"g{i}"])) for i in range(len(wl.NS))]

    flops_step = sum(wl.gemm_flops)
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[wl.compute_dtype]
    # dominant kernel: the GEMM; per launch = mean algorithmic FLOPs / mean duration
    gemm_avg_ms = float(np.mean(g_ms))
    gemm_avg_flops = float(np.mean(wl.gemm_flops))
    achieved = gemm_avg_flops / (gemm_avg_ms * 1e-3) / 1e12
    traffic = None
    rec = traffic_record("gemm.hip")
    if rec and rec.get("workload") == wl.config()["workload"]:
        traffic = rec.get("bytes_per_launch")
    roofline = {"bound": "mfma", "kernel": wl.gemm_kernel, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                "avg_launch_ms": round(gemm_avg_ms, 4), "algorithmic_flops_per_launch": gemm_avg_flops}
    mrec = traffic_record("gemm.hip", "mfma_busy.json")
    if mrec and mrec.get("workload") == wl.config()["workload"]:
        # counters of the same kernel: the MFMA pipes' busy fraction and the
        # shader clock during it (the published peak assumes 2.4 GHz)
        roofline.update({"mfma_busy": round(mrec["mfma_busy"], 4), "sclk_GHz": round(mrec["sclk_GHz"], 3)})
    qrec = traffic_record("quantize.hip", "traffic_quantize.json")
    q_traffic = qrec.get("bytes_per_launch") if qrec and qrec.get("workload") == wl.config()["workload"] else None
    quant_gbs = wl.quant_bytes / (q_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.compute_dtype,
        "data": "synthetic",
        "config": wl.config(),
        "quantize": {"kernel": wl.quant_kernel, "avg_launch_ms": round(q_ms, 4), "timing": "graph replay",
                     "step_interval_ms": round(q_interval_ms, 4), "bytes": wl.quant_bytes, "traffic": q_traffic,
                     "GB/s": round(quant_gbs, 1), "frac_hbm": round(quant_gbs / HBM_PEAK_GBS, 4)},
        "gemm": [{"N": n, "avg_launch_ms": round(t, 4), "TFLOP/s": round(f / (t * 1e-3) / 1e12, 1),
                  "frac": round(f / (t * 1e-3) / 1e12 / peak, 4)} for n, t, f in zip(wl.NS, g_ms, wl.gemm_flops)],
        "roofline": roofline,
    }
    if isinstance(wl, RazerDecode):
        log("[bench] decode batch sizes")
        out["decode_small_m"] = wl.small_m()
    if not args.no_rows and isinstance(wl, Prefill):
        # the other rows of the path, each at its own workload, on the same GPU after the step
        del wl.w
        torch.cuda.empty_cache()
        rows = {}
        for name, fn in (("mxfp4_linear", measure_mxfp4_linear), ("razer_decode", measure_decode),
                         ("scale_variants", measure_variants), ("macaq", measure_macaq)):
            log(f"[bench] row {name}")
            rows[name] = fn(B)
        out["rows"] = rows
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out))
    sys.stdout.flush()


if __name__ == "__main__":
    main()
