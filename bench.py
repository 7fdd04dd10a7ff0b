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
    quant_kernel = "quantize_kernel"

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

    def step(self, ev=None):
        B = self.B
        if ev: ev.mark("q0")
        self.quantize_call()
        if ev: ev.mark("q1")
        for i, (wc, ws, wg, out) in enumerate(self.w):
            if ev: ev.mark(f"g{i}s")
            B.gemm("nvfp4", self.codes, self.scales, self.g_act, "nvfp4", wc, ws, wg, out=out)
            if ev: ev.mark(f"g{i}")


class MxLinear:
    name = "mxfp4_linear"
    M, K, N = 4096, 4096, 14336
    compute_dtype = "fp4"
    gemm_kernel = "gemm_tile_kernel"
    quant_kernel = "quantize_kernel"

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

    def step(self, ev=None):
        B = self.B
        if ev: ev.mark("q0")
        self.quantize_call()
        if ev: ev.mark("q1")
        if ev: ev.mark("g0s")
        B.gemm("mxfp4", self.codes, self.scales, None, "mxfp4", self.wc, self.ws, None, out=self.out)
        if ev: ev.mark("g0")


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

    def step(self, ev=None):
        B = self.B
        if ev: ev.mark("q0")
        self.quantize_call()
        if ev: ev.mark("q1")
        if ev: ev.mark("g0s")
        B.gemm("razer_a", self.codes, self.scales, self.g, "razer_w", self.wc, self.ws, self.wg, self.sp, out=self.out)
        if ev: ev.mark("g0")


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


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(wl, budget_s: float = 20.0):
    """The oracle, as it is, on a bounded sample of the same workload, single
    thread; extrapolated linearly to one whole step."""
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
    return {
        "value": flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"single-thread oracle: quantize of {rows} x {K} rows, GEMM of 1 activation row against "
                   f"2048 weight rows per projection repeated for ~{budget_s / 2:.0f} s; per-element and per-MAC "
                   f"times extrapolated linearly to the full step"),
        "step_s_extrapolated": t_step,
    }


# ---------------------------------------------------------------- traffic from PMC runs
def traffic_record(kernel_source: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, only if
    they were taken from the current kernel source"""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "block_scaled_fp4_e4m3_amd", "csrc", kernel_source), "rb").read()
    if rec.get("source_sha256") != hashlib.sha256(src).hexdigest():
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


def _counter_means(csv_path: str, counter: str, name_part: str):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no {counter} samples for kernels matching {name_part!r} in {csv_path}")
    return float(np.mean(vals)), len(vals)


def traffic_from_pmc(workload: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str,
                     out_json: str, kernel: str = "gemm_tile_kernel") -> dict:
    """HBM bytes per launch of `kernel` from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the copy probe"""
    fk, nf = _counter_means(fetch_csv, "FETCH_SIZE", kernel)
    wk, nw = _counter_means(write_csv, "WRITE_SIZE", kernel)
    cf, _ = _counter_means(copy_fetch_csv, "FETCH_SIZE", "neg")
    cw, _ = _counter_means(copy_write_csv, "WRITE_SIZE", "neg")
    f_scale = cf * 1024.0 / COPY_PROBE_BYTES   # counter KiB per true KiB
    w_scale = cw * 1024.0 / COPY_PROBE_BYTES
    fetch_b = fk * 1024.0 / f_scale
    write_b = wk * 1024.0 / w_scale
    src = open(os.path.join(ROOT, "block_scaled_fp4_e4m3_amd", "csrc", "gemm.hip"), "rb").read()
    rec = {"workload": workload, "kernel": kernel, "source_sha256": hashlib.sha256(src).hexdigest(),
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
    ap.add_argument("--copy-probe", action="store_true", help="run the counter-scaling copy kernel and exit")
    ap.add_argument("--quant-sweep", action="store_true",
                    help="time the NVFP4 quantizer over rules x block sizes on 4096 x 4096 FP32, print one JSON line, exit")
    ap.add_argument("--summarize-stats", nargs=4, metavar=("STATS_CSV", "OUT_MD", "TITLE", "COMMAND"),
                    help="write a markdown summary of a rocprofv3 kernel_stats.csv and exit")
    ap.add_argument("--traffic-record", nargs=5,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "OUT_JSON"),
                    help="HBM bytes per GEMM launch of --workload from rocprofv3 --pmc CSVs, then exit")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.traffic_record:
        wl_name = {"prefill": "prefill_hybrid_layer_M32768_K5120_N10240-17408-5120",
                   "mxfp4_linear": "mxfp4_linear_M4096_K4096_N14336",
                   "razer_decode": "razer_decode_M128_K5120_N17408"}[args.workload]
        print(json.dumps(traffic_from_pmc(wl_name, *args.traffic_record)))
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

    wl = WORKLOADS[args.workload](B)
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
                     "step_interval_ms": round(q_interval_ms, 4), "bytes": wl.quant_bytes,
                     "GB/s": round(quant_gbs, 1), "frac_hbm": round(quant_gbs / HBM_PEAK_GBS, 4)},
        "gemm": [{"N": n, "avg_launch_ms": round(t, 4), "TFLOP/s": round(f / (t * 1e-3) / 1e12, 1),
                  "frac": round(f / (t * 1e-3) / 1e12 / peak, 4)} for n, t, f in zip(wl.NS, g_ms, wl.gemm_flops)],
        "roofline": roofline,
    }
    if isinstance(wl, RazerDecode):
        log("[bench] decode batch sizes")
        out["decode_small_m"] = wl.small_m()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out))
    sys.stdout.flush()


if __name__ == "__main__":
    main()
