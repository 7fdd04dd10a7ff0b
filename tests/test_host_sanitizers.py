"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the oracle (every entry point on small inputs of every format, rule,
global mode and transform) and the C ABI's argument validation (every entry
point with valid arguments, every documented error, and extreme sizes that
an unchecked product would overflow).  The ABI is linked against recording
stubs of the launchers, so no GPU code is built or run; `gcc`/`g++` only."""
import os
import shutil
import subprocess
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")

ORACLE_DRIVER = textwrap.dedent(r'''
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "oracle.h"

static uint32_t st = 12345u;
static float urand(void) { st = st * 1664525u + 1013904223u; return (float)((st >> 8) & 0xFFFF) / 65536.0f; }

int main(void) {
  enum { R = 5, C = 128 };
  float x[R * C], t[C], sp[4] = {5.f, -5.f, 2.5f, -2.5f}, out[R * C], g;
  uint16_t xb[R * C];
  uint8_t codes[R * C / 2], scales[R * C / 4];
  for (int i = 0; i < R * C; ++i) {
    x[i] = (urand() - 0.5f) * ldexpf(1.0f, (int)(urand() * 20) - 10);
    uint32_t u; memcpy(&u, &x[i], 4); xb[i] = (uint16_t)(u >> 16);
  }
  x[3] = 0.f; x[7] = 6.0f; x[8] = -0.f;
  for (int j = 0; j < C; ++j) t[j] = 0.5f + urand();
  int fails = 0;
  const int blocks[4] = {4, 8, 16, 32};
  for (int fmt = 0; fmt <= 4; ++fmt)
    for (int bi = 0; bi < 4; ++bi)
      for (int rule = 0; rule <= 3; ++rule)
        for (int gm = 0; gm <= 2; ++gm)
          for (int had = 0; had <= 32; had += 16)
            for (int dt = 0; dt <= 1; ++dt) {
              g = 0.01f;
              int rc = or_quantize(fmt, blocks[bi], rule | (rule == 0 && bi == 1 ? OR_PREVENT_ZERO : 0), gm,
                                   (had == 16) ? t : NULL, had, sp, dt ? (const void*)xb : (const void*)x, dt,
                                   R, C, C, codes, scales, &g);
              if (rc == 0) {
                if (or_dequantize(fmt, blocks[bi], sp, codes, scales, g, R, C, out) != 0) ++fails;
              }
            }
  /* matmuls */
  float cw[3 * 3];
  uint8_t ac[3 * C / 2], as[3 * C / 16], wc[3 * C / 2], ws[3 * C / 16];
  g = 1.f;
  if (or_quantize(0, 16, 1, 0, NULL, 0, NULL, x, 0, 3, C, C, ac, as, &g)) ++fails;
  if (or_quantize(3, 16, 0, 1, NULL, 0, sp, x + C, 0, 3, C, C, wc, ws, &g)) ++fails;
  if (or_gemm_rows(0, ac, as, 1.f, 3, wc, ws, g, sp, 3, 3, C, 0, 3, cw)) ++fails;
  long ms[2] = {0, 2}, ns[2] = {1, 2};
  if (or_gemm_entries(0, ac, as, 1.f, 3, wc, ws, g, sp, 3, 3, C, ms, ns, 2, cw)) ++fails;
  if (or_gemm_w4a16_rows(xb, C, 3, wc, ws, g, sp, 3, 3, C, 1, 3, cw)) ++fails;
  double pair[OR_RAZER_NPAIRS];
  if (or_razer_table_search(x, 0, R, C, C, 1.f, pair) < 0) ++fails;
  if (or_razer_table_search(xb, 1, R, C, C, 0.5f, pair) < 0) ++fails;
  /* MACaQ */
  enum { K = 64, N = 3 };
  double h[K * K], obj[2 * N];
  int moves[N];
  for (int i = 0; i < K; ++i)
    for (int j = 0; j < K; ++j) h[i * K + j] = (i == j ? 2.0 : 0.0) + 0.1 * (double)(urand() - 0.5f) * (i != j);
  for (int i = 0; i < K; ++i) for (int j = 0; j < i; ++j) h[i * K + j] = h[j * K + i];
  uint8_t mc[N * K / 2], msc[N * K / 32];
  if (or_macaq_quantize(x, N, K, C, h, K, 2 * K, mc, msc, moves, obj)) ++fails;
  or_channel_scale(xb, 1, R, C, x, 0, R, C, C, 0.75, t, out);
  /* bad arguments are refused, not read */
  if (or_quantize(9, 16, 0, 0, NULL, 0, NULL, x, 0, R, C, C, codes, scales, &g) == 0) ++fails;
  if (or_gemm_w4a16_rows(xb, C, 1, wc, ws, g, sp, 3, 3, C, 0, 3, cw) == 0) ++fails;
  if (or_razer_table_search(x, 0, R, 40, C, 1.f, pair) >= 0) ++fails;
  printf("oracle driver: %d failures\n", fails);
  return fails != 0;
}
''')

ABI_STUBS = textwrap.dedent(r'''
#include "fp4q_internal.hpp"
namespace fp4q {
static int calls = 0;
int stub_calls() { return calls; }
hipError_t launch_quantize(int, int, int, int, const QuantParams&, hipStream_t) { ++calls; return hipSuccess; }
hipError_t launch_dequantize(int, int, const DequantParams&, hipStream_t) { ++calls; return hipSuccess; }
hipError_t launch_gemm(int, int, const GemmParams& p, hipStream_t, const Workspace&) {
  ++calls;
  for (int i = 0; i < p.nseg; ++i) if (p.seg_end[i] > p.N) return hipErrorInvalidValue;
  return hipSuccess;
}
hipError_t launch_gemm_w4a16(int, const GemmParams&, hipStream_t, const Workspace&) { ++calls; return hipSuccess; }
hipError_t launch_gemm_act_bf16(int, int, const GemmParams&, hipStream_t, const Workspace&) { ++calls; return hipSuccess; }
float* split_workspace(hipStream_t) { return nullptr; }
float* noalloc_scratch() { static float f[4]; return f; }
hipError_t launch_channel_scale(const ChanScaleParams&, hipStream_t) { ++calls; return hipSuccess; }
hipError_t launch_razer_search(const QuantParams&, int, double*, double*, float*, hipStream_t) { ++calls; return hipSuccess; }
hipError_t launch_macaq(const MacaqParams&, void*, size_t, hipStream_t) { ++calls; return hipSuccess; }
int64_t macaq_max_k() { return 5120; }
}  // namespace fp4q
''')

ABI_DRIVER = textwrap.dedent(r'''
#include <stdint.h>
#include <stdio.h>
#include <vector>
#include "fp4q.h"
namespace fp4q { int stub_calls(); }

int main() {
  const int64_t BIG = INT64_MAX, HUGE = (int64_t)1 << 62;
  // aligned fake device addresses: the stubs never touch them
  uint8_t* P = (uint8_t*)(uintptr_t)0x100000;
  float* F = (float*)(uintptr_t)0x200000;
  fp4q_quant_desc d{};
  d.struct_size = sizeof(d); d.format = FP4Q_NVFP4; d.block = 16; d.rule = FP4Q_RULE_4OVER6;
  d.global_mode = FP4Q_GLOBAL_GIVEN; d.special[0] = 5; d.special[1] = -5; d.special[2] = 2.5f; d.special[3] = -2.5f;
  int bad = 0;
  auto expect = [&](int got, int want, const char* what) {
    if (got != want) { printf("%s: %d, expected %d\n", what, got, want); ++bad; }
  };
  // valid calls reach the launchers
  expect(fp4q_quantize(&d, P, FP4Q_BF16, 64, 512, 512, P, P, F, nullptr), 0, "quantize");
  expect(fp4q_dequantize(&d, P, P, F, 64, 512, P, FP4Q_F32, 512, nullptr), 0, "dequantize");
  expect(fp4q_gemm_w4a4(FP4Q_NVFP4, P, P, F, FP4Q_NVFP4, P, P, F, nullptr, 64, 64, 512, P, FP4Q_F32, 64, nullptr), 0,
         "gemm");
  expect(fp4q_gemm_w4a4_noalloc(FP4Q_NVFP4, P, P, F, FP4Q_NVFP4, P, P, F, nullptr, 64, 64, 512, P, FP4Q_F32, 64,
                                nullptr), 0, "noalloc");
  int64_t seg[3] = {32, 16, 16};
  expect(fp4q_gemm_w4a4_segmented(FP4Q_NVFP4, P, P, F, FP4Q_NVFP4, P, P, F, seg, 3, nullptr, 64, 64, 512, P,
                                  FP4Q_F32, 64, nullptr), 0, "segmented");
  expect(fp4q_gemm_w4a4_act_bf16((const uint16_t*)P, 512, FP4Q_RULE_4OVER6, F, P, P, FP4Q_NVFP4, P, P, F, seg, 3,
                                 nullptr, 8, 64, 512, P, FP4Q_BF16, 64, nullptr), 0, "act_bf16");
  expect(fp4q_gemm_w4a16((const uint16_t*)P, 512, FP4Q_NVFP4, P, P, F, nullptr, 8, 64, 512, P, FP4Q_F32, 64,
                         nullptr), 0, "w4a16");
  expect(fp4q_razer_table_search(P, FP4Q_F32, 4, 64, 64, FP4Q_GLOBAL_AUTO, F, (double*)P, F, P, 4 * 28 * 8,
                                 nullptr), 0, "search");
  expect(fp4q_macaq_quantize(F, 4, 64, 64, (const double*)P, 64, 10, P, P, nullptr, P, 1 << 20, nullptr), 0,
         "macaq");
  expect(fp4q_channel_scale(P, FP4Q_BF16, 4, 8, P, FP4Q_F32, 4, 8, 8, 0.75, F, F, nullptr), 0, "channel_scale");
  const int launched = fp4q::stub_calls();
  // sizes whose byte counts or tile counts would overflow 64 bits are refused
  // before any product is formed
  expect(fp4q_quantize(&d, P, FP4Q_F32, 4, 64, BIG, P, P, F, nullptr) != 0, 1, "quantize huge pitch");
  expect(fp4q_quantize(&d, P, FP4Q_F32, BIG, 64, 64, P, P, F, nullptr) != 0, 1, "quantize huge rows");
  expect(fp4q_quantize(&d, P, FP4Q_F32, 4, HUGE, HUGE, P, P, F, nullptr) != 0, 1, "quantize huge cols");
  expect(fp4q_dequantize(&d, P, P, F, 4, 64, P, FP4Q_F32, BIG, nullptr) != 0, 1, "dequantize huge pitch");
  expect(fp4q_gemm_w4a4(FP4Q_NVFP4, P, P, F, FP4Q_NVFP4, P, P, F, nullptr, BIG, BIG, 512, P, FP4Q_F32, BIG, nullptr)
         != 0, 1, "gemm huge");
  expect(fp4q_gemm_w4a4(FP4Q_NVFP4, P, P, F, FP4Q_NVFP4, P, P, F, nullptr, 64, 64, 512, P, FP4Q_F32, BIG, nullptr)
         != 0, 1, "gemm huge ldc");
  int64_t segbig[2] = {BIG, BIG};
  expect(fp4q_gemm_w4a4_segmented(FP4Q_NVFP4, P, P, F, FP4Q_NVFP4, P, P, F, segbig, 2, nullptr, 64, 64, 512, P,
                                  FP4Q_F32, 64, nullptr), 2, "segments overflow");
  expect(fp4q_gemm_w4a16((const uint16_t*)P, 512, FP4Q_NVFP4, P, P, F, nullptr, BIG, BIG, 512, P, FP4Q_F32, BIG,
                         nullptr) != 0, 1, "w4a16 huge");
  expect(fp4q_gemm_w4a4_act_bf16((const uint16_t*)P, 512, 1, F, nullptr, nullptr, FP4Q_NVFP4, P, P, F, nullptr, 0,
                                 nullptr, BIG, 64, 512, P, FP4Q_F32, BIG, nullptr) != 0, 1, "act huge");
  expect(fp4q_razer_table_search(P, FP4Q_F32, BIG, 64, 64, FP4Q_GLOBAL_NONE, F, (double*)P, F, P, 1 << 20, nullptr)
         != 0, 1, "search huge rows");
  expect(fp4q_razer_table_search(P, FP4Q_F32, 4, 64, BIG, FP4Q_GLOBAL_NONE, F, (double*)P, F, P, 1 << 20, nullptr)
         != 0, 1, "search huge pitch");
  expect(fp4q_macaq_quantize(F, BIG, 64, BIG, (const double*)P, BIG, 10, P, P, nullptr, P, 1 << 20, nullptr) != 0,
         1, "macaq huge");
  expect(fp4q_channel_scale(P, FP4Q_BF16, BIG, BIG, P, FP4Q_F32, BIG, BIG, BIG, 0.75, F, F, nullptr) != 0, 1,
         "channel_scale huge");
  expect(fp4q::stub_calls(), launched, "no launch after a refused call");
  printf("abi driver: %d failures, %d launches\n", bad, launched);
  return bad != 0;
}
''')


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("no host compiler")
    return tmp_path_factory.mktemp("sanitize")


def _check(res):
    out = res.stdout + res.stderr
    assert "runtime error" not in out, out[-4000:]
    assert "AddressSanitizer" not in out and "LeakSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]


def test_oracle_under_sanitizers(workdir):
    src = workdir / "oracle_driver.c"
    src.write_text(ORACLE_DRIVER)
    exe = workdir / "oracle_driver"
    res = _run(["gcc", "-std=c11", "-ffp-contract=off", *SAN, "-I", os.path.join(ROOT, "oracle"), str(src),
                os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", str(exe)])
    assert res.returncode == 0, res.stderr[-4000:]
    res = _run([str(exe)], env=ENV)
    _check(res)
    assert "0 failures" in res.stdout


def test_abi_validation_under_sanitizers(workdir):
    csrc = os.path.join(ROOT, "block_scaled_fp4_e4m3_amd", "csrc")
    (workdir / "stubs.cpp").write_text(ABI_STUBS)
    (workdir / "driver.cpp").write_text(ABI_DRIVER)
    exe = workdir / "abi_driver"
    res = _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", *SAN, "-I/opt/rocm/include", "-I", csrc,
                "-I", os.path.join(ROOT, "include"), os.path.join(csrc, "abi.cpp"), str(workdir / "stubs.cpp"),
                str(workdir / "driver.cpp"), "-o", str(exe)])
    if res.returncode != 0 and "hip/hip_runtime.h" in res.stderr:
        pytest.skip("HIP headers not installed")
    assert res.returncode == 0, res.stderr[-4000:]
    res = _run([str(exe)], env=ENV)
    _check(res)
    assert "0 failures" in res.stdout
