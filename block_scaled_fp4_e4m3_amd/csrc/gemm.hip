// W4A4 block-scaled matmul on gfx950 matrix cores.
//
// Pages: NVFP4 W4A4 -- "Why Gated DeltaNet Survives 4-Bit Quantization"
// review, section 1; RaZeR weight-activation GEMM -- RaZeR summary 2.3 (two
// tensor-core passes on Blackwell; here the special value decodes exactly, so
// one pass suffices); MXFP4 W4A4 -- MACaQ review, section 3.
//
// MXFP4: codes and E8M0 exponents go straight into the block-scaled FP4 MFMA
// (V_MFMA_SCALE_F32_32X32X64_F8F6F4): one lane supplies the 32 codes of one
// MX block of its row and that block's exponent byte.
//
// NVFP4 family: value * E4M3 (or E3M3) scale has at most 8 significant bits
// and lies in [2^-10, 3360], so it is exact in f16; products of two are exact
// in FP32.  Each lane decodes its 8 codes with the gfx950 FP4 -> f16 convert
// (the convert applies only a power-of-two scale, 2^8 or 2^12) and one packed
// f16 multiply by the scale, whose f16 bit pattern is the scale byte shifted
// left by 7 (= scale * 2^-8 for E4M3, * 2^-12 for E3M3).  RaZeR's code 0x8
// (-0 after the convert) is then replaced by special * scale.  The f16 MFMA
// accumulates in FP32; the epilogue multiplies by RN32(g_a * g_w).
#include "fp4q_internal.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kTile = 128;  // workgroup tile (M and N); 4 waves of 64 x 64

template <int F>
__device__ __forceinline__ half8 decode8(uint32_t codes, uint32_t sb, const float* wspecial) {
  constexpr float kCvt = (F == RAZER_W) ? 4096.0f : 256.0f;
  const uint32_t k = (F == RAZER_W) ? (sb & 0x3Fu) : (sb & 0x7Fu);
  const _Float16 s16 = __builtin_bit_cast(_Float16, (uint16_t)(k << 7));
  const half2v s2 = {s16, s16};
  half8 out;
  static_for<0, 4>([&](auto ic) {
    constexpr int b = decltype(ic)::value;
    half2v v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, kCvt, b);
    v = v * s2;  // exact: value * scale
    out[2 * b] = v[0];
    out[2 * b + 1] = v[1];
  });
  if constexpr (F == RAZER_A || F == RAZER_W) {
    float v = (F == RAZER_A) ? ((sb & 0x80u) ? -5.0f : 5.0f) : wspecial[sb >> 6];
    const _Float16 vs = (_Float16)(v * kCvt) * s16;  // exact
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (((codes >> (4 * i)) & 15u) == 8u) out[i] = vs;
  }
  return out;
}

__device__ __forceinline__ void store_c(const GemmParams& p, int64_t row, int64_t col, float v) {
  if (row < p.M && col < p.N) {
    if (p.c_bf16) {
      uint32_t a = __float_as_uint(v);
      a = (a + 0x7FFFu + ((a >> 16) & 1u)) >> 16;
      ((uint16_t*)p.c)[row * p.ldc + col] = (uint16_t)a;
    } else {
      ((float*)p.c)[row * p.ldc + col] = v;
    }
  }
}

template <int FA, int FW>
__global__ __launch_bounds__(kThreads) void gemm_nv_kernel(GemmParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t m0 = (int64_t)blockIdx.y * kTile + (wave >> 1) * 64;
  const int64_t n0 = (int64_t)blockIdx.x * kTile + (wave & 1) * 64;
  const int r32 = lane & 31, kh = lane >> 5;
  const int64_t krow = p.K / 2, kb = p.K / 16;
  int64_t am[2], wn[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    am[t] = min(m0 + 32 * t + r32, p.M - 1);
    wn[t] = min(n0 + 32 * t + r32, p.N - 1);
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};
  for (int64_t kk = 0; kk < p.K; kk += 16) {
    half8 a[2], b[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t ca = *(const uint32_t*)(p.a_codes + am[t] * krow + kk / 2 + kh * 4);
      uint32_t sa = p.a_scales[am[t] * kb + kk / 16];
      a[t] = decode8<FA>(ca, sa, nullptr);
      uint32_t cw = *(const uint32_t*)(p.w_codes + wn[t] * krow + kk / 2 + kh * 4);
      uint32_t sw = p.w_scales[wn[t] * kb + kk / 16];
      b[t] = decode8<FW>(cw, sw, p.w_special);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  const float ga = p.a_global ? *p.a_global : 1.0f;
  const float gw = p.w_global ? *p.w_global : 1.0f;
  const float gg = ga * gw;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int64_t row = m0 + 32 * i + (r / 4) * 8 + kh * 4 + (r % 4);
        int64_t col = n0 + 32 * j + r32;
        store_c(p, row, col, gg * acc[i][j][r]);
      }
}

__global__ __launch_bounds__(kThreads) void gemm_mx_kernel(GemmParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t m0 = (int64_t)blockIdx.y * kTile + (wave >> 1) * 64;
  const int64_t n0 = (int64_t)blockIdx.x * kTile + (wave & 1) * 64;
  const int r32 = lane & 31, kh = lane >> 5;
  const int64_t krow = p.K / 2, kb = p.K / 32;
  int64_t am[2], wn[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    am[t] = min(m0 + 32 * t + r32, p.M - 1);
    wn[t] = min(n0 + 32 * t + r32, p.N - 1);
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};
  for (int64_t kk = 0; kk < p.K; kk += 64) {
    const int64_t k0 = kk + 32 * kh;  // this lane's MX block
    const bool live = k0 < p.K;       // K % 64 == 32: the upper half is empty
    i32x8 a[2], b[2];
    int sa[2], sw[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint4 ca = live ? *(const uint4*)(p.a_codes + am[t] * krow + k0 / 2) : make_uint4(0, 0, 0, 0);
      uint4 cw = live ? *(const uint4*)(p.w_codes + wn[t] * krow + k0 / 2) : make_uint4(0, 0, 0, 0);
      sa[t] = live ? (int)p.a_scales[am[t] * kb + k0 / 32] : 127;
      sw[t] = live ? (int)p.w_scales[wn[t] * kb + k0 / 32] : 127;
      a[t] = (i32x8){(int)ca.x, (int)ca.y, (int)ca.z, (int)ca.w, 0, 0, 0, 0};
      b[t] = (i32x8){(int)cw.x, (int)cw.y, (int)cw.z, (int)cw.w, 0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, sa[i], 0, sw[j]);
  }
  const float ga = p.a_global ? *p.a_global : 1.0f;
  const float gw = p.w_global ? *p.w_global : 1.0f;
  const float gg = ga * gw;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int64_t row = m0 + 32 * i + (r / 4) * 8 + kh * 4 + (r % 4);
        int64_t col = n0 + 32 * j + r32;
        store_c(p, row, col, gg * acc[i][j][r]);
      }
}

template <int FA>
hipError_t launch_nv_a(int fw, const GemmParams& p, dim3 grid, hipStream_t s) {
  switch (fw) {
    case RAZER_A: hipLaunchKernelGGL((gemm_nv_kernel<FA, RAZER_A>), grid, dim3(kThreads), 0, s, p); break;
    case RAZER_W: hipLaunchKernelGGL((gemm_nv_kernel<FA, RAZER_W>), grid, dim3(kThreads), 0, s, p); break;
    default: hipLaunchKernelGGL((gemm_nv_kernel<FA, NVFP4>), grid, dim3(kThreads), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int fa, int fw, const GemmParams& p, hipStream_t s) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  dim3 grid((unsigned)((p.N + kTile - 1) / kTile), (unsigned)((p.M + kTile - 1) / kTile));
  if (fa == MXFP4) {
    hipLaunchKernelGGL(gemm_mx_kernel, grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
  }
  if (fa == RAZER_A) return launch_nv_a<RAZER_A>(fw, p, grid, s);
  return launch_nv_a<NVFP4>(fw, p, grid, s);
}

}  // namespace fp4q
