// Internal declarations of libfp4q: launch parameters and launchers shared by
// the C ABI (abi.cpp) and the kernels (quantize.hip, gemm.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fp4q {

enum Fmt : int { NVFP4 = 0, MXFP4 = 1, RAZER_A = 2, RAZER_W = 3 };
enum Rule : int { ABSMAX = 0, FOUR6 = 1, BRUTE = 2 };
enum GMode : int { G_NONE = 0, G_AUTO = 1, G_GIVEN = 2 };

struct QuantParams {
  const void* x;          // rows x cols, pitch ld (elements)
  int64_t rows, cols, ld;
  int x_bf16;             // 0 fp32, 1 bf16
  uint8_t* codes;         // rows x cols/2
  uint8_t* scales;        // rows x cols/block
  float* global;          // device scalar or nullptr (= 1.0)
  const float* chan_scale;// device, cols, or nullptr
  int hadamard;           // 0 or 32
  int prevent_zero;
  float special[4];       // RAZER_W table
  float fused_denom;      // > 0: one workgroup that first sets *global = amax / fused_denom (automatic g)
};

struct DequantParams {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global;
  int64_t rows, cols, ld_out;
  void* out;
  int out_bf16;
  float special[4];
};

struct GemmParams {
  const uint8_t* a_codes; const uint8_t* a_scales; const float* a_global;
  const uint8_t* w_codes; const uint8_t* w_scales; const float* w_global;
  float w_special[4];
  int64_t M, N, K;
  void* c; int64_t ldc; int c_bf16;
  int splits;  // K-splits per output tile (1, or > 1 with FP32 atomics into a zeroed C)
};

struct ChanScaleParams {
  const void* x; int x_bf16; int64_t rows_x, ldx;
  const void* w; int w_bf16; int64_t rows_w, ldw;
  int64_t cols; double alpha;
  float* t; float* r;
};

// launchers: return hipSuccess or the launch error
hipError_t launch_quantize(int fmt, int block, int rule, int gmode, const QuantParams& p,
                           hipStream_t s);
hipError_t launch_dequantize(int fmt, int block, const DequantParams& p, hipStream_t s);
hipError_t launch_gemm(int fa, int fw, const GemmParams& p, hipStream_t s);
hipError_t launch_channel_scale(const ChanScaleParams& p, hipStream_t s);

// compile-time loop: f(std::integral_constant<int, I>) for I in [B, E); used
// where a builtin needs an immediate operand (the FP4 convert's byte select)
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace fp4q
