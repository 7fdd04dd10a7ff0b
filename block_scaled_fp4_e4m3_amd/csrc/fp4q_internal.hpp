// Internal declarations of libfp4q: launch parameters and launchers shared by
// the C ABI (abi.cpp) and the kernels (quantize.hip, gemm.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fp4q {

enum Fmt : int { NVFP4 = 0, MXFP4 = 1, RAZER_A = 2, RAZER_W = 3, UE5M3 = 4 };
enum Rule : int { ABSMAX = 0, FOUR6 = 1, BRUTE = 2, EXPSEARCH = 3 };
enum GMode : int { G_NONE = 0, G_AUTO = 1, G_GIVEN = 2 };

struct QuantParams {
  const void* x;          // rows x cols, pitch ld (elements)
  int64_t rows, cols, ld;
  int x_bf16;             // 0 fp32, 1 bf16
  uint8_t* codes;         // rows x cols/2
  uint8_t* scales;        // rows x cols/block
  float* global;          // device scalar or nullptr (= 1.0)
  const float* chan_scale;// device, cols, or nullptr
  int hadamard;           // 0, 16 or 32
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
  const uint16_t* a_bf16; int64_t lda;  // bf16 activations (M x K, pitch lda): weight-only, or quantized on load
  uint8_t* aq_codes; uint8_t* aq_scales;  // quantized on load: the activations' codes and scales, or nullptr
  // W row segments with their own global scales: segment i covers the
  // output columns [seg_end[i-1], seg_end[i]) (seg_end[-1] = 0) and takes
  // seg_global[i] in place of w_global; nseg = 0: w_global everywhere
  int nseg;
  const float* seg_global;
  int64_t seg_end[8];
  int splits;       // K-splits per output tile (set by the launcher)
  float* partials;  // splits > 1: the splits' RN32(g * acc_s), dense M x N slices, added in split order
};
constexpr int kMaxSegments = 8;

// bytes of the split-K workspace a matmul may use (per stream, or the
// library's own array for the non-allocating entry point)
constexpr size_t kSplitWorkspaceBytes = size_t(32) << 20;

struct MacaqParams {
  const float* w; int64_t N, K, ldw;      // weight, row n = output channel
  const double* h; int64_t ldh;           // Hessian X^T X, K x K
  int64_t max_moves;                      // per row
  uint8_t* codes; uint8_t* scales;        // N x K/2, N x K/32
  int32_t* moves;                         // N, or nullptr
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
// Device memory for the partial results of K splits: `fixed` if set, else
// the stream's own workspace, allocated when a launch first splits K (see
// split_workspace); bytes = 0: no splits.
struct Workspace {
  float* fixed;
  size_t bytes;
};
hipError_t launch_gemm(int fa, int fw, const GemmParams& p, hipStream_t s, const Workspace& ws);
// weight-only matmul (bf16 activations in p.a_bf16), fw NVFP4 or RAZER_W;
// needs K % 512 == 0 and 16-byte aligned rows
hipError_t launch_gemm_w4a16(int fw, const GemmParams& p, hipStream_t s, const Workspace& ws);
// W4A4 matmul whose NVFP4 activations are quantized from bf16 (p.a_bf16) as
// they are loaded, rule ABSMAX or FOUR6 under *p.a_global (or 1); fw of the
// NVFP4 family; needs K % 512 == 0 and 16-byte aligned rows
hipError_t launch_gemm_act_bf16(int rule, int fw, const GemmParams& p, hipStream_t s, const Workspace& ws);
// the split-K workspace of stream s on the current device (allocated on first
// use, kept until the process ends), or nullptr
float* split_workspace(hipStream_t s);
// the device address of the library's own split-K array on the current
// device (looked up once per device), or nullptr if the lookup failed
float* noalloc_scratch();
hipError_t launch_channel_scale(const ChanScaleParams& p, hipStream_t s);
constexpr int kRazerPairs = 28;  // special-value pairs the search compares
// RaZeR special-value search over p.x (rows x cols, block 16) under *p.global
// (AUTO: computed first); row_sums: rows x 28 doubles of workspace
hipError_t launch_razer_search(const QuantParams& p, int gmode, double* row_sums, double* pair_sse, float* table,
                               hipStream_t s);
// MACaQ calibration; workspace holds the r rows of one pass (K doubles per row)
hipError_t launch_macaq(const MacaqParams& p, void* workspace, size_t ws_bytes, hipStream_t s);
int64_t macaq_max_k();

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
