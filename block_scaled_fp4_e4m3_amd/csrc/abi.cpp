// extern "C" entry points of libfp4q: argument validation on the host, then
// dispatch to the HIP launchers.  Validation touches no HIP API, so every
// argument error is reported before anything is enqueued (and on machines
// without a GPU).
#include "../../include/fp4q.h"

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "fp4q_internal.hpp"

namespace {

using namespace fp4q;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_format(int f) { return f >= FP4Q_NVFP4 && f <= FP4Q_UE5M3; }
// formats the matmul consumes (UE5M3 is quantize/dequantize only)
bool gemm_format(int f) { return f >= FP4Q_NVFP4 && f <= FP4Q_NVFP4_RAZER_W; }

// RaZeR special value: multiple of 0.5 (RaZeR summary 2.2), 0 < |v| <= 7.5 so
// that value * scale stays exact in the matmul's f16 decode, and not one of
// the standard E2M1 magnitudes
bool valid_special(float v) {
  if (!std::isfinite(v)) return false;
  float a = std::fabs(v);
  if (!(a > 0.0f && a <= 7.5f)) return false;
  float twice = a * 2.0f;
  if (twice != std::floor(twice)) return false;
  static const float kStd[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  for (float s : kStd)
    if (a == s) return false;
  return true;
}

fp4q_status check_desc(const fp4q_quant_desc* d, bool quantizing) {
  if (!d) return FP4Q_ERR_NULL;
  if (d->struct_size != sizeof(fp4q_quant_desc)) return FP4Q_ERR_ARG;
  if (!valid_format(d->format)) return FP4Q_ERR_FORMAT;
  if (d->format == FP4Q_MXFP4) {
    if (d->block != 32) return FP4Q_ERR_ARG;
  } else if (d->block != 4 && d->block != 8 && d->block != 16 && d->block != 32) {
    return FP4Q_ERR_ARG;
  }
  if (d->format == FP4Q_NVFP4_RAZER_W)
    for (int i = 0; i < 4; ++i)
      if (!valid_special(d->special[i])) return FP4Q_ERR_ARG;
  if (!quantizing) return FP4Q_OK;
  const uint32_t rule = d->rule & 0xFFu, flags = d->rule & ~0xFFu;
  if (flags & ~(uint32_t)FP4Q_FLAG_PREVENT_ZERO) return FP4Q_ERR_ARG;
  if (rule > FP4Q_RULE_EXPSEARCH) return FP4Q_ERR_ARG;
  switch (d->format) {
    case FP4Q_NVFP4:
    case FP4Q_UE5M3:
      if (rule > FP4Q_RULE_BRUTE) return FP4Q_ERR_ARG;
      break;
    case FP4Q_MXFP4:
      if (rule != FP4Q_RULE_ABSMAX && rule != FP4Q_RULE_EXPSEARCH) return FP4Q_ERR_ARG;
      break;
    default:  // RaZeR: abs-max scale, the special value by block error
      if (rule != FP4Q_RULE_ABSMAX) return FP4Q_ERR_ARG;
  }
  if (d->format == FP4Q_MXFP4 && flags) return FP4Q_ERR_ARG;
  if (d->global_mode < FP4Q_GLOBAL_NONE || d->global_mode > FP4Q_GLOBAL_GIVEN) return FP4Q_ERR_ARG;
  if (d->format == FP4Q_MXFP4 && d->global_mode != FP4Q_GLOBAL_NONE) return FP4Q_ERR_ARG;
  if (d->format == FP4Q_UE5M3 && d->global_mode == FP4Q_GLOBAL_AUTO) return FP4Q_ERR_ARG;
  if (d->hadamard != 0 && d->hadamard != 16 && d->hadamard != 32) return FP4Q_ERR_ARG;
  return FP4Q_OK;
}

fp4q_status device_status(hipError_t e) { return e == hipSuccess ? FP4Q_OK : FP4Q_ERR_DEVICE; }

size_t elem_size(fp4q_dtype t) { return t == FP4Q_BF16 ? 2 : 4; }

// A rows x pitch matrix the kernels can address: each extent at most 2^40
// and the element count at most 2^46 (far above one GPU's memory), so that
// no byte offset or size formed from them overflows 64 bits.  Checked
// before any product of the two is formed.
bool dims_ok(int64_t rows, int64_t pitch) {
  constexpr int64_t kMaxExtent = int64_t(1) << 40, kMaxElems = int64_t(1) << 46;
  if (rows < 0 || pitch < 0 || rows > kMaxExtent || pitch > kMaxExtent) return false;
  return rows == 0 || pitch <= kMaxElems / rows;
}

// Validation shared by the two matmul entry points, then the launch
// parameters.  Touches no HIP API.
fp4q_status gemm_params(fp4q_format fa, const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                        fp4q_format fw, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                        const float* w_special, int64_t M, int64_t N, int64_t K, void* c, fp4q_dtype c_dtype,
                        int64_t ldc, GemmParams& p) {
  if (!gemm_format(fa) || !gemm_format(fw)) return FP4Q_ERR_FORMAT;
  if ((fa == FP4Q_MXFP4) != (fw == FP4Q_MXFP4) || fa == FP4Q_NVFP4_RAZER_W) return FP4Q_ERR_FORMAT;
  if (c_dtype != FP4Q_F32 && c_dtype != FP4Q_BF16) return FP4Q_ERR_ARG;
  if (!a_codes || !a_scales || !w_codes || !w_scales || !c) return FP4Q_ERR_NULL;
  if (fw == FP4Q_NVFP4_RAZER_W && !w_special) return FP4Q_ERR_NULL;
  const int64_t block = fa == FP4Q_MXFP4 ? 32 : 16;
  if (M < 0 || N < 0 || K <= 0 || K % block != 0 || K > (int64_t(1) << 24) || ldc < N) return FP4Q_ERR_SHAPE;
  if (!dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, ldc)) return FP4Q_ERR_SHAPE;
  const int64_t tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
  if (tiles_n > 0 && tiles_m > INT32_MAX / tiles_n) return FP4Q_ERR_SHAPE;
  if (fw == FP4Q_NVFP4_RAZER_W)
    for (int i = 0; i < 4; ++i)
      if (!valid_special(w_special[i])) return FP4Q_ERR_ARG;
  if (!aligned16(a_codes) || !aligned16(w_codes) || !aligned16(c) ||
      (ldc * (int64_t)elem_size(c_dtype)) % 16 != 0)
    return FP4Q_ERR_ALIGN;
  if ((a_global && ((uintptr_t)a_global & 3u)) || (w_global && ((uintptr_t)w_global & 3u)))
    return FP4Q_ERR_ALIGN;
  p.a_codes = a_codes;
  p.a_scales = a_scales;
  p.a_global = a_global;
  p.w_codes = w_codes;
  p.w_scales = w_scales;
  p.w_global = w_global;
  for (int i = 0; i < 4; ++i) p.w_special[i] = (fw == FP4Q_NVFP4_RAZER_W) ? w_special[i] : 0.0f;
  p.M = M;
  p.N = N;
  p.K = K;
  p.c = c;
  p.ldc = ldc;
  p.c_bf16 = c_dtype == FP4Q_BF16;
  return FP4Q_OK;
}

// W row segments: nseg == 0 keeps the single w_global; 1..8 segments of
// seg_rows[i] >= 0 rows summing to N take w_global[i] each
fp4q_status segment_params(const float* w_global, const int64_t* seg_rows, int nseg, int64_t N, GemmParams& p) {
  p.nseg = 0;
  p.seg_global = nullptr;
  if (nseg == 0) return FP4Q_OK;
  if (nseg < 0 || nseg > kMaxSegments) return FP4Q_ERR_ARG;
  if (!seg_rows || !w_global) return FP4Q_ERR_NULL;
  int64_t end = 0;
  for (int i = 0; i < nseg; ++i) {
    if (seg_rows[i] < 0 || seg_rows[i] > N - end) return FP4Q_ERR_SHAPE;
    end += seg_rows[i];
    p.seg_end[i] = end;
  }
  if (end != N) return FP4Q_ERR_SHAPE;
  for (int i = nseg; i < kMaxSegments; ++i) p.seg_end[i] = N;
  p.nseg = nseg;
  p.seg_global = w_global;
  return FP4Q_OK;
}

}  // namespace

extern "C" {

fp4q_status fp4q_quantize(const fp4q_quant_desc* desc, const void* x, fp4q_dtype x_dtype,
                          int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                          uint8_t* scales, float* global, void* stream) {
  fp4q_status st = check_desc(desc, true);
  if (st != FP4Q_OK) return st;
  if (x_dtype != FP4Q_F32 && x_dtype != FP4Q_BF16) return FP4Q_ERR_ARG;
  if (!x || !codes || !scales) return FP4Q_ERR_NULL;
  if (desc->global_mode != FP4Q_GLOBAL_NONE && !global) return FP4Q_ERR_NULL;
  if (rows < 0 || cols <= 0 || ld_x < cols || cols % desc->block != 0) return FP4Q_ERR_SHAPE;
  if (!dims_ok(rows, ld_x)) return FP4Q_ERR_SHAPE;
  if (desc->hadamard != 0 && cols % desc->hadamard != 0) return FP4Q_ERR_SHAPE;
  if (!aligned16(x) || (ld_x * (int64_t)elem_size(x_dtype)) % 16 != 0 || !aligned16(codes))
    return FP4Q_ERR_ALIGN;
  if (desc->chan_scale && !aligned16(desc->chan_scale)) return FP4Q_ERR_ALIGN;
  if (global && ((uintptr_t)global & 3u)) return FP4Q_ERR_ALIGN;

  QuantParams p{};
  p.x = x;
  p.rows = rows;
  p.cols = cols;
  p.ld = ld_x;
  p.x_bf16 = x_dtype == FP4Q_BF16;
  p.codes = codes;
  p.scales = scales;
  p.global = desc->global_mode == FP4Q_GLOBAL_NONE ? nullptr : global;
  p.chan_scale = desc->chan_scale;
  p.hadamard = desc->hadamard;
  p.prevent_zero = (desc->rule & FP4Q_FLAG_PREVENT_ZERO) != 0;
  for (int i = 0; i < 4; ++i) p.special[i] = desc->special[i];
  return device_status(launch_quantize(desc->format, desc->block, (int)(desc->rule & 0xFFu),
                                       desc->global_mode, p, (hipStream_t)stream));
}

fp4q_status fp4q_dequantize(const fp4q_quant_desc* desc, const uint8_t* codes,
                            const uint8_t* scales, const float* global, int64_t rows,
                            int64_t cols, void* out, fp4q_dtype out_dtype, int64_t ld_out,
                            void* stream) {
  fp4q_status st = check_desc(desc, false);
  if (st != FP4Q_OK) return st;
  if (out_dtype != FP4Q_F32 && out_dtype != FP4Q_BF16) return FP4Q_ERR_ARG;
  if (!codes || !scales || !out) return FP4Q_ERR_NULL;
  if (rows < 0 || cols <= 0 || ld_out < cols || cols % desc->block != 0) return FP4Q_ERR_SHAPE;
  if (!dims_ok(rows, ld_out)) return FP4Q_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(out) || (ld_out * (int64_t)elem_size(out_dtype)) % 16 != 0)
    return FP4Q_ERR_ALIGN;
  if (global && ((uintptr_t)global & 3u)) return FP4Q_ERR_ALIGN;
  DequantParams p{};
  p.codes = codes;
  p.scales = scales;
  p.global = global;
  p.rows = rows;
  p.cols = cols;
  p.ld_out = ld_out;
  p.out = out;
  p.out_bf16 = out_dtype == FP4Q_BF16;
  for (int i = 0; i < 4; ++i) p.special[i] = desc->special[i];
  return device_status(launch_dequantize(desc->format, desc->block, p, (hipStream_t)stream));
}

fp4q_status fp4q_gemm_w4a4(fp4q_format fa, const uint8_t* a_codes, const uint8_t* a_scales,
                           const float* a_global, fp4q_format fw, const uint8_t* w_codes,
                           const uint8_t* w_scales, const float* w_global,
                           const float* w_special, int64_t M, int64_t N, int64_t K, void* c,
                           fp4q_dtype c_dtype, int64_t ldc, void* stream) {
  GemmParams p{};
  fp4q_status st = gemm_params(fa, a_codes, a_scales, a_global, fw, w_codes, w_scales, w_global, w_special, M, N,
                               K, c, c_dtype, ldc, p);
  if (st != FP4Q_OK || M == 0 || N == 0) return st;
  return device_status(launch_gemm(fa, fw, p, (hipStream_t)stream, Workspace{nullptr, kSplitWorkspaceBytes}));
}

fp4q_status fp4q_gemm_w4a4_noalloc(fp4q_format fa, const uint8_t* a_codes, const uint8_t* a_scales,
                                   const float* a_global, fp4q_format fw, const uint8_t* w_codes,
                                   const uint8_t* w_scales, const float* w_global,
                                   const float* w_special, int64_t M, int64_t N, int64_t K, void* c,
                                   fp4q_dtype c_dtype, int64_t ldc, void* stream) {
  GemmParams p{};
  fp4q_status st = gemm_params(fa, a_codes, a_scales, a_global, fw, w_codes, w_scales, w_global, w_special, M, N,
                               K, c, c_dtype, ldc, p);
  if (st != FP4Q_OK || M == 0 || N == 0) return st;
  float* scratch = noalloc_scratch();
  if (!scratch) return FP4Q_ERR_DEVICE;
  return device_status(launch_gemm(fa, fw, p, (hipStream_t)stream, Workspace{scratch, kSplitWorkspaceBytes}));
}

fp4q_status fp4q_gemm_w4a4_segmented(fp4q_format fa, const uint8_t* a_codes, const uint8_t* a_scales,
                                     const float* a_global, fp4q_format fw, const uint8_t* w_codes,
                                     const uint8_t* w_scales, const float* w_global, const int64_t* seg_rows,
                                     int nseg, const float* w_special, int64_t M, int64_t N, int64_t K, void* c,
                                     fp4q_dtype c_dtype, int64_t ldc, void* stream) {
  GemmParams p{};
  fp4q_status st = gemm_params(fa, a_codes, a_scales, a_global, fw, w_codes, w_scales, nullptr, w_special, M, N,
                               K, c, c_dtype, ldc, p);
  if (st != FP4Q_OK) return st;
  if (nseg == 0) p.w_global = w_global;
  if ((st = segment_params(w_global, seg_rows, nseg, N, p)) != FP4Q_OK) return st;
  if (w_global && ((uintptr_t)w_global & 3u)) return FP4Q_ERR_ALIGN;
  if (M == 0 || N == 0) return FP4Q_OK;
  return device_status(launch_gemm(fa, fw, p, (hipStream_t)stream, Workspace{nullptr, kSplitWorkspaceBytes}));
}

fp4q_status fp4q_gemm_w4a4_act_bf16(const uint16_t* a, int64_t lda, uint32_t a_rule, const float* a_global,
                                    uint8_t* a_codes_out, uint8_t* a_scales_out, fp4q_format fw,
                                    const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                                    const int64_t* seg_rows, int nseg, const float* w_special, int64_t M,
                                    int64_t N, int64_t K, void* c, fp4q_dtype c_dtype, int64_t ldc, void* stream) {
  if (fw != FP4Q_NVFP4 && fw != FP4Q_NVFP4_RAZER_A && fw != FP4Q_NVFP4_RAZER_W) return FP4Q_ERR_FORMAT;
  if (a_rule != FP4Q_RULE_ABSMAX && a_rule != FP4Q_RULE_4OVER6) return FP4Q_ERR_ARG;
  if (c_dtype != FP4Q_F32 && c_dtype != FP4Q_BF16) return FP4Q_ERR_ARG;
  if (!a || !w_codes || !w_scales || !c) return FP4Q_ERR_NULL;
  if ((a_codes_out == nullptr) != (a_scales_out == nullptr)) return FP4Q_ERR_NULL;
  if (fw == FP4Q_NVFP4_RAZER_W && !w_special) return FP4Q_ERR_NULL;
  if (M < 0 || N < 0 || K <= 0 || K % 512 != 0 || K > (int64_t(1) << 24) || lda < K || lda > (int64_t(1) << 24) ||
      ldc < N)
    return FP4Q_ERR_SHAPE;
  if (!dims_ok(M, lda) || !dims_ok(N, K) || !dims_ok(M, ldc)) return FP4Q_ERR_SHAPE;
  if (fw == FP4Q_NVFP4_RAZER_W)
    for (int i = 0; i < 4; ++i)
      if (!valid_special(w_special[i])) return FP4Q_ERR_ARG;
  GemmParams p{};
  fp4q_status st = segment_params(w_global, seg_rows, nseg, N, p);
  if (st != FP4Q_OK) return st;
  if (!aligned16(a) || lda % 8 != 0 || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(c) ||
      !aligned16(a_codes_out) || !aligned16(a_scales_out) || (ldc * (int64_t)elem_size(c_dtype)) % 16 != 0)
    return FP4Q_ERR_ALIGN;
  if ((a_global && ((uintptr_t)a_global & 3u)) || (w_global && ((uintptr_t)w_global & 3u))) return FP4Q_ERR_ALIGN;
  if (M == 0 || N == 0) return FP4Q_OK;
  p.a_bf16 = a;
  p.lda = lda;
  p.a_global = a_global;
  p.aq_codes = a_codes_out;
  p.aq_scales = a_scales_out;
  p.w_codes = w_codes;
  p.w_scales = w_scales;
  p.w_global = nseg == 0 ? w_global : nullptr;
  for (int i = 0; i < 4; ++i) p.w_special[i] = (fw == FP4Q_NVFP4_RAZER_W) ? w_special[i] : 0.0f;
  p.M = M;
  p.N = N;
  p.K = K;
  p.c = c;
  p.ldc = ldc;
  p.c_bf16 = c_dtype == FP4Q_BF16;
  return device_status(launch_gemm_act_bf16(a_rule == FP4Q_RULE_4OVER6 ? FOUR6 : ABSMAX, fw, p, (hipStream_t)stream,
                                            Workspace{nullptr, kSplitWorkspaceBytes}));
}

fp4q_status fp4q_gemm_w4a16(const uint16_t* a, int64_t lda, fp4q_format fw, const uint8_t* w_codes,
                            const uint8_t* w_scales, const float* w_global, const float* w_special, int64_t M,
                            int64_t N, int64_t K, void* c, fp4q_dtype c_dtype, int64_t ldc, void* stream) {
  if (fw != FP4Q_NVFP4 && fw != FP4Q_NVFP4_RAZER_W) return FP4Q_ERR_FORMAT;
  if (c_dtype != FP4Q_F32 && c_dtype != FP4Q_BF16) return FP4Q_ERR_ARG;
  if (!a || !w_codes || !w_scales || !c) return FP4Q_ERR_NULL;
  if (fw == FP4Q_NVFP4_RAZER_W && !w_special) return FP4Q_ERR_NULL;
  if (M < 0 || N < 0 || K <= 0 || K % 512 != 0 || K > (int64_t(1) << 24) || lda < K || lda > (int64_t(1) << 24) ||
      ldc < N)
    return FP4Q_ERR_SHAPE;
  if (!dims_ok(M, lda) || !dims_ok(N, K) || !dims_ok(M, ldc)) return FP4Q_ERR_SHAPE;
  if (fw == FP4Q_NVFP4_RAZER_W)
    for (int i = 0; i < 4; ++i)
      if (!valid_special(w_special[i])) return FP4Q_ERR_ARG;
  if (!aligned16(a) || lda % 8 != 0 || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(c) ||
      (ldc * (int64_t)elem_size(c_dtype)) % 16 != 0)
    return FP4Q_ERR_ALIGN;
  if (w_global && ((uintptr_t)w_global & 3u)) return FP4Q_ERR_ALIGN;
  if (M == 0 || N == 0) return FP4Q_OK;
  GemmParams p{};
  p.a_bf16 = a;
  p.lda = lda;
  p.w_codes = w_codes;
  p.w_scales = w_scales;
  p.w_global = w_global;
  for (int i = 0; i < 4; ++i) p.w_special[i] = (fw == FP4Q_NVFP4_RAZER_W) ? w_special[i] : 0.0f;
  p.M = M;
  p.N = N;
  p.K = K;
  p.c = c;
  p.ldc = ldc;
  p.c_bf16 = c_dtype == FP4Q_BF16;
  return device_status(launch_gemm_w4a16(fw, p, (hipStream_t)stream, Workspace{nullptr, kSplitWorkspaceBytes}));
}

fp4q_status fp4q_razer_table_search(const void* w, fp4q_dtype w_dtype, int64_t rows, int64_t cols, int64_t ld_w,
                                    fp4q_global_mode global_mode, float* global, double* pair_sse, float* table,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (w_dtype != FP4Q_F32 && w_dtype != FP4Q_BF16) return FP4Q_ERR_ARG;
  if (global_mode < FP4Q_GLOBAL_NONE || global_mode > FP4Q_GLOBAL_GIVEN) return FP4Q_ERR_ARG;
  if (!pair_sse || !table) return FP4Q_ERR_NULL;
  if (global_mode != FP4Q_GLOBAL_NONE && !global) return FP4Q_ERR_NULL;
  if (rows < 0 || cols <= 0 || cols % 16 != 0 || ld_w < cols || !dims_ok(rows, ld_w)) return FP4Q_ERR_SHAPE;
  if (rows > 0 && (!w || !workspace)) return FP4Q_ERR_NULL;
  if ((uint64_t)rows > (uint64_t)(SIZE_MAX / (kRazerPairs * sizeof(double))) ||
      workspace_bytes < (size_t)rows * kRazerPairs * sizeof(double))
    return FP4Q_ERR_ARG;
  if (!aligned16(w) || (ld_w * (int64_t)elem_size(w_dtype)) % 16 != 0) return FP4Q_ERR_ALIGN;
  if (((uintptr_t)pair_sse & 7u) || ((uintptr_t)table & 3u) || ((uintptr_t)workspace & 7u) ||
      (global && ((uintptr_t)global & 3u)))
    return FP4Q_ERR_ALIGN;
  QuantParams p{};
  p.x = w;
  p.rows = rows;
  p.cols = cols;
  p.ld = ld_w;
  p.x_bf16 = w_dtype == FP4Q_BF16;
  p.global = global_mode == FP4Q_GLOBAL_NONE ? nullptr : global;
  return device_status(launch_razer_search(p, global_mode, (double*)workspace, pair_sse, table, (hipStream_t)stream));
}

fp4q_status fp4q_macaq_quantize(const float* w, int64_t N, int64_t K, int64_t ldw, const double* h,
                                int64_t ldh, int64_t max_moves, uint8_t* codes, uint8_t* scales,
                                int32_t* moves, void* workspace, size_t workspace_bytes, void* stream) {
  if (!w || !h || !codes || !scales || !workspace) return FP4Q_ERR_NULL;
  if (N < 0 || K <= 0 || K % 32 != 0 || K > macaq_max_k() || ldw < K || ldh < K) return FP4Q_ERR_SHAPE;
  if (!dims_ok(N, ldw) || !dims_ok(K, ldh)) return FP4Q_ERR_SHAPE;
  if (max_moves < 0 || workspace_bytes < (size_t)K * sizeof(double)) return FP4Q_ERR_ARG;
  if (((uintptr_t)w & 3u) || ((uintptr_t)h & 7u) || ((uintptr_t)workspace & 7u) || ((uintptr_t)moves & 3u))
    return FP4Q_ERR_ALIGN;
  if (N == 0) return FP4Q_OK;
  MacaqParams p{};
  p.w = w;
  p.N = N;
  p.K = K;
  p.ldw = ldw;
  p.h = h;
  p.ldh = ldh;
  p.max_moves = max_moves;
  p.codes = codes;
  p.scales = scales;
  p.moves = moves;
  return device_status(launch_macaq(p, workspace, workspace_bytes, (hipStream_t)stream));
}

fp4q_status fp4q_channel_scale(const void* x, fp4q_dtype x_dtype, int64_t rows_x, int64_t ldx,
                               const void* w, fp4q_dtype w_dtype, int64_t rows_w, int64_t ldw,
                               int64_t cols, double alpha, float* t, float* r, void* stream) {
  if ((x_dtype != FP4Q_F32 && x_dtype != FP4Q_BF16) || (w_dtype != FP4Q_F32 && w_dtype != FP4Q_BF16))
    return FP4Q_ERR_ARG;
  if (!x || !w || !t || !r) return FP4Q_ERR_NULL;
  if (rows_x <= 0 || rows_w <= 0 || cols <= 0 || ldx < cols || ldw < cols) return FP4Q_ERR_SHAPE;
  if (!dims_ok(rows_x, ldx) || !dims_ok(rows_w, ldw)) return FP4Q_ERR_SHAPE;
  if (!std::isfinite(alpha)) return FP4Q_ERR_ARG;
  if (((uintptr_t)x % elem_size(x_dtype)) || ((uintptr_t)w % elem_size(w_dtype)) ||
      ((uintptr_t)t & 3u) || ((uintptr_t)r & 3u))
    return FP4Q_ERR_ALIGN;
  ChanScaleParams p{};
  p.x = x;
  p.x_bf16 = x_dtype == FP4Q_BF16;
  p.rows_x = rows_x;
  p.ldx = ldx;
  p.w = w;
  p.w_bf16 = w_dtype == FP4Q_BF16;
  p.rows_w = rows_w;
  p.ldw = ldw;
  p.cols = cols;
  p.alpha = alpha;
  p.t = t;
  p.r = r;
  return device_status(launch_channel_scale(p, (hipStream_t)stream));
}

const char* fp4q_status_string(fp4q_status s) {
  switch (s) {
    case FP4Q_OK: return "ok";
    case FP4Q_ERR_NULL: return "a required pointer is NULL";
    case FP4Q_ERR_SHAPE: return "sizes are negative or not divisible as required";
    case FP4Q_ERR_ALIGN: return "a pointer or row pitch is not 16-byte aligned";
    case FP4Q_ERR_FORMAT: return "unknown format or unsupported format pair";
    case FP4Q_ERR_ARG: return "bad rule, mode, block, transform or special value";
    case FP4Q_ERR_UNSUPPORTED: return "combination not implemented";
    case FP4Q_ERR_DEVICE: return "the HIP runtime reported an error";
  }
  return "unknown status";
}

uint32_t fp4q_abi_version(void) { return FP4Q_ABI_VERSION; }

}  // extern "C"
