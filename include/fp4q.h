/*
 * fp4q.h -- C ABI of libfp4q: block-scaled FP4 quantization and the W4A4
 * matmul on AMD Instinct MI355X (gfx950).
 *
 * Formats, byte for byte, as the pages define them:
 *   NVFP4    E2M1 elements, one E4M3 scale per block of 16 (4, 8 and 32 are
 *            accepted by quantize/dequantize), optional FP32 per-tensor global
 *            scale.  "Why Gated DeltaNet Survives 4-Bit Quantization" review,
 *            section 1; "Finer is Better (with the Right Scaling)", Method 2.
 *   MXFP4    E2M1 elements, one E8M0 exponent per block of 32.  MACaQ review,
 *            section 1.
 *   RAZER_A  NVFP4 whose E4M3 sign bit picks the block's special value from
 *            {+5, -5}; code 0x8 (the redundant -0) decodes to it.  RaZeR
 *            summary, sections 2.1-2.2.
 *   RAZER_W  E2M1 elements with a 6-bit E3M3 scale; the top two bits of the
 *            scale byte pick one of four special values; code 0x8 decodes to
 *            it.  RaZeR summary, sections 2.1-2.2.
 *   UE5M3    E2M1 elements with an unsigned 8-bit UE5M3 scale per block of 4,
 *            8, 16 or 32 (5 exponent bits, bias 15, 3 mantissa bits,
 *            subnormals, no special codes: 0 .. 122880); the wide-exponent
 *            scale "Finer is Better" compares with E4M3 + 4-over-6 +
 *            hierarchical scaling (findings, claims).  Global mode NONE or
 *            GIVEN; quantize and dequantize only.
 *
 * Layout (every buffer row-major, blocks run along the last, contiguous
 * dimension):
 *   codes   rows x cols/2 bytes; byte j/2 of a row holds element j, the even
 *           element in the low nibble.  E2M1 code = sign<<3 | magnitude, with
 *           magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; a zero is always 0x0.
 *   scales  rows x cols/block bytes:
 *             NVFP4    E4M3 code (bit 7 = 0)
 *             MXFP4    E8M0 code (2^(code-127))
 *             RAZER_A  bit 7 = pick (0: +5, 1: -5), bits 6:0 = E4M3 code
 *             RAZER_W  bits 7:6 = index into special[4], bits 5:0 = E3M3 code
 *             UE5M3    UE5M3 code
 *   global  one FP32 on the device; an element decodes to value * scale * g.
 *
 * Ownership: the caller allocates and owns every buffer it passes.  The only
 * device memory libfp4q allocates itself is a split-K workspace of 32 MiB per
 * (device, stream), taken with hipMalloc when fp4q_gemm_w4a4 or fp4q_gemm_w4a16
 * first splits K on that stream and kept until the process ends.  Calls are
 * thread-safe.
 *
 * Asynchrony: every call validates its arguments on the host, enqueues its
 * kernels on `stream` (a hipStream_t passed as void*, NULL = default stream)
 * and returns without synchronising.  An argument error returns its status
 * and enqueues nothing; a failed launch returns FP4Q_ERR_DEVICE.
 *
 * Sizes: every row count, column count and pitch is at most 2^40 and every
 * matrix holds at most 2^46 elements (rows x pitch), else FP4Q_ERR_SHAPE, so
 * that no offset formed from them overflows.
 *
 * Non-finite inputs, and a GIVEN global scale that is not a positive finite
 * number, are outside the contract: the outputs are then unspecified.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4Q_ABI_VERSION 1u

typedef enum {
  FP4Q_OK = 0,
  FP4Q_ERR_NULL = 1,        /* a required pointer is NULL                       */
  FP4Q_ERR_SHAPE = 2,       /* sizes negative, or not divisible as required     */
  FP4Q_ERR_ALIGN = 3,       /* pointer or row pitch not 16-byte aligned         */
  FP4Q_ERR_FORMAT = 4,      /* unknown format, or a format pair not supported   */
  FP4Q_ERR_ARG = 5,         /* bad rule, mode, block, transform or special value */
  FP4Q_ERR_UNSUPPORTED = 6, /* valid combination not implemented by libfp4q   */
  FP4Q_ERR_DEVICE = 7       /* the HIP runtime reported an error                */
} fp4q_status;

typedef enum {
  FP4Q_NVFP4 = 0,
  FP4Q_MXFP4 = 1,
  FP4Q_NVFP4_RAZER_A = 2,
  FP4Q_NVFP4_RAZER_W = 3,
  FP4Q_UE5M3 = 4          /* quantize / dequantize only                        */
} fp4q_format;

typedef enum { FP4Q_F32 = 0, FP4Q_BF16 = 1 } fp4q_dtype;

/* scale rules (low byte of fp4q_quant_desc.rule) and OR-able flags, from
 * "Finer is Better (with the Right Scaling)", Method 2 */
enum {
  FP4Q_RULE_ABSMAX = 0,        /* block max maps to 6, nearest E4M3 scale          */
  FP4Q_RULE_4OVER6 = 1,        /* max maps to 4 or 6, lower block error kept       */
  FP4Q_RULE_BRUTE = 2,         /* every positive scale, lowest error kept         */
  FP4Q_RULE_EXPSEARCH = 3,     /* MXFP4: shared exponent E, E+1 or E-1, lowest
                                  block error kept (ties: that order)             */
  FP4Q_FLAG_PREVENT_ZERO = 0x100 /* a zero scale is raised to the smallest positive */
};

typedef enum {
  FP4Q_GLOBAL_NONE = 0,  /* g = 1; `global` may be NULL                          */
  FP4Q_GLOBAL_AUTO = 1,  /* g = amax/(6*448) (E3M3: amax/(6*30)) of the transformed
                            tensor, written to *global on the device             */
  FP4Q_GLOBAL_GIVEN = 2  /* g read from *global on the device                    */
} fp4q_global_mode;

/* Description of one quantization.  Set struct_size = sizeof(fp4q_quant_desc). */
typedef struct {
  uint32_t struct_size;
  fp4q_format format;
  int32_t block;               /* NVFP4 family: 4, 8, 16 or 32; MXFP4: 32        */
  uint32_t rule;               /* rule | flags.  NVFP4, UE5M3: ABSMAX, 4OVER6,
                                  BRUTE (+ PREVENT_ZERO); MXFP4: ABSMAX or
                                  EXPSEARCH; RaZeR: ABSMAX (+ PREVENT_ZERO)      */
  fp4q_global_mode global_mode;/* MXFP4: NONE; UE5M3: NONE or GIVEN              */
  const float* chan_scale;     /* device, `cols` floats, or NULL: x_j *= t_j
                                  before quantization (MACaQ online scaling)     */
  int32_t hadamard;            /* 0, 32 or 16: orthonormal block-Hadamard of
                                  that size after the channel scale (MACaQ
                                  micro-rotation; 16 matches the NVFP4 block);
                                  needs cols % hadamard == 0                     */
  float special[4];            /* RAZER_W: the four special values; each a
                                  multiple of 0.5 with 0 < |v| <= 7.5 that is
                                  not an E2M1 magnitude.  Ignored otherwise.     */
} fp4q_quant_desc;

/*
 * Quantize a rows x cols tensor x (fp32 or bf16, row pitch ld_x elements).
 * Steps: widen to fp32; x_j *= chan_scale[j] (if given); block-Hadamard
 * (if hadamard is 16 or 32); global scale per global_mode; per-block
 * scale by the rule; E2M1 encode (RaZeR: with the special value); pack.
 * Pages: scale rules -- "Finer is Better", Method 2; RaZeR picks -- RaZeR
 * summary 2.2; transforms -- MACaQ review, sections 1 and 3; MXFP4 -- MACaQ
 * review, section 1.
 *   x       device, 16-byte aligned, ld_x * sizeof(elem) a multiple of 16
 *   codes   device, rows*(cols/2) bytes, 16-byte aligned, written
 *   scales  device, rows*(cols/block) bytes, written
 *   global  device FP32: read (GIVEN), written (AUTO) or unused (NONE, may be NULL)
 * Errors: NULL desc/x/codes/scales (or global with AUTO/GIVEN) -> ERR_NULL;
 * rows < 0, cols <= 0, cols % block, ld_x < cols, cols % hadamard
 * -> ERR_SHAPE; misalignment -> ERR_ALIGN; bad format -> ERR_FORMAT; bad rule,
 * flag, block, mode, struct_size, hadamard or special value -> ERR_ARG.
 * rows == 0 is valid and enqueues nothing (AUTO then writes nothing).
 */
fp4q_status fp4q_quantize(const fp4q_quant_desc* desc, const void* x, fp4q_dtype x_dtype,
                          int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                          uint8_t* scales, float* global, void* stream);

/*
 * Dequantize codes/scales (layout above) to out = RN32(value * scale * g),
 * stored as fp32, or as bf16 rounded to nearest even from that fp32 value.
 * desc supplies format, block and (RAZER_W) special; its rule and transform
 * fields are ignored.  global: device FP32, NULL means g = 1.
 *   out     device, rows x cols with row pitch ld_out elements, 16-byte aligned
 * Errors as for fp4q_quantize (ld_out < cols -> ERR_SHAPE).
 */
fp4q_status fp4q_dequantize(const fp4q_quant_desc* desc, const uint8_t* codes,
                            const uint8_t* scales, const float* global, int64_t rows,
                            int64_t cols, void* out, fp4q_dtype out_dtype, int64_t ld_out,
                            void* stream);

/*
 * W4A4 block-scaled matmul C = (g_a * g_w) * A^ W^T  with A^ (M x K) and W^
 * (N x K, row n = output channel) given as codes and scales; accumulation in
 * FP32; C = RN32(g * acc) with g = RN32(g_a*g_w), stored fp32 or bf16 (RNE of
 * that FP32 value), row pitch ldc.  On launches with few output tiles the
 * library may split K into S contiguous ranges with accumulators acc_0 ..
 * acc_{S-1}; then C = (...((p_0 + p_1) + p_2) ... + p_{S-1}) with
 * p_s = RN32(g * acc_s), each addition rounded to FP32, in that order, and
 * stored as above.  S depends only on the shape, the formats and the device
 * (S = 1 if the stream's workspace could not be allocated), so every launch of
 * the same arguments gives the same bytes.  The summation order inside each
 * acc_s is the kernel's and is not specified.
 * Pages: NVFP4 W4A4 -- "Why Gated DeltaNet Survives..." review, section 1;
 * RaZeR weight-activation GEMM -- RaZeR summary 2.3; MXFP4 W4A4 -- MACaQ
 * review, section 3.
 *   fa, fw    both MXFP4 (block 32), or both of the NVFP4 family (block 16):
 *             fa in {NVFP4, RAZER_A}, fw in {NVFP4, RAZER_A, RAZER_W}
 *             (RAZER_W needs a special table, which only the W side carries)
 *   a_global, w_global  device FP32 or NULL (= 1.0)
 *   w_special host, 4 floats, required when fw == RAZER_W, else ignored
 *   c         device, M x N (pitch ldc elements), 16-byte aligned
 * Errors: NULL pointer -> ERR_NULL; M, N < 0, K <= 0, K % block, K > 2^24
 * (operand offsets within a 256-row panel are 32-bit), more than 2^31 - 1
 * tiles of 256 x 256, or ldc < N -> ERR_SHAPE; a mixed MXFP4/NVFP4 pair,
 * fa == RAZER_W, or a UE5M3 operand -> ERR_FORMAT;
 * bad special value
 * -> ERR_ARG; misalignment -> ERR_ALIGN.  M == 0 or N == 0 enqueues nothing.
 */
fp4q_status fp4q_gemm_w4a4(fp4q_format fa, const uint8_t* a_codes, const uint8_t* a_scales,
                           const float* a_global, fp4q_format fw, const uint8_t* w_codes,
                           const uint8_t* w_scales, const float* w_global,
                           const float* w_special, int64_t M, int64_t N, int64_t K, void* c,
                           fp4q_dtype c_dtype, int64_t ldc, void* stream);

/*
 * fp4q_gemm_w4a4 for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops, harnesses that forbid hipMalloc): the same
 * arguments, checks, kernels and result -- the same bytes as fp4q_gemm_w4a4 --
 * but the partial results of K splits go to an array that is part of the
 * library's code object, 32 MiB per device, instead of a per-stream workspace.
 * It calls no allocating routine.  Its device address is looked up on the
 * first call on each device (FP4Q_ERR_DEVICE if that fails).  The split count
 * is capped so that the partials fit the array, the same cap fp4q_gemm_w4a4
 * applies to its workspace, so no shape needs more than the array holds.
 * Every call on a device shares that device's array, and nothing in it has to
 * start at zero; calls that overlap on one device (on different streams, or
 * from several threads) race on it and must be ordered by the caller.
 */
fp4q_status fp4q_gemm_w4a4_noalloc(fp4q_format fa, const uint8_t* a_codes, const uint8_t* a_scales,
                                   const float* a_global, fp4q_format fw, const uint8_t* w_codes,
                                   const uint8_t* w_scales, const float* w_global,
                                   const float* w_special, int64_t M, int64_t N, int64_t K, void* c,
                                   fp4q_dtype c_dtype, int64_t ldc, void* stream);

/*
 * fp4q_gemm_w4a4 for fused projections: W^ is the row-wise concatenation of
 * nseg weights (say Q, K and V), each quantized under its own global scale.
 * Segment i holds the seg_rows[i] rows after those of segments 0 .. i-1 and
 * its output columns take w_global[i]: C[m][n] = RN32(RN32(g_a g_i) acc),
 * with the split rule of fp4q_gemm_w4a4, so each segment's columns are those
 * of fp4q_gemm_w4a4 on that segment alone (bit for bit when both launches
 * split K alike).  The "Why Gated DeltaNet Survives..." review (section 3)
 * reports a global-scale mismatch when serving fused GEMMs; a per-segment
 * scale serves the fused product without requantizing any weight under a
 * shared scale.
 *   w_global  device, nseg FP32 (nseg >= 1); with nseg == 0 it is the single
 *             w_global of fp4q_gemm_w4a4 (device FP32 or NULL = 1.0)
 *   seg_rows  host, nseg counts >= 0 summing to N (ignored when nseg == 0)
 * Errors as fp4q_gemm_w4a4; nseg < 0 or > 8 -> ERR_ARG; seg_rows or
 * w_global NULL with nseg > 0 -> ERR_NULL; a negative count or a sum other
 * than N -> ERR_SHAPE.
 */
fp4q_status fp4q_gemm_w4a4_segmented(fp4q_format fa, const uint8_t* a_codes, const uint8_t* a_scales,
                                     const float* a_global, fp4q_format fw, const uint8_t* w_codes,
                                     const uint8_t* w_scales, const float* w_global, const int64_t* seg_rows,
                                     int nseg, const float* w_special, int64_t M, int64_t N, int64_t K, void* c,
                                     fp4q_dtype c_dtype, int64_t ldc, void* stream);

/*
 * W4A4 matmul whose activations arrive in bf16 and are quantized to NVFP4
 * (block 16) as the matmul loads them: the online activation quantization
 * ("Finer is Better", Method 2: abs-max or 4-over-6; hierarchical scaling
 * with a GIVEN global scale) fused into the matmul's A prologue.  The codes,
 * scales and C are those of fp4q_quantize (NVFP4, block 16, a_rule, GLOBAL
 * GIVEN a_global, or NONE when a_global is NULL) followed by
 * fp4q_gemm_w4a4_segmented (C bit for bit when both launches split K alike).
 * Meant for decode-sized M: every workgroup quantizes the activation rows it
 * multiplies, so the quantization is repeated once per 128 or 256 output
 * columns; for large M (prefill) quantize first and call fp4q_gemm_w4a4.
 *   a            device bf16 (uint16 bit patterns) M x K, pitch lda; 16-byte
 *                aligned, lda % 8 == 0
 *   a_rule       FP4Q_RULE_ABSMAX or FP4Q_RULE_4OVER6 (no flags)
 *   a_global     device FP32 (GIVEN) or NULL (g = 1)
 *   a_codes_out, a_scales_out  device M x K/2 and M x K/16 bytes, 16-byte
 *                aligned, written with the quantized activations; or both NULL
 *   fw           NVFP4, RAZER_A or RAZER_W (block 16); w_global, seg_rows,
 *                nseg as fp4q_gemm_w4a4_segmented; w_special as fp4q_gemm_w4a4
 * Errors: NULL pointer (or only one of the two outputs) -> ERR_NULL; another
 * fw -> ERR_FORMAT; M, N < 0, K <= 0, K % 512, K > 2^24, lda < K, lda > 2^24
 * or ldc < N -> ERR_SHAPE; another rule, a bad special value or segment
 * count -> ERR_ARG; misalignment -> ERR_ALIGN.  M == 0 or N == 0 enqueues
 * nothing.
 */
fp4q_status fp4q_gemm_w4a4_act_bf16(const uint16_t* a, int64_t lda, uint32_t a_rule, const float* a_global,
                                    uint8_t* a_codes_out, uint8_t* a_scales_out, fp4q_format fw,
                                    const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                                    const int64_t* seg_rows, int nseg, const float* w_special, int64_t M,
                                    int64_t N, int64_t K, void* c, fp4q_dtype c_dtype, int64_t ldc, void* stream);

/*
 * Weight-only matmul C = g_w * A W^^T with bf16 activations A (M x K, row
 * pitch lda elements) and a block-16 weight W^ (N x K) in NVFP4 or RAZER_W
 * (RaZeR summary 2.3: the weight-only kernel next to the weight-activation
 * one).  The weight decodes exactly to bf16 (value * scale, or the block's
 * special value * scale at code 0x8); products accumulate in FP32 and
 * C = RN32(g_w * acc), stored fp32 or bf16 (RNE).  K may be split as in
 * fp4q_gemm_w4a4, with the same summation rule, determinism and workspace.
 *   a         device bf16 (uint16 bit patterns), 16-byte aligned, lda % 8 == 0
 *   fw        NVFP4 or RAZER_W
 *   w_codes, w_scales  device, as fp4q_quantize writes them (block 16), 16-byte aligned
 *   w_global  device FP32 or NULL (= 1.0)
 *   w_special host, 4 floats, required when fw == RAZER_W
 *   c         device, M x N (pitch ldc elements), 16-byte aligned
 * Errors: NULL pointer -> ERR_NULL; another format -> ERR_FORMAT; M, N < 0,
 * K <= 0, K % 512 (the kernel's K window), K > 2^24, lda < K, lda > 2^24 or
 * ldc < N -> ERR_SHAPE; bad special value -> ERR_ARG; misalignment ->
 * ERR_ALIGN.  M == 0 or N == 0 enqueues nothing.
 */
fp4q_status fp4q_gemm_w4a16(const uint16_t* a, int64_t lda, fp4q_format fw, const uint8_t* w_codes,
                            const uint8_t* w_scales, const float* w_global, const float* w_special, int64_t M,
                            int64_t N, int64_t K, void* c, fp4q_dtype c_dtype, int64_t ldc, void* stream);

/*
 * Per-channel scale of MACaQ's online scaling (MACaQ review, section 3):
 *   t_j = (rms_j(W) / rms_j(X))^alpha, r_j = RN32(1 / t_j),
 * rms over the rows of each column, computed in binary64 and rounded to fp32;
 * t_j = 1 where either rms is 0.  Activations then take chan_scale = t, the
 * weights chan_scale = r (W D^-1 B absorbed offline).
 *   x  device, rows_x x cols, pitch ldx;  w  device, rows_w x cols, pitch ldw
 *   t, r  device, cols floats each, written
 * Errors: NULL -> ERR_NULL; rows_x, rows_w <= 0, cols <= 0, pitches < cols
 * -> ERR_SHAPE; alpha not finite -> ERR_ARG.
 */
fp4q_status fp4q_channel_scale(const void* x, fp4q_dtype x_dtype, int64_t rows_x, int64_t ldx,
                               const void* w, fp4q_dtype w_dtype, int64_t rows_w, int64_t ldw,
                               int64_t cols, double alpha, float* t, float* r, void* stream);

/*
 * MACaQ weight calibration for MXFP4 (MACaQ review, sections 1 and 3): the
 * weight's codes and E8M0 exponents chosen for the layer-output error
 * ||X W^T - X W^^T||_F^2 = sum_n (w_n - w^_n)^T H (w_n - w^_n), H = X^T X.
 *   1. Hessian-weighted exponent screening: per 32-element block, the
 *      standard exponent E (as fp4q_quantize's MXFP4) and E + 1, E - 1, in
 *      that order, each with round-to-nearest codes, compared by e^T H_bb e
 *      (H_bb the block's 32 x 32 diagonal block of H, e the block error); the
 *      strictly smallest is kept.
 *   2. Flip-Refinement: per row, repeatedly the single move of one code to
 *      an adjacent E2M1 level with the largest gain
 *      -(2 delta (H d)_k + delta^2 H_kk) (d = w^ - w) is taken while the gain
 *      is positive (a tie keeps the smaller k, then the move up), at most
 *      max_moves times; H d is updated by delta times row k of H.
 * All arithmetic is binary64 in a fixed order: every sum over j runs j
 * ascending; e^T H_bb e adds the 32 products e_i (H_bb e)_i by a balanced
 * pairwise tree in index order; the gain is -(2 (delta r_k) + (delta delta)
 * H_kk).  The weight is taken as given: apply any channel scale or rotation
 * (W D^-1 B) before, and pass the Hessian of the transformed activations.
 *   w          device fp32, N x K, row pitch ldw (row n = output channel)
 *   h          device binary64, K x K, row pitch ldh (rows are read)
 *   codes      device, N x K/2 (layout as fp4q_quantize), written
 *   scales     device, N x K/32 E8M0 codes, written
 *   moves      device int32 per row (moves taken), or NULL
 *   workspace  device, 8-byte aligned; holds H d for workspace_bytes / (8 K)
 *              rows at a time (at least one row: 8 K bytes)
 * Errors: NULL pointer -> ERR_NULL; N < 0, K <= 0, K % 32, K > 5120,
 * ldw < K or ldh < K -> ERR_SHAPE; max_moves < 0 or a workspace below one
 * row -> ERR_ARG; misaligned w (4), h, workspace (8), moves (4) -> ERR_ALIGN.
 * N == 0 enqueues nothing.
 */
fp4q_status fp4q_macaq_quantize(const float* w, int64_t N, int64_t K, int64_t ldw, const double* h,
                                int64_t ldh, int64_t max_moves, uint8_t* codes, uint8_t* scales,
                                int32_t* moves, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Offline choice of RaZeR-W's special values (RaZeR summary 2.2: the weight
 * table's four values are precomputed offline, multiples of 0.5, by
 * quantization error).  Candidates are the magnitudes a in {2.5, 3.5, 4.5, 5,
 * 5.5, 6.5, 7, 7.5} (the multiples of 0.5 up to 7.5 that are not E2M1
 * magnitudes); a table is {+a, -a, +b, -b} for a pair a < b, 28 pairs in
 * lexicographic order (a, b) = (2.5, 3.5), (2.5, 4.5), ... (7, 7.5).  Each
 * 16-element block of w takes RaZeR-W quantization under the global scale
 * (abs-max E3M3 scale, round-to-nearest codes, the element rule of
 * fp4q_quantize) with the one signed candidate of the table that gives the
 * lowest block error (the FP32 error of fp4q_quantize's RaZeR-W).  A pair's
 * error is the binary64 sum over rows, ascending, of the binary64 sum over
 * each row's blocks, ascending, of that lowest block error.
 *   w           device, rows x cols, pitch ld_w (fp32 or bf16), 16-byte aligned
 *   global_mode NONE (g = 1), AUTO (g = RN32(amax / 180), 1 for an all-zero
 *               w, written to *global as fp4q_quantize's RAZER_W does),
 *               GIVEN (*global read)
 *   pair_sse    device, 28 doubles: each pair's error, written
 *   table       device, 4 floats: {+a, -a, +b, -b} of the pair with the
 *               lowest error (a tie keeps the earlier pair), written; pass it
 *               (copied to the host) as fp4q_quant_desc.special
 *   workspace   device, 8-byte aligned, at least rows * 28 * 8 bytes
 * Errors: NULL pointer -> ERR_NULL; rows < 0, cols <= 0, cols % 16 or
 * ld_w < cols -> ERR_SHAPE; bad dtype or mode, or a small workspace ->
 * ERR_ARG; misalignment -> ERR_ALIGN.  rows == 0 (w and workspace may then
 * be NULL) writes zero errors and the first pair.
 */
fp4q_status fp4q_razer_table_search(const void* w, fp4q_dtype w_dtype, int64_t rows, int64_t cols, int64_t ld_w,
                                    fp4q_global_mode global_mode, float* global, double* pair_sse, float* table,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code; never NULL. */
const char* fp4q_status_string(fp4q_status s);

/* FP4Q_ABI_VERSION of the loaded library. */
uint32_t fp4q_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FP4Q_H */
