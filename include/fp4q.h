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
 *   global  one FP32 on the device; an element decodes to value * scale * g.
 *
 * Ownership: the caller allocates and owns every buffer; libfp4q never
 * allocates or frees device memory and keeps no state beyond its loaded code.
 * Calls are thread-safe.
 *
 * Asynchrony: every call validates its arguments on the host, enqueues its
 * kernels on `stream` (a hipStream_t passed as void*, NULL = default stream)
 * and returns without synchronising.  An argument error returns its status
 * and enqueues nothing; a failed launch returns FP4Q_ERR_DEVICE.
 *
 * Non-finite inputs, and a GIVEN global scale that is not a positive finite
 * number, are outside the contract: the outputs are then unspecified.
 */
#ifndef FP4Q_H
#define FP4Q_H

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
  FP4Q_NVFP4_RAZER_W = 3
} fp4q_format;

typedef enum { FP4Q_F32 = 0, FP4Q_BF16 = 1 } fp4q_dtype;

/* scale rules (low byte of fp4q_quant_desc.rule) and OR-able flags, from
 * "Finer is Better (with the Right Scaling)", Method 2 */
enum {
  FP4Q_RULE_ABSMAX = 0,        /* block max maps to 6, nearest E4M3 scale          */
  FP4Q_RULE_4OVER6 = 1,        /* max maps to 4 or 6, lower block error kept       */
  FP4Q_RULE_BRUTE = 2,         /* all 126 positive E4M3 scales, lowest error kept  */
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
  uint32_t rule;               /* rule | flags; RaZeR formats and MXFP4 take
                                  ABSMAX (RaZeR may add PREVENT_ZERO)            */
  fp4q_global_mode global_mode;/* MXFP4: must be NONE                            */
  const float* chan_scale;     /* device, `cols` floats, or NULL: x_j *= t_j
                                  before quantization (MACaQ online scaling)     */
  int32_t hadamard;            /* 0, or 32: size-32 block-Hadamard after the
                                  channel scale (MACaQ micro-rotation);
                                  needs cols % 32 == 0                           */
  float special[4];            /* RAZER_W: the four special values; each a
                                  multiple of 0.5 with 0 < |v| <= 7.5 that is
                                  not an E2M1 magnitude.  Ignored otherwise.     */
} fp4q_quant_desc;

/*
 * Quantize a rows x cols tensor x (fp32 or bf16, row pitch ld_x elements).
 * Steps: widen to fp32; x_j *= chan_scale[j] (if given); size-32
 * block-Hadamard (if hadamard == 32); global scale per global_mode; per-block
 * scale by the rule; E2M1 encode (RaZeR: with the special value); pack.
 * Pages: scale rules -- "Finer is Better", Method 2; RaZeR picks -- RaZeR
 * summary 2.2; transforms -- MACaQ review, sections 1 and 3; MXFP4 -- MACaQ
 * review, section 1.
 *   x       device, 16-byte aligned, ld_x * sizeof(elem) a multiple of 16
 *   codes   device, rows*(cols/2) bytes, 16-byte aligned, written
 *   scales  device, rows*(cols/block) bytes, written
 *   global  device FP32: read (GIVEN), written (AUTO) or unused (NONE, may be NULL)
 * Errors: NULL desc/x/codes/scales (or global with AUTO/GIVEN) -> ERR_NULL;
 * rows < 0, cols <= 0, cols % block, ld_x < cols, hadamard with cols % 32
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
 * FP32; C = RN32(RN32(g_a*g_w) * acc), stored fp32 or bf16 (RNE), row pitch ldc.
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
 * tiles of 256 x 256, or ldc < N -> ERR_SHAPE; a mixed MXFP4/NVFP4 pair or fa == RAZER_W -> ERR_FORMAT;
 * bad special value
 * -> ERR_ARG; misalignment -> ERR_ALIGN.  M == 0 or N == 0 enqueues nothing.
 */
fp4q_status fp4q_gemm_w4a4(fp4q_format fa, const uint8_t* a_codes, const uint8_t* a_scales,
                           const float* a_global, fp4q_format fw, const uint8_t* w_codes,
                           const uint8_t* w_scales, const float* w_global,
                           const float* w_special, int64_t M, int64_t N, int64_t K, void* c,
                           fp4q_dtype c_dtype, int64_t ldc, void* stream);

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

/* Static text for a status code; never NULL. */
const char* fp4q_status_string(fp4q_status s);

/* FP4Q_ABI_VERSION of the loaded library. */
uint32_t fp4q_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FP4Q_H */
