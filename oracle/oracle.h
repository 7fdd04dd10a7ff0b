/*
 * oracle.h -- plain CPU oracle for block-scaled FP4 quantization and the W4A4
 * matmul.  TEST INFRASTRUCTURE ONLY: nothing on the product path may include,
 * link or call this.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or table with the HIP library.
 *
 * Sources (cited by page title and section throughout):
 *   [NVFP4-GDN]  "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 ..."
 *                review, section 1 (NVFP4 definition), section 3 (fused GEMMs,
 *                shared global scale).
 *   [RaZeR]      "RaZeR - breaking the NVFP4 limit by redundant zero remapping"
 *                summary, section 1 (problem), 2.1 (scale redundancy),
 *                2.2 (remapping the redundant zero), 2.3 (implementation).
 *   [MACaQ]      "MACaQ: Fast, Model Agnostic Calibrated Quantization ..." review,
 *                section 1 (MXFP4, online scaling and micro-rotation), section 3.
 *   [Finer]      "Finer is Better (with the Right Scaling)" summary, Method 1
 *                (numerical study) and Method 2 (the five scaling strategies).
 *
 * Precision: every rounding decision (scale -> scale format, element -> E2M1)
 * is decided exactly in real arithmetic; the comparisons are carried out in
 * binary64 on operands that are exact there.  The per-block error used to pick
 * between candidates ("MSE" on the pages) is the binary32 sum of squares with a
 * fixed balanced pairwise tree, the precision the device kernel computes it in.
 * Transforms (channel scale, block-Hadamard) are the binary32 steps listed at
 * or_transform.  The matmul accumulates in binary64.
 */
#ifndef FP4_ORACLE_H
#define FP4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* container formats */
#define OR_NVFP4   0   /* E2M1 + E4M3 per block (+ FP32 global)          */
#define OR_MXFP4   1   /* E2M1 + E8M0 per 32-element block                */
#define OR_RAZER_A 2   /* NVFP4, E4M3 sign bit = pick of +5 / -5          */
#define OR_RAZER_W 3   /* E3M3 scale + 2-bit pick among 4 special values   */
#define OR_UE5M3   4   /* E2M1 + UE5M3 (unsigned, 5-bit exponent) per block */

/* scale rules (low byte) and flags */
#define OR_ABSMAX       0
#define OR_4OVER6       1
#define OR_BRUTE        2
#define OR_EXPSEARCH    3   /* MXFP4: shared exponent E_std, E_std+1, E_std-1 by block error */
#define OR_PREVENT_ZERO 0x100

/* global scale modes */
#define OR_G_NONE  0
#define OR_G_AUTO  1
#define OR_G_GIVEN 2

/* element dtypes of the input tensor */
#define OR_F32  0
#define OR_BF16 1

/* scale formats for or_round_scale */
#define OR_SF_E4M3 0
#define OR_SF_E3M3 1
#define OR_SF_UE5M3 2

/* -- number formats --------------------------------------------------------- */
double or_e2m1_value(int code);   /* signed value of a 4-bit E2M1 code          */
double or_e4m3_value(int k);      /* k in 0..126 (OCP E4M3, sign bit clear)     */
double or_e3m3_value(int k);      /* k in 0..63  (6-bit, bias 3)                */
double or_e8m0_value(int k);      /* k in 0..254                                */
double or_ue5m3_value(int k);     /* k in 0..255 (unsigned, bias 15)            */

/* -- rounding primitives ------------------------------------------------------ */
/* nearest code of scale format sf to a/(T*g); ties to the even code; saturates */
int or_round_scale(int sf, double a, double T, double g);
/* E2M1 round-to-nearest of x/(s*g); ties to even mantissa; saturates at 6;
 * a zero magnitude is always +0; s == 0 gives code 0 */
int or_rtn(float x, double s, double g);
/* RaZeR element rounding: nearest of the 15 standard values and v (code 0x8);
 * a tie between v and a standard value keeps the standard value */
int or_rtn_special(float x, double s, double g, double v);
/* binary32 sum of squared errors of one block of n (power of two) elements;
 * code 0x8 decodes to v when has_special, else to -0 */
float or_block_sse(const float* x, const int* codes, int n, double s, float g,
                   int has_special, double v);

/* -- whole-tensor operations -------------------------------------------------- */
/* widen (bf16 -> fp32), channel scale x_j*t_j, then the block-Hadamard of
 * size 16 or 32 (orthonormal).  t may be NULL; hadamard is 0, 16 or 32.  out
 * is rows x cols fp32, contiguous. */
void or_transform(const void* x, int xdtype, long rows, long cols, long ld,
                  const float* t, int hadamard, float* out);

/* g for AUTO mode from the transformed tensor (max |x'|): a/2688 for E4M3
 * scales, a/180 for E3M3 scales, 1 when the tensor is all zero */
float or_auto_global(const float* xt, long rows, long cols, int format);

/* quantize rows of an already transformed fp32 tensor (contiguous, cols per
 * row) with global scale g.  Writes codes (rows x cols/2, low nibble = even
 * element) and scales (rows x cols/block).  Returns 0, or -1 on a bad argument. */
int or_quantize_rows(int format, int block, int rule, const float* special4,
                     const float* xt, long rows, long cols, float g,
                     uint8_t* codes, uint8_t* scales);

/* full quantize as the library defines it: transform, global scale, encode.
 * g_inout is read for GIVEN, written for AUTO and NONE (1.0). */
int or_quantize(int format, int block, int rule, int gmode, const float* chan_scale,
                int hadamard, const float* special4, const void* x, int xdtype,
                long rows, long cols, long ld, uint8_t* codes, uint8_t* scales,
                float* g_inout);

/* dequantize to fp32: RN32((value * scale) * g) */
int or_dequantize(int format, int block, const float* special4, const uint8_t* codes,
                  const uint8_t* scales, float g, long rows, long cols, float* out);

/* decoded element values without the global scale (value * block scale),
 * exact in binary64; one row */
int or_decode_row(int format, int block, const float* special4, const uint8_t* codes_row,
                  const uint8_t* scales_row, long cols, double* out);

/* W4A4 matmul C = (g_a*g_w) * A^ W^T for rows [m0, m1) of C.  A is M x K, W is
 * N x K (row n = output channel).  Accumulates in binary64, then
 * C = RN32(RN32(g_a*g_w) * acc).  c has (m1-m0) rows of N floats. */
int or_gemm_rows(int fa, const uint8_t* a_codes, const uint8_t* a_scales, float g_a,
                 int fw, const uint8_t* w_codes, const uint8_t* w_scales, float g_w,
                 const float* w_special4, long M, long N, long K, long m0, long m1,
                 float* c);

/* same, for an explicit list of (m, n) entries */
int or_gemm_entries(int fa, const uint8_t* a_codes, const uint8_t* a_scales, float g_a,
                    int fw, const uint8_t* w_codes, const uint8_t* w_scales, float g_w,
                    const float* w_special4, long M, long N, long K, const long* ms,
                    const long* ns, long count, float* out);

/* RaZeR weight-only matmul ([RaZeR] 2.3, W4A16): C = g_w * A W^^T for rows
 * [m0, m1) with A in bf16 (bit patterns, M x K, pitch lda) and W (N x K) given
 * as codes/scales of format fw (NVFP4 or RaZeR-W, block 16).  Accumulates the
 * exact products in binary64, then C = RN32(g_w * acc). */
int or_gemm_w4a16_rows(const uint16_t* a, long lda, int fw, const uint8_t* w_codes,
                       const uint8_t* w_scales, float g_w, const float* w_special4,
                       long M, long N, long K, long m0, long m1, float* c);

/* RaZeR offline special-value search ([RaZeR] 2.2): the candidate magnitudes
 * are the multiples of 0.5 in (0, 7.5] that are not E2M1 magnitudes,
 * {2.5, 3.5, 4.5, 5, 5.5, 6.5, 7, 7.5}; a table is {+a, -a, +b, -b} for a pair
 * a < b (28 pairs, lexicographic).  For a table, each 16-element block of the
 * weight (RaZeR-W: abs-max E3M3 scale under g) takes the table value with the
 * smallest block error (or_block_sse), and the tensor error is the binary64
 * sum over rows (ascending) of the binary64 sum over the row's blocks
 * (ascending).  Writes the 28 tensor errors and returns the index of the
 * smallest (a tie keeps the earlier pair), or -1 on a bad argument. */
#define OR_RAZER_NCAND 8
#define OR_RAZER_NPAIRS 28
int or_razer_table_search(const void* x, int xdtype, long rows, long cols, long ld, float g,
                          double* pair_sse);
/* magnitudes of pair p (0 .. 27) */
void or_razer_pair(int p, float* a, float* b);

/* MACaQ weight calibration for MXFP4 ([MACaQ] sections 1 and 3): for each
 * row of W (N x K, row n = output channel, fp32) and the layer-input Hessian
 * H = X^T X (K x K, binary64, row-major, pitch ldh):
 *  1. exponent screening: per 32-element block the standard exponent E and
 *     E + 1, E - 1 are compared by the Hessian-weighted error e^T H_bb e of
 *     the block's RTN codes (H_bb the block's 32 x 32 diagonal block);
 *  2. Flip-Refinement: starting from the screened RTN codes, the single move
 *     of one code to an adjacent E2M1 level with the largest gain in
 *     f = (w - w^)^T H (w - w^) is taken, repeatedly, while a move gains
 *     (at most max_moves per row).
 * Writes codes (N x K/2), scales (E8M0 codes, N x K/32); moves[n] = moves
 * taken on row n and objective[2n], [2n+1] = f before and after refinement
 * (either may be NULL).  Returns 0, or -1 on a bad argument. */
int or_macaq_quantize(const float* w, long N, long K, long ldw, const double* h, long ldh,
                      long max_moves, uint8_t* codes, uint8_t* scales, int* moves,
                      double* objective);

/* per-channel scale t_j = (rms_j(W) / rms_j(X))^alpha in binary64, rounded to
 * fp32, and r_j = RN32(1 / t_j).  X is rows_x x cols, W is rows_w x cols. */
void or_channel_scale(const void* x, int xdtype, long rows_x, long ldx,
                      const void* w, int wdtype, long rows_w, long ldw, long cols,
                      double alpha, float* t, float* r);

#ifdef __cplusplus
}
#endif
#endif
