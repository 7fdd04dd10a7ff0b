/*
 * oracle.c -- plain, slow CPU oracle for block-scaled FP4 quantization and the
 * W4A4 matmul.  TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline of
 * the benchmark).  Shares no code with the HIP library.  Build flags:
 * -O2 -ffp-contract=off -fno-fast-math, so every binary32 operation below is
 * one IEEE round-to-nearest-even operation (fmaf is the correctly rounded
 * fused multiply-add of the C library).
 *
 * Page citations use the tags of oracle.h: [NVFP4-GDN], [RaZeR], [MACaQ], [Finer].
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Number formats                                                            */
/* ------------------------------------------------------------------------- */

/* E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit.  The magnitudes are the
 * set {0, 0.5, 1, 1.5, 2, 3, 4, 6} listed in [RaZeR] section 1; the bit layout
 * s|ee|m is the OCP one named in [MACaQ] section 1 and [Finer] Method 1. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double or_e2m1_value(int code) {
  double m = E2M1_MAG[code & 7];
  return (code & 8) ? -m : m;
}

/* OCP E4M3 ("FN": bias 7, subnormals, max 448, code 127 is NaN and never
 * produced).  Block scale of NVFP4 per [NVFP4-GDN] section 1 and [RaZeR] section 1. */
double or_e4m3_value(int k) {
  int e = k >> 3, m = k & 7;
  if (e == 0) return ldexp((double)m, -9);
  return ldexp((double)(8 + m), e - 10);
}

/* E3M3 6-bit weight scale of [RaZeR] section 2.1; the page gives only the
 * width, read here as bias 3 with subnormals and no special codes (max 30). */
double or_e3m3_value(int k) {
  int e = k >> 3, m = k & 7;
  if (e == 0) return ldexp((double)m, -5);
  return ldexp((double)(8 + m), e - 6);
}

/* E8M0: a bare power of two, the MXFP4 shared scale of [MACaQ] section 1. */
double or_e8m0_value(int k) { return ldexp(1.0, k - 127); }

/* UE5M3: the unsigned wide-exponent block scale that [Finer] findings and
 * claims compare with E4M3 + 4-over-6 + hierarchical scaling.  The page gives
 * only the name; read here as 5 exponent bits (bias 15, the half-precision
 * bias) and 3 mantissa bits, subnormals, no sign and no special codes: 256
 * values from 0 to 1.875 * 2^16 = 122880, smallest positive 2^-17. */
double or_ue5m3_value(int k) {
  int e = k >> 3, m = k & 7;
  if (e == 0) return ldexp((double)m, -17);
  return ldexp((double)(8 + m), e - 18);
}

static double sf_value(int sf, int k) {
  if (sf == OR_SF_E4M3) return or_e4m3_value(k);
  if (sf == OR_SF_E3M3) return or_e3m3_value(k);
  return or_ue5m3_value(k);
}
static int sf_max_code(int sf) { return sf == OR_SF_E4M3 ? 126 : sf == OR_SF_E3M3 ? 63 : 255; }

/* ------------------------------------------------------------------------- */
/* Rounding primitives                                                       */
/* ------------------------------------------------------------------------- */

/* Nearest scale-format value to y = a / (T*g), scanning the codes upward.
 * [Finer] Method 2 "abs-max": the block maximum mapped to the largest E2M1
 * value, rounded to the nearest representable E4M3 value.  Instead of forming
 * y, a is compared with each midpoint times T*g; the midpoint has at most 5
 * significant bits, T (4 or 6) at most 2 and g 24, so the product is exact in
 * binary64 and so is the comparison.  A tie goes to the even code; values past
 * the largest code saturate to it. */
int or_round_scale(int sf, double a, double T, double g) {
  int kmax = sf_max_code(sf);
  for (int k = 0; k < kmax; ++k) {
    double mid = 0.5 * (sf_value(sf, k) + sf_value(sf, k + 1));
    double M = mid * T * g;
    if (a < M) return k;
    if (a == M) return (k % 2 == 0) ? k : k + 1;
  }
  return kmax;
}

/* E2M1 round-to-nearest ("RTN", [MACaQ] section 1) of x / (s*g): the
 * midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 times s*g are exact in
 * binary64 (at most 3 + 4 + 24 bits), so each comparison is exact.  A tie goes
 * to the neighbour with an even mantissa bit; |x| past 6*s*g saturates to 6. */
int or_rtn(float x, double s, double g) {
  if (s == 0.0) return 0;
  double ax = fabs((double)x);
  int m = 7;
  for (int j = 0; j < 7; ++j) {
    double M = 0.5 * (E2M1_MAG[j] + E2M1_MAG[j + 1]) * s * g;
    if (ax < M) { m = j; break; }
    if (ax == M) { m = (j % 2 == 0) ? j : j + 1; break; }
  }
  if (m == 0) return 0;              /* zero magnitude: always +0 */
  return (x < 0.0f ? 8 : 0) | m;
}

/* [RaZeR] section 2.2: the redundant zero (code 0x8) stands for the block's
 * special value v.  The element takes the nearest of the 15 standard values
 * and v.  The nearest standard value is or_rtn's; v replaces it only when x is
 * strictly nearer to v, decided against the exact midpoint (q+v)/2*s*g (at
 * most 5 + 4 + 24 bits).  A tie keeps the standard value. */
int or_rtn_special(float x, double s, double g, double v) {
  if (s == 0.0) return 0;
  int c = or_rtn(x, s, g);
  double q = or_e2m1_value(c);
  double mid = 0.5 * (q + v) * s * g;
  double xd = (double)x;
  if (v > q) return (xd > mid) ? 8 : c;
  if (v < q) return (xd < mid) ? 8 : c;
  return c;
}

/* binary32 balanced pairwise sum: T(p[0..n)) = T(left half) + T(right half) */
static float tree_sum(const float* p, int n) {
  if (n == 1) return p[0];
  float l = tree_sum(p, n / 2);
  float r = tree_sum(p + n / 2, n - n / 2);
  return l + r;
}

/* Block error used by the MSE-based rules ([Finer] Method 2, [RaZeR] 2.2):
 * e_i = fma(-(value_i*s), g, x_i) with value_i*s exact in binary32 (at most
 * 8 significant bits), p_i = e_i*e_i, summed by the balanced tree.  Dividing
 * by the block size would not change any comparison, so the sum is compared. */
float or_block_sse(const float* x, const int* codes, int n, double s, float g,
                   int has_special, double v) {
  float p[32];
  for (int i = 0; i < n; ++i) {
    double val = (has_special && codes[i] == 8) ? v : or_e2m1_value(codes[i]);
    float q = (float)(val * s);
    float e = fmaf(-q, g, x[i]);
    p[i] = e * e;
  }
  return tree_sum(p, n);
}

/* ------------------------------------------------------------------------- */
/* One block                                                                  */
/* ------------------------------------------------------------------------- */

static double block_absmax(const float* x, int B) {
  double a = 0.0;
  for (int i = 0; i < B; ++i) {
    double v = fabs((double)x[i]);
    if (v > a) a = v;
  }
  return a;
}

static void encode_plain(const float* x, int B, double s, double g, int* codes) {
  for (int i = 0; i < B; ++i) codes[i] = or_rtn(x[i], s, g);
}

static void encode_special(const float* x, int B, double s, double g, double v, int* codes) {
  for (int i = 0; i < B; ++i) codes[i] = or_rtn_special(x[i], s, g, v);
}

/* floor(log2 a) for a finite a > 0, read exactly through frexp */
static int floor_log2(double a) {
  int ex;
  (void)frexp(a, &ex);  /* a = f * 2^ex, f in [0.5, 1) */
  return ex - 1;
}

/* Quantize one block; writes B codes and returns the scale byte. */
static uint8_t quant_block(int format, int B, int rule, const float* special4,
                           const float* x, float g, int* codes) {
  int pz = (rule & OR_PREVENT_ZERO) != 0;
  int r = rule & 0xff;
  double a = block_absmax(x, B);
  double gd = (double)g;

  if (format == OR_MXFP4) {
    /* [MACaQ] section 1: one E8M0 exponent per 32 elements.  The "standard
     * exponent" is read as the OCP rule floor(log2 amax) - 2 (2 = the largest
     * E2M1 exponent), clamped to the E8M0 range; elements past 6 saturate. */
    int E = (a == 0.0) ? -127 : floor_log2(a) - 2;
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    encode_plain(x, B, ldexp(1.0, E), 1.0, codes);
    if (r != OR_EXPSEARCH) return (uint8_t)(E + 127);
    /* [MACaQ] section 1 compares the standard exponent with offsets +1 and
     * -1 by a Hessian-weighted error; with a plain block error (unit
     * Hessian) that is the search below.  Candidates in the order E, E+1,
     * E-1 (those inside the E8M0 range); the strictly smallest block error
     * wins, a tie keeps the earlier candidate. */
    float best = or_block_sse(x, codes, B, ldexp(1.0, E), 1.0f, 0, 0.0);
    int bestE = E;
    const int off[2] = {1, -1};
    int tmp[32];
    for (int t = 0; t < 2; ++t) {
      int Ec = E + off[t];
      if (Ec < -127 || Ec > 127) continue;
      encode_plain(x, B, ldexp(1.0, Ec), 1.0, tmp);
      float e = or_block_sse(x, tmp, B, ldexp(1.0, Ec), 1.0f, 0, 0.0);
      if (e < best) {
        best = e;
        bestE = Ec;
        memcpy(codes, tmp, sizeof(int) * B);
      }
    }
    return (uint8_t)(bestE + 127);
  }

  if (format == OR_NVFP4 || format == OR_UE5M3) {
    const int sf = format == OR_NVFP4 ? OR_SF_E4M3 : OR_SF_UE5M3;
    if (r == OR_BRUTE) {
      /* [Finer] Method 2 "brute-force": every positive finite scale of the
       * format is tried; the strictly smallest error wins, a tie keeps the
       * smaller code. */
      int best_k = 1;
      float best = 0.0f;
      int tmp[32];
      for (int k = 1; k <= sf_max_code(sf); ++k) {
        double s = sf_value(sf, k);
        encode_plain(x, B, s, gd, tmp);
        float e = or_block_sse(x, tmp, B, s, g, 0, 0.0);
        if (k == 1 || e < best) {
          best = e;
          best_k = k;
          memcpy(codes, tmp, sizeof(int) * B);
        }
      }
      return (uint8_t)best_k;
    }
    /* [Finer] Method 2 "abs-max": the block max maps to 6.0 */
    int k6 = or_round_scale(sf, a, 6.0, gd);
    /* [Finer] Method 2 "prevent-zero": a zero scale is raised to the smallest
     * positive representable scale (2^-9 for E4M3, 2^-17 for UE5M3) */
    if (pz && k6 == 0) k6 = 1;
    encode_plain(x, B, sf_value(sf, k6), gd, codes);
    if (r == OR_ABSMAX) return (uint8_t)k6;
    /* [Finer] Method 2 "4-over-6": the block max maps to 4.0 or to 6.0,
     * whichever block error is lower; both candidates are quantized.  A tie
     * keeps 6. */
    int k4 = or_round_scale(sf, a, 4.0, gd);
    if (pz && k4 == 0) k4 = 1;
    int c4[32];
    encode_plain(x, B, sf_value(sf, k4), gd, c4);
    float e6 = or_block_sse(x, codes, B, sf_value(sf, k6), g, 0, 0.0);
    float e4 = or_block_sse(x, c4, B, sf_value(sf, k4), g, 0, 0.0);
    if (e4 < e6) {
      memcpy(codes, c4, sizeof(int) * B);
      return (uint8_t)k4;
    }
    return (uint8_t)k6;
  }

  if (format == OR_RAZER_A) {
    /* [RaZeR] 2.1/2.2: activations keep the E4M3 abs-max scale; its unused
     * sign bit selects the special value of the pair {+5, -5}; the block is
     * quantized with each and the lower error is kept (a tie keeps +5). */
    int k = or_round_scale(OR_SF_E4M3, a, 6.0, gd);
    if (pz && k == 0) k = 1;
    if (k == 0) {
      for (int i = 0; i < B; ++i) codes[i] = 0;
      return 0;
    }
    double s = or_e4m3_value(k);
    int cm[32];
    encode_special(x, B, s, gd, 5.0, codes);
    encode_special(x, B, s, gd, -5.0, cm);
    float ep = or_block_sse(x, codes, B, s, g, 1, 5.0);
    float en = or_block_sse(x, cm, B, s, g, 1, -5.0);
    if (en < ep) {
      memcpy(codes, cm, sizeof(int) * B);
      return (uint8_t)(0x80 | k);
    }
    return (uint8_t)k;
  }

  /* OR_RAZER_W: [RaZeR] 2.1/2.2: weights use a 6-bit E3M3 abs-max scale and
   * the two freed bits pick one of four offline special values; the lowest
   * block error wins, a tie keeps the lower index. */
  {
    int k = or_round_scale(OR_SF_E3M3, a, 6.0, gd);
    if (pz && k == 0) k = 1;
    if (k == 0) {
      for (int i = 0; i < B; ++i) codes[i] = 0;
      return 0;
    }
    double s = or_e3m3_value(k);
    int best_p = 0;
    float best = 0.0f;
    int tmp[32];
    for (int p = 0; p < 4; ++p) {
      double v = (double)special4[p];
      encode_special(x, B, s, gd, v, tmp);
      float e = or_block_sse(x, tmp, B, s, g, 1, v);
      if (p == 0 || e < best) {
        best = e;
        best_p = p;
        memcpy(codes, tmp, sizeof(int) * B);
      }
    }
    return (uint8_t)((best_p << 6) | k);
  }
}

/* ------------------------------------------------------------------------- */
/* Tensors                                                                    */
/* ------------------------------------------------------------------------- */

static float load_elem(const void* x, int dt, long idx) {
  if (dt == OR_F32) return ((const float*)x)[idx];
  /* bf16 -> fp32 is exact: the 16 bits become the high half */
  uint32_t u = (uint32_t)((const uint16_t*)x)[idx] << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Sylvester-ordered fast Walsh-Hadamard transform of n (16 or 32) values in
 * binary32: for h = 1, 2, 4, ... < n the pairs (j, j+h) become (u+w, u-w). */
static void fwht(float* y, int n) {
  for (int h = 1; h < n; h *= 2)
    for (int i = 0; i < n; i += 2 * h)
      for (int j = i; j < i + h; ++j) {
        float u = y[j], w = y[j + h];
        y[j] = u + w;
        y[j + h] = u - w;
      }
}

/* [MACaQ] sections 1 and 3: the online per-channel scale D (x_j * t_j) and
 * then the size-32 block-Hadamard B, normalised to be orthonormal by
 * c = RN32(2^-2.5); the weight side absorbs W D^-1 B, i.e. the same call with
 * t_j replaced by 1/t_j.  hadamard = 16 is the NVFP4-block-sized variant
 * ("Finer is Better" claims compare scale formats; the MACaQ page sizes the
 * rotation to the block): groups of 16, normalised by exactly 1/4. */
void or_transform(const void* x, int xdtype, long rows, long cols, long ld,
                  const float* t, int hadamard, float* out) {
  uint32_t cbits = 0x3E3504F3u;
  float c;
  memcpy(&c, &cbits, 4);
  if (hadamard == 16) c = 0.25f;
  for (long r = 0; r < rows; ++r) {
    float* y = out + r * cols;
    for (long j = 0; j < cols; ++j) {
      float v = load_elem(x, xdtype, r * ld + j);
      y[j] = t ? v * t[j] : v;
    }
    if (hadamard == 16 || hadamard == 32)
      for (long j0 = 0; j0 < cols; j0 += hadamard) {
        fwht(y + j0, hadamard);
        for (int i = 0; i < hadamard; ++i) y[j0 + i] = y[j0 + i] * c;
      }
  }
}

/* [Finer] Method 2 "hierarchical": a per-tensor FP32 scale over the local
 * block scales.  Read as a decode multiplier g with the tensor maximum mapped
 * to the top of the two-level range: g = amax / (6 * 448) for E4M3 block
 * scales, amax / (6 * 30) for E3M3. */
float or_auto_global(const float* xt, long rows, long cols, int format) {
  float a = 0.0f;
  for (long i = 0; i < rows * cols; ++i) {
    float v = fabsf(xt[i]);
    if (v > a) a = v;
  }
  if (a == 0.0f) return 1.0f;
  return format == OR_RAZER_W ? a / 180.0f : a / 2688.0f;
}

static int check_format(int format, int block, int rule, int hadamard, long cols) {
  if (format < OR_NVFP4 || format > OR_UE5M3) return -1;
  if (format == OR_MXFP4) {
    if (block != 32 || (rule != OR_ABSMAX && rule != OR_EXPSEARCH)) return -1;
  } else {
    if (block != 4 && block != 8 && block != 16 && block != 32) return -1;
    int r = rule & 0xff;
    if ((rule & ~0x1ff) != 0 || r > OR_BRUTE) return -1;
    if ((format == OR_RAZER_A || format == OR_RAZER_W) && r != OR_ABSMAX) return -1;
  }
  if (hadamard != 0 && hadamard != 16 && hadamard != 32) return -1;
  if (cols <= 0 || cols % block != 0 || (hadamard && cols % hadamard != 0)) return -1;
  return 0;
}

int or_quantize_rows(int format, int block, int rule, const float* special4,
                     const float* xt, long rows, long cols, float g,
                     uint8_t* codes, uint8_t* scales) {
  if (check_format(format, block, rule, 0, cols)) return -1;
  int cb[32];
  long nb = cols / block;
  for (long r = 0; r < rows; ++r) {
    for (long b = 0; b < nb; ++b) {
      const float* xb = xt + r * cols + b * block;
      scales[r * nb + b] = quant_block(format, block, rule, special4, xb, g, cb);
      for (int i = 0; i < block; i += 2) {
        long j = b * block + i;
        /* two codes per byte, the even element in the low nibble */
        codes[r * (cols / 2) + j / 2] = (uint8_t)(cb[i] | (cb[i + 1] << 4));
      }
    }
  }
  return 0;
}

int or_quantize(int format, int block, int rule, int gmode, const float* chan_scale,
                int hadamard, const float* special4, const void* x, int xdtype,
                long rows, long cols, long ld, uint8_t* codes, uint8_t* scales,
                float* g_inout) {
  if (check_format(format, block, rule, hadamard, cols)) return -1;
  if (format == OR_MXFP4 && gmode != OR_G_NONE) return -1;
  /* UE5M3's range needs no hierarchical scale ([Finer] claims): no AUTO */
  if (format == OR_UE5M3 && gmode == OR_G_AUTO) return -1;
  float* xt = (float*)malloc(sizeof(float) * (size_t)(rows > 0 ? rows : 1) * (size_t)cols);
  if (!xt) return -2;
  or_transform(x, xdtype, rows, cols, ld, chan_scale, hadamard, xt);
  float g = 1.0f;
  if (gmode == OR_G_AUTO) g = or_auto_global(xt, rows, cols, format);
  else if (gmode == OR_G_GIVEN) g = *g_inout;
  if (g_inout && gmode != OR_G_GIVEN) *g_inout = g;
  int rc = or_quantize_rows(format, block, rule, special4, xt, rows, cols, g, codes, scales);
  free(xt);
  return rc;
}

/* value of code c in a block whose scale byte is sb; returns value * scale,
 * exact in binary64 */
static double decode_elem(int format, const float* special4, int c, uint8_t sb) {
  switch (format) {
    case OR_NVFP4: return or_e2m1_value(c) * or_e4m3_value(sb & 0x7f);
    case OR_MXFP4: return or_e2m1_value(c) * or_e8m0_value(sb);
    case OR_UE5M3: return or_e2m1_value(c) * or_ue5m3_value(sb);
    case OR_RAZER_A: {
      double s = or_e4m3_value(sb & 0x7f);
      if (c == 8) return ((sb & 0x80) ? -5.0 : 5.0) * s;
      return or_e2m1_value(c) * s;
    }
    default: {
      double s = or_e3m3_value(sb & 0x3f);
      if (c == 8) return (double)special4[sb >> 6] * s;
      return or_e2m1_value(c) * s;
    }
  }
}

int or_decode_row(int format, int block, const float* special4, const uint8_t* codes_row,
                  const uint8_t* scales_row, long cols, double* out) {
  if (format < OR_NVFP4 || format > OR_UE5M3 || block <= 0 || cols % block) return -1;
  for (long j = 0; j < cols; ++j) {
    int c = (codes_row[j / 2] >> (4 * (j & 1))) & 15;
    out[j] = decode_elem(format, special4, c, scales_row[j / block]);
  }
  return 0;
}

int or_dequantize(int format, int block, const float* special4, const uint8_t* codes,
                  const uint8_t* scales, float g, long rows, long cols, float* out) {
  if (format < OR_NVFP4 || format > OR_UE5M3 || block <= 0 || cols % block) return -1;
  double* row = (double*)malloc(sizeof(double) * (size_t)cols);
  if (!row) return -2;
  for (long r = 0; r < rows; ++r) {
    or_decode_row(format, block, special4, codes + r * (cols / 2), scales + r * (cols / block), cols, row);
    for (long j = 0; j < cols; ++j) out[r * cols + j] = (float)(row[j] * (double)g);
  }
  free(row);
  return 0;
}

static int gemm_block(int f) { return f == OR_MXFP4 ? 32 : 16; }

static int gemm_check(int fa, int fw, long K) {
  if (fa < 0 || fa > 3 || fw < 0 || fw > 3) return -1;
  if ((fa == OR_MXFP4) != (fw == OR_MXFP4)) return -1;
  if (K <= 0 || K % gemm_block(fa)) return -1;
  return 0;
}

/* The W4A4 matmul consumes codes and scales as packed ([NVFP4-GDN] section 1,
 * [RaZeR] 2.3, [MACaQ] section 3): C[m][n] = g_a g_w sum_k A^[m][k] W^[n][k]. */
int or_gemm_rows(int fa, const uint8_t* a_codes, const uint8_t* a_scales, float g_a,
                 int fw, const uint8_t* w_codes, const uint8_t* w_scales, float g_w,
                 const float* w_special4, long M, long N, long K, long m0, long m1,
                 float* c) {
  if (gemm_check(fa, fw, K) || m0 < 0 || m1 > M || m0 > m1) return -1;
  int ba = gemm_block(fa), bw = gemm_block(fw);
  long rows = m1 - m0;
  double* ad = (double*)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) * (size_t)K);
  double* wd = (double*)malloc(sizeof(double) * (size_t)K);
  if (!ad || !wd) { free(ad); free(wd); return -2; }
  for (long i = 0; i < rows; ++i)
    or_decode_row(fa, ba, NULL, a_codes + (m0 + i) * (K / 2), a_scales + (m0 + i) * (K / ba), K, ad + i * K);
  float gg = g_a * g_w;
  for (long n = 0; n < N; ++n) {
    or_decode_row(fw, bw, w_special4, w_codes + n * (K / 2), w_scales + n * (K / bw), K, wd);
    for (long i = 0; i < rows; ++i) {
      const double* ar = ad + i * K;
      double acc = 0.0;
      for (long k = 0; k < K; ++k) acc += ar[k] * wd[k];
      c[i * N + n] = (float)((double)gg * acc);
    }
  }
  free(ad);
  free(wd);
  return 0;
}

int or_gemm_entries(int fa, const uint8_t* a_codes, const uint8_t* a_scales, float g_a,
                    int fw, const uint8_t* w_codes, const uint8_t* w_scales, float g_w,
                    const float* w_special4, long M, long N, long K, const long* ms,
                    const long* ns, long count, float* out) {
  if (gemm_check(fa, fw, K)) return -1;
  int ba = gemm_block(fa), bw = gemm_block(fw);
  double* ad = (double*)malloc(sizeof(double) * (size_t)K);
  double* wd = (double*)malloc(sizeof(double) * (size_t)K);
  if (!ad || !wd) { free(ad); free(wd); return -2; }
  float gg = g_a * g_w;
  for (long i = 0; i < count; ++i) {
    long m = ms[i], n = ns[i];
    if (m < 0 || m >= M || n < 0 || n >= N) { free(ad); free(wd); return -1; }
    or_decode_row(fa, ba, NULL, a_codes + m * (K / 2), a_scales + m * (K / ba), K, ad);
    or_decode_row(fw, bw, w_special4, w_codes + n * (K / 2), w_scales + n * (K / bw), K, wd);
    double acc = 0.0;
    for (long k = 0; k < K; ++k) acc += ad[k] * wd[k];
    out[i] = (float)((double)gg * acc);
  }
  free(ad);
  free(wd);
  return 0;
}

/* [MACaQ] section 3 "online scaling": t_j proportional to
 * (sigma_j^W / rms_j^x)^alpha.  Read with proportionality constant 1, rms over
 * the other dimension for both operands, and t_j = 1 where either rms is 0. */
void or_channel_scale(const void* x, int xdtype, long rows_x, long ldx,
                      const void* w, int wdtype, long rows_w, long ldw, long cols,
                      double alpha, float* t, float* r) {
  for (long j = 0; j < cols; ++j) {
    double sx = 0.0, sw = 0.0;
    for (long i = 0; i < rows_x; ++i) {
      double v = (double)load_elem(x, xdtype, i * ldx + j);
      sx += v * v;
    }
    for (long i = 0; i < rows_w; ++i) {
      double v = (double)load_elem(w, wdtype, i * ldw + j);
      sw += v * v;
    }
    double rx = sqrt(sx / (double)rows_x), rw = sqrt(sw / (double)rows_w);
    double tj = (rx == 0.0 || rw == 0.0) ? 1.0 : pow(rw / rx, alpha);
    t[j] = (float)tj;
    r[j] = 1.0f / t[j];
  }
}

/* ------------------------------------------------------------------------- */
/* RaZeR weight-only matmul and the offline special-value search              */
/* ------------------------------------------------------------------------- */

int or_gemm_w4a16_rows(const uint16_t* a, long lda, int fw, const uint8_t* w_codes,
                       const uint8_t* w_scales, float g_w, const float* w_special4,
                       long M, long N, long K, long m0, long m1, float* c) {
  if ((fw != OR_NVFP4 && fw != OR_RAZER_W) || K <= 0 || K % 16 || m0 < 0 || m1 > M || m0 > m1 || lda < K)
    return -1;
  double* wd = (double*)malloc(sizeof(double) * (size_t)K);
  if (!wd) return -2;
  for (long n = 0; n < N; ++n) {
    or_decode_row(fw, 16, w_special4, w_codes + n * (K / 2), w_scales + n * (K / 16), K, wd);
    for (long m = m0; m < m1; ++m) {
      double acc = 0.0;
      for (long k = 0; k < K; ++k) acc += (double)load_elem(a, OR_BF16, m * lda + k) * wd[k];
      c[(m - m0) * N + n] = (float)((double)g_w * acc);
    }
  }
  free(wd);
  return 0;
}

static const float RAZER_CAND[OR_RAZER_NCAND] = {2.5f, 3.5f, 4.5f, 5.0f, 5.5f, 6.5f, 7.0f, 7.5f};

void or_razer_pair(int p, float* a, float* b) {
  int q = 0;
  for (int i = 0; i < OR_RAZER_NCAND; ++i)
    for (int j = i + 1; j < OR_RAZER_NCAND; ++j, ++q)
      if (q == p) {
        *a = RAZER_CAND[i];
        *b = RAZER_CAND[j];
      }
}

int or_razer_table_search(const void* x, int xdtype, long rows, long cols, long ld, float g,
                          double* pair_sse) {
  if (rows < 0 || cols <= 0 || cols % 16 || ld < cols) return -1;
  float* xr = (float*)malloc(sizeof(float) * (size_t)cols);
  double* row_sum = (double*)malloc(sizeof(double) * OR_RAZER_NPAIRS);
  if (!xr || !row_sum) { free(xr); free(row_sum); return -2; }
  for (int p = 0; p < OR_RAZER_NPAIRS; ++p) pair_sse[p] = 0.0;
  for (long r = 0; r < rows; ++r) {
    for (long j = 0; j < cols; ++j) xr[j] = load_elem(x, xdtype, r * ld + j);
    for (int p = 0; p < OR_RAZER_NPAIRS; ++p) row_sum[p] = 0.0;
    for (long b = 0; b < cols / 16; ++b) {
      const float* xb = xr + 16 * b;
      /* the RaZeR-W block scale (abs-max E3M3) and the error of each signed
       * candidate as the block's special value */
      int k = or_round_scale(OR_SF_E3M3, block_absmax(xb, 16), 6.0, (double)g);
      double s = or_e3m3_value(k);
      float err[2 * OR_RAZER_NCAND];
      int codes[16];
      for (int c = 0; c < 2 * OR_RAZER_NCAND; ++c) {
        double v = (c & 1) ? -RAZER_CAND[c / 2] : RAZER_CAND[c / 2];
        if (k == 0) {
          for (int i = 0; i < 16; ++i) codes[i] = 0;
        } else {
          encode_special(xb, 16, s, (double)g, v, codes);
        }
        err[c] = or_block_sse(xb, codes, 16, s, g, 1, v);
      }
      int p = 0;
      for (int i = 0; i < OR_RAZER_NCAND; ++i)
        for (int j = i + 1; j < OR_RAZER_NCAND; ++j, ++p) {
          float m = err[2 * i];
          if (err[2 * i + 1] < m) m = err[2 * i + 1];
          if (err[2 * j] < m) m = err[2 * j];
          if (err[2 * j + 1] < m) m = err[2 * j + 1];
          row_sum[p] = row_sum[p] + (double)m;
        }
    }
    for (int p = 0; p < OR_RAZER_NPAIRS; ++p) pair_sse[p] = pair_sse[p] + row_sum[p];
  }
  int best = 0;
  for (int p = 1; p < OR_RAZER_NPAIRS; ++p)
    if (pair_sse[p] < pair_sse[best]) best = p;
  free(xr);
  free(row_sum);
  return best;
}

/* ------------------------------------------------------------------------- */
/* MACaQ weight calibration                                                   */
/* ------------------------------------------------------------------------- */

/* The 15 distinct E2M1 values in increasing order, with their codes; a code's
 * adjacent levels are its neighbours in this list ([MACaQ] section 1:
 * Flip-Refinement moves a code to the immediately adjacent E2M1 level). */
static const double LEVELS[15] = {-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6};
static const int LEVEL_CODE[15] = {15, 14, 13, 12, 11, 10, 9, 0, 1, 2, 3, 4, 5, 6, 7};

static int level_of(int code) {
  for (int i = 0; i < 15; ++i)
    if (LEVEL_CODE[i] == code || (code == 8 && i == 7)) return i;
  return 7;
}

/* Hessian-weighted error of one block: e_i = x_i - v_i 2^E (exact in
 * binary64), u_i = sum_j H[i][j] e_j with j ascending, then the balanced
 * pairwise tree (index order) of e_i u_i, every step a binary64 operation. */
static double block_hcost(const float* x, const int* codes, int E, const double* hbb, long ldh) {
  double e[32], p[32];
  for (int i = 0; i < 32; ++i) e[i] = (double)x[i] - or_e2m1_value(codes[i]) * ldexp(1.0, E);
  for (int i = 0; i < 32; ++i) {
    double u = 0.0;
    for (int j = 0; j < 32; ++j) u = u + hbb[i * ldh + j] * e[j];
    p[i] = e[i] * u;
  }
  for (int n = 32; n > 1; n /= 2)   /* balanced tree: T(0..n) = T(left) + T(right) */
    for (int i = 0; i < n / 2; ++i) p[i] = p[2 * i] + p[2 * i + 1];
  return p[0];
}

int or_macaq_quantize(const float* w, long N, long K, long ldw, const double* h, long ldh,
                      long max_moves, uint8_t* codes, uint8_t* scales, int* moves,
                      double* objective) {
  if (N < 0 || K <= 0 || K % 32 || ldw < K || ldh < K || max_moves < 0) return -1;
  int* cd = (int*)malloc(sizeof(int) * (size_t)K);
  int* ex = (int*)malloc(sizeof(int) * (size_t)(K / 32));
  double* d = (double*)malloc(sizeof(double) * (size_t)K);
  double* r = (double*)malloc(sizeof(double) * (size_t)K);
  if (!cd || !ex || !d || !r) { free(cd); free(ex); free(d); free(r); return -2; }
  for (long n = 0; n < N; ++n) {
    const float* x = w + n * ldw;
    /* 1. exponent screening, per block: candidates E, E+1, E-1 in that order,
     * the strictly smallest Hessian-weighted error kept */
    for (long b = 0; b < K / 32; ++b) {
      const float* xb = x + 32 * b;
      const double* hbb = h + (32 * b) * ldh + 32 * b;
      double a = block_absmax(xb, 32);
      int E = (a == 0.0) ? -127 : floor_log2(a) - 2;
      if (E < -127) E = -127;
      if (E > 127) E = 127;
      int best_c[32], tmp[32];
      encode_plain(xb, 32, ldexp(1.0, E), 1.0, best_c);
      double best = block_hcost(xb, best_c, E, hbb, ldh);
      int bestE = E;
      const int off[2] = {1, -1};
      for (int t = 0; t < 2; ++t) {
        int Ec = E + off[t];
        if (Ec < -127 || Ec > 127) continue;
        encode_plain(xb, 32, ldexp(1.0, Ec), 1.0, tmp);
        double c = block_hcost(xb, tmp, Ec, hbb, ldh);
        if (c < best) {
          best = c;
          bestE = Ec;
          memcpy(best_c, tmp, sizeof(best_c));
        }
      }
      ex[b] = bestE;
      for (int i = 0; i < 32; ++i) cd[32 * b + i] = best_c[i];
    }
    /* 2. Flip-Refinement on f = d^T H d, d = w^ - w: r = H d (j ascending);
     * a move of code k by one level changes w^_k by delta and f by
     * 2 delta r_k + delta^2 H_kk; its gain is the negative of that.  The
     * largest gain wins (k ascending, the move up before the move down, a
     * tie keeps the earlier); it is taken while it is positive. */
    for (long k = 0; k < K; ++k) d[k] = or_e2m1_value(cd[k]) * ldexp(1.0, ex[k / 32]) - (double)x[k];
    for (long k = 0; k < K; ++k) {
      double s = 0.0;
      for (long j = 0; j < K; ++j) s = s + h[k * ldh + j] * d[j];
      r[k] = s;
    }
    double f0 = 0.0;
    if (objective)
      for (long k = 0; k < K; ++k) f0 = f0 + d[k] * r[k];
    long taken = 0;
    while (taken < max_moves) {
      double best = 0.0;
      long bk = -1;
      double bdelta = 0.0;
      int blevel = 0;
      for (long k = 0; k < K; ++k) {
        const int lv = level_of(cd[k]);
        const double sc = ldexp(1.0, ex[k / 32]);
        for (int dir = 0; dir < 2; ++dir) {
          const int nl = dir == 0 ? lv + 1 : lv - 1;
          if (nl < 0 || nl > 14) continue;
          const double delta = (LEVELS[nl] - LEVELS[lv]) * sc;
          const double t1 = delta * r[k];
          const double t2 = delta * delta;
          const double q = 2.0 * t1 + t2 * h[k * ldh + k];
          const double gain = -q;
          if (gain > best) {
            best = gain;
            bk = k;
            bdelta = delta;
            blevel = nl;
          }
        }
      }
      if (bk < 0) break;   /* no move gains: the row leaves the active set */
      cd[bk] = LEVEL_CODE[blevel];
      for (long j = 0; j < K; ++j) r[j] = r[j] + bdelta * h[bk * ldh + j];
      ++taken;
    }
    if (moves) moves[n] = (int)taken;
    if (objective) {
      double f1 = 0.0;
      for (long k = 0; k < K; ++k) d[k] = or_e2m1_value(cd[k]) * ldexp(1.0, ex[k / 32]) - (double)x[k];
      for (long k = 0; k < K; ++k) {
        double s = 0.0;
        for (long j = 0; j < K; ++j) s = s + h[k * ldh + j] * d[j];
        f1 = f1 + d[k] * s;
      }
      objective[2 * n] = f0;
      objective[2 * n + 1] = f1;
    }
    for (long b = 0; b < K / 32; ++b) scales[n * (K / 32) + b] = (uint8_t)(ex[b] + 127);
    for (long k = 0; k < K; k += 2) codes[n * (K / 2) + k / 2] = (uint8_t)(cd[k] | (cd[k + 1] << 4));
  }
  free(cd);
  free(ex);
  free(d);
  free(r);
  return 0;
}
