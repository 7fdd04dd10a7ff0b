// Exact FP4 element and scale decisions shared by the quantizer and the
// matmul that quantizes its activations as it loads them.
//
// Every rounding decision is the exact real-arithmetic one.  A decision "is
// |x| past T" with T = m * s * g (m a midpoint of at most 5 significant bits,
// s a scale of at most 4, g an FP32) is reduced to one unsigned compare of
// FP32 bit patterns: |x| > T  <=>  |x| > RD32(T), and |x| >= T  <=>  |x| >=
// RU32(T); T is formed exactly in binary64.  Where the hardware converts are
// used, they are bracketed (multipliers 1 -/+ 2^-20 around a reciprocal within
// one ulp) and an element whose two bracketed codes differ is settled by the
// exact midpoint test.  A tie goes to the even neighbour.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_internal.hpp"

namespace fp4q {
namespace {

__device__ __forceinline__ uint32_t fbits(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __uint_as_float(u); }

// value of lane ^ D within a quad (D = 1, 2) through a DPP quad permutation;
// other distances through the LDS crossbar
template <int D>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (D == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // [1,0,3,2]
  else if constexpr (D == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // [2,3,0,1]
  else return (uint32_t)__shfl_xor((int)v, D);
}
__device__ __forceinline__ float lane_xor_f(float v, int d) {
  if (d == 1) return bitsf(lane_xor<1>(fbits(v)));
  if (d == 2) return bitsf(lane_xor<2>(fbits(v)));
  return __shfl_xor(v, d);
}

// strict-greater threshold bits for "round up past T" decisions:
// tie_up = false:  |x| > T  <=>  bits(|x|) > bits(RD32(T))
// tie_up = true :  |x| >= T <=>  bits(|x|) > bits(RU32(T)) - 1
__device__ __forceinline__ uint32_t thr_bits(double T, bool tie_up) {
  float f = (float)T;  // nearest
  uint32_t b = fbits(f);
  if (!tie_up) {
    if ((double)f > T) b -= 1;  // RD
    return b;
  }
  if ((double)f < T) b += 1;    // RU
  return b - 1;
}
// |x| < T  <=>  bits(|x|) < bits(RU32(T))
__device__ __forceinline__ uint32_t ru_bits(double T) {
  float f = (float)T;
  uint32_t b = fbits(f);
  if ((double)f < T) b += 1;
  return b;
}

// scale-format values (binary64, exact)
template <int SF>  // 0: E4M3 (codes 0..126), 1: E3M3 (codes 0..63), 2: UE5M3 (codes 0..255)
__device__ __forceinline__ double sf_val(int k) {
  int e = k >> 3, m = k & 7;
  if (SF == 0) return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  if (SF == 1) return e == 0 ? ldexp((double)m, -5) : ldexp((double)(8 + m), e - 6);
  return e == 0 ? ldexp((double)m, -17) : ldexp((double)(8 + m), e - 18);
}
template <int SF>
constexpr int sf_kmax() { return SF == 0 ? 126 : SF == 1 ? 63 : 255; }

// E2M1 magnitudes and the midpoints between neighbours
// (compile-time arrays, indexed with constants only: literals, no memory loads)
constexpr float kMid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
constexpr double kMidD[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
constexpr float kMag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};

template <int FMT> struct FmtTraits;
template <> struct FmtTraits<NVFP4>   { static constexpr int SF = 0, KMAX = 126, NSP = 0; };
template <> struct FmtTraits<RAZER_A> { static constexpr int SF = 0; };
template <> struct FmtTraits<RAZER_W> { static constexpr int SF = 1, KMAX = 63,  NSP = 4; };
template <> struct FmtTraits<UE5M3>   { static constexpr int SF = 2, KMAX = 255, NSP = 0; };

// LDS tables, built once per workgroup for the launch's global scale g
template <int FMT>
struct Tables {
  static constexpr int KN = FmtTraits<FMT>::KMAX + 1;
  static constexpr int NSP = FmtTraits<FMT>::NSP > 0 ? FmtTraits<FMT>::NSP : 1;
  uint32_t elt[KN][8];        // per scale code: 7 element thresholds (strict >)
  uint32_t smid6[KN];         // scale midpoints for T = 6 (strict >), last unused
  uint32_t smid4[KN];         // scale midpoints for T = 4
  uint32_t sp_lo[KN][NSP];    // special interval, strict >
  uint32_t sp_hi[KN][NSP];    // special interval, strict <
  float spv[NSP];             // special values
};
template <> struct Tables<MXFP4> { uint32_t dummy; };  // kernels without tables

// Nearest standard E2M1 magnitudes below/above |v| (|v| in (2, 7.5], not on the grid)
__device__ __forceinline__ void special_bounds(float av, float& lo, float& hi, bool& open_hi) {
  float below = 0.f, above = 0.f;
  open_hi = true;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (kMag[m] < av) below = kMag[m];
    if (kMag[m] > av && open_hi) { above = kMag[m]; open_hi = false; }
  }
  lo = 0.5f * (below + av);
  hi = 0.5f * (above + av);
}

template <int FMT>
__device__ void build_tables(Tables<FMT>& T, float g, const float* special) {
  if constexpr (FMT != MXFP4) {
    constexpr int SF = FmtTraits<FMT>::SF;
    constexpr int KN = Tables<FMT>::KN;
    constexpr int NSP = FmtTraits<FMT>::NSP;
    const double gd = (double)g;
    for (int k = threadIdx.x; k < KN; k += blockDim.x) {
      const double sg = sf_val<SF>(k) * gd;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t v = 0x7F800000u;  // never passed by a finite |x|
        if (k > 0 && j < 7) v = thr_bits(kMidD[j] * sg, (j & 1) != 0);
        T.elt[k][j] = v;
      }
    }
    for (int i = threadIdx.x; i < 2 * KN; i += blockDim.x) {
      int k = i % KN, which = i / KN;
      uint32_t v = 0xFFFFFFFFu;
      if (k < KN - 1) {
        double mid = 0.5 * (sf_val<SF>(k) + sf_val<SF>(k + 1));
        v = thr_bits(mid * (which ? 4.0 : 6.0) * gd, (k & 1) != 0);  // tie -> even code
      }
      if (which) T.smid4[k] = v; else T.smid6[k] = v;
    }
    if constexpr (NSP > 0) {
      for (int i = threadIdx.x; i < KN * NSP; i += blockDim.x) {
        int k = i / NSP, p = i % NSP;
        float v = (FMT == RAZER_A) ? (p == 0 ? 5.0f : -5.0f) : special[p];
        float lo, hi; bool open_hi;
        special_bounds(fabsf(v), lo, hi, open_hi);
        double s = sf_val<SF>(k) * gd;
        T.sp_lo[k][p] = (k == 0) ? 0x7F800000u : thr_bits((double)lo * s, false);
        T.sp_hi[k][p] = (k == 0 || open_hi) ? 0x7F800000u : ru_bits((double)hi * s);
        if (k == 0) T.spv[p] = v;
      }
    }
  }
}

// scale code guess for a/(T g) in binary64, off by at most one
template <int SF>
__device__ __forceinline__ int select_scale_guess(float a, double inv_Tg) {
  constexpr int KMAX = sf_kmax<SF>();
  // largest value, smallest normal, subnormal quantum (as a power of two), bias
  constexpr double MAXV = SF == 0 ? 448.0 : SF == 1 ? 30.0 : 122880.0;
  constexpr double MINN = SF == 0 ? 0.015625 : SF == 1 ? 0.25 : 0x1p-14;
  constexpr double SUBQ = SF == 0 ? 512.0 : SF == 1 ? 32.0 : 131072.0;
  constexpr int BIAS = SF == 0 ? 7 : SF == 1 ? 3 : 15;
  double y = (double)a * inv_Tg;
  int k;
  if (!(y < MAXV)) k = KMAX;
  else if (y < MINN) k = (int)(y * SUBQ);
  else {
    uint64_t b = (uint64_t)__double_as_longlong(y);
    int e = (int)((b >> 52) & 0x7FF) - 1023;
    k = ((e + BIAS) << 3) | (int)((b >> 49) & 7);
  }
  return k;
}

// nearest scale code to a/(T g) from the midpoint table
template <int SF>
__device__ __forceinline__ int select_scale(float a, const uint32_t* smid, double inv_Tg) {
  constexpr int KMAX = sf_kmax<SF>();
  int k = select_scale_guess<SF>(a, inv_Tg);
  uint32_t ab = fbits(a);
  if (k < KMAX && ab > smid[k]) ++k;
  else if (k > 0 && ab <= smid[k - 1]) --k;
  return k;
}

// E2M1 magnitude index of |x| (bits xb) against 7 non-decreasing thresholds
__device__ __forceinline__ int rtn_mag(uint32_t xb, const uint32_t t[7]) {
  bool c2 = xb > t[3];
  uint32_t s1 = c2 ? t[5] : t[1];
  bool c1 = xb > s1;
  uint32_t s0 = c2 ? (c1 ? t[6] : t[4]) : (c1 ? t[2] : t[0]);
  bool c0 = xb > s0;
  return (c2 ? 4 : 0) | (c1 ? 2 : 0) | (c0 ? 1 : 0);
}

// the same decision against thresholds held in scalars: a kernel whose
// threshold array would be indexed through selected addresses gets the array
// placed in LDS, and that alone costs its launches about 12 us here
__device__ __forceinline__ int rtn_mag_v(uint32_t xb, uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3,
                                         uint32_t t4, uint32_t t5, uint32_t t6) {
  const bool c2 = xb > t3;
  const bool c1 = xb > (c2 ? t5 : t1);
  const bool c0 = xb > (c2 ? (c1 ? t6 : t4) : (c1 ? t2 : t0));
  return (c2 ? 4 : 0) | (c1 ? 2 : 0) | (c0 ? 1 : 0);
}

template <int L>
struct Chunk {
  float x[L];
};

template <int L>
__device__ __forceinline__ float tree_sum(const float* p) {
  if constexpr (L == 4) return (p[0] + p[1]) + (p[2] + p[3]);
  else return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

// encode L elements with thresholds t; returns packed nibbles
template <int L>
__device__ __forceinline__ uint32_t encode_plain(const float* x, const uint32_t t[7]) {
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    uint32_t b = fbits(x[i]);
    int m = rtn_mag(b & 0x7FFFFFFFu, t);
    uint32_t c = m ? ((uint32_t)m | ((b >> 28) & 8u)) : 0u;
    packed |= c << (4 * i);
  }
  return packed;
}

template <int L>
__device__ __forceinline__ uint32_t encode_plain_v(const float* x, uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3,
                                                   uint32_t t4, uint32_t t5, uint32_t t6) {
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const uint32_t b = fbits(x[i]);
    const int m = rtn_mag_v(b & 0x7FFFFFFFu, t0, t1, t2, t3, t4, t5, t6);
    const uint32_t c = m ? ((uint32_t)m | ((b >> 28) & 8u)) : 0u;
    packed |= c << (4 * i);
  }
  return packed;
}

// RaZeR: standard code unless |x| lies strictly inside the special interval
// with the special value's sign, then 0x8
template <int L>
__device__ __forceinline__ uint32_t encode_special(const float* x, const uint32_t t[7], uint32_t lo,
                                                   uint32_t hi, uint32_t vsign) {
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    uint32_t b = fbits(x[i]);
    uint32_t xb = b & 0x7FFFFFFFu;
    int m = rtn_mag(xb, t);
    uint32_t c = m ? ((uint32_t)m | ((b >> 28) & 8u)) : 0u;
    bool sp = ((b & 0x80000000u) == vsign) && xb > lo && xb < hi;
    packed |= (sp ? 8u : c) << (4 * i);
  }
  return packed;
}

// E4M3 scale code (0..126) -> its value as FP32: the hardware FP8 decode
// (OCP E4M3, exact) with unit scale
__device__ __forceinline__ float e4m3_f32(int k) { return __builtin_amdgcn_cvt_scalef32_f32_fp8(k, 1.0f, 0); }
// UE5M3 scale code (0..255) -> its value as FP32 (exact: every value is a
// normal FP32 number)
__device__ __forceinline__ float ue5m3_f32(int k) {
  const int e = k >> 3, m = k & 7;
  return e == 0 ? (float)m * 0x1p-17f : bitsf((uint32_t)(e + 112) << 23 | (uint32_t)m << 20);
}
template <int SF>
__device__ __forceinline__ float sf_f32(int k) { return SF == 0 ? e4m3_f32(k) : ue5m3_f32(k); }

// codes whose magnitude rounded to 0 carry the sign of x in the hardware
// convert (code 0x8); the format writes them as 0
__device__ __forceinline__ uint32_t clear_neg_zero(uint32_t packed) {
  const uint32_t nz = ((packed & 0x77777777u) + 0x77777777u) & 0x88888888u;  // bit 3: magnitude != 0
  return packed & ~(packed & 0x88888888u & ~nz);
}

template <int LPB>
__device__ __forceinline__ bool group_all(bool v) {
  uint32_t b = v ? 1u : 0u;
  if constexpr (LPB >= 2) b &= lane_xor<1>(b);
  if constexpr (LPB >= 4) b &= lane_xor<2>(b);
  return b != 0;
}

// true on every lane when `pred` holds on all lanes of the wave (all lanes
// are active here): the exact paths below are taken per wave, uniformly
__device__ __forceinline__ bool wave_all(bool pred) { return __builtin_amdgcn_ballot_w64(!pred) == 0; }

// E2M1 magnitude index of |x| (bits xb) as the number of thresholds passed
// (the thresholds are non-decreasing); no indexing into t
__device__ __forceinline__ int rtn_count(uint32_t xb, const uint32_t t[7]) {
  int m = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) m += xb > t[j] ? 1 : 0;
  return m;
}

// element thresholds of scale code k (format SF) under g, formed in binary64
// (the same values the LDS tables hold)
template <int SF>
__device__ __forceinline__ void nv_thresholds(int k, double gd, uint32_t t[7]) {
  const double sv = sf_val<SF>(k) * gd;
#pragma unroll
  for (int j = 0; j < 7; ++j) t[j] = k > 0 ? thr_bits((double)kMidD[j] * sv, (j & 1) != 0) : 0x7F800000u;
}

// nearest code of scale format SF to a / (T g) (T = 6 or 4), ties to the
// even code, saturating at the largest: binary64 guess corrected by the exact
// scale midpoints
template <int SF>
__device__ __forceinline__ int select_sf_exact(float a, double inv_Tg, double Tg) {
  constexpr int KMAX = sf_kmax<SF>();
  int k = select_scale_guess<SF>(a, inv_Tg);
  const uint32_t ab = fbits(a);
  auto mid = [&](int j) { return thr_bits(0.5 * (sf_val<SF>(j) + sf_val<SF>(j + 1)) * Tg, (j & 1) != 0); };
  if (k < KMAX && ab > mid(k)) ++k;
  else if (k > 0 && ab <= mid(k - 1)) --k;
  return k;
}
__device__ __forceinline__ int select_e4m3_exact(float a, double inv_Tg, double Tg) {
  return select_sf_exact<0>(a, inv_Tg, Tg);
}

// Exact side of a rounding midpoint.  The midpoint threshold is T = Q g
// with Q = (midpoint value) * (scale value) exact in FP32 (at most 8
// significant bits).  Split T = Phi + Plo exactly (Phi = RN(Q g), Plo the
// FMA residual); near T, |x| - Phi is exact (the operands are within a
// factor of two), so comparing it with Plo is the exact comparison of |x|
// with T, equality included.  `odd`: a tie rounds up (to the even neighbour).
__device__ __forceinline__ bool past_midpoint(float ax, float Q, float g, bool odd) {
  const float phi = Q * g;
  const float plo = __builtin_fmaf(Q, g, -phi);
  const float r1 = ax - phi;
  return r1 > plo || (r1 == plo && odd);
}

// MXFP4 codes by the exact threshold search (a wave with a non-finite block,
// or a shared exponent below the normal range): thresholds 2^E times the E2M1
// midpoints (exact), as bit patterns, strict > for the even ones and >= (one
// below) for the odd ones (ties to even).  Out of line for the same reason as
// the NVFP4 search below.
template <int L>
__device__ __attribute__((noinline)) uint32_t encode_mx_thresholds(float __attribute__((ext_vector_type(L))) xv,
                                                                   int E) {
  float x[L];
#pragma unroll
  for (int i = 0; i < L; ++i) x[i] = xv[i];
  const uint32_t t0 = fbits(ldexpf(kMid[0], E)), t1 = fbits(ldexpf(kMid[1], E)) - 1u;
  const uint32_t t2 = fbits(ldexpf(kMid[2], E)), t3 = fbits(ldexpf(kMid[3], E)) - 1u;
  const uint32_t t4 = fbits(ldexpf(kMid[4], E)), t5 = fbits(ldexpf(kMid[5], E)) - 1u;
  const uint32_t t6 = fbits(ldexpf(kMid[6], E));
  return encode_plain_v<L>(x, t0, t1, t2, t3, t4, t5, t6);
}

// NVFP4 codes by the exact threshold search (a wave with a non-finite block,
// or s g near the ends of the FP32 range).  Kept out of line: inlined, its
// 7 x L comparison masks claim the scalar registers of the whole kernel.
template <int L, int SF = 0>
__device__ __attribute__((noinline)) uint32_t encode_nv_thresholds(float __attribute__((ext_vector_type(L))) x, int k,
                                                                   float g) {
  uint32_t t[7];
  nv_thresholds<SF>(k, (double)g, t);
  uint32_t plo = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const uint32_t b = fbits(x[i]);
    const int m = rtn_count(b & 0x7FFFFFFFu, t);
    plo |= (m ? ((uint32_t)m | ((b >> 28) & 8u)) : 0u) << (4 * i);
  }
  return plo;
}

// Elements whose codes at x * rlo and x * rhi differ sit on or near a
// rounding midpoint.  Each one's exact code is its low-side code or one
// magnitude step above (the bracket is far narrower than the gap between
// midpoints); the exact midpoint test decides.  One element per lane per pass,
// in a wave-uniform loop that almost always runs once.  Out of line, with the
// elements by value: inlined, the selection of the element by its index makes
// the compiler keep the caller's element array in LDS.
template <int L>
__device__ __attribute__((noinline)) uint32_t resolve_ambiguous(float __attribute__((ext_vector_type(L))) x,
                                                                uint32_t plo, uint32_t phi, float s, float g) {
  uint32_t amb = plo ^ phi;
  while (!wave_all(amb == 0)) {
    const int sh = amb ? (int)(__builtin_ctz(amb) & ~3) : 0;  // 4 * element index
    float xi = x[0];
#pragma unroll
    for (int j = 1; j < L; ++j) xi = (sh == 4 * j) ? x[j] : xi;
    const uint32_t mag = (plo >> sh) & 7u;
    typedef float f2v __attribute__((ext_vector_type(2)));
    const f2v v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(mag | ((mag + 1u) << 4), 0.5f, 0);
    const bool go = amb != 0 && mag != 7u && past_midpoint(fabsf(xi), (v[0] + v[1]) * s, g, (mag & 1u) != 0);
    plo += go ? (1u << sh) : 0u;  // magnitude + 1 (at most 7: no carry)
    amb &= ~(0xFu << sh);
  }
  return plo;
}

// Bracketed hardware encode.  The gfx950 FP4 convert rounds to nearest even
// (saturating) after dividing by the power-of-two part of its scale, which is
// 1 here.  Each element is converted at x * rlo and x * rhi, where
// rlo < 1/(s g) < rhi with a relative margin far above the rounding errors of
// forming them and of the product, so the exact ratio |x| / (s g) lies
// strictly between the two converted values.  Rounding is monotone: equal
// codes at both ends are the exact decision.
//
// NVFP4 codes of a lane's L elements for scale code k (value s) under global
// g: the bracketed convert; when some element of the wave cannot be decided
// that way, the whole wave resolves its ambiguous elements exactly.  The
// bracket is used only for finite blocks with s g well inside the normal
// range; a wave with any other block takes the threshold search.
template <int L, int LPB, int SF = 0>
__device__ __forceinline__ uint32_t encode_nv(const float* x, int k, float s, float g, bool finite) {
  const float sg = s * g;
  const float r = __builtin_amdgcn_rcpf(sg);  // within 1 ulp of 1 / RN(s g)
  const bool ok = finite && sg > 0x1p-120f && sg < 0x1p120f;
  const float rlo = r * (1.0f - 0x1p-20f), rhi = r * (1.0f + 0x1p-20f);
  uint32_t plo = 0, phi = 0;
  static_for<0, L / 2>([&](auto ic) {
    constexpr int b = decltype(ic)::value;
    plo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(plo, x[2 * b] * rlo, x[2 * b + 1] * rlo, 1.0f, b);
    phi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(phi, x[2 * b] * rhi, x[2 * b + 1] * rhi, 1.0f, b);
  });
  if (!wave_all(ok && plo == phi)) {
    typedef float fLv __attribute__((ext_vector_type(L)));
    fLv xv;
#pragma unroll
    for (int i = 0; i < L; ++i) xv[i] = x[i];
    if (wave_all(ok)) plo = resolve_ambiguous<L>(xv, plo, phi, s, g);
    else return encode_nv_thresholds<L, SF>(xv, k, g);
  }
  return clear_neg_zero(plo);
}

// nearest E4M3 code to a / (T g) (T = 6 or 4), ties to the even code,
// saturating at 126: the hardware convert of a * lo (lo < 1/(T g)) gives the
// exact code or one below; step up where a is past the midpoint
__device__ __forceinline__ int e4m3_from_low(uint32_t wl_byte, float a, float T, float g) {
  const int klo = min((int)wl_byte, 126);
  if (klo == 126) return 126;
  typedef float f2v __attribute__((ext_vector_type(2)));
  const f2v v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)klo | ((uint32_t)(klo + 1) << 8), 0.5f, false);
  const float mid = v[0] + v[1];  // exact: at most 5 significant bits
  return past_midpoint(a, mid * T, g, (klo & 1) != 0) ? klo + 1 : klo;
}

// block error of a lane's L elements (lane part of the balanced tree);
// value of a code via the hardware FP4 -> FP32 convert (scale 1.0 is exact)
template <int L>
__device__ __forceinline__ float lane_sse(const float* x, uint32_t packed, float s, float g,
                                          bool has_sp, float vs) {
  float p[L];
  static_for<0, L / 2>([&](auto ic) {
    constexpr int b = decltype(ic)::value;  // byte b holds elements 2b, 2b+1
    auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, b);
    float q0 = v2[0] * s, q1 = v2[1] * s;
    if (has_sp) {
      if (((packed >> (8 * b)) & 15u) == 8u) q0 = vs;
      if (((packed >> (8 * b + 4)) & 15u) == 8u) q1 = vs;
    }
    float e0 = __builtin_fmaf(-q0, g, x[2 * b]);
    float e1 = __builtin_fmaf(-q1, g, x[2 * b + 1]);
    p[2 * b] = e0 * e0;
    p[2 * b + 1] = e1 * e1;
  });
  return tree_sum<L>(p);
}

template <int LPB>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPB >= 2) v = v + bitsf(lane_xor<1>(fbits(v)));
  if constexpr (LPB >= 4) v = v + bitsf(lane_xor<2>(fbits(v)));
  static_assert(LPB <= 4, "blocks span at most 4 lanes");
  return v;
}
template <int LPB>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  if constexpr (LPB >= 2) v = max(v, lane_xor<1>(v));
  if constexpr (LPB >= 4) v = max(v, lane_xor<2>(v));
  return v;
}

// codes of 16 elements as two words (elements 0-7, 8-15), -0 not yet cleared
template <int LPB, int SF = 0>
__device__ __forceinline__ uint2 encode_nv16(const float* x, int k, float s, float g, bool finite) {
  const float sg = s * g;
  const float r = __builtin_amdgcn_rcpf(sg);  // within 1 ulp of 1 / RN(s g)
  const bool ok = finite && sg > 0x1p-120f && sg < 0x1p120f;
  const float rlo = r * (1.0f - 0x1p-20f), rhi = r * (1.0f + 0x1p-20f);
  uint32_t l0 = 0, l1 = 0, h0 = 0, h1 = 0;
  static_for<0, 4>([&](auto ic) {
    constexpr int b = decltype(ic)::value;
    l0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(l0, x[2 * b] * rlo, x[2 * b + 1] * rlo, 1.0f, b);
    h0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h0, x[2 * b] * rhi, x[2 * b + 1] * rhi, 1.0f, b);
    l1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(l1, x[8 + 2 * b] * rlo, x[9 + 2 * b] * rlo, 1.0f, b);
    h1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h1, x[8 + 2 * b] * rhi, x[9 + 2 * b] * rhi, 1.0f, b);
  });
  if (!wave_all(ok && l0 == h0 && l1 == h1)) {
    typedef float f8v __attribute__((ext_vector_type(8)));
    f8v xa, xb;
#pragma unroll
    for (int i = 0; i < 8; ++i) { xa[i] = x[i]; xb[i] = x[8 + i]; }
    if (wave_all(ok)) {
      l0 = resolve_ambiguous<8>(xa, l0, h0, s, g);
      l1 = resolve_ambiguous<8>(xb, l1, h1, s, g);
    } else {
      l0 = encode_nv_thresholds<8, SF>(xa, k, g);
      l1 = encode_nv_thresholds<8, SF>(xb, k, g);
    }
  }
  return make_uint2(l0, l1);
}

// block error of a lane's 16 elements: the balanced tree of the two halves
__device__ __forceinline__ float lane_sse16(const float* x, uint2 c, float s, float g) {
  return lane_sse<8>(x, c.x, s, g, false, 0.f) + lane_sse<8>(x + 8, c.y, s, g, false, 0.f);
}

}  // namespace
}  // namespace fp4q
