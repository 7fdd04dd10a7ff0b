// Block-scaled FP4 quantization, dequantization, global amax and channel
// scale kernels for gfx950.
//
// Pages: scale rules -- "Finer is Better (with the Right Scaling)", Method 2
// (abs-max, prevent-zero, 4-over-6, brute-force, hierarchical); RaZeR picks --
// RaZeR summary, sections 2.1 and 2.2; MXFP4 and the online transforms --
// MACaQ review, sections 1 and 3.
//
// Exactness.  Every rounding decision is the exact real-arithmetic one.  A
// decision "is |x| past T" with T = m * s * g (m a midpoint of at most 5
// significant bits, s a scale of at most 4, g an FP32) is reduced to one
// unsigned compare of FP32 bit patterns: |x| > T  <=>  |x| > RD32(T), and
// |x| >= T  <=>  |x| >= RU32(T).  T is formed exactly in binary64 and rounded
// down or up to FP32 once per workgroup, into LDS tables indexed by the scale
// code.  A tie goes to the even neighbour, so each threshold is stored as the
// strict-greater form of either RD (tie stays low) or RU (tie goes up).
//
// Work mapping.  One lane owns L = 8 consecutive elements of a row (L = 4 for
// blocks of 4): one 128-bit load of bf16 (two of fp32).  A block of B >= L
// elements spans B/L adjacent lanes; block maxima and error sums cross lanes
// with xor shuffles, which reproduces the balanced pairwise error tree
// (each lane sums its L elements as a balanced tree first).
#include "fp4q_internal.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

namespace {

constexpr int kThreads = 256;

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
template <int SF>  // 0: E4M3 (codes 0..126), 1: E3M3 (codes 0..63)
__device__ __forceinline__ double sf_val(int k) {
  int e = k >> 3, m = k & 7;
  if (SF == 0) return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return e == 0 ? ldexp((double)m, -5) : ldexp((double)(8 + m), e - 6);
}

// E2M1 magnitudes and the midpoints between neighbours
// (compile-time arrays, indexed with constants only: literals, no memory loads)
constexpr float kMid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
constexpr double kMidD[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
constexpr float kMag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};

template <int FMT> struct FmtTraits;
template <> struct FmtTraits<NVFP4>   { static constexpr int SF = 0, KMAX = 126, NSP = 0; };
template <> struct FmtTraits<RAZER_A> { static constexpr int SF = 0; };
template <> struct FmtTraits<RAZER_W> { static constexpr int SF = 1, KMAX = 63,  NSP = 4; };
template <> struct FmtTraits<MXFP4>   { static constexpr int SF = 2; };

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
template <> struct Tables<MXFP4> { uint32_t dummy; };

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
  constexpr int KMAX = SF == 0 ? 126 : 63;
  double y = (double)a * inv_Tg;
  int k;
  if (SF == 0) {
    if (!(y < 448.0)) k = KMAX;
    else if (y < 0.015625) k = (int)(y * 512.0);
    else {
      uint64_t b = (uint64_t)__double_as_longlong(y);
      int e = (int)((b >> 52) & 0x7FF) - 1023;
      k = ((e + 7) << 3) | (int)((b >> 49) & 7);
    }
  } else {
    if (!(y < 30.0)) k = KMAX;
    else if (y < 0.25) k = (int)(y * 32.0);
    else {
      uint64_t b = (uint64_t)__double_as_longlong(y);
      int e = (int)((b >> 52) & 0x7FF) - 1023;
      k = ((e + 3) << 3) | (int)((b >> 49) & 7);
    }
  }
  return k;
}

// nearest scale code to a/(T g) from the midpoint table
template <int SF>
__device__ __forceinline__ int select_scale(float a, const uint32_t* smid, double inv_Tg) {
  constexpr int KMAX = SF == 0 ? 126 : 63;
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

// the raw input words of one chunk (L bf16 or L fp32 values)
template <int L, bool BF16>
struct Raw {
  static constexpr int W = BF16 ? L / 2 : L;  // 32-bit words
  uint32_t w[W];
  float t[L];  // the chunk's channel scales, when loaded with the chunk
};

// buffer view of the channel scales; with none, a view of no bytes, whose
// reads return zeros without touching memory
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chan_view(const QuantParams& p) {
  const bool on = p.chan_scale != nullptr;
  return __builtin_amdgcn_make_buffer_rsrc((void*)p.chan_scale, (short)0, on ? (int)(p.cols * 4) : 0,
                                           (int)0x00020000);
}

// the chunk's channel scales, issued with the chunk's load so that one wait
// covers both
template <int L, bool BF16>
__device__ __forceinline__ void load_t(__amdgpu_buffer_rsrc_t tv, int64_t j0, Raw<L, BF16>& raw) {
#pragma unroll
  for (int i = 0; i < L; i += 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(tv, (int)((j0 + i) * 4), 0, 0);
    raw.t[i] = bitsf(v[0]); raw.t[i + 1] = bitsf(v[1]); raw.t[i + 2] = bitsf(v[2]); raw.t[i + 3] = bitsf(v[3]);
  }
}

template <int L, bool BF16>
__device__ __forceinline__ void load_raw(const QuantParams& p, int64_t r, int64_t j0, Raw<L, BF16>& raw) {
  if constexpr (BF16) {
    const uint16_t* src = (const uint16_t*)p.x + r * p.ld + j0;
    if constexpr (L == 8) {
      const uint4 v = *(const uint4*)src;
      raw.w[0] = v.x; raw.w[1] = v.y; raw.w[2] = v.z; raw.w[3] = v.w;
    } else {
      const uint2 v = *(const uint2*)src;
      raw.w[0] = v.x; raw.w[1] = v.y;
    }
  } else {
    const float* src = (const float*)p.x + r * p.ld + j0;
#pragma unroll
    for (int i = 0; i < L; i += 4) {
      const uint4 v = *(const uint4*)(src + i);
      raw.w[i] = v.x; raw.w[i + 1] = v.y; raw.w[i + 2] = v.z; raw.w[i + 3] = v.w;
    }
  }
}

// widen a raw chunk, apply the channel scale and the size-32 block-Hadamard
// (lanes of a 32-group are adjacent)
template <int L, bool BF16, bool PRE_T = false>
__device__ __forceinline__ void finish_chunk(const QuantParams& p, int64_t j0, const Raw<L, BF16>& raw, float* x,
                                             bool chan, bool had) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < L / 2; ++i) {
      x[2 * i] = bitsf(raw.w[i] << 16);
      x[2 * i + 1] = bitsf(raw.w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < L; ++i) x[i] = bitsf(raw.w[i]);
  }
  if (chan) {
    if constexpr (PRE_T) {
#pragma unroll
      for (int i = 0; i < L; ++i) x[i] = x[i] * raw.t[i];
    } else {
#pragma unroll
      for (int i = 0; i < L; i += 4) {
        float4 t = *(const float4*)(p.chan_scale + j0 + i);
        x[i] = x[i] * t.x; x[i + 1] = x[i + 1] * t.y; x[i + 2] = x[i + 2] * t.z; x[i + 3] = x[i + 3] * t.w;
      }
    }
  }
  if (had) {
    // in-lane stages h < L
#pragma unroll
    for (int h = 1; h < L; h *= 2) {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        if ((i & h) == 0) {
          float u = x[i], w = x[i + h];
          x[i] = u + w;
          x[i + h] = u - w;
        }
      }
    }
    // cross-lane stages h = L .. 16 with partner lane ^ (h / L)
    // butterfly with the partner lane: the lower lane keeps x + o, the upper
    // o - x, written as o + (+-x) (the same IEEE operations)
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 32 / L; d *= 2) {
      const uint32_t neg = (lane & d) ? 0x80000000u : 0u;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const float o = lane_xor_f(x[i], d);
        x[i] = o + bitsf(fbits(x[i]) ^ neg);
      }
    }
    const float c = bitsf(0x3E3504F3u);  // RN32(2^-2.5)
#pragma unroll
    for (int i = 0; i < L; ++i) x[i] = x[i] * c;
  }
}

template <int L, bool BF16>
__device__ __forceinline__ void load_chunk(const QuantParams& p, int64_t r, int64_t j0, float* x,
                                           bool chan, bool had) {
  Raw<L, BF16> raw;
  load_raw<L, BF16>(p, r, j0, raw);
  finish_chunk<L, BF16>(p, j0, raw, x, chan, had);
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

// codes whose magnitude rounded to 0 carry the sign of x in the hardware
// convert (code 0x8); the format writes them as 0
__device__ __forceinline__ uint32_t clear_neg_zero(uint32_t packed) {
  const uint32_t nz = ((packed & 0x77777777u) + 0x77777777u) & 0x88888888u;  // bit 3: magnitude != 0
  return packed & ~(packed & 0x88888888u & ~nz);
}

// Bracketed hardware encode.  The gfx950 FP4 convert rounds to nearest even
// (saturating) after dividing by the power-of-two part of its scale, which is
// 1 here.  Each element is converted at x * rlo and x * rhi, where
// rlo < 1/(s g) < rhi with a relative margin far above the rounding errors of
// forming them and of the product, so the exact ratio |x| / (s g) lies
// strictly between the two converted values.  Rounding is monotone: equal
// codes at both ends are the exact decision.  `ok` is false when some element
// may sit on or near a rounding midpoint; that block then takes the threshold
// path.
template <int L>
__device__ __forceinline__ uint32_t encode_bracket(const float* x, float rlo, float rhi, bool& ok) {
  uint32_t plo = 0, phi = 0;
  static_for<0, L / 2>([&](auto ic) {
    constexpr int b = decltype(ic)::value;
    plo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(plo, x[2 * b] * rlo, x[2 * b + 1] * rlo, 1.0f, b);
    phi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(phi, x[2 * b] * rhi, x[2 * b + 1] * rhi, 1.0f, b);
  });
  ok = plo == phi;
  return clear_neg_zero(plo);
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

// element thresholds of E4M3 scale code k under g, formed in binary64 (the
// same values the LDS tables hold)
__device__ __forceinline__ void nv_thresholds(int k, double gd, uint32_t t[7]) {
  const double sv = sf_val<0>(k) * gd;
#pragma unroll
  for (int j = 0; j < 7; ++j) t[j] = k > 0 ? thr_bits((double)kMidD[j] * sv, (j & 1) != 0) : 0x7F800000u;
}

// nearest E4M3 code to a / (T g) (T = 6 or 4), ties to the even code,
// saturating at 126: binary64 guess corrected by the exact scale midpoints
__device__ __forceinline__ int select_e4m3_exact(float a, double inv_Tg, double Tg) {
  int k = select_scale_guess<0>(a, inv_Tg);
  const uint32_t ab = fbits(a);
  auto mid = [&](int j) { return thr_bits(0.5 * (sf_val<0>(j) + sf_val<0>(j + 1)) * Tg, (j & 1) != 0); };
  if (k < 126 && ab > mid(k)) ++k;
  else if (k > 0 && ab <= mid(k - 1)) --k;
  return k;
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

// Exact codes from low-side codes.  `plo` holds the codes of x * rlo with
// rlo < 1/(s g): every element's exact code is its low-side code or one
// magnitude step above (the exact ratio exceeds the low-side ratio by far less
// than the gap between midpoints).  Step up where |x| is past the midpoint
// above the low-side magnitude; magnitude 7 (6.0) is the top.
template <int L>
__device__ __forceinline__ uint32_t resolve_codes(const float* x, uint32_t plo, float s, float g) {
  const uint32_t inc = (plo & 0x77777777u) + 0x11111111u;  // magnitude + 1 per nibble
  uint32_t up = 0;
  static_for<0, L / 2>([&](auto ic) {
    constexpr int b = decltype(ic)::value;
    // half values of the low-side and next magnitudes: their sum is the midpoint
    const auto vl = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(plo, 0.5f, b);
    const auto vu = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(inc, 0.5f, b);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * b + h;
      const uint32_t mag = (plo >> (4 * i)) & 7u;
      const float mid = fabsf(vl[h]) + vu[h];
      const bool go = mag != 7u && past_midpoint(fabsf(x[i]), mid * s, g, (mag & 1u) != 0);
      up |= go ? (0xFu << (4 * i)) : 0u;
    }
  });
  return (plo & ~up) | (((inc & 0x77777777u) | (plo & 0x88888888u)) & up);
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
template <int L>
__device__ __attribute__((noinline)) uint32_t encode_nv_thresholds(float __attribute__((ext_vector_type(L))) x, int k,
                                                                   float g) {
  uint32_t t[7];
  nv_thresholds(k, (double)g, t);
  uint32_t plo = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const uint32_t b = fbits(x[i]);
    const int m = rtn_count(b & 0x7FFFFFFFu, t);
    plo |= (m ? ((uint32_t)m | ((b >> 28) & 8u)) : 0u) << (4 * i);
  }
  return plo;
}

// NVFP4 codes of a lane's L elements for scale code k (value s) under global
// g: bracketed convert; when some element of the wave cannot be decided that
// way (on or near a midpoint), the whole wave resolves its elements exactly
// from the low-side codes.  The bracket is used only for finite blocks with
// s g well inside the normal range; a wave with any other block takes the
// threshold search.
template <int L, int LPB>
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
    if (wave_all(ok)) {
      // elements whose two ends differ, one per lane per pass (usually one pass)
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
    } else {
      typedef float fLv __attribute__((ext_vector_type(L)));
      fLv xv;
#pragma unroll
      for (int i = 0; i < L; ++i) xv[i] = x[i];
      return encode_nv_thresholds<L>(xv, k, g);
    }
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

// Automatic global scale inside a single-workgroup launch (small tensors,
// where the separate abs-max, finalize and zeroing launches would dominate):
// the abs-max of the transformed tensor as an integer maximum of magnitude
// bits (order-free, so equal to the grid-wide reduction), then amax /
// fused_denom, or 1 for an all-zero tensor, written to *global.  Every thread
// returns g.  The chunk width and the Hadamard stage order do not change the
// transformed values, so the maximum is that of the separate abs-max pass.
template <int L, bool BF16>
__device__ float fused_auto_global(const QuantParams& p) {
  __shared__ uint32_t part[kThreads / 64];
  const bool chan = p.chan_scale != nullptr;
  const bool had = p.hadamard == 32;
  const int64_t cpr = p.cols / L;
  const int64_t total = p.rows * cpr;
  uint32_t m = 0;
  // four chunks per thread per pass, all loads issued before the first wait;
  // whole waves stay in the loop (Hadamard shuffles), and lanes past the end
  // load the last chunk and do not count it
  constexpr int U = 4;
  for (int64_t c0 = 0; c0 < total; c0 += U * kThreads) {
    Raw<L, BF16> raw[U];
    int64_t cu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kThreads + threadIdx.x;
      cu[u] = c < total ? c : -1;
      const int64_t cc = c < total ? c : total - 1;
      load_raw<L, BF16>(p, cc / cpr, (cc % cpr) * L, raw[u]);
      load_t<L, BF16>(chan_view(p), (cc % cpr) * L, raw[u]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[L];
      const int64_t cc = cu[u] >= 0 ? cu[u] : total - 1;
      finish_chunk<L, BF16, true>(p, (cc % cpr) * L, raw[u], x, chan, had);
      if (cu[u] >= 0)
#pragma unroll
        for (int i = 0; i < L; ++i) m = max(m, fbits(x[i]) & 0x7FFFFFFFu);
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d *= 2) m = max(m, (uint32_t)__shfl_xor((int)m, d));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t a = part[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) a = max(a, part[w]);
  const float g = (a == 0u) ? 1.0f : bitsf(a) / p.fused_denom;
  if (threadIdx.x == 0) *p.global = g;
  return g;
}

// CONTIG: rows are contiguous (ld == cols) and there is no channel scale, so
// the tensor is walked as one row of rows * cols elements
template <int FMT, int B, int RULE, bool BF16, bool CONTIG>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantParams p) {
  constexpr int L = (B == 4) ? 4 : 8;
  constexpr int LPB = B / L;  // lanes per block
  // LDS tables serve RaZeR-W (E3M3 scales) and the brute-force search;
  // NVFP4 (abs-max, 4-over-6), RaZeR-A and MXFP4 form their rare exact
  // decisions on the fly
  constexpr bool TABLES = (FMT == RAZER_W || RULE == BRUTE);
  __shared__ Tables<TABLES ? FMT : MXFP4> T;
  const float g = (p.fused_denom > 0.0f) ? fused_auto_global<L, BF16>(p) : (p.global ? *p.global : 1.0f);
  if constexpr (TABLES) {
    build_tables<FMT>(T, g, p.special);
    __syncthreads();
  }

  const bool chan = p.chan_scale != nullptr;
  const bool had = p.hadamard == 32;
  const int64_t cpr = p.cols / L;            // chunks per row
  const int64_t total = p.rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const double inv6 = 1.0 / (6.0 * (double)g);
  const double inv4 = 1.0 / (4.0 * (double)g);
  constexpr int SF = FmtTraits<FMT>::SF;

  // E4M3 scale selection by the hardware FP32 -> E4M3 convert (nearest even;
  // above 464 it gives the NaN code, which stands for the saturated 126):
  // amax / (6 g) and amax / (4 g) are bracketed like the element ratios in
  // encode_nv, and equal codes at both ends are the exact choice
  const bool fast_scale = g > 0x1p-100f && g < 0x1p100f;
  const float r6 = __builtin_amdgcn_rcpf(6.0f * g), r4 = __builtin_amdgcn_rcpf(4.0f * g);
  const float lo6 = r6 * (1.0f - 0x1p-20f), lo4 = r4 * (1.0f - 0x1p-20f);

  // chunk c = r * cpr + cj; the division happens once, then (r, cj) advance.
  // Each iteration issues the loads of U chunks (c, c + stride, ...) before
  // working on the first, to keep enough bytes in flight per CU.
  constexpr int U = (FMT == MXFP4 && CONTIG) ? 1 : 2;
  const __amdgpu_buffer_rsrc_t tv = chan_view(p);
  int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  int64_t r0 = CONTIG ? 0 : c / cpr, cj0 = CONTIG ? c : c % cpr;
  const int64_t sr = CONTIG ? 0 : stride / cpr, sc = CONTIG ? stride : stride % cpr;
  for (; c - threadIdx.x < total; c += U * stride) {
    // whole waves stay in the loop so that shuffles see their partners; lanes
    // past the end work on a clamped chunk and store nothing
    Raw<L, BF16> raw[U];
    int64_t ru[U], cu[U];
    bool vu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vu[u] = c + u * stride < total;
      if constexpr (CONTIG) {
        ru[u] = 0;
        cu[u] = vu[u] ? c + u * stride : total - 1;
      } else {
        ru[u] = vu[u] ? r0 : p.rows - 1;
        cu[u] = vu[u] ? cj0 : cpr - 1;
        r0 += sr;
        cj0 += sc;
        if (cj0 >= cpr) {
          cj0 -= cpr;
          ++r0;
        }
      }
      load_raw<L, BF16>(p, ru[u], cu[u] * L, raw[u]);
      if constexpr (!CONTIG) load_t<L, BF16>(tv, cu[u] * L, raw[u]);
    }
    __builtin_amdgcn_sched_barrier(0);  // all of the iteration's loads before the first wait
#pragma unroll
    for (int u = 0; u < U; ++u) {
    const bool valid = vu[u];
    const int64_t r = ru[u], cj = cu[u];
    float x[L];
    finish_chunk<L, BF16, !CONTIG>(p, cj * L, raw[u], x, chan, had);

    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) amax = max(amax, fbits(x[i]) & 0x7FFFFFFFu);
    amax = group_max<LPB>(amax);

    uint32_t packed;
    uint8_t sbyte;
    if constexpr (FMT == MXFP4) {
      // MACaQ section 1: shared exponent E = floor(log2 amax) - 2, clamped
      int E;
      if (amax == 0) E = -127;
      else {
        int ex = (int)(amax >> 23);
        int fl = ex ? ex - 127 : (31 - __clz((int)amax)) - 149;
        E = max(-127, fl - 2);
      }
      // the convert divides by 2^E exactly (E >= -126: a normal FP32 scale)
      // and rounds to nearest even, which is the format's rounding
      if (wave_all(E >= -126 && amax < 0x7F800000u)) {
        packed = 0;
        const float sc = bitsf((uint32_t)(E + 127) << 23);
        static_for<0, L / 2>([&](auto ic) {
          constexpr int b = decltype(ic)::value;
          packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, x[2 * b], x[2 * b + 1], sc, b);
        });
        packed = clear_neg_zero(packed);
      } else {
        typedef float fLv __attribute__((ext_vector_type(L)));
        fLv xv;
#pragma unroll
        for (int i = 0; i < L; ++i) xv[i] = x[i];
        packed = encode_mx_thresholds<L>(xv, E);
      }
      sbyte = (uint8_t)(E + 127);
    } else if constexpr (FMT == NVFP4) {
      if constexpr (RULE == BRUTE) {
        // every positive E4M3 scale; strict minimum, ties keep the smaller code
        float best = 0.f;
        int bestk = 1;
        packed = 0;
        for (int k = 1; k <= 126; ++k) {
          uint32_t t[7];
#pragma unroll
          for (int j = 0; j < 7; ++j) t[j] = T.elt[k][j];
          uint32_t pk = encode_plain<L>(x, t);
          float e = group_sum<LPB>(lane_sse<L>(x, pk, (float)sf_val<0>(k), g, false, 0.f));
          if (k == 1 || e < best) { best = e; bestk = k; packed = pk; }
        }
        sbyte = (uint8_t)bestk;
      } else {
        const bool finite = amax < 0x7F800000u;
        int k6 = 0, k4 = 0;
        if (wave_all(fast_scale && finite)) {
          typedef short s2v __attribute__((ext_vector_type(2)));
          const float a = bitsf(amax);
          const s2v z = {0, 0};
          const s2v clo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a * lo6, a * lo4, 1.0f, false);
          const uint32_t wl = (uint16_t)clo[0];
          k6 = e4m3_from_low(wl & 0xFFu, a, 6.0f, g);
          if constexpr (RULE == FOUR6) k4 = e4m3_from_low(wl >> 8, a, 4.0f, g);
        } else {
          k6 = select_e4m3_exact(bitsf(amax), inv6, 6.0 * (double)g);
          if constexpr (RULE == FOUR6) k4 = select_e4m3_exact(bitsf(amax), inv4, 4.0 * (double)g);
        }
        if (p.prevent_zero && k6 == 0) k6 = 1;
        const float s6 = e4m3_f32(k6);
        packed = encode_nv<L, LPB>(x, k6, s6, g, finite);
        sbyte = (uint8_t)k6;
        if constexpr (RULE == FOUR6) {
          if (p.prevent_zero && k4 == 0) k4 = 1;
          const float s4 = e4m3_f32(k4);
          uint32_t pk4 = encode_nv<L, LPB>(x, k4, s4, g, finite);
          float e6 = group_sum<LPB>(lane_sse<L>(x, packed, s6, g, false, 0.f));
          float e4 = group_sum<LPB>(lane_sse<L>(x, pk4, s4, g, false, 0.f));
          if (e4 < e6) { packed = pk4; sbyte = (uint8_t)k4; }
        }
      }
    } else if constexpr (FMT == RAZER_A) {
      // RaZeR-A: the abs-max E4M3 scale and element codes of NVFP4 (the same
      // rule: nearest E4M3 to amax / (6 g), ties to even), then the special
      // value +5 or -5 with the lower block error (ties keep +5).  A special
      // takes the elements of its sign strictly inside (4.5, 5.5) s g, the
      // midpoints to its neighbours 4 and 6; both bounds are exact products in
      // binary64, rounded down (strict >) and up (strict <) to FP32 patterns.
      const bool finite = amax < 0x7F800000u;
      int k;
      if (wave_all(fast_scale && finite)) {
        typedef short s2v __attribute__((ext_vector_type(2)));
        const float a = bitsf(amax);
        const s2v z = {0, 0};
        const s2v clo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a * lo6, a, 1.0f, false);
        k = e4m3_from_low((uint16_t)clo[0] & 0xFFu, a, 6.0f, g);
      } else {
        k = select_e4m3_exact(bitsf(amax), inv6, 6.0 * (double)g);
      }
      if (p.prevent_zero && k == 0) k = 1;
      const float s = e4m3_f32(k);
      const uint32_t base = encode_nv<L, LPB>(x, k, s, g, finite);
      const double sg = (double)s * (double)g;
      const uint32_t lo = thr_bits(4.5 * sg, false), hi = ru_bits(5.5 * sg);
      float best = 0.f;
      int bestp = 0;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t vsign = q ? 0x80000000u : 0u;
        uint32_t pk = base;
#pragma unroll
        for (int i = 0; i < L; ++i) {
          const uint32_t b = fbits(x[i]), xb = b & 0x7FFFFFFFu;
          const bool sp = ((b & 0x80000000u) == vsign) && xb > lo && xb < hi;
          pk = sp ? ((pk & ~(0xFu << (4 * i))) | (8u << (4 * i))) : pk;
        }
        const float v = q ? -5.0f : 5.0f;
        const float e = group_sum<LPB>(lane_sse<L>(x, pk, s, g, true, v * s));
        if (q == 0 || e < best) { best = e; bestp = q; packed = pk; }
      }
      if (k == 0) {
        packed = 0;
        bestp = 0;
      }
      sbyte = (uint8_t)((bestp << 7) | k);
    } else {
      // RaZeR: abs-max scale (E4M3 for activations, E3M3 for weights), then
      // the special value with the lowest block error (ties keep the first)
      int k = select_scale<SF>(bitsf(amax), T.smid6, inv6);
      if (p.prevent_zero && k == 0) k = 1;
      uint32_t t[7];
#pragma unroll
      for (int j = 0; j < 7; ++j) t[j] = T.elt[k][j];
      const float s = (float)sf_val<SF>(k);
      constexpr int NSP = FmtTraits<FMT>::NSP;
      float best = 0.f;
      int bestp = 0;
      packed = 0;
      if (k == 0) {
        packed = 0;
      } else {
#pragma unroll
        for (int q = 0; q < NSP; ++q) {
          float v = T.spv[q];
          uint32_t pk = encode_special<L>(x, t, T.sp_lo[k][q], T.sp_hi[k][q], fbits(v) & 0x80000000u);
          float e = group_sum<LPB>(lane_sse<L>(x, pk, s, g, true, v * s));
          if (q == 0 || e < best) { best = e; bestp = q; packed = pk; }
        }
      }
      if (FMT == RAZER_A) sbyte = (uint8_t)((bestp << 7) | k);
      else sbyte = (uint8_t)((bestp << 6) | k);
    }

    if (valid) {
      uint8_t* dst = p.codes + (CONTIG ? 0 : r * (p.cols / 2)) + cj * (L / 2);
      if constexpr (L == 8) *(uint32_t*)dst = packed;
      else *(uint16_t*)dst = (uint16_t)packed;
      if (cj % LPB == 0) p.scales[(CONTIG ? 0 : r * (p.cols / B)) + cj / LPB] = sbyte;
    }
    }  // u
  }
}

// ---------------------------------------------------------------- global amax
__global__ void zero_global_kernel(float* g) { *(uint32_t*)g = 0u; }

// workgroup maximum, then one atomic per workgroup
__device__ __forceinline__ void block_max_to_global(uint32_t m, unsigned int* dst) {
  __shared__ uint32_t part[kThreads / 64];
#pragma unroll
  for (int d = 1; d < 64; d *= 2) m = max(m, (uint32_t)__shfl_xor((int)m, d));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = part[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) v = max(v, part[w]);
    atomicMax(dst, v);
  }
}

// CONTIG: rows are contiguous (ld == cols) and there is no channel scale, so
// chunk c starts at element c * L, and two chunks are loaded per iteration
template <bool BF16, bool CONTIG>
__global__ __launch_bounds__(kThreads) void amax_kernel(QuantParams p) {
  constexpr int L = 8;
  constexpr int U = CONTIG ? 2 : 1;
  const bool chan = p.chan_scale != nullptr;
  const bool had = p.hadamard == 32;
  const int64_t cpr = p.cols / L;
  const int64_t total = p.rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t m = 0;
  // whole waves stay in the loop so that the Hadamard exchanges see their
  // partners; lanes past the end work on the last chunk and are not counted
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c - threadIdx.x < total; c += U * stride) {
    if constexpr (CONTIG) {
      Raw<L, BF16> raw[U];
      int64_t cu[U];
      bool vu[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        vu[u] = c + u * stride < total;
        cu[u] = vu[u] ? c + u * stride : total - 1;
        load_raw<L, BF16>(p, 0, cu[u] * L, raw[u]);
      }
      __builtin_amdgcn_sched_barrier(0);  // both chunks' loads before the first wait
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[L];
        finish_chunk<L, BF16, false>(p, cu[u] * L, raw[u], x, false, had);
        if (vu[u])
#pragma unroll
          for (int i = 0; i < L; ++i) m = max(m, fbits(x[i]) & 0x7FFFFFFFu);
      }
    } else {
      const bool valid = c < total;
      const int64_t cc = valid ? c : total - 1;
      float x[L];
      load_chunk<L, BF16>(p, cc / cpr, (cc % cpr) * L, x, chan, had);
      if (valid)
#pragma unroll
        for (int i = 0; i < L; ++i) m = max(m, fbits(x[i]) & 0x7FFFFFFFu);
    }
  }
  block_max_to_global(m, (unsigned int*)p.global);
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void amax4_kernel(QuantParams p) {
  // columns that are a multiple of 4 but not 8 (blocks of 4 without Hadamard)
  constexpr int L = 4;
  const bool chan = p.chan_scale != nullptr;
  const int64_t cpr = p.cols / L;
  const int64_t total = p.rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t m = 0;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < total; c += stride) {
    float x[L];
    load_chunk<L, BF16>(p, c / cpr, (c % cpr) * L, x, chan, false);
#pragma unroll
    for (int i = 0; i < L; ++i) m = max(m, fbits(x[i]) & 0x7FFFFFFFu);
  }
  block_max_to_global(m, (unsigned int*)p.global);
}

// "Finer is Better" Method 2 hierarchical scaling: g maps the tensor maximum
// to the top of the two-level range: amax / (6*448) for E4M3 block scales,
// amax / (6*30) for E3M3; 1 for an all-zero tensor
__global__ void finalize_global_kernel(float* g, float denom) {
  float a = bitsf(*(const uint32_t*)g);
  *g = (a == 0.0f) ? 1.0f : a / denom;
}

// ---------------------------------------------------------------- dequantize
template <int FMT, int B>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(DequantParams p) {
  constexpr int L = (B == 4) ? 4 : 8;
  const float g = p.global ? *p.global : 1.0f;
  const int64_t cpr = p.cols / L;
  const int64_t total = p.rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < total; c += stride) {
    const int64_t r = c / cpr, cj = c % cpr, j0 = cj * L;
    const uint8_t* src = p.codes + r * (p.cols / 2) + j0 / 2;
    uint32_t packed = (L == 8) ? *(const uint32_t*)src : (uint32_t)*(const uint16_t*)src;
    const uint8_t sb = p.scales[r * (p.cols / B) + j0 / B];
    float s, v = 0.f;
    if constexpr (FMT == MXFP4) s = ldexpf(1.0f, (int)sb - 127);
    else if constexpr (FMT == RAZER_W) { s = (float)sf_val<1>(sb & 0x3F); v = p.special[sb >> 6]; }
    else { s = (float)sf_val<0>(sb & 0x7F); v = (sb & 0x80) ? -5.0f : 5.0f; }
    float out[L];
    static_for<0, L / 2>([&](auto ic) {
      constexpr int b = decltype(ic)::value;
      auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, b);
      float q0 = v2[0] * s, q1 = v2[1] * s;  // exact (at most 8 significant bits)
      if (FMT == RAZER_A || FMT == RAZER_W) {
        if (((packed >> (8 * b)) & 15u) == 8u) q0 = v * s;
        if (((packed >> (8 * b + 4)) & 15u) == 8u) q1 = v * s;
      }
      out[2 * b] = q0 * g;
      out[2 * b + 1] = q1 * g;
    });
    if (p.out_bf16) {
      uint16_t* dst = (uint16_t*)p.out + r * p.ld_out + j0;
      uint32_t w[L / 2];
#pragma unroll
      for (int i = 0; i < L; i += 2) {
        uint32_t a = fbits(out[i]), b = fbits(out[i + 1]);
        a = (a + 0x7FFFu + ((a >> 16) & 1u)) >> 16;  // RNE to bf16 (finite)
        b = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
        w[i / 2] = a | (b << 16);
      }
      if constexpr (L == 8) *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
      else *(uint2*)dst = make_uint2(w[0], w[1]);
    } else {
      float* dst = (float*)p.out + r * p.ld_out + j0;
#pragma unroll
      for (int i = 0; i < L; i += 4) *(float4*)(dst + i) = make_float4(out[i], out[i + 1], out[i + 2], out[i + 3]);
    }
  }
}

// ---------------------------------------------------------------- channel scale
// MACaQ section 3: t_j = (rms_j(W) / rms_j(X))^alpha.  A workgroup owns 16
// columns, so that a 4096-column calibration fills 256 CUs: thread (slice y,
// column x) sums the squares of rows y, y + 64, ... in binary64 (a wave reads
// 4 rows of its 16 columns per step), then the 64 row slices of a column
// combine in a fixed pairwise order.
constexpr int kCsThreads = 1024, kCsCols = 16, kCsSlices = kCsThreads / kCsCols;

__device__ __forceinline__ double load_any(const void* base, int bf16, int64_t idx) {
  if (bf16) return (double)bitsf((uint32_t)((const uint16_t*)base)[idx] << 16);
  return (double)((const float*)base)[idx];
}

__global__ __launch_bounds__(kCsThreads) void channel_scale_kernel(ChanScaleParams p) {
  __shared__ double part[2][kCsSlices][kCsCols];
  const int tx = threadIdx.x % kCsCols, ty = threadIdx.x / kCsCols;
  const int64_t j = (int64_t)blockIdx.x * kCsCols + tx;
  double sx = 0.0, sw = 0.0;
  if (j < p.cols) {
#pragma unroll 4
    for (int64_t i = ty; i < p.rows_x; i += kCsSlices) { double v = load_any(p.x, p.x_bf16, i * p.ldx + j); sx += v * v; }
#pragma unroll 4
    for (int64_t i = ty; i < p.rows_w; i += kCsSlices) { double v = load_any(p.w, p.w_bf16, i * p.ldw + j); sw += v * v; }
  }
  part[0][ty][tx] = sx;
  part[1][ty][tx] = sw;
  // pairwise tree over the slices: level h adds slice k + h into slice k
  for (int h = kCsSlices / 2; h >= 1; h /= 2) {
    __syncthreads();
    if (ty < h) {
      part[0][ty][tx] = part[0][ty][tx] + part[0][ty + h][tx];
      part[1][ty][tx] = part[1][ty][tx] + part[1][ty + h][tx];
    }
  }
  __syncthreads();
  if (ty == 0 && j < p.cols) {
    double rx = sqrt(part[0][0][tx] / (double)p.rows_x), rw = sqrt(part[1][0][tx] / (double)p.rows_w);
    double tj = (rx == 0.0 || rw == 0.0) ? 1.0 : pow(rw / rx, p.alpha);
    float tf = (float)tj;
    p.t[j] = tf;
    p.r[j] = 1.0f / tf;
  }
}

// automatic g in the quantize launch itself up to this many elements: one
// pass of four chunks per thread of one workgroup for the maximum (one load
// latency), which beats three extra launches; larger tensors need more
// dependent passes than the launches cost
constexpr int64_t kFusedAutoMax = 8192;

int grid_for(int64_t work_items, int64_t cap = 256 * 16) {  // default: 16 workgroups per CU on 256 CUs
  int64_t blocks = (work_items + kThreads - 1) / kThreads;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

template <int FMT, int B, int RULE>
hipError_t launch_q3(bool bf16, const QuantParams& p, hipStream_t s) {
  constexpr int L = (B == 4) ? 4 : 8;
  const int64_t chunks = p.rows * (p.cols / L);
  int grid = p.fused_denom > 0.0f ? 1 : grid_for(chunks);
  // kernels that build LDS tables per workgroup: a few chunks per thread
  // (2 for small tensors, where the grid is short of the CUs anyway, 4 above)
  if (FMT == RAZER_W || RULE == BRUTE) {
    const int64_t per = chunks <= 65536 ? 2 : 4;
    const int64_t cap = (chunks + kThreads * per - 1) / (kThreads * per);
    if (grid > cap) grid = (int)(cap < 1 ? 1 : cap);
  }
  // the brute-force search is compute-bound: one addressing variant suffices
  const bool contig = RULE != BRUTE && p.ld == p.cols && p.chan_scale == nullptr;
  if (contig) {
    if (bf16) hipLaunchKernelGGL((quantize_kernel<FMT, B, RULE, true, RULE != BRUTE>), dim3(grid), dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((quantize_kernel<FMT, B, RULE, false, RULE != BRUTE>), dim3(grid), dim3(kThreads), 0, s, p);
  } else {
    if (bf16) hipLaunchKernelGGL((quantize_kernel<FMT, B, RULE, true, false>), dim3(grid), dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((quantize_kernel<FMT, B, RULE, false, false>), dim3(grid), dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

template <int FMT, int RULE>
hipError_t launch_q2(int block, bool bf16, const QuantParams& p, hipStream_t s) {
  switch (block) {
    case 4: return launch_q3<FMT, 4, RULE>(bf16, p, s);
    case 8: return launch_q3<FMT, 8, RULE>(bf16, p, s);
    case 16: return launch_q3<FMT, 16, RULE>(bf16, p, s);
    default: return launch_q3<FMT, 32, RULE>(bf16, p, s);
  }
}

}  // namespace

hipError_t launch_quantize(int fmt, int block, int rule, int gmode, const QuantParams& p,
                           hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  const bool bf16 = p.x_bf16 != 0;
  QuantParams q = p;
  q.fused_denom = 0.0f;
  const float denom = fmt == RAZER_W ? 180.0f : 2688.0f;
  if (gmode == G_AUTO && p.rows * p.cols <= kFusedAutoMax) {
    // small tensor: one workgroup finds g and quantizes, in one launch
    q.fused_denom = denom;
  } else if (gmode == G_AUTO) {
    hipLaunchKernelGGL(zero_global_kernel, dim3(1), dim3(1), 0, s, p.global);
    if (p.cols % 8 == 0) {
      int grid = grid_for(p.rows * (p.cols / 8), 256 * 4);
      const bool contig = p.ld == p.cols && p.chan_scale == nullptr;
      if (contig) {
        if (bf16) hipLaunchKernelGGL((amax_kernel<true, true>), dim3(grid), dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((amax_kernel<false, true>), dim3(grid), dim3(kThreads), 0, s, p);
      } else {
        if (bf16) hipLaunchKernelGGL((amax_kernel<true, false>), dim3(grid), dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((amax_kernel<false, false>), dim3(grid), dim3(kThreads), 0, s, p);
      }
    } else {
      int grid = grid_for(p.rows * (p.cols / 4), 256 * 4);
      if (bf16) hipLaunchKernelGGL(amax4_kernel<true>, dim3(grid), dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL(amax4_kernel<false>, dim3(grid), dim3(kThreads), 0, s, p);
    }
    hipLaunchKernelGGL(finalize_global_kernel, dim3(1), dim3(1), 0, s, p.global, denom);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (fmt) {
    case MXFP4: return launch_q3<MXFP4, 32, ABSMAX>(bf16, q, s);
    case RAZER_A: return launch_q2<RAZER_A, ABSMAX>(block, bf16, q, s);
    case RAZER_W: return launch_q2<RAZER_W, ABSMAX>(block, bf16, q, s);
    default:
      if (rule == FOUR6) return launch_q2<NVFP4, FOUR6>(block, bf16, q, s);
      if (rule == BRUTE) return launch_q2<NVFP4, BRUTE>(block, bf16, q, s);
      return launch_q2<NVFP4, ABSMAX>(block, bf16, q, s);
  }
}

hipError_t launch_dequantize(int fmt, int block, const DequantParams& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  const int L = (block == 4) ? 4 : 8;
  int grid = grid_for(p.rows * (p.cols / L));
#define FP4Q_DQ(F, BB) hipLaunchKernelGGL((dequantize_kernel<F, BB>), dim3(grid), dim3(kThreads), 0, s, p)
  switch (fmt) {
    case MXFP4: FP4Q_DQ(MXFP4, 32); break;
    case NVFP4:
      if (block == 4) FP4Q_DQ(NVFP4, 4); else if (block == 8) FP4Q_DQ(NVFP4, 8);
      else if (block == 16) FP4Q_DQ(NVFP4, 16); else FP4Q_DQ(NVFP4, 32);
      break;
    case RAZER_A:
      if (block == 4) FP4Q_DQ(RAZER_A, 4); else if (block == 8) FP4Q_DQ(RAZER_A, 8);
      else if (block == 16) FP4Q_DQ(RAZER_A, 16); else FP4Q_DQ(RAZER_A, 32);
      break;
    default:
      if (block == 4) FP4Q_DQ(RAZER_W, 4); else if (block == 8) FP4Q_DQ(RAZER_W, 8);
      else if (block == 16) FP4Q_DQ(RAZER_W, 16); else FP4Q_DQ(RAZER_W, 32);
      break;
  }
#undef FP4Q_DQ
  return hipGetLastError();
}

hipError_t launch_channel_scale(const ChanScaleParams& p, hipStream_t s) {
  int grid = (int)((p.cols + kCsCols - 1) / kCsCols);
  hipLaunchKernelGGL(channel_scale_kernel, dim3(grid), dim3(kCsThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fp4q
