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
#include "nv_encode.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace fp4q {

namespace {

constexpr int kThreads = 256;

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
    if constexpr (L >= 8) {
#pragma unroll
      for (int i = 0; i < L / 2; i += 4) {
        const uint4 v = *(const uint4*)(src + 2 * i);
        raw.w[i] = v.x; raw.w[i + 1] = v.y; raw.w[i + 2] = v.z; raw.w[i + 3] = v.w;
      }
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

// Block-Hadamard of size HS (16 or 32) over a lane's L consecutive elements
// and, when HS > L, its neighbours' (the HS / L lanes of a group are
// adjacent): the natural-order FWHT, in-lane stages h < L, then cross-lane
// stages with partner lane ^ (h / L); then the orthonormal factor
// RN32(2^-2.5) for 32, exactly 1/4 for 16.
template <int L, int HS>
__device__ __forceinline__ void block_hadamard(float* x) {
#pragma unroll
  for (int h = 1; h < L && h < HS; h *= 2) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if ((i & h) == 0) {
        float u = x[i], w = x[i + h];
        x[i] = u + w;
        x[i + h] = u - w;
      }
    }
  }
  // butterfly with the partner lane: the lower lane keeps x + o, the upper
  // o - x, written as o + (+-x) (the same IEEE operations)
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < HS / L; d *= 2) {
    const uint32_t neg = (lane & d) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const float o = lane_xor_f(x[i], d);
      x[i] = o + bitsf(fbits(x[i]) ^ neg);
    }
  }
  const float c = HS == 32 ? bitsf(0x3E3504F3u) : 0.25f;
#pragma unroll
  for (int i = 0; i < L; ++i) x[i] = x[i] * c;
}

// widen a raw chunk, apply the channel scale and the block-Hadamard of size
// had (0, 16 or 32)
template <int L, bool BF16, bool PRE_T = false>
__device__ __forceinline__ void finish_chunk(const QuantParams& p, int64_t j0, const Raw<L, BF16>& raw, float* x,
                                             bool chan, int had) {
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
  if (had == 32) block_hadamard<L, 32>(x);
  else if (had == 16) block_hadamard<L, 16>(x);
}

template <int L, bool BF16>
__device__ __forceinline__ void load_chunk(const QuantParams& p, int64_t r, int64_t j0, float* x,
                                           bool chan, int had) {
  Raw<L, BF16> raw;
  load_raw<L, BF16>(p, r, j0, raw);
  finish_chunk<L, BF16>(p, j0, raw, x, chan, had);
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
  const int had = p.hadamard;
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
  const int had = p.hadamard;
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
  constexpr int U = 2;
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
    if constexpr (FMT == NVFP4 || FMT == UE5M3) {
      if constexpr (RULE == BRUTE) {
        // every positive scale of the format; strict minimum, ties keep the
        // smaller code
        float best = 0.f;
        int bestk = 1;
        packed = 0;
        for (int k = 1; k <= FmtTraits<FMT>::KMAX; ++k) {
          uint32_t t[7];
#pragma unroll
          for (int j = 0; j < 7; ++j) t[j] = T.elt[k][j];
          uint32_t pk = encode_plain<L>(x, t);
          float e = group_sum<LPB>(lane_sse<L>(x, pk, (float)sf_val<SF>(k), g, false, 0.f));
          if (k == 1 || e < best) { best = e; bestk = k; packed = pk; }
        }
        sbyte = (uint8_t)bestk;
      } else {
        const bool finite = amax < 0x7F800000u;
        int k6 = 0, k4 = 0;
        if (FMT == NVFP4 && wave_all(fast_scale && finite)) {
          typedef short s2v __attribute__((ext_vector_type(2)));
          const float a = bitsf(amax);
          const s2v z = {0, 0};
          const s2v clo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a * lo6, a * lo4, 1.0f, false);
          const uint32_t wl = (uint16_t)clo[0];
          k6 = e4m3_from_low(wl & 0xFFu, a, 6.0f, g);
          if constexpr (RULE == FOUR6) k4 = e4m3_from_low(wl >> 8, a, 4.0f, g);
        } else {
          // UE5M3 has no hardware convert; E4M3 outside the convert's range
          k6 = select_sf_exact<SF>(bitsf(amax), inv6, 6.0 * (double)g);
          if constexpr (RULE == FOUR6) k4 = select_sf_exact<SF>(bitsf(amax), inv4, 4.0 * (double)g);
        }
        if (p.prevent_zero && k6 == 0) k6 = 1;
        const float s6 = sf_f32<SF>(k6);
        packed = encode_nv<L, LPB, SF>(x, k6, s6, g, finite);
        sbyte = (uint8_t)k6;
        if constexpr (RULE == FOUR6) {
          if (p.prevent_zero && k4 == 0) k4 = 1;
          const float s4 = sf_f32<SF>(k4);
          uint32_t pk4 = encode_nv<L, LPB, SF>(x, k4, s4, g, finite);
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
      // RaZeR-W: the abs-max E3M3 scale, then the special value of the table
      // with the lowest block error (ties keep the first)
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
      sbyte = (uint8_t)((bestp << 6) | k);
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

// ---------------------------------------------------------------- NVFP4, 16 elements per lane
// Abs-max and 4-over-6 with blocks of 16 or 32 on contiguous rows without a
// channel scale (the layout of every activation and weight workload here).
// The tensor is walked as one row of 16-element runs; lane l of a wave owns
// run (wave base + l).  A block of 16 is one lane and a block of 32 two
// adjacent lanes, so the per-block work (abs-max, both scale decisions, the
// reciprocals) is paid once per 16 elements and the error sums of 16-blocks
// need no lane exchange.  The run splits into two 8-element words for the
// FP4 converts; the decisions and the error tree are those of the 8-element
// kernel: tree(16) = tree(first 8) + tree(last 8).


template <int FMT, int B, int RULE, bool BF16>
__global__ __launch_bounds__(kThreads) void nv16_kernel(QuantParams p) {
  constexpr int L = 16, LPB = B / L;
  constexpr int SF = FmtTraits<FMT>::SF;
  static_assert(LPB == 1 || LPB == 2, "blocks of 16 or 32");
  const float g = p.global ? *p.global : 1.0f;
  const int had = p.hadamard;
  const int64_t total = p.rows * (p.cols / L);  // runs
  const double inv6 = 1.0 / (6.0 * (double)g);
  const double inv4 = 1.0 / (4.0 * (double)g);
  // scale selection as in quantize_kernel: the hardware FP32 -> E4M3 convert of
  // amax / (T g) bracketed from below, one exact midpoint test
  const bool fast_scale = g > 0x1p-100f && g < 0x1p100f;
  const float r6 = __builtin_amdgcn_rcpf(6.0f * g), r4 = __builtin_amdgcn_rcpf(4.0f * g);
  const float lo6 = r6 * (1.0f - 0x1p-20f), lo4 = r4 * (1.0f - 0x1p-20f);

  constexpr int U = 2;  // runs whose loads are issued before the first is worked on
  const int lane = threadIdx.x & 63;
  const int64_t pass = (int64_t)gridDim.x * kThreads;
  // wave-uniform base run; whole waves stay in the loop (Hadamard exchanges)
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads + (threadIdx.x & ~63); c0 < total; c0 += U * pass) {
    Raw<L, BF16> raw[U];
    int64_t cu[U];
    bool vu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * pass + lane;
      vu[u] = c < total;
      cu[u] = vu[u] ? c : total - 1;
      if (c0 + u * pass < total) load_raw<L, BF16>(p, 0, cu[u] * L, raw[u]);  // uniform: the wave has work
    }
    __builtin_amdgcn_sched_barrier(0);  // all of the iteration's loads before the first wait
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u * pass >= total) break;  // uniform: no run of the wave is left
      float x[L];
      finish_chunk<L, BF16, false>(p, cu[u] * L, raw[u], x, false, had);
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < L; ++i) amax = max(amax, fbits(x[i]) & 0x7FFFFFFFu);
      amax = group_max<LPB>(amax);
      const bool finite = amax < 0x7F800000u;
      int k6 = 0, k4 = 0;
      if (FMT == NVFP4 && wave_all(fast_scale && finite)) {
        typedef short s2v __attribute__((ext_vector_type(2)));
        const float a = bitsf(amax);
        const s2v z = {0, 0};
        const s2v clo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a * lo6, a * lo4, 1.0f, false);
        const uint32_t wl = (uint16_t)clo[0];
        k6 = e4m3_from_low(wl & 0xFFu, a, 6.0f, g);
        if constexpr (RULE == FOUR6) k4 = e4m3_from_low(wl >> 8, a, 4.0f, g);
      } else {
        // UE5M3 has no hardware convert; E4M3 outside the convert's range
        k6 = select_sf_exact<SF>(bitsf(amax), inv6, 6.0 * (double)g);
        if constexpr (RULE == FOUR6) k4 = select_sf_exact<SF>(bitsf(amax), inv4, 4.0 * (double)g);
      }
      if (p.prevent_zero && k6 == 0) k6 = 1;
      const float s6 = sf_f32<SF>(k6);
      uint2 packed = encode_nv16<LPB, SF>(x, k6, s6, g, finite);
      int sbyte = k6;
      if constexpr (RULE == FOUR6) {
        if (p.prevent_zero && k4 == 0) k4 = 1;
        const float s4 = sf_f32<SF>(k4);
        const uint2 pk4 = encode_nv16<LPB, SF>(x, k4, s4, g, finite);
        // a -0 code (0x8) decodes to -0 and gives the same error as +0
        const float e6 = group_sum<LPB>(lane_sse16(x, packed, s6, g));
        const float e4 = group_sum<LPB>(lane_sse16(x, pk4, s4, g));
        if (e4 < e6) { packed = pk4; sbyte = k4; }
      }
      packed.x = clear_neg_zero(packed.x);
      packed.y = clear_neg_zero(packed.y);
      if (vu[u]) {
        *(uint2*)(p.codes + cu[u] * (L / 2)) = packed;
        if (LPB == 1 || (lane & 1) == 0) p.scales[cu[u] / LPB] = (uint8_t)sbyte;
      }
    }
  }
}

// ---------------------------------------------------------------- NVFP4 4-over-6, decided from estimates
// 4-over-6 ("Finer is Better", Method 2) keeps the scale whose FP32 block
// error is lower.  nv16_kernel forms both candidates' exact codes (two
// bracketed converts each) and both exact errors.  Here each candidate is
// encoded once, at y = x * rlo (rlo just below 1/(s g)), and its error is
// estimated in units of s g as S = sum (y - v(y))^2, where v(y) is the value
// of y's code.  Only the chosen candidate's codes get the upper bracket.
//
// Why the estimate decides exactly.  Let t = x / (s g) and v(t) its exact
// E2M1 code value; the oracle's error is E = (s g)^2 T (1 + th) with
// T = sum (t - v(t))^2 and |th| < 8 u (u = 2^-24: one rounding of e, one of
// e^2, a tree of depth 4).  |y - t| <= |t| 1.32 2^-20 (the bracket factor,
// the reciprocal's ulp and three roundings), so with y_max = a * rlo every
// element has |y - t| <= dl = 1.5 2^-20 y_max.  Both v are nearest values,
// so ||y - v(y)| - |t - v(t)|| <= dl, and by Cauchy-Schwarz over 16 terms
// |S - T| <= 8 dl sqrt(S) + 16 dl^2 (plus the sum's own roundings, below
// 12 u relative).  P = s^2 S and Q = s^2 (that bound) then give: E4 < E6
// surely when P4 + Q4 + rho < P6 - Q6, and E4 > E6 surely when
// P4 - Q4 > P6 + Q6 + rho, with rho = 2^-17 (P4 + P6) covering every other
// rounding.  The codes of y at an element that sits on a midpoint may be
// either neighbour; both are dl-close in error, which the bound covers.
// Ranges that keep every step normal and finite (s g in [2^-50, 2^50],
// y_max < 64, a finite error) are required as well; a lane outside them, or
// whose estimates are too close, takes the exact 4-over-6 of nv16_kernel.

struct Four6Block {
  uint32_t lo, hi;  // codes of elements 0-7 and 8-15
  int sbyte;
};

// the exact 4-over-6 of one 16-element NVFP4 block (nv16_kernel's steps)
__device__ __attribute__((noinline)) Four6Block four6_exact16(float __attribute__((ext_vector_type(16))) xv,
                                                               float g, int pz) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = xv[i];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, fbits(x[i]) & 0x7FFFFFFFu);
  const bool finite = amax < 0x7F800000u;
  const double gd = (double)g;
  int k6 = select_sf_exact<0>(bitsf(amax), 1.0 / (6.0 * gd), 6.0 * gd);
  int k4 = select_sf_exact<0>(bitsf(amax), 1.0 / (4.0 * gd), 4.0 * gd);
  if (pz && k6 == 0) k6 = 1;
  if (pz && k4 == 0) k4 = 1;
  const float s6 = e4m3_f32(k6), s4 = e4m3_f32(k4);
  const uint2 c6 = encode_nv16<1, 0>(x, k6, s6, g, finite);
  const uint2 c4 = encode_nv16<1, 0>(x, k4, s4, g, finite);
  const float e6 = lane_sse16(x, c6, s6, g);
  const float e4 = lane_sse16(x, c4, s4, g);
  Four6Block o;
  if (e4 < e6) { o.lo = c4.x; o.hi = c4.y; o.sbyte = k4; }
  else { o.lo = c6.x; o.hi = c6.y; o.sbyte = k6; }
  return o;
}

// max(|a|, |b|, |c|) in one instruction (the compiler would first quiet each
// input); a NaN input is dropped, and its block then fails the finite-error
// test below
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// one candidate: codes of y = x * rl (elements 0-7, 8-15) and
// S = sum (y - v(y))^2 as two FMA chains
__device__ __forceinline__ float four6_candidate(const float* x, float rl, uint32_t& ca, uint32_t& cb) {
  float y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = x[i] * rl;
  ca = 0;
  cb = 0;
  static_for<0, 4>([&](auto ic) {
    constexpr int b = decltype(ic)::value;
    ca = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ca, y[2 * b], y[2 * b + 1], 1.0f, b);
    cb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cb, y[8 + 2 * b], y[9 + 2 * b], 1.0f, b);
  });
  float sa = 0.0f, sb = 0.0f;
  static_for<0, 4>([&](auto ic) {
    constexpr int b = decltype(ic)::value;
    const auto va = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ca, 1.0f, b);
    const auto vb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cb, 1.0f, b);
    const float d0 = y[2 * b] - va[0], d1 = y[2 * b + 1] - va[1];
    const float d2 = y[8 + 2 * b] - vb[0], d3 = y[9 + 2 * b] - vb[1];
    sa = __builtin_fmaf(d0, d0, sa);
    sb = __builtin_fmaf(d2, d2, sb);
    sa = __builtin_fmaf(d1, d1, sa);
    sb = __builtin_fmaf(d3, d3, sb);
  });
  return sa + sb;
}

// Codes of a lane's 16 elements whose two bracketed codes differ (the exact
// code is the low one or one magnitude step above).  The element is past its
// midpoint Q g (Q = midpoint * s, exact) by the sign of fma(-Q, g, |x|), a
// single rounding of the exact difference, which lies far from the underflow
// range for s g in [2^-50, 2^50]; a tie rounds up from an odd magnitude (to
// the even one).  The 16 positions are visited in order, each only when some
// lane of the wave has it ambiguous: every element is named by a constant
// index (an element chosen by a run-time index would put the elements in
// memory), and nothing is called (a call waits for the loads in flight).
__device__ __forceinline__ void resolve16(const float* x, uint32_t& wa, uint32_t& wb, uint32_t ha, uint32_t hb,
                                          float s, float g) {
  const uint32_t aa = wa ^ ha, ab = wb ^ hb;
  static_for<0, 16>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    constexpr int sh = 4 * (i & 7);
    const uint32_t am = (i < 8 ? aa : ab) & (0xFu << sh);
    if (!wave_all(am == 0)) {
      uint32_t& w = i < 8 ? wa : wb;
      const uint32_t mag = (w >> sh) & 7u;
      typedef float f2v __attribute__((ext_vector_type(2)));
      const f2v v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(mag | ((mag + 1u) << 4), 0.5f, 0);
      const float Q = (v[0] + v[1]) * s;  // exact: at most 8 significant bits
      const float e = __builtin_fmaf(-Q, g, fabsf(x[i]));
      const bool go = am != 0 && mag != 7u && (e > 0.0f || (e == 0.0f && (mag & 1u) != 0));
      w += go ? (1u << sh) : 0u;  // magnitude + 1 (at most 7: no carry)
    }
  });
}

// NVFP4, blocks of 16, rule 4-over-6, contiguous rows, optional
// block-Hadamard of 16 (HAD = 0 or 16); same walk as nv16_kernel
template <bool BF16, int HAD>
__global__ __launch_bounds__(kThreads) void nv16_four6_kernel(QuantParams p) {
  constexpr int L = 16;
  const float g = p.global ? *p.global : 1.0f;
  const int pz = p.prevent_zero;
  const int64_t total = p.rows * (p.cols / L);
  const bool gok = g > 0x1p-100f && g < 0x1p100f;
  // scale codes by the hardware FP32 -> E4M3 convert bracketed on both sides
  const float r6 = __builtin_amdgcn_rcpf(6.0f * g), r4 = __builtin_amdgcn_rcpf(4.0f * g);
  const float lo6 = r6 * (1.0f - 0x1p-20f), hi6 = r6 * (1.0f + 0x1p-20f);
  const float lo4 = r4 * (1.0f - 0x1p-20f), hi4 = r4 * (1.0f + 0x1p-20f);
  const float ag = __builtin_amdgcn_rcpf(g) * (1.0f + 0x1p-20f);  // above 1 / g

  constexpr int U = 2;
  const int lane = threadIdx.x & 63;
  const int64_t pass = (int64_t)gridDim.x * kThreads;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads + (threadIdx.x & ~63); c0 < total; c0 += U * pass) {
    Raw<L, BF16> raw[U];
    int64_t cu[U];
    bool vu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * pass + lane;
      vu[u] = c < total;
      cu[u] = vu[u] ? c : total - 1;
      if (c0 + u * pass < total) load_raw<L, BF16>(p, 0, cu[u] * L, raw[u]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u * pass >= total) break;
      float x[L];
      finish_chunk<L, BF16, false>(p, cu[u] * L, raw[u], x, false, HAD);
      float a = max3_abs(x[0], x[1], x[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) a = max3_abs(a, x[i], x[i + 1]);
      a = max3_abs(a, x[15], x[15]);

      typedef short s2v __attribute__((ext_vector_type(2)));
      const s2v z = {0, 0};
      const s2v clo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a * lo6, a * lo4, 1.0f, false);
      const s2v chi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a * hi6, a * hi4, 1.0f, false);
      const uint32_t wl = (uint16_t)clo[0], wh = (uint16_t)chi[0];
      // codes past 126 (the NaN code, above 464) stand for the saturated 126;
      // where the two ends differ, a / (T g) lies on or next to a scale
      // midpoint (calibrated global scales make exact midpoints common), and
      // one exact midpoint test settles it
      int k6 = min((int)(wl & 0xFFu), 126), k4 = min((int)(wl >> 8), 126);
      const bool m6 = k6 != min((int)(wh & 0xFFu), 126), m4 = k4 != min((int)(wh >> 8), 126);
      if (!wave_all(!gok || !(m6 || m4))) {
        if (gok && m6) k6 = e4m3_from_low(k6, a, 6.0f, g);
        if (gok && m4) k4 = e4m3_from_low(k4, a, 4.0f, g);
      }
      bool valid = gok;
      if (pz) { k6 = max(k6, 1); k4 = max(k4, 1); }
      valid = valid && k6 > 0;  // k4 >= k6
      const float s6 = e4m3_f32(k6), s4 = e4m3_f32(k4);
      const float sg6 = s6 * g, sg4 = s4 * g;
      valid = valid && sg6 >= 0x1p-50f && sg4 <= 0x1p50f;  // s6 <= s4
      const float q6 = __builtin_amdgcn_rcpf(sg6), q4 = __builtin_amdgcn_rcpf(sg4);
      const float rl6 = q6 * (1.0f - 0x1p-20f), rl4 = q4 * (1.0f - 0x1p-20f);

      uint32_t c6a, c6b, c4a, c4b;
      const float S6 = four6_candidate(x, rl6, c6a, c6b);
      const float S4 = four6_candidate(x, rl4, c4a, c4b);
      // the combined bound: s^2 dl sqrt(S) = 1.5 2^-20 (a / g) sqrt(P) (a / g
      // rounded up through ag), the dl^2 and absolute terms below 2^-31 (a / g)^2
      // (s <= a / (2 g) for both candidates)
      const float P6 = (s6 * s6) * S6, P4 = (s4 * s4) * S4;  // s^2 exact: at most 8 significant bits
      const float A = a * ag;
      const float M = 0x1.9p-17f * A * (__builtin_amdgcn_sqrtf(P4) + __builtin_amdgcn_sqrtf(P6)) +
                      0x1p-31f * (A * A) + 0x1p-17f * (P4 + P6);
      valid = valid && a * rl6 < 64.0f && P4 + P6 < 0x1p100f;  // rl4 <= rl6
      const bool pick4 = valid && k4 != k6 && P4 + M < P6;
      const bool pick6 = valid && (k4 == k6 || P4 > P6 + M);
      const bool dec = pick4 || pick6;

      uint32_t wa = pick4 ? c4a : c6a, wb = pick4 ? c4b : c6b;
      int sbyte = pick4 ? k4 : k6;
      // the chosen codes at the upper end of the bracket
      const float rh = (pick4 ? q4 : q6) * (1.0f + 0x1p-20f);
      uint32_t ha = 0, hb = 0;
      static_for<0, 4>([&](auto ic) {
        constexpr int b = decltype(ic)::value;
        ha = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ha, x[2 * b] * rh, x[2 * b + 1] * rh, 1.0f, b);
        hb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hb, x[8 + 2 * b] * rh, x[9 + 2 * b] * rh, 1.0f, b);
      });
      if (!dec) { ha = wa; hb = wb; }
      if (!wave_all(ha == wa && hb == wb)) resolve16(x, wa, wb, ha, hb, pick4 ? s4 : s6, g);
      if (!wave_all(dec)) {
        if (!dec) {
          typedef float f16v __attribute__((ext_vector_type(16)));
          f16v xv;
#pragma unroll
          for (int i = 0; i < 16; ++i) xv[i] = x[i];
          const Four6Block o = four6_exact16(xv, g, pz);
          wa = o.lo;
          wb = o.hi;
          sbyte = o.sbyte;
        }
      }
      if (vu[u]) {
        *(uint2*)(p.codes + cu[u] * (L / 2)) = make_uint2(clear_neg_zero(wa), clear_neg_zero(wb));
        p.scales[cu[u]] = (uint8_t)sbyte;
      }
    }
  }
}

// ---------------------------------------------------------------- MXFP4, 32 elements per lane
// One lane owns a 32-element run: one MXFP4 block and one Hadamard group, so
// the rotation runs in registers and the block maximum needs no exchange.
// A thread keeps its run position within the row and walks rows: the grid's
// thread count is a multiple of the runs per row (the launcher sizes it so),
// so thread t owns run t mod rpr of rows t / rpr, t / rpr + rstep, ... and
// loads the run's 32 channel scales once.
template <bool BF16>
__device__ __forceinline__ void load_run32(const QuantParams& p, int64_t r, int64_t j0, uint32_t (&w)[BF16 ? 16 : 32]) {
  constexpr int W = BF16 ? 16 : 32;
  const uint8_t* src = (const uint8_t*)p.x + (r * p.ld + j0) * (BF16 ? 2 : 4);
#pragma unroll
  for (int i = 0; i < W; i += 4) {
    const uint4 v = *(const uint4*)(src + 4 * i);
    w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
  }
}

// MXFP4 codes of 32 elements at shared exponent E >= -126 (a normal FP32
// scale, which the convert divides by exactly, rounding to nearest even)
__device__ __forceinline__ void mx_encode32(const float* x, int E, uint32_t (&pk)[4]) {
  const float sc = bitsf((uint32_t)(E + 127) << 23);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w = 0;
    static_for<0, 4>([&](auto ic) {
      constexpr int b = decltype(ic)::value;
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[8 * q + 2 * b], x[8 * q + 2 * b + 1], sc, b);
    });
    pk[q] = clear_neg_zero(w);
  }
}

// block error of 32 elements with codes pk at exponent E: value * 2^E is
// exact, e = x - value * 2^E in one rounding (the oracle's fma with g = 1),
// squares, the balanced tree
__device__ __forceinline__ float mx_sse32(const float* x, const uint32_t (&pk)[4], float sc) {
  float part[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float pp[8];
    static_for<0, 4>([&](auto ic) {
      constexpr int b = decltype(ic)::value;
      const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[q], 1.0f, b);
      const float e0 = x[8 * q + 2 * b] - v2[0] * sc, e1 = x[8 * q + 2 * b + 1] - v2[1] * sc;
      pp[2 * b] = e0 * e0;
      pp[2 * b + 1] = e1 * e1;
    });
    part[q] = tree_sum<8>(pp);
  }
  return (part[0] + part[1]) + (part[2] + part[3]);
}

// The same for any E in [-127, 127] (a block near the bottom of the FP32
// range): the exact threshold encode, and value * 2^E formed by ldexpf
// (exact, subnormal results included).  Out of line: rare.
struct MxCand {
  uint32_t pk[4];
  float sse;
};
__device__ __attribute__((noinline)) MxCand mx_candidate_exact(float __attribute__((ext_vector_type(32))) xv, int E) {
  MxCand out;
  uint32_t* pk = out.pk;
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = xv[i];
  typedef float f8v __attribute__((ext_vector_type(8)));
  float part[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f8v w;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = x[8 * q + i];
    pk[q] = encode_mx_thresholds<8>(w, E);
    float pp[8];
    static_for<0, 4>([&](auto ic) {
      constexpr int b = decltype(ic)::value;
      const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[q], 1.0f, b);
      const float e0 = x[8 * q + 2 * b] - ldexpf(v2[0], E), e1 = x[8 * q + 2 * b + 1] - ldexpf(v2[1], E);
      pp[2 * b] = e0 * e0;
      pp[2 * b + 1] = e1 * e1;
    });
    part[q] = tree_sum<8>(pp);
  }
  out.sse = (part[0] + part[1]) + (part[2] + part[3]);
  return out;
}

// HS: block-Hadamard size (0, 16, 32).  RULE: ABSMAX (the standard
// exponent), or EXPSEARCH: the standard exponent E and the offsets E + 1 and
// E - 1 (MACaQ section 1's candidates) compared by plain block error, in that
// order, the strictly smallest kept.
template <bool BF16, bool CHAN, int HS, int RULE>
__global__ __launch_bounds__(kThreads) void mx32_kernel(QuantParams p) {
  constexpr int L = 32, W = BF16 ? 16 : 32;
  const int64_t rpr = p.cols / L;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t rstep = (int64_t)gridDim.x * kThreads / rpr;
  const int64_t cj = t % rpr, j0 = cj * L;
  float tc[L];
  if constexpr (CHAN) {
#pragma unroll
    for (int i = 0; i < L; i += 4) {
      const float4 v = *(const float4*)(p.chan_scale + j0 + i);
      tc[i] = v.x; tc[i + 1] = v.y; tc[i + 2] = v.z; tc[i + 3] = v.w;
    }
  }
  constexpr int U = 2;  // rows whose loads are issued before the first is worked on
  for (int64_t r0 = t / rpr; r0 < p.rows; r0 += U * rstep) {
    // no lane exchange in this kernel, so a lane past the last row simply
    // loads nothing
    uint32_t raw[U][W];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (r0 + u * rstep < p.rows) load_run32<BF16>(p, r0 + u * rstep, j0, raw[u]);
      else
#pragma unroll
        for (int i = 0; i < W; ++i) raw[u][i] = 0u;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + u * rstep;
      float x[L];
      if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < W; ++i) {
          x[2 * i] = bitsf(raw[u][i] << 16);
          x[2 * i + 1] = bitsf(raw[u][i] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < L; ++i) x[i] = bitsf(raw[u][i]);
      }
      if constexpr (CHAN) {
#pragma unroll
        for (int i = 0; i < L; ++i) x[i] = x[i] * tc[i];
      }
      if constexpr (HS > 0) block_hadamard<L, HS>(x);
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < L; ++i) amax = max(amax, fbits(x[i]) & 0x7FFFFFFFu);
      // MACaQ section 1: shared exponent E = floor(log2 amax) - 2, clamped
      int E;
      if (amax == 0) E = -127;
      else {
        const int ex = (int)(amax >> 23);
        const int fl = ex ? ex - 127 : (31 - __clz((int)amax)) - 149;
        E = max(-127, fl - 2);
      }
      const bool finite = amax < 0x7F800000u;
      uint32_t pk[4];
      if constexpr (RULE == EXPSEARCH) {
        // the lowest candidate E - 1 must be a normal scale for the fast path;
        // E + 1 <= 126 always holds for a finite block
        int Eb = E;
        if (E - 1 >= -126 && finite) {
          mx_encode32(x, E, pk);
          float best = mx_sse32(x, pk, bitsf((uint32_t)(E + 127) << 23));
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int Ec = c == 0 ? E + 1 : E - 1;
            uint32_t pc[4];
            mx_encode32(x, Ec, pc);
            const float e = mx_sse32(x, pc, bitsf((uint32_t)(Ec + 127) << 23));
            if (e < best) {
              best = e;
              Eb = Ec;
#pragma unroll
              for (int q = 0; q < 4; ++q) pk[q] = pc[q];
            }
          }
        } else {
          typedef float f32v __attribute__((ext_vector_type(32)));
          f32v xv;
#pragma unroll
          for (int i = 0; i < L; ++i) xv[i] = x[i];
          MxCand best = mx_candidate_exact(xv, E);
          for (int c = 0; c < 2; ++c) {
            const int Ec = c == 0 ? E + 1 : E - 1;
            if (Ec < -127 || Ec > 127) continue;
            const MxCand cand = mx_candidate_exact(xv, Ec);
            if (cand.sse < best.sse) {
              best = cand;
              Eb = Ec;
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) pk[q] = best.pk[q];
        }
        E = Eb;
      } else if (E >= -126 && finite) {
        mx_encode32(x, E, pk);
      } else {
        typedef float f8v __attribute__((ext_vector_type(8)));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f8v xv;
#pragma unroll
          for (int i = 0; i < 8; ++i) xv[i] = x[8 * q + i];
          pk[q] = encode_mx_thresholds<8>(xv, E);
        }
      }
      if (r < p.rows) {
        *(uint4*)(p.codes + r * (p.cols / 2) + cj * (L / 2)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        p.scales[r * rpr + cj] = (uint8_t)(E + 127);
      }
    }
  }
}

// grid for mx32_kernel: a thread count that is a multiple of the runs per row,
// near the usual cap
int mx32_grid(int64_t rows, int64_t rpr) {
  int64_t a = rpr, b = kThreads;
  while (b) { const int64_t t = a % b; a = b; b = t; }  // a = gcd(rpr, kThreads)
  const int64_t base = rpr / a;                          // the fewest workgroups covering whole rows
  // two rows per thread (one iteration of two rows in flight), at most 8
  // workgroups per CU
  const int64_t want = std::min<int64_t>((rows * rpr + 2 * kThreads - 1) / (2 * kThreads), 256 * 8);
  return (int)std::max(base, want / base * base);
}

// ---------------------------------------------------------------- RaZeR special-value search
// RaZeR summary 2.2: the weight table's special values are chosen offline,
// multiples of 0.5, by quantization error.  The candidate magnitudes are the
// multiples of 0.5 in (0, 7.5] that are not E2M1 magnitudes; a table is
// {+a, -a, +b, -b} for a pair a < b (28 pairs, lexicographic).  Every 16-element
// block (RaZeR-W: abs-max E3M3 scale under g) takes the table's value with the
// lowest block error, and a table's tensor error is the binary64 sum over
// rows (ascending) of the binary64 sum over each row's blocks (ascending).
// One wave per row, one lane per block of a 64-block chunk: the lane forms
// the block error of each of the 16 signed candidates (the block error of
// RaZeR-W quantization) and the 28 pair minima; the wave stages the minima in
// LDS and lanes 0..27 add their pair's column in block order.
constexpr int kSearchCand = 8, kSearchPairs = kRazerPairs;
// the candidate magnitudes times 2, one nibble each: 5, 7, 9, 10, 11, 13, 14, 15
constexpr uint32_t kSearchMag2 = 0xFEDBA975u;
__host__ __device__ constexpr float search_mag(int i) { return 0.5f * (float)((kSearchMag2 >> (4 * i)) & 15u); }

struct SearchTables {
  uint32_t elt[64][8];                // per E3M3 code: 7 element thresholds (strict >)
  uint32_t smid6[64];                 // scale midpoints for T = 6
  uint32_t lo[64][kSearchCand];       // special interval of each magnitude, strict >
  uint32_t hi[64][kSearchCand];       // ... strict <
};

constexpr int kSearchWaves = kThreads / 64;  // rows per workgroup

template <bool BF16>
__global__ __launch_bounds__(kThreads) void razer_search_rows_kernel(QuantParams p, double* row_sums) {
  __shared__ SearchTables T;
  __shared__ float mins[kSearchWaves][kSearchPairs][64];
  const float g = p.global ? *p.global : 1.0f;
  const double gd = (double)g;
  for (int k = threadIdx.x; k < 64; k += blockDim.x) {
    const double sg = sf_val<1>(k) * gd;
#pragma unroll
    for (int j = 0; j < 8; ++j) T.elt[k][j] = (k > 0 && j < 7) ? thr_bits(kMidD[j] * sg, (j & 1) != 0) : 0x7F800000u;
    T.smid6[k] = k < 63 ? thr_bits(0.5 * (sf_val<1>(k) + sf_val<1>(k + 1)) * 6.0 * gd, (k & 1) != 0) : 0xFFFFFFFFu;
#pragma unroll
    for (int c = 0; c < kSearchCand; ++c) {
      float lo, hi;
      bool open_hi;
      special_bounds(search_mag(c), lo, hi, open_hi);
      T.lo[k][c] = k == 0 ? 0x7F800000u : thr_bits((double)lo * sg, false);
      T.hi[k][c] = (k == 0 || open_hi) ? 0x7F800000u : ru_bits((double)hi * sg);
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * kSearchWaves + wave;
  const bool live = r0 < p.rows;
  const int64_t r = live ? r0 : p.rows - 1;  // waves past the end read the last row and write nothing
  const double inv6 = 1.0 / (6.0 * gd);
  const int64_t nb = p.cols / 16;
  double acc = 0.0;  // lanes 0..27: pair `lane`
  // every wave of the workgroup runs the same chunks (equal rows), so the
  // workgroup barriers below are reached by all
  for (int64_t b0 = 0; b0 < nb; b0 += 64) {
    const int64_t b = b0 + lane;
    const bool has = b < nb;
    Raw<16, BF16> raw;
    load_raw<16, BF16>(p, r, 16 * (has ? b : nb - 1), raw);
    float x[16];
    finish_chunk<16, BF16, false>(p, 16 * b, raw, x, false, 0);
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = max(amax, fbits(x[i]) & 0x7FFFFFFFu);
    const int k = select_scale<1>(bitsf(amax), T.smid6, inv6);
    const float s = (float)sf_val<1>(k);
    // thresholds in scalars: an array read through selected elements would
    // be placed in memory
    const uint32_t t0 = T.elt[k][0], t1 = T.elt[k][1], t2 = T.elt[k][2], t3 = T.elt[k][3], t4 = T.elt[k][4],
                   t5 = T.elt[k][5], t6 = T.elt[k][6];
    // the standard codes, then per candidate the RaZeR element rule of
    // encode_special: 0x8 inside the special value's interval with its sign
    uint32_t std0 = 0, std1 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t bb = fbits(x[i]);
      const int mm = rtn_mag_v(bb & 0x7FFFFFFFu, t0, t1, t2, t3, t4, t5, t6);
      const uint32_t cc = mm ? ((uint32_t)mm | ((bb >> 28) & 8u)) : 0u;
      if (i < 8) std0 |= cc << (4 * i);
      else std1 |= cc << (4 * (i - 8));
    }
    float m[kSearchCand];  // per magnitude: the smaller block error of its two signs
#pragma unroll
    for (int c = 0; c < kSearchCand; ++c) {
      const uint32_t lo = T.lo[k][c], hi = T.hi[k][c];
      float e2[2];
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        const uint32_t vsign = sg ? 0x80000000u : 0u;
        uint32_t p0 = std0, p1 = std1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t bb = fbits(x[i]), xb = bb & 0x7FFFFFFFu;
          const bool sp = ((bb & 0x80000000u) == vsign) && xb > lo && xb < hi;
          if (i < 8) p0 = sp ? ((p0 & ~(0xFu << (4 * i))) | (8u << (4 * i))) : p0;
          else p1 = sp ? ((p1 & ~(0xFu << (4 * (i - 8)))) | (8u << (4 * (i - 8)))) : p1;
        }
        if (k == 0) p0 = p1 = 0u;
        const float v = sg ? -search_mag(c) : search_mag(c);
        e2[sg] = lane_sse<8>(x, p0, s, g, true, v * s) + lane_sse<8>(x + 8, p1, s, g, true, v * s);
      }
      m[c] = fminf(e2[0], e2[1]);
    }
    {
      int q = 0;
#pragma unroll
      for (int i = 0; i < kSearchCand; ++i)
#pragma unroll
        for (int j = i + 1; j < kSearchCand; ++j, ++q) mins[wave][q][lane] = fminf(m[i], m[j]);
    }
    __syncthreads();
    if (lane < kSearchPairs) {
      const int n = (int)min((int64_t)64, nb - b0);
      for (int l = 0; l < n; ++l) acc = acc + (double)mins[wave][lane][l];
    }
    __syncthreads();
  }
  if (live && lane < kSearchPairs) row_sums[r * kSearchPairs + lane] = acc;
}

// per pair, the sum over rows in ascending order; then the smallest (a tie
// keeps the earlier pair) as the table {+a, -a, +b, -b}.  The workgroup
// stages 128 rows of sums at a time in LDS with coalesced loads (the next
// chunk's loads in flight while the current one is summed); threads 0..27
// add their pair's column in row order.
constexpr int kReduceRows = 128;
__global__ __launch_bounds__(256) void razer_search_reduce_kernel(const double* row_sums, int64_t rows,
                                                                  double* pair_sse, float* table) {
  __shared__ double buf[2][kReduceRows * kSearchPairs];
  __shared__ double tot[kSearchPairs];
  const int tid = threadIdx.x;
  constexpr int kChunk = kReduceRows * kSearchPairs;  // doubles per chunk
  const int64_t total = rows * kSearchPairs;
  const int64_t nchunks = (rows + kReduceRows - 1) / kReduceRows;
  double acc = 0.0;
  double pre[(kChunk + 255) / 256];
  auto fetch = [&](int64_t ch) {
#pragma unroll
    for (int i = 0; i < (kChunk + 255) / 256; ++i) {
      const int64_t idx = ch * kChunk + i * 256 + tid;
      pre[i] = (i * 256 + tid < kChunk && idx < total) ? row_sums[idx] : 0.0;
    }
  };
  auto stage = [&](int slot) {
#pragma unroll
    for (int i = 0; i < (kChunk + 255) / 256; ++i)
      if (i * 256 + tid < kChunk) buf[slot][i * 256 + tid] = pre[i];
  };
  if (nchunks > 0) fetch(0);
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int slot = (int)(ch & 1);
    stage(slot);
    __syncthreads();
    if (ch + 1 < nchunks) fetch(ch + 1);  // in flight while the column sums run
    if (tid < kSearchPairs) {
      const int64_t n = min((int64_t)kReduceRows, rows - ch * kReduceRows);
#pragma unroll 8
      for (int64_t r = 0; r < n; ++r) acc = acc + buf[slot][r * kSearchPairs + tid];
    }
    // the slot written next iteration is the other one; the one after that
    // waits for this barrier
    __syncthreads();
  }
  if (tid < kSearchPairs) {
    tot[tid] = acc;
    pair_sse[tid] = acc;
  }
  __syncthreads();
  if (tid == 0) {
    int best = 0;
    for (int i = 1; i < kSearchPairs; ++i)
      if (tot[i] < tot[best]) best = i;
    int n = 0;
    for (int i = 0; i < kSearchCand; ++i)
      for (int j = i + 1; j < kSearchCand; ++j, ++n)
        if (n == best) {
          table[0] = search_mag(i);
          table[1] = -search_mag(i);
          table[2] = search_mag(j);
          table[3] = -search_mag(j);
        }
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
  const int had = p.hadamard;
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
    else if constexpr (FMT == UE5M3) s = ue5m3_f32(sb);
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
  if constexpr ((FMT == NVFP4 || FMT == UE5M3) && RULE != BRUTE && B >= 16) {
    if (contig && p.fused_denom == 0.0f) {
      // two runs per thread and iteration: at least one whole iteration each
      const int g16 = grid_for((p.rows * (p.cols / 16) + 1) / 2);
      if constexpr (FMT == NVFP4 && B == 16 && RULE == FOUR6) {
        if (p.hadamard == 0 || p.hadamard == 16) {
          if (p.hadamard == 16) {
            if (bf16) hipLaunchKernelGGL((nv16_four6_kernel<true, 16>), dim3(g16), dim3(kThreads), 0, s, p);
            else hipLaunchKernelGGL((nv16_four6_kernel<false, 16>), dim3(g16), dim3(kThreads), 0, s, p);
          } else {
            if (bf16) hipLaunchKernelGGL((nv16_four6_kernel<true, 0>), dim3(g16), dim3(kThreads), 0, s, p);
            else hipLaunchKernelGGL((nv16_four6_kernel<false, 0>), dim3(g16), dim3(kThreads), 0, s, p);
          }
          return hipGetLastError();
        }
      }
      if (bf16) hipLaunchKernelGGL((nv16_kernel<FMT, B, RULE, true>), dim3(g16), dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL((nv16_kernel<FMT, B, RULE, false>), dim3(g16), dim3(kThreads), 0, s, p);
      return hipGetLastError();
    }
  }
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

// automatic global scale of the transformed tensor into *p.global: zero it,
// the abs-max pass, then g = amax / denom (1 for an all-zero tensor)
hipError_t launch_auto_global(const QuantParams& p, float denom, hipStream_t s) {
  const bool bf16 = p.x_bf16 != 0;
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
  return hipGetLastError();
}

template <int RULE, bool BF16, bool CHAN>
hipError_t launch_mx_hs(const QuantParams& q, int grid, hipStream_t s) {
  if (q.hadamard == 32) hipLaunchKernelGGL((mx32_kernel<BF16, CHAN, 32, RULE>), dim3(grid), dim3(kThreads), 0, s, q);
  else if (q.hadamard == 16) hipLaunchKernelGGL((mx32_kernel<BF16, CHAN, 16, RULE>), dim3(grid), dim3(kThreads), 0, s, q);
  else hipLaunchKernelGGL((mx32_kernel<BF16, CHAN, 0, RULE>), dim3(grid), dim3(kThreads), 0, s, q);
  return hipGetLastError();
}

template <int RULE>
hipError_t launch_mx(bool bf16, const QuantParams& q, int grid, hipStream_t s) {
  const bool chan = q.chan_scale != nullptr;
  if (bf16) return chan ? launch_mx_hs<RULE, true, true>(q, grid, s) : launch_mx_hs<RULE, true, false>(q, grid, s);
  return chan ? launch_mx_hs<RULE, false, true>(q, grid, s) : launch_mx_hs<RULE, false, false>(q, grid, s);
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
    const hipError_t e = launch_auto_global(p, denom, s);
    if (e != hipSuccess) return e;
  }
  switch (fmt) {
    case MXFP4: {
      const int64_t rpr = q.cols / 32;
      const int grid = mx32_grid(q.rows, rpr);
      return rule == EXPSEARCH ? launch_mx<EXPSEARCH>(bf16, q, grid, s) : launch_mx<ABSMAX>(bf16, q, grid, s);
    }
    case RAZER_A: return launch_q2<RAZER_A, ABSMAX>(block, bf16, q, s);
    case RAZER_W: return launch_q2<RAZER_W, ABSMAX>(block, bf16, q, s);
    case UE5M3:
      if (rule == FOUR6) return launch_q2<UE5M3, FOUR6>(block, bf16, q, s);
      if (rule == BRUTE) return launch_q2<UE5M3, BRUTE>(block, bf16, q, s);
      return launch_q2<UE5M3, ABSMAX>(block, bf16, q, s);
    default:
      if (rule == FOUR6) return launch_q2<NVFP4, FOUR6>(block, bf16, q, s);
      if (rule == BRUTE) return launch_q2<NVFP4, BRUTE>(block, bf16, q, s);
      return launch_q2<NVFP4, ABSMAX>(block, bf16, q, s);
  }
}

hipError_t launch_razer_search(const QuantParams& p, int gmode, double* row_sums, double* pair_sse, float* table,
                               hipStream_t s) {
  if (gmode == G_AUTO) {
    const hipError_t e = launch_auto_global(p, 180.0f, s);
    if (e != hipSuccess) return e;
  }
  const unsigned grid = (unsigned)((p.rows + kSearchWaves - 1) / kSearchWaves);  // one wave per row
  if (p.rows > 0) {
    if (p.x_bf16) hipLaunchKernelGGL(razer_search_rows_kernel<true>, dim3(grid), dim3(kThreads), 0, s, p, row_sums);
    else hipLaunchKernelGGL(razer_search_rows_kernel<false>, dim3(grid), dim3(kThreads), 0, s, p, row_sums);
  }
  hipLaunchKernelGGL(razer_search_reduce_kernel, dim3(1), dim3(256), 0, s, (const double*)row_sums, p.rows, pair_sse,
                     table);
  return hipGetLastError();
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
    case UE5M3:
      if (block == 4) FP4Q_DQ(UE5M3, 4); else if (block == 8) FP4Q_DQ(UE5M3, 8);
      else if (block == 16) FP4Q_DQ(UE5M3, 16); else FP4Q_DQ(UE5M3, 32);
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
