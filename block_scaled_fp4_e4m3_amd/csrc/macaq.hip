// MACaQ weight calibration for MXFP4 on gfx950 (MACaQ review, sections 1 and
// 3): Hessian-weighted exponent screening, then Flip-Refinement.
//
// For a weight W (N x K, row n = output channel) and the layer-input Hessian
// H = X^T X (K x K, binary64):
//   1. macaq_screen_kernel: per 32-element block, the standard exponent E
//      and E + 1, E - 1 (in that order) are compared by e^T H_bb e, the error
//      of the block's round-to-nearest codes weighted by the block's 32 x 32
//      diagonal block of H; the strictly smallest is kept.
//   2. macaq_hd_kernel: r = H d for every row, d = w^ - w, each entry summed
//      over j in ascending order.
//   3. macaq_refine_kernel: per row, the one-level move of one code with the
//      largest gain -(2 delta r_k + delta^2 H_kk) is taken while it gains, and
//      r is updated by delta * (row k of H).
// Every floating-point step is a binary64 operation in a fixed order (no
// contraction), so the codes and exponents do not depend on the launch.
#include "fp4q_internal.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace fp4q {

namespace {

__device__ __forceinline__ uint32_t fbits(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __uint_as_float(u); }

// E2M1 magnitudes; the adjacent levels of a code are its neighbours among the
// 15 distinct values -6 .. 6 (level index 0 .. 14, 7 = zero)
constexpr float kMag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
constexpr double kMidD[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};

__device__ __forceinline__ int level_of(uint32_t code) {
  const int m = (int)(code & 7u);
  return (code & 8u) ? 7 - m : 7 + m;
}
__device__ __forceinline__ uint32_t code_of(int level) {
  return level >= 7 ? (uint32_t)(level - 7) : (8u | (uint32_t)(7 - level));
}
__device__ __forceinline__ double level_value(int level) {
  const double m = (double)kMag[level >= 7 ? level - 7 : 7 - level];
  return level >= 7 ? m : -m;
}

__device__ __forceinline__ double shfl_d(double v, int src, int width = 64) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)u, src, width);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(u >> 32), src, width);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double shfl_xor_d(double v, int d, int width = 64) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)u, d, width);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(u >> 32), d, width);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// round-to-nearest E2M1 code of x at scale 2^E (ties to the even mantissa,
// saturating, a zero magnitude is +0): the hardware convert, which divides by
// the normal power of two exactly and rounds to nearest even, for E >= -126;
// for lower E the exact comparison with the midpoints 2^E * m (binary64)
__device__ __forceinline__ uint32_t rtn_code(float x, int E) {
  uint32_t c;
  if (E >= -126) {
    const float sc = bitsf((uint32_t)(E + 127) << 23);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x, 0.0f, sc, 0) & 0xFu;
  } else {
    const double ax = fabs((double)x);
    int m = 7;
    for (int j = 0; j < 7; ++j) {
      const double M = kMidD[j] * ldexp(1.0, E);
      if (ax < M) { m = j; break; }
      if (ax == M) { m = (j & 1) ? j + 1 : j; break; }
    }
    c = m ? ((uint32_t)m | (x < 0.0f ? 8u : 0u)) : 0u;
  }
  return (c & 7u) ? c : 0u;  // a magnitude of zero is always +0
}

// value * 2^E of code c, exact in binary64
__device__ __forceinline__ double code_value(uint32_t c, int E) {
  const double m = (double)kMag[c & 7u];
  return ((c & 8u) ? -m : m) * ldexp(1.0, E);
}

// ---------------------------------------------------------------- 1. screening
// A half-wave per block: lane i owns element i.  Each candidate's error e_i is
// exact in binary64; u_i = sum_j H[i][j] e_j takes e_j from lane j in order;
// the butterfly over lanes adds e_i u_i as the balanced index-order tree.
__global__ __launch_bounds__(256) void macaq_screen_kernel(MacaqParams p) {
  const int64_t nblk = p.K / 32;
  const int64_t blk = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 5;  // uniform per half-wave
  const int i = threadIdx.x & 31;
  const bool live = blk < p.N * nblk;
  const int64_t n = live ? blk / nblk : 0, b = live ? blk % nblk : 0;
  const float x = p.w[n * p.ldw + 32 * b + i];
  uint32_t am = fbits(x) & 0x7FFFFFFFu;
#pragma unroll
  for (int d = 1; d < 32; d *= 2) am = max(am, (uint32_t)__shfl_xor((int)am, d, 32));
  // MACaQ section 1: the standard exponent floor(log2 amax) - 2, clamped
  int E;
  if (am == 0) E = -127;
  else {
    const int ex = (int)(am >> 23);
    const int fl = ex ? ex - 127 : (31 - __clz((int)am)) - 149;
    E = max(-127, min(127, fl - 2));
  }
  const double* hrow = p.h + (32 * b + i) * p.ldh + 32 * b;
  double hr[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) hr[j] = hrow[j];
  auto cost = [&](uint32_t c, int Ec) {
    const double e = (double)x - code_value(c, Ec);
    double u = 0.0;
#pragma unroll
    for (int j = 0; j < 32; ++j) u = u + hr[j] * shfl_d(e, j, 32);
    double t = e * u;
#pragma unroll
    for (int d = 1; d < 32; d *= 2) t = t + shfl_xor_d(t, d, 32);
    return t;
  };
  uint32_t best_c = rtn_code(x, E);
  double best = cost(best_c, E);
  int bestE = E;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int Ec = t == 0 ? E + 1 : E - 1;
    if (Ec < -127 || Ec > 127) continue;  // uniform across the half-wave
    const uint32_t c = rtn_code(x, Ec);
    const double v = cost(c, Ec);
    if (v < best) {
      best = v;
      bestE = Ec;
      best_c = c;
    }
  }
  const uint32_t hi = (uint32_t)__shfl_xor((int)best_c, 1, 32);
  if (live) {
    if ((i & 1) == 0) p.codes[n * (p.K / 2) + 16 * b + i / 2] = (uint8_t)(best_c | (hi << 4));
    if (i == 0) p.scales[n * nblk + b] = (uint8_t)(bestE + 127);
  }
}

// ---------------------------------------------------------------- 2. r = H d
// R[n][k] = sum_j d[n][j] H[k][j], j ascending, for rows [n0, n0 + rows): a
// 64 x 64 tile of (n, k) per workgroup, 4 x 4 per thread, j in steps of 16
// staged in LDS (d formed from W, codes and exponents on the way in).
constexpr int kHdTile = 64, kHdStep = 16;

__global__ __launch_bounds__(256) void macaq_hd_kernel(MacaqParams p, int64_t n0, int64_t rows, double* R) {
  __shared__ double Ds[kHdTile][kHdStep + 1];
  __shared__ double Hs[kHdTile][kHdStep + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t nb = (int64_t)blockIdx.y * kHdTile, kb = (int64_t)blockIdx.x * kHdTile;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.0;
  for (int64_t j0 = 0; j0 < p.K; j0 += kHdStep) {
    __syncthreads();
    for (int e = threadIdx.x; e < kHdTile * kHdStep; e += 256) {
      const int rr = e / kHdStep, jj = e % kHdStep;
      const int64_t n = nb + rr, k = kb + rr, j = j0 + jj;
      double dv = 0.0, hv = 0.0;
      if (n < rows && j < p.K) {
        const int64_t row = n0 + n;
        const uint32_t c = (p.codes[row * (p.K / 2) + j / 2] >> (4 * (j & 1))) & 0xFu;
        const int E = (int)p.scales[row * (p.K / 32) + j / 32] - 127;
        dv = code_value(c, E) - (double)p.w[row * p.ldw + j];
      }
      if (k < p.K && j < p.K) hv = p.h[k * p.ldh + j];
      Ds[rr][jj] = dv;
      Hs[rr][jj] = hv;
    }
    __syncthreads();
    const int jn = (int)min<int64_t>(kHdStep, p.K - j0);
    for (int jj = 0; jj < jn; ++jj) {
      double dn[4], hk[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) dn[a] = Ds[ty * 4 + a][jj];
#pragma unroll
      for (int c = 0; c < 4; ++c) hk[c] = Hs[tx * 4 + c][jj];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = acc[a][c] + hk[c] * dn[a];
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t n = nb + ty * 4 + a, k = kb + tx * 4 + c;
      if (n < rows && k < p.K) R[n * p.K + k] = acc[a][c];
    }
}

// ---------------------------------------------------------------- 3. refinement
// One workgroup of four waves per row.  Wave w owns the elements
// j = 64 (4 i + w) + lane (i = 0, 1, ...) and keeps their r (binary64), levels
// and exponents in registers; the diagonal of H sits in LDS.  A move: every
// lane adds delta * H[k][j] to its r_j and, in the same pass, forms the two
// gains of each of its elements from the updated r (up before down; strict >
// keeps the first, so a tie keeps the smaller j, then up); each wave takes its
// best by a butterfly (largest gain, then the smaller index), and the four
// wave bests meet in LDS under the same rule, so every thread knows the next
// move.  The LDS slots alternate between two sets, one barrier per move.
constexpr int kMacaqMaxK = 80 * 64;
constexpr int kRowWaves = 4;
constexpr int kPer = kMacaqMaxK / (64 * kRowWaves);  // elements per lane, at most

struct MoveBest {
  double gain;
  int64_t idx;  // 2 j + (0 up, 1 down); INT64_MAX: none
  double delta;
};

__device__ __forceinline__ bool better(double g, int64_t i, double bg, int64_t bi) {
  return g > bg || (g == bg && i < bi);
}

__global__ __launch_bounds__(64 * kRowWaves) void macaq_refine_kernel(MacaqParams p, int64_t n0, const double* R) {
  __shared__ MoveBest slot[2][kRowWaves];
  __shared__ double hd[kMacaqMaxK];
  const int64_t K = p.K;
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int64_t nr = blockIdx.x, row = n0 + nr;
  double r[kPer];
  int st[kPer];  // level (bits 3:0) and exponent + 128 (bits 15:4)
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t j = 64 * (kRowWaves * (int64_t)i + wave) + lane;
    r[i] = 0.0;
    st[i] = 7 | (128 << 4);
    if (j < K) {
      r[i] = R[nr * K + j];
      hd[j] = p.h[j * p.ldh + j];
      const int lv = level_of((p.codes[row * (K / 2) + j / 2] >> (4 * (j & 1))) & 0xFu);
      const int e = (int)p.scales[row * (K / 32) + j / 32] - 127;
      st[i] = lv | ((e + 128) << 4);
    }
  }
  // the step between adjacent levels l and l + 1 (l in 0..13): 2 for the
  // outer pairs (-6/-4, 4/6), 1 for -4/-3, -3/-2, 2/3, 3/4, 0.5 otherwise
  auto step_up = [](int l) -> double {
    const int t = l >= 7 ? l - 7 : 6 - l;
    return t < 4 ? 0.5 : (t < 6 ? 1.0 : 2.0);
  };
  MoveBest b{0.0, INT64_MAX, 0.0};
  __syncthreads();  // the diagonal is in LDS
  auto consider = [&](int i, int64_t j) {
    const int li = st[i] & 15;
    const double hjj = hd[j];
    const double sc = ldexp(1.0, (st[i] >> 4) - 128);
    if (li < 14) {
      const double delta = step_up(li) * sc;
      const double q = 2.0 * (delta * r[i]) + (delta * delta) * hjj;
      const double gain = -q;
      if (gain > b.gain) b = MoveBest{gain, 2 * j, delta};
    }
    if (li > 0) {
      const double delta = -step_up(li - 1) * sc;
      const double q = 2.0 * (delta * r[i]) + (delta * delta) * hjj;
      const double gain = -q;
      if (gain > b.gain) b = MoveBest{gain, 2 * j + 1, delta};
    }
  };
  // the row's best: a butterfly per wave, then the four waves through LDS
  auto row_best = [&](int par) {
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
      const double og = shfl_xor_d(b.gain, d), od = shfl_xor_d(b.delta, d);
      const int64_t oi = (int64_t)(((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)((uint64_t)b.idx >> 32), d) << 32) |
                                   (uint32_t)__shfl_xor((int)(uint32_t)b.idx, d));
      if (better(og, oi, b.gain, b.idx)) b = MoveBest{og, oi, od};
    }
    if (lane == 0) slot[par][wave] = b;
    __syncthreads();
    MoveBest g = slot[par][0];
#pragma unroll
    for (int w = 1; w < kRowWaves; ++w) {
      const MoveBest o = slot[par][w];
      if (better(o.gain, o.idx, g.gain, g.idx)) g = o;
    }
    b = g;
  };
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t j = 64 * (kRowWaves * (int64_t)i + wave) + lane;
    if (j < K) consider(i, j);
  }
  row_best(0);
  int64_t taken = 0;
  while (taken < p.max_moves && b.gain > 0.0) {
    const int64_t k = b.idx >> 1;
    const bool down = (b.idx & 1) != 0;
    const double delta = b.delta;
    const double* hrow = p.h + k * p.ldh;
    double hv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t j = 64 * (kRowWaves * (int64_t)i + wave) + lane;
      hv[i] = j < K ? hrow[j] : 0.0;
    }
    // the moved element's new level, in its owner's registers
    if (wave == (int)((k >> 6) % kRowWaves) && lane == (int)(k & 63)) {
      const int ki = (int)(k >> 8);
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (i == ki) st[i] += down ? -1 : 1;
    }
    b = MoveBest{0.0, INT64_MAX, 0.0};
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t j = 64 * (kRowWaves * (int64_t)i + wave) + lane;
      if (j < K) {
        r[i] = r[i] + delta * hv[i];
        consider(i, j);
      }
    }
    ++taken;
    row_best((int)(taken & 1));
  }
  if (p.moves && threadIdx.x == 0) p.moves[row] = (int32_t)taken;
  // codes: element j (even lane) and j + 1 (the next lane) share a byte
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t j = 64 * (kRowWaves * (int64_t)i + wave) + lane;
    const uint32_t c = code_of(st[i] & 15);
    const uint32_t hi = (uint32_t)__shfl_down((int)c, 1);
    if (j < K && (lane & 1) == 0) p.codes[row * (K / 2) + j / 2] = (uint8_t)(c | (hi << 4));
  }
}

}  // namespace

int64_t macaq_max_k() { return kMacaqMaxK; }

hipError_t launch_macaq(const MacaqParams& p, void* workspace, size_t ws_bytes, hipStream_t s) {
  if (p.N == 0) return hipSuccess;
  const int64_t blocks = p.N * (p.K / 32);
  hipLaunchKernelGGL(macaq_screen_kernel, dim3((unsigned)((blocks + 7) / 8)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t chunk = std::min<int64_t>(p.N, (int64_t)(ws_bytes / ((size_t)p.K * sizeof(double))));
  double* R = (double*)workspace;
  for (int64_t n0 = 0; n0 < p.N; n0 += chunk) {
    const int64_t rows = std::min(chunk, p.N - n0);
    const dim3 g((unsigned)((p.K + kHdTile - 1) / kHdTile), (unsigned)((rows + kHdTile - 1) / kHdTile));
    hipLaunchKernelGGL(macaq_hd_kernel, g, dim3(256), 0, s, p, n0, rows, R);
    hipLaunchKernelGGL(macaq_refine_kernel, dim3((unsigned)rows), dim3(64 * kRowWaves), 0, s, p, n0, (const double*)R);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp4q
