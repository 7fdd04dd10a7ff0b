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
// One wave per row; the waves of a workgroup share the diagonal of H in LDS,
// and each keeps its row's r (binary64), levels (0..14) and exponents in LDS.
// Lane l scans elements k = l, l + 64, ... (k ascending, the move up before
// the move down); the wave takes the largest gain (a tie keeps the smaller k,
// then up) and adds delta * H[k][j] to every r_j.
constexpr int kMacaqMaxK = 80 * 64;
constexpr size_t kMacaqLds = 160 * 1024;

__host__ __device__ __forceinline__ size_t refine_wave_bytes(int64_t K) { return (size_t)K * 9 + (size_t)K / 32; }

__global__ __launch_bounds__(256) void macaq_refine_kernel(MacaqParams p, int64_t n0, int64_t rows, const double* R) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int64_t K = p.K;
  const int waves = (int)(blockDim.x >> 6), wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  double* diag = (double*)lds;
  double* r = (double*)(lds + (size_t)K * 8 + (size_t)wave * refine_wave_bytes(K));
  uint8_t* lv = (uint8_t*)(r + K);
  int8_t* ex = (int8_t*)(lv + K);
  for (int64_t k = threadIdx.x; k < K; k += blockDim.x) diag[k] = p.h[k * p.ldh + k];
  const int64_t nr = (int64_t)blockIdx.x * waves + wave;
  const bool live = nr < rows;
  const int64_t row = n0 + (live ? nr : 0);
  if (live) {
    for (int64_t k = lane; k < K; k += 64) {
      r[k] = R[nr * K + k];
      lv[k] = (uint8_t)level_of((p.codes[row * (K / 2) + k / 2] >> (4 * (k & 1))) & 0xFu);
    }
    for (int64_t b = lane; b < K / 32; b += 64) ex[b] = (int8_t)((int)p.scales[row * (K / 32) + b] - 127);
  }
  __syncthreads();
  if (!live) return;  // uniform per wave; no barrier follows
  // the gain of each one-level move of element j (up, then down; strict >
  // keeps the first, so a tie keeps the smaller j, then up) into the lane's
  // (best, bidx); the step between adjacent levels l and l + 1 is 2 for the
  // outer pairs (-6/-4, 4/6), 1 for -4/-3, -3/-2, 2/3, 3/4 and 0.5 otherwise
  double best = 0.0;
  int64_t bidx = INT64_MAX;  // 2 j + (0 up, 1 down)
  auto step_up = [](int l) -> double {
    const int t = l >= 7 ? l - 7 : 6 - l;
    return t < 4 ? 0.5 : (t < 6 ? 1.0 : 2.0);
  };
  auto consider = [&](int64_t j, double rj) {
    const int li = lv[j];
    const double sc = ldexp(1.0, ex[j / 32]);
    const double hjj = diag[j];
    if (li < 14) {
      const double delta = step_up(li) * sc;
      const double q = 2.0 * (delta * rj) + (delta * delta) * hjj;
      const double gain = -q;
      if (gain > best) {
        best = gain;
        bidx = 2 * j;
      }
    }
    if (li > 0) {
      const double delta = -step_up(li - 1) * sc;
      const double q = 2.0 * (delta * rj) + (delta * delta) * hjj;
      const double gain = -q;
      if (gain > best) {
        best = gain;
        bidx = 2 * j + 1;
      }
    }
  };
  // the wave's best: largest gain, then the smaller index
  auto wave_best = [&]() {
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
      const double og = shfl_xor_d(best, d);
      const int64_t oi = (int64_t)(((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)((uint64_t)bidx >> 32), d) << 32) |
                                   (uint32_t)__shfl_xor((int)(uint32_t)bidx, d));
      if (og > best || (og == best && oi < bidx)) {
        best = og;
        bidx = oi;
      }
    }
  };
  for (int64_t k = lane; k < K; k += 64) consider(k, r[k]);
  wave_best();
  // Each move: r_j += delta * H[k][j] for every j, and the next move's gains
  // from the updated r in the same pass.  Lane l owns j = l + 64 i; the row
  // of H comes in groups of kGroup elements per lane, the next group's loads
  // in flight while the current one is used.
  constexpr int kGroup = 16;
  const int64_t nper = (K + 63) / 64, ngroups = (nper + kGroup - 1) / kGroup;
  int64_t taken = 0;
  while (taken < p.max_moves && best > 0.0) {
    const int64_t k = bidx >> 1;
    const int li = lv[k];
    const int nl = (bidx & 1) ? li - 1 : li + 1;
    const double delta = ((bidx & 1) ? -step_up(nl) : step_up(li)) * ldexp(1.0, ex[k / 32]);
    const double* hrow = p.h + k * p.ldh;
    double cur[kGroup], nxt[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const int64_t j = lane + 64 * (int64_t)i;
      cur[i] = j < K ? hrow[j] : 0.0;
    }
    // the whole wave has read lv[k] before the write; LDS operations of one
    // wave complete in order, so the pass below sees the new level
    __builtin_amdgcn_wave_barrier();
    if (lane == (int)(k & 63)) lv[k] = (uint8_t)nl;
    __builtin_amdgcn_wave_barrier();
    best = 0.0;
    bidx = INT64_MAX;
    for (int64_t g = 0; g < ngroups; ++g) {
      if (g + 1 < ngroups) {
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
          const int64_t j = lane + 64 * ((g + 1) * kGroup + i);
          nxt[i] = j < K ? hrow[j] : 0.0;
        }
      }
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const int64_t j = lane + 64 * (g * kGroup + i);
        if (j < K) {
          const double rj = r[j] + delta * cur[i];
          r[j] = rj;
          consider(j, rj);
        }
      }
#pragma unroll
      for (int i = 0; i < kGroup; ++i) cur[i] = nxt[i];
    }
    wave_best();
    __builtin_amdgcn_wave_barrier();
    ++taken;
  }
  if (p.moves && lane == 0) p.moves[row] = (int32_t)taken;
  __builtin_amdgcn_wave_barrier();
  for (int64_t m = lane; m < K / 2; m += 64)
    p.codes[row * (K / 2) + m] = (uint8_t)(code_of(lv[2 * m]) | (code_of(lv[2 * m + 1]) << 4));
}

int refine_waves(int64_t K) {
  for (int w = 4; w > 1; --w)
    if ((size_t)K * 8 + (size_t)w * refine_wave_bytes(K) <= kMacaqLds) return w;
  return 1;
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
  const int waves = refine_waves(p.K);
  const size_t lds = (size_t)p.K * 8 + (size_t)waves * refine_wave_bytes(p.K);
  // the refinement's LDS can exceed the default limit of a launch
  e = hipFuncSetAttribute((const void*)macaq_refine_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMacaqLds);
  if (e != hipSuccess) return e;
  for (int64_t n0 = 0; n0 < p.N; n0 += chunk) {
    const int64_t rows = std::min(chunk, p.N - n0);
    const dim3 g((unsigned)((p.K + kHdTile - 1) / kHdTile), (unsigned)((rows + kHdTile - 1) / kHdTile));
    hipLaunchKernelGGL(macaq_hd_kernel, g, dim3(256), 0, s, p, n0, rows, R);
    hipLaunchKernelGGL(macaq_refine_kernel, dim3((unsigned)((rows + waves - 1) / waves)), dim3(64 * waves), lds, s, p,
                       n0, rows, (const double*)R);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp4q
