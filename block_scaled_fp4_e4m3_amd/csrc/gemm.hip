// W4A4 block-scaled matmul on gfx950 matrix cores.
//
// Pages: NVFP4 W4A4 -- "Why Gated DeltaNet Survives 4-Bit Quantization"
// review, section 1; RaZeR weight-activation GEMM -- RaZeR summary 2.3 (two
// tensor-core passes on Blackwell; here the special value decodes exactly, so
// one pass suffices); MXFP4 W4A4 -- MACaQ review, section 3.
//
// C[m][n] = RN32(g_a g_w) * sum_k A^[m][k] W^[n][k]; A^ is M x K and W^ is
// N x K (row n = output channel), both stored as packed codes (K/2 bytes per
// row) and per-block scale bytes, K contiguous ("NT" layout).
//
// Tiling.  A workgroup of 4 waves computes a 256 x 256 tile; each wave owns a
// 128 x 128 sub-tile as 4 x 4 MFMA 32x32 accumulators (256 FP32 per lane).
// K advances in stages of 128 elements: the packed codes (64 bytes per row)
// and scale bytes of both operands are loaded with coalesced 16-byte global
// loads into registers, written to one of two LDS buffers (row stride 80
// bytes, which keeps ds_read_b128 of 32 consecutive rows free of bank
// conflicts), and read back per wave while the next stage's loads are in
// flight.  Workgroup ids are remapped so that each XCD works on a contiguous,
// grouped range of tiles and its L2 sees shared operand panels.
//
// MXFP4: codes and E8M0 exponents go straight into the block-scaled FP4 MFMA
// (V_MFMA_SCALE_F32_32X32X64_F8F6F4); a lane supplies the 32 codes of one MX
// block of its row and that block's exponent byte.
//
// NVFP4 family: value * E4M3 (or E3M3) scale has at most 8 significant bits
// and lies in [2^-10, 3360], so it is exact in f16, and products of two are
// exact in FP32.  Each lane decodes 8 codes with the gfx950 FP4 -> f16
// convert (which applies only a power-of-two scale: 2^8 or 2^12) and one
// packed f16 multiply by the scale, whose f16 bit pattern is the scale byte
// shifted left by 7 (= scale * 2^-8 for E4M3, * 2^-12 for E3M3).  RaZeR's code
// 0x8 (-0 after the convert) is then replaced by special * scale.  The f16
// MFMA (32x32x16) accumulates in FP32.  Within each 64-element chunk the
// contraction index is permuted identically for both operands, so that the
// 8 codes a lane feeds one MFMA always lie in one 16-element block: lane
// (row, h) owns elements [32h, 32h + 32) of the chunk and MFMA j of the chunk
// takes its elements [8j, 8j + 8).
#include "fp4q_internal.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256;   // workgroup tile
constexpr int BK = 128;             // K elements per stage
constexpr int KB = BK / 2;          // code bytes per row per stage
constexpr int ROWB = KB + 16;       // LDS row stride of the codes
constexpr int SB = 8;               // LDS scale bytes per row per stage
constexpr int kXcds = 8;
constexpr int kGroupM = 8;          // tile rows per group in the tile order

struct Smem {
  uint8_t a[2][BM * ROWB];
  uint8_t w[2][BN * ROWB];
  uint8_t sa[2][BM * SB];
  uint8_t sw[2][BN * SB];
};

// ---------------------------------------------------------------- decode
template <int F>
__device__ __forceinline__ half8 decode8(uint32_t codes, uint32_t sb, const float* wspecial) {
  constexpr float kCvt = (F == RAZER_W) ? 4096.0f : 256.0f;
  const uint32_t k = (F == RAZER_W) ? (sb & 0x3Fu) : (sb & 0x7Fu);
  const _Float16 s16 = __builtin_bit_cast(_Float16, (uint16_t)(k << 7));
  const half2v s2 = {s16, s16};
  half8 out;
  static_for<0, 4>([&](auto ic) {
    constexpr int b = decltype(ic)::value;
    half2v v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, kCvt, b);
    v = v * s2;  // exact: value * scale
    out[2 * b] = v[0];
    out[2 * b + 1] = v[1];
  });
  if constexpr (F == RAZER_A || F == RAZER_W) {
    float v = (F == RAZER_A) ? ((sb & 0x80u) ? -5.0f : 5.0f) : wspecial[sb >> 6];
    const _Float16 vs = (_Float16)(v * kCvt) * s16;  // exact
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (((codes >> (4 * i)) & 15u) == 8u) out[i] = vs;
  }
  return out;
}

// ---------------------------------------------------------------- tile order
__device__ __forceinline__ void tile_coords(int64_t M, int64_t N, int& tm, int& tn) {
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  const int T = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  // workgroup bid runs on XCD bid % 8: give every XCD a contiguous range of tiles
  const int q = T / kXcds, r = T % kXcds;
  const int x = bid % kXcds, loc = bid / kXcds;
  const int t = x * q + min(x, r) + loc;
  // grouped order: kGroupM tile rows advance together along N
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group, first_m = g * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in = t % per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// ---------------------------------------------------------------- staging
struct Stage {
  uint4 a[4], w[4];
  uint2 sa, sw;
};

// 16 bytes of codes at byte offset `off` of a row holding `rowbytes` bytes;
// bytes past the row end read as zero codes
__device__ __forceinline__ uint4 load_codes16(const uint8_t* row, int64_t off, int64_t rowbytes) {
  if (off + 16 <= rowbytes) return *(const uint4*)(row + off);
  uint4 v = make_uint4(0, 0, 0, 0);
  if (off + 8 <= rowbytes) {
    uint2 h = *(const uint2*)(row + off);
    v.x = h.x;
    v.y = h.y;
  }
  return v;
}

// NS scale bytes (8 for 16-element blocks, 4 for 32-element blocks) of one
// row starting at block b0; blocks past the row read as 0 (they multiply zero codes)
template <int NS>
__device__ __forceinline__ uint2 load_scales(const uint8_t* row, int64_t b0, int64_t nblocks, bool vec) {
  if (vec && b0 + NS <= nblocks) {
    if constexpr (NS == 8) return *(const uint2*)(row + b0);
    else return make_uint2(*(const uint32_t*)(row + b0), 0u);
  }
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    uint32_t v = (b0 + i < nblocks) ? (uint32_t)row[b0 + i] : 0u;
    if (i < 4) lo |= v << (8 * i);
    else hi |= v << (8 * (i - 4));
  }
  return make_uint2(lo, hi);
}

template <int BLK>
__device__ __forceinline__ void load_stage(const GemmParams& p, int64_t m0, int64_t n0, int64_t k0, bool vec_scales,
                                           Stage& s) {
  const int t = threadIdx.x;
  const int64_t rowbytes = p.K / 2, nblocks = p.K / BLK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = i * kThreads + t;
    const int row = q >> 2, c16 = q & 3;
    const int64_t am = min(m0 + row, p.M - 1), wn = min(n0 + row, p.N - 1);
    const int64_t off = k0 / 2 + 16 * c16;
    s.a[i] = load_codes16(p.a_codes + am * rowbytes, off, rowbytes);
    s.w[i] = load_codes16(p.w_codes + wn * rowbytes, off, rowbytes);
  }
  constexpr int NS = BK / BLK;
  const int64_t am = min(m0 + t, p.M - 1), wn = min(n0 + t, p.N - 1);
  s.sa = load_scales<NS>(p.a_scales + am * nblocks, k0 / BLK, nblocks, vec_scales);
  s.sw = load_scales<NS>(p.w_scales + wn * nblocks, k0 / BLK, nblocks, vec_scales);
}

__device__ __forceinline__ void store_stage(Smem& sm, int buf, const Stage& s) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = i * kThreads + t;
    const int row = q >> 2, c16 = q & 3;
    *(uint4*)&sm.a[buf][row * ROWB + 16 * c16] = s.a[i];
    *(uint4*)&sm.w[buf][row * ROWB + 16 * c16] = s.w[i];
  }
  *(uint2*)&sm.sa[buf][t * SB] = s.sa;
  *(uint2*)&sm.sw[buf][t * SB] = s.sw;
}

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------- compute on one stage
template <int FA, int FW>
__device__ __forceinline__ void compute_stage_nv(const Smem& sm, int buf, int wm, int wn, const float* wspecial,
                                                 f32x16 (&acc)[4][4]) {
  const int lane = threadIdx.x & 63, r32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    uint4 ca[4], cw[4];
    uint32_t sa[4], sw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + 32 * i + r32, rw = wn * 128 + 32 * i + r32;
      ca[i] = *(const uint4*)&sm.a[buf][ra * ROWB + kc * 32 + kh * 16];
      cw[i] = *(const uint4*)&sm.w[buf][rw * ROWB + kc * 32 + kh * 16];
      sa[i] = *(const uint16_t*)&sm.sa[buf][ra * SB + kc * 4 + kh * 2];
      sw[i] = *(const uint16_t*)&sm.sw[buf][rw * SB + kc * 4 + kh * 2];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = decode8<FA>(u4_get(ca[i], j), (sa[i] >> (8 * (j >> 1))) & 0xFFu, nullptr);
        b[i] = decode8<FW>(u4_get(cw[i], j), (sw[i] >> (8 * (j >> 1))) & 0xFFu, wspecial);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[jj], acc[i][jj], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void compute_stage_mx(const Smem& sm, int buf, int wm, int wn, f32x16 (&acc)[4][4]) {
  const int lane = threadIdx.x & 63, r32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    i32x8 a[4], b[4];
    int sa[4], sw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + 32 * i + r32, rw = wn * 128 + 32 * i + r32;
      const uint4 ca = *(const uint4*)&sm.a[buf][ra * ROWB + kc * 32 + kh * 16];
      const uint4 cw = *(const uint4*)&sm.w[buf][rw * ROWB + kc * 32 + kh * 16];
      a[i] = (i32x8){(int)ca.x, (int)ca.y, (int)ca.z, (int)ca.w, 0, 0, 0, 0};
      b[i] = (i32x8){(int)cw.x, (int)cw.y, (int)cw.z, (int)cw.w, 0, 0, 0, 0};
      sa[i] = sm.sa[buf][ra * SB + kc * 2 + kh];
      sw[i] = sm.sw[buf][rw * SB + kc * 2 + kh];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[jj], acc[i][jj], 4, 4, 0, sa[i], 0,
                                                                     sw[jj]);
  }
}

// ---------------------------------------------------------------- kernel
// FA, FW: operand formats; FA == MXFP4 selects the block-scaled FP4 MFMA path
template <int FA, int FW, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_tile_kernel(GemmParams p) {
  constexpr bool MX = (FA == MXFP4);
  constexpr int BLK = MX ? 32 : 16;
  __shared__ __align__(16) Smem sm;
  int tm, tn;
  tile_coords(p.M, p.N, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t nblocks = p.K / BLK;
  constexpr int NS = BK / BLK;
  const bool vec_scales =
      (nblocks % NS == 0) && ((((uintptr_t)p.a_scales | (uintptr_t)p.w_scales) % (NS == 8 ? 8 : 4)) == 0);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};

  const int64_t nstages = (p.K + BK - 1) / BK;
  Stage st;
  load_stage<BLK>(p, m0, n0, 0, vec_scales, st);
  store_stage(sm, 0, st);
  __syncthreads();
  for (int64_t s = 0; s < nstages; ++s) {
    const int buf = (int)(s & 1);
    const bool more = s + 1 < nstages;
    if (more) load_stage<BLK>(p, m0, n0, (s + 1) * BK, vec_scales, st);
    if constexpr (MX) compute_stage_mx(sm, buf, wm, wn, acc);
    else compute_stage_nv<FA, FW>(sm, buf, wm, wn, p.w_special, acc);
    if (more) store_stage(sm, buf ^ 1, st);
    __syncthreads();
  }

  const float ga = p.a_global ? *p.a_global : 1.0f;
  const float gw = p.w_global ? *p.w_global : 1.0f;
  const float gg = ga * gw;
  const int r32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + 32 * j + r32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + 32 * i + (r / 4) * 8 + kh * 4 + (r % 4);
        if (row >= p.M || col >= p.N) continue;
        const float v = gg * acc[i][j][r];
        if constexpr (OUT_BF16) {
          uint32_t u = __float_as_uint(v);
          u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
          ((uint16_t*)p.c)[row * p.ldc + col] = (uint16_t)u;
        } else {
          ((float*)p.c)[row * p.ldc + col] = v;
        }
      }
    }
  }
}

template <int FA, int FW>
hipError_t launch_tile(const GemmParams& p, hipStream_t s) {
  const int64_t T = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (p.c_bf16) hipLaunchKernelGGL((gemm_tile_kernel<FA, FW, true>), dim3((unsigned)T), dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((gemm_tile_kernel<FA, FW, false>), dim3((unsigned)T), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int FA>
hipError_t launch_nv_a(int fw, const GemmParams& p, hipStream_t s) {
  switch (fw) {
    case RAZER_A: return launch_tile<FA, RAZER_A>(p, s);
    case RAZER_W: return launch_tile<FA, RAZER_W>(p, s);
    default: return launch_tile<FA, NVFP4>(p, s);
  }
}

}  // namespace

hipError_t launch_gemm(int fa, int fw, const GemmParams& p, hipStream_t s) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (fa == MXFP4) return launch_tile<MXFP4, MXFP4>(p, s);
  if (fa == RAZER_A) return launch_nv_a<RAZER_A>(fw, p, s);
  return launch_nv_a<NVFP4>(fw, p, s);
}

}  // namespace fp4q
