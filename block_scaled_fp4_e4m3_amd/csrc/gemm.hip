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
constexpr int kXcds = 8;
constexpr int kGroupM = 8;          // tile rows per group in the tile order

// Per-format stage geometry: K elements per stage, code bytes per row, LDS
// row stride (padded by 16 bytes against bank conflicts), scale bytes per row.
template <bool MX>
struct Geo {
  static constexpr int BLK = MX ? 32 : 16;    // elements per scale block
  static constexpr int BK = 128;               // K elements per stage
  static constexpr int KB = BK / 2;           // code bytes per row per stage
  static constexpr int ROWB = KB + 16;        // LDS row stride
  static constexpr int CPR = KB / 16;         // 16-byte chunks per row
  static constexpr int NCH = BM * CPR / kThreads;  // chunks per thread per operand
  static constexpr int NS = BK / BLK;         // scale bytes per row per stage
  static constexpr int NKC = BK / 64;         // 64-element chunks per stage
};

template <bool MX>
struct Smem {
  using G = Geo<MX>;
  uint8_t a[2][BM * G::ROWB];
  uint8_t w[2][BN * G::ROWB];
  uint8_t sa[2][BM * G::NS];
  uint8_t sw[2][BN * G::NS];
};

// ---------------------------------------------------------------- decode
// scale byte -> f16 bit pattern of scale * 2^-8 (E4M3) or scale * 2^-12 (E3M3)
template <int F>
__device__ __forceinline__ uint32_t scale_f16_bits(uint32_t sb) {
  return (F == RAZER_W ? (sb & 0x3Fu) : (sb & 0x7Fu)) << 7;
}

template <int F>
__device__ __forceinline__ half8 decode8(uint32_t codes, uint32_t s16bits, uint32_t sb, const float* wspecial) {
  constexpr float kCvt = (F == RAZER_W) ? 4096.0f : 256.0f;
  const _Float16 s16 = __builtin_bit_cast(_Float16, (uint16_t)s16bits);
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
// Each thread moves NCH 16-byte chunks of codes per operand per stage (chunk
// q = i * 256 + tid covers row q / CPR, bytes 16 * (q % CPR)) and the NS scale
// bytes of row tid.  Row indices past M (N) are clamped to the last row; those
// rows are computed and never stored.
template <bool MX>
struct Loader {
  using G = Geo<MX>;
  const uint8_t* a_base;     // codes of the tile's first row
  const uint8_t* w_base;
  const uint8_t* sa_row;     // scales of this thread's row
  const uint8_t* sw_row;
  uint32_t a_off[G::NCH], w_off[G::NCH];  // byte offsets of the chunks at k = 0
  int64_t rowbytes, nblocks;
  bool vec_scales;

  __device__ void init(const GemmParams& p, int64_t m0, int64_t n0) {
    const int t = threadIdx.x;
    rowbytes = p.K / 2;
    nblocks = p.K / G::BLK;
    a_base = p.a_codes + m0 * rowbytes;
    w_base = p.w_codes + n0 * rowbytes;
#pragma unroll
    for (int i = 0; i < G::NCH; ++i) {
      const int q = i * kThreads + t;
      const int row = q / G::CPR, c16 = q % G::CPR;
      const int64_t ra = min((int64_t)row, p.M - 1 - m0), rw = min((int64_t)row, p.N - 1 - n0);
      a_off[i] = (uint32_t)(ra * rowbytes + 16 * c16);
      w_off[i] = (uint32_t)(rw * rowbytes + 16 * c16);
    }
    sa_row = p.a_scales + min(m0 + t, p.M - 1) * nblocks;
    sw_row = p.w_scales + min(n0 + t, p.N - 1) * nblocks;
    vec_scales = (nblocks % G::NS == 0) && ((((uintptr_t)p.a_scales | (uintptr_t)p.w_scales) & 3u) == 0);
  }
};

template <bool MX>
struct Stage {
  static constexpr int NSW = Geo<MX>::NS / 4;  // 32-bit words of scale bytes per row
  uint4 a[Geo<MX>::NCH], w[Geo<MX>::NCH];
  uint32_t sa[NSW], sw[NSW];
};

// NS scale bytes of one row from block b0; blocks past the row read as 0
template <int NS>
__device__ __forceinline__ void scales_bytes(const uint8_t* row, int64_t b0, int64_t nblocks, uint32_t* out) {
#pragma unroll
  for (int w = 0; w < NS / 4; ++w) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t b = b0 + 4 * w + i;
      v |= (b < nblocks ? (uint32_t)row[b] : 0u) << (8 * i);
    }
    out[w] = v;
  }
}

// a stage entirely inside K: unconditional 16-byte loads
template <bool MX>
__device__ __forceinline__ void load_full(const Loader<MX>& L, int64_t k0, Stage<MX>& s) {
  using G = Geo<MX>;
  const uint8_t* ab = L.a_base + k0 / 2;
  const uint8_t* wb = L.w_base + k0 / 2;
#pragma unroll
  for (int i = 0; i < G::NCH; ++i) {
    s.a[i] = *(const uint4*)(ab + L.a_off[i]);
    s.w[i] = *(const uint4*)(wb + L.w_off[i]);
  }
  const int64_t b0 = k0 / G::BLK;
  if (L.vec_scales) {
#pragma unroll
    for (int w = 0; w < G::NS / 4; ++w) {
      s.sa[w] = *(const uint32_t*)(L.sa_row + b0 + 4 * w);
      s.sw[w] = *(const uint32_t*)(L.sw_row + b0 + 4 * w);
    }
  } else {
    scales_bytes<G::NS>(L.sa_row, b0, L.nblocks, s.sa);
    scales_bytes<G::NS>(L.sw_row, b0, L.nblocks, s.sw);
  }
}

// the last, partial stage: bytes past the row end read as zero codes
__device__ __forceinline__ uint4 load_codes_tail(const uint8_t* p, int64_t off, int64_t rowbytes) {
  uint4 v = make_uint4(0, 0, 0, 0);
  if (off + 16 <= rowbytes) return *(const uint4*)p;
  if (off + 8 <= rowbytes) {
    uint2 h = *(const uint2*)p;
    v.x = h.x;
    v.y = h.y;
  }
  return v;
}

template <bool MX>
__device__ __forceinline__ void load_tail(const Loader<MX>& L, int64_t k0, Stage<MX>& s) {
  using G = Geo<MX>;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < G::NCH; ++i) {
    const int c16 = (i * kThreads + t) % G::CPR;
    const int64_t off = k0 / 2 + 16 * c16;  // offset within the row
    s.a[i] = load_codes_tail(L.a_base + k0 / 2 + L.a_off[i], off, L.rowbytes);
    s.w[i] = load_codes_tail(L.w_base + k0 / 2 + L.w_off[i], off, L.rowbytes);
  }
  scales_bytes<G::NS>(L.sa_row, k0 / G::BLK, L.nblocks, s.sa);
  scales_bytes<G::NS>(L.sw_row, k0 / G::BLK, L.nblocks, s.sw);
}

template <bool MX>
__device__ __forceinline__ void store_stage(Smem<MX>& sm, int buf, const Stage<MX>& s) {
  using G = Geo<MX>;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < G::NCH; ++i) {
    const int q = i * kThreads + t;
    const int row = q / G::CPR, c16 = q % G::CPR;
    *(uint4*)&sm.a[buf][row * G::ROWB + 16 * c16] = s.a[i];
    *(uint4*)&sm.w[buf][row * G::ROWB + 16 * c16] = s.w[i];
  }
#pragma unroll
  for (int w = 0; w < G::NS / 4; ++w) {
    *(uint32_t*)&sm.sa[buf][t * G::NS + 4 * w] = s.sa[w];
    *(uint32_t*)&sm.sw[buf][t * G::NS + 4 * w] = s.sw[w];
  }
}

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// interleave: one MFMA, then n VALU instructions, `count` times
template <int COUNT, int NVALU>
__device__ __forceinline__ void interleave_mfma_valu() {
  static_for<0, COUNT>([&](auto) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);
  });
}

// ---------------------------------------------------------------- compute on one stage
// NVFP4 family: 2 chunks of 64 x 4 MFMA steps; the decode of step s+1 is
// interleaved with the 16 MFMAs of step s
template <int FA, int FW>
__device__ __forceinline__ void compute_stage_nv(const Smem<false>& sm, int buf, int wm, int wn,
                                                 const float* wspecial, f32x16 (&acc)[4][4]) {
  using G = Geo<false>;
  const int lane = threadIdx.x & 63, r32 = lane & 31, kh = lane >> 5;
  uint4 ca[2][4], cw[2][4];
  uint32_t sa[2][4], sw[2][4];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + 32 * i + r32, rw = wn * 128 + 32 * i + r32;
      ca[kc][i] = *(const uint4*)&sm.a[buf][ra * G::ROWB + kc * 32 + kh * 16];
      cw[kc][i] = *(const uint4*)&sm.w[buf][rw * G::ROWB + kc * 32 + kh * 16];
      sa[kc][i] = *(const uint16_t*)&sm.sa[buf][ra * G::NS + kc * 4 + kh * 2];
      sw[kc][i] = *(const uint16_t*)&sm.sw[buf][rw * G::NS + kc * 4 + kh * 2];
    }
  half8 da[2][4], db[2][4];
  auto decode_step = [&](int step, half8 (&a)[4], half8 (&b)[4]) {
    const int kc = step >> 2, j = step & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t sba = (sa[kc][i] >> (8 * (j >> 1))) & 0xFFu;
      const uint32_t sbw = (sw[kc][i] >> (8 * (j >> 1))) & 0xFFu;
      a[i] = decode8<FA>(u4_get(ca[kc][i], j), scale_f16_bits<FA>(sba), sba, nullptr);
      b[i] = decode8<FW>(u4_get(cw[kc][i], j), scale_f16_bits<FW>(sbw), sbw, wspecial);
    }
  };
  decode_step(0, da[0], db[0]);
  static_for<0, 8>([&](auto sc) {
    constexpr int step = decltype(sc)::value;
    constexpr int cur = step & 1;
    if constexpr (step + 1 < 8) decode_step(step + 1, da[cur ^ 1], db[cur ^ 1]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[cur][i], db[cur][jj], acc[i][jj], 0, 0, 0);
    if constexpr (step + 1 < 8) interleave_mfma_valu<16, 4>();
  });
}

// MXFP4: 4 chunks of 64 per stage, 16 block-scaled MFMAs per chunk
__device__ __forceinline__ void compute_stage_mx(const Smem<true>& sm, int buf, int wm, int wn,
                                                 f32x16 (&acc)[4][4]) {
  using G = Geo<true>;
  const int lane = threadIdx.x & 63, r32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int kc = 0; kc < G::NKC; ++kc) {
    uint4 ca[4], cw[4];
    int sa[4], sw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + 32 * i + r32, rw = wn * 128 + 32 * i + r32;
      ca[i] = *(const uint4*)&sm.a[buf][ra * G::ROWB + kc * 32 + kh * 16];
      cw[i] = *(const uint4*)&sm.w[buf][rw * G::ROWB + kc * 32 + kh * 16];
      sa[i] = sm.sa[buf][ra * G::NS + kc * 2 + kh];
      sw[i] = sm.sw[buf][rw * G::NS + kc * 2 + kh];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const i32x8 a = {(int)ca[i].x, (int)ca[i].y, (int)ca[i].z, (int)ca[i].w, 0, 0, 0, 0};
        const i32x8 b = {(int)cw[jj].x, (int)cw[jj].y, (int)cw[jj].z, (int)cw[jj].w, 0, 0, 0, 0};
        acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][jj], 4, 4, 0, sa[i], 0, sw[jj]);
      }
  }
}

// ---------------------------------------------------------------- kernel
// FA, FW: operand formats; FA == MXFP4 selects the block-scaled FP4 MFMA path
template <int FA, int FW, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_tile_kernel(GemmParams p) {
  constexpr bool MX = (FA == MXFP4);
  using G = Geo<MX>;
  __shared__ __align__(16) Smem<MX> sm;
  int tm, tn;
  tile_coords(p.M, p.N, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;

  Loader<MX> L;
  L.init(p, m0, n0);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};

  // stages entirely inside K run branch-free; the last stage may be partial
  const int64_t nfull = p.K / G::BK;
  const int64_t nstages = (p.K + G::BK - 1) / G::BK;
  Stage<MX> st;
  if (nfull > 0) load_full<MX>(L, 0, st);
  else load_tail<MX>(L, 0, st);
  store_stage<MX>(sm, 0, st);
  __syncthreads();
  auto compute = [&](int buf) {
    if constexpr (MX) compute_stage_mx(sm, buf, wm, wn, acc);
    else compute_stage_nv<FA, FW>(sm, buf, wm, wn, p.w_special, acc);
  };
  int64_t s = 0;
  for (; s + 1 < nfull; ++s) {          // next stage is a full one
    const int buf = (int)(s & 1);
    load_full<MX>(L, (s + 1) * G::BK, st);
    compute(buf);
    store_stage<MX>(sm, buf ^ 1, st);
    __syncthreads();
  }
  for (; s < nstages; ++s) {            // at most two stages: the last full one and the tail
    const int buf = (int)(s & 1);
    const bool more = s + 1 < nstages;
    if (more) load_tail<MX>(L, (s + 1) * G::BK, st);
    compute(buf);
    if (more) store_stage<MX>(sm, buf ^ 1, st);
    __syncthreads();
  }

  const float ga = p.a_global ? *p.a_global : 1.0f;
  const float gw = p.w_global ? *p.w_global : 1.0f;
  const float gg = ga * gw;
  const int r32 = lane & 31, kh = lane >> 5;
  const int64_t row0 = m0 + wm * 128, col0 = n0 + wn * 128;
  const bool inside = row0 + 128 <= p.M && col0 + 128 <= p.N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = col0 + 32 * j + r32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + 32 * i + (r / 4) * 8 + kh * 4 + (r % 4);
        if (!inside && (row >= p.M || col >= p.N)) continue;
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
