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
// 128 x 128 sub-tile as 4 x 4 MFMA 32x32 accumulators (256 FP32 per lane, in
// the accumulation registers).  K advances in stages of 128 elements.  When K
// and the operand alignment allow (K % 256 == 0, or 512 for MXFP4), global
// loads write the packed codes and scale bytes straight into LDS (LDS-DMA),
// two stages of each row per load; otherwise 16-byte buffer loads bring them
// into registers, which are written to one of two LDS stage buffers in MFMA
// fragment order (below), so that every fragment read is one ds_read_b128.
// Workgroup ids are remapped so that each XCD works on a contiguous, grouped
// range of tiles and its L2 sees shared operand panels.
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
#include "nv_encode.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <algorithm>
#include <mutex>
#include <map>

namespace fp4q {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256;   // workgroup tile

// global scale of output column col: the segment's, or w_global
__device__ __forceinline__ float col_w_global(const GemmParams& p, float gw, int64_t col) {
  if (p.nseg == 0) return gw;
  int sidx = 0;
#pragma unroll
  for (int i = 0; i < kMaxSegments - 1; ++i) sidx += (i < p.nseg - 1 && col >= p.seg_end[i]) ? 1 : 0;
  return p.seg_global[sidx];
}
constexpr int kXcds = 8;
constexpr int kGroupM = 8;          // tile rows per group in the tile order
constexpr int BK = 128;             // K elements per stage
constexpr int KB = BK / 2;          // code bytes per row per stage
constexpr int CPR = KB / 16;        // 16-byte code chunks per row per stage
constexpr int NCH = BM * CPR / kThreads;  // code chunks per thread per operand per stage
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer resource, gfx9 family

// ---------------------------------------------------------------- LDS stage layout
// One stage buffer: [A codes][W codes][A scales][W scales].
//   codes: 256 rows x 64 bytes as 16-byte slots.  Row r = 32 g + r32, chunk
//     c = 2 kc + kh (kc: 64-element chunk, kh: its half).  Slot
//     128 g + 32 c + (r32 ^ 4c): the 64 lanes (r32, kh) of a fragment read of
//     tile g, chunk kc touch 64 consecutive slots (one ds_read_b128 over a
//     contiguous KiB), and the XOR keeps the stores, where 16 consecutive
//     threads write 4 rows x 4 chunks, on 16 distinct slots mod 16.
//   scales: one dword per (row, kh), dword slot 64 g + 32 kh + r32, holding
//     the scale bytes lane (r32, kh) needs for the whole stage:
//     NVFP4 family: blocks 2kh, 2kh+1 (chunk 0), 4+2kh, 5+2kh (chunk 1);
//     MXFP4: blocks kh (chunk 0), 2+kh (chunk 1), then two zero bytes.
constexpr int kCodeBytes = BM * KB;                              // 16 KiB
constexpr int kScaleBytes = BM * 2 * 4;                          // 2 KiB
constexpr int kBufBytes = 2 * kCodeBytes + 2 * kScaleBytes;      // 36 KiB
constexpr int kNbuf = 2;

__device__ __forceinline__ int code_slot(int row, int c) {
  return (row >> 5) * 128 + c * 32 + ((row & 31) ^ (c << 2));
}

// ---------------------------------------------------------------- decode
// f16 bit patterns of scale * 2^-8 (E4M3) or scale * 2^-12 (E3M3) for the two
// scale bytes of chunk KC in a stage scale dword, packed in the two halves
template <int F, int KC>
__device__ __forceinline__ uint32_t scale_pair_f16(uint32_t raw4) {
  constexpr uint32_t m = (F == RAZER_W) ? 0x3Fu : 0x7Fu;
  const uint32_t two = __builtin_amdgcn_perm(0u, raw4, KC ? 0x0C030C02u : 0x0C010C00u);
  return (two & (m | (m << 16))) << 7;
}

// RaZeR: f16 patterns of special * scale * 2^-8 (or 2^-12) for the two blocks
// of chunk KC, from the chunk's scale pair and raw scale bytes.  RaZeR-A: the
// scale byte's top bit picks -5 or +5.  RaZeR-W: its top two bits index the
// four specials, held as f16 in sp_lo (specials 0, 1) and sp_hi (2, 3).
// Exact: special (at most 4 significant bits, a multiple of 1/2) times the
// scale pattern (at most 4 bits, a multiple of 2^-17) is a multiple of 2^-18
// with at most 8 significant bits.
template <int F, int KC>
__device__ __forceinline__ uint32_t special_pair_f16(uint32_t raw4, uint32_t scl2, uint32_t sp_lo, uint32_t sp_hi) {
  if constexpr (F == RAZER_A) {
    const half2v five = __builtin_bit_cast(half2v, scl2) * (half2v){(_Float16)5.0f, (_Float16)5.0f};
    // bytes 2KC, 2KC+1 to the high bytes of the two halves: their top bits are the signs
    const uint32_t sg = __builtin_amdgcn_perm(0u, raw4, KC ? 0x030C020Cu : 0x010C000Cu) & 0x80008000u;
    return __builtin_bit_cast(uint32_t, five) ^ sg;
  } else if constexpr (F == RAZER_W) {
    const uint32_t i0 = (raw4 >> (16 * KC + 6)) & 3u, i1 = (raw4 >> (16 * KC + 14)) & 3u;
    // byte selectors of the 8-byte table {sp_hi, sp_lo}: special i at bytes 2i, 2i+1
    const uint32_t sel = (2u * i0) | ((2u * i0 + 1u) << 8) | ((2u * i1) << 16) | ((2u * i1 + 1u) << 24);
    const half2v v = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(sp_hi, sp_lo, sel));
    return __builtin_bit_cast(uint32_t, v * __builtin_bit_cast(half2v, scl2));
  } else {
    return 0u;
  }
}

// 8 codes -> 8 f16 values value * scale; H selects the block (half of scl2).
// RaZeR: the convert turns code 0x8 into -0; a second word with code 0x2
// (+1.0) exactly there and 0 elsewhere is converted too and added times the
// block's special pattern (spec2, half H): u * special + v is special * scale
// at those codes (v = -0) and v elsewhere (u = +0), each exact.
template <int F, int H>
__device__ __forceinline__ half8 decode8(uint32_t codes, uint32_t scl2, uint32_t spec2) {
  constexpr float kCvt = (F == RAZER_W) ? 4096.0f : 256.0f;
  const _Float16 s16 = __builtin_bit_cast(half2v, scl2)[H];
  const half2v s2 = {s16, s16};
  uint32_t t = 0;
  half2v x2 = {};
  if constexpr (F == RAZER_A || F == RAZER_W) {
    const uint32_t y = codes ^ 0x88888888u;                          // nibble 0 where the code is 0x8
    const uint32_t nz = ((y & 0x77777777u) + 0x77777777u) | y;       // bit 3: nibble != 0
    t = (~nz & 0x88888888u) >> 2;                                    // 0x2 where the code is 0x8
    const _Float16 x16 = __builtin_bit_cast(half2v, spec2)[H];
    x2 = (half2v){x16, x16};
  }
  half8 out;
  static_for<0, 4>([&](auto ic) {
    constexpr int b = decltype(ic)::value;
    half2v v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, kCvt, b);
    v = v * s2;  // exact: value * scale
    if constexpr (F == RAZER_A || F == RAZER_W) {
      const half2v u = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(t, kCvt, b);
      v = __builtin_elementwise_fma(u, x2, v);
    }
    out[2 * b] = v[0];
    out[2 * b + 1] = v[1];
  });
  return out;
}

// ---------------------------------------------------------------- tile order
__device__ __forceinline__ void tile_coords(int64_t M, int64_t N, int bid, int& tm, int& tn) {
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  const int T = tiles_m * tiles_n;
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
// q = i * 256 + tid covers row q / 4, bytes 16 * (q % 4)) and the scale bytes
// of row tid.  Row indices past M (N) are clamped to the last row; those rows
// are computed and never stored.
template <bool MX>
struct Loader {
  static constexpr int BLK = MX ? 32 : 16;   // elements per scale block
  static constexpr int NS = BK / BLK;        // scale bytes per row per stage
  const uint8_t* a_base;     // codes of the tile's first row
  const uint8_t* w_base;
  const uint8_t* sa_row;     // scales of this thread's row
  const uint8_t* sw_row;
  __amdgpu_buffer_rsrc_t ra, rw, rsa, rsw;  // buffer views of the same
  uint32_t a_off[NCH], w_off[NCH];  // byte offsets of the chunks at k = 0
  uint32_t sa_off, sw_off;          // byte offsets of this thread's scale rows
  int64_t rowbytes, nblocks;
  bool vec_scales;

  __device__ void init(const GemmParams& p, int64_t m0, int64_t n0) {
    const int t = threadIdx.x;
    rowbytes = p.K / 2;
    nblocks = p.K / BLK;
    a_base = p.a_codes + m0 * rowbytes;
    w_base = p.w_codes + n0 * rowbytes;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = i * kThreads + t;
      const int row = q / CPR, c16 = q % CPR;
      const int64_t rA = min((int64_t)row, p.M - 1 - m0), rW = min((int64_t)row, p.N - 1 - n0);
      a_off[i] = (uint32_t)(rA * rowbytes + 16 * c16);
      w_off[i] = (uint32_t)(rW * rowbytes + 16 * c16);
    }
    const uint8_t* sa0 = p.a_scales + m0 * nblocks;
    const uint8_t* sw0 = p.w_scales + n0 * nblocks;
    sa_off = (uint32_t)(min((int64_t)t, p.M - 1 - m0) * nblocks);
    sw_off = (uint32_t)(min((int64_t)t, p.N - 1 - n0) * nblocks);
    sa_row = sa0 + sa_off;
    sw_row = sw0 + sw_off;
    ra = __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, -1, (int)kRsrcWord3);
    rw = __builtin_amdgcn_make_buffer_rsrc((void*)w_base, (short)0, -1, (int)kRsrcWord3);
    rsa = __builtin_amdgcn_make_buffer_rsrc((void*)sa0, (short)0, -1, (int)kRsrcWord3);
    rsw = __builtin_amdgcn_make_buffer_rsrc((void*)sw0, (short)0, -1, (int)kRsrcWord3);
    vec_scales = (nblocks % NS == 0) && ((((uintptr_t)p.a_scales | (uintptr_t)p.w_scales) & 3u) == 0);
  }
};

template <bool MX>
struct Stage {
  static constexpr int NSW = Loader<MX>::NS / 4;  // 32-bit words of scale bytes per row
  uint4 a[NCH], w[NCH];
  uint32_t sa[NSW], sw[NSW];
};

__device__ __forceinline__ uint4 as_uint4(u32x4 v) {
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Staging items of a stage: 0..3 the A code chunks, 4..7 the W code chunks,
// 8 the A scale words, 9 the W scale words.
constexpr int kItems = 2 * NCH + 2;

// items [I0, I1) of a stage entirely inside K with word-aligned scale rows:
// buffer loads whose only per-stage change is the scalar offset
template <bool MX, int I0 = 0, int I1 = kItems>
__device__ __forceinline__ void load_fast(const Loader<MX>& L, int64_t k0, Stage<MX>& s) {
  const int kb = (int)(k0 / 2), b0 = (int)(k0 / Loader<MX>::BLK);
  static_for<I0, I1>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i < NCH) {
      s.a[i] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(L.ra, (int)L.a_off[i], kb, 0));
    } else if constexpr (i < 2 * NCH) {
      s.w[i - NCH] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(L.rw, (int)L.w_off[i - NCH], kb, 0));
    } else {
      const __amdgpu_buffer_rsrc_t r = (i == 2 * NCH) ? L.rsa : L.rsw;
      const int off = (int)((i == 2 * NCH) ? L.sa_off : L.sw_off);
      uint32_t* dst = (i == 2 * NCH) ? s.sa : s.sw;
      if constexpr (MX) {
        dst[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, b0, 0);
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, b0, 0);
        dst[0] = v[0];
        dst[1] = v[1];
      }
    }
  });
}

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

// any stage: per-chunk bounds and byte-wise scale loads
template <bool MX>
__device__ __forceinline__ void load_any(const Loader<MX>& L, int64_t k0, Stage<MX>& s) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c16 = (i * kThreads + t) % CPR;
    const int64_t off = k0 / 2 + 16 * c16;  // offset within the row
    s.a[i] = load_codes_tail(L.a_base + k0 / 2 + L.a_off[i], off, L.rowbytes);
    s.w[i] = load_codes_tail(L.w_base + k0 / 2 + L.w_off[i], off, L.rowbytes);
  }
  scales_bytes<Loader<MX>::NS>(L.sa_row, k0 / Loader<MX>::BLK, L.nblocks, s.sa);
  scales_bytes<Loader<MX>::NS>(L.sw_row, k0 / Loader<MX>::BLK, L.nblocks, s.sw);
}

// items [I0, I1) of a stage -> LDS buffer at `buf` in fragment order
template <bool MX, int I0 = 0, int I1 = kItems>
__device__ __forceinline__ void store_stage(uint8_t* buf, const Stage<MX>& s) {
  const int t = threadIdx.x;
  uint8_t* ca = buf + code_slot(t / CPR, t % CPR) * 16;
  uint32_t* sc = (uint32_t*)(buf + 2 * kCodeBytes) + (t >> 5) * 64 + (t & 31);
  static_for<I0, I1>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i < NCH) {  // chunk i holds rows 64 i + t / 4: slot + 256 i
      *(uint4*)(ca + i * 4096) = s.a[i];
    } else if constexpr (i < 2 * NCH) {
      *(uint4*)(ca + kCodeBytes + (i - NCH) * 4096) = s.w[i - NCH];
    } else {
      const uint32_t* src = (i == 2 * NCH) ? s.sa : s.sw;
      uint32_t* d = sc + ((i == 2 * NCH) ? 0 : kScaleBytes / 4);
      if constexpr (MX) {
        d[0] = __builtin_amdgcn_perm(0u, src[0], 0x0C0C0200u);
        d[32] = __builtin_amdgcn_perm(0u, src[0], 0x0C0C0301u);
      } else {
        d[0] = __builtin_amdgcn_perm(src[1], src[0], 0x05040100u);
        d[32] = __builtin_amdgcn_perm(src[1], src[0], 0x07060302u);
      }
    }
  });
}

// LDS-only workgroup barrier: waits for this wave's LDS operations, not for
// its global loads in flight
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Scheduling of one MFMA step (16 MFMAs): each MFMA is followed by up to one
// LDS write, one global load and one LDS read (for the first NDSW / NVMEM /
// NDSR MFMAs) and NVALU vector instructions; nothing crosses the step.
template <int NDSW, int NVMEM, int NDSR, int NVALU>
__device__ __forceinline__ void sched_step() {
  static_for<0, 16>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (k < NDSW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    if constexpr (k < NVMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    if constexpr (k < NDSR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);
  });
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------- NVFP4-family K loop
// Per-wave registers: the codes of the stage's two chunks for the wave's 4 A
// row tiles and 4 W column tiles, the stage scale dwords, and the f16 scale
// pairs of each chunk.
struct NvRegs {
  uint4 ca0[4], cw0[4], ca1[4], cw1[4];
  uint32_t ra[4], rw[4];     // stage scale dwords (read one stage ahead)
  uint32_t pa0[4], pw0[4], pa1[4], pw1[4];  // f16 scale pairs per chunk
  uint32_t xa0[4], xw0[4], xa1[4], xw1[4];  // f16 special pairs per chunk (RaZeR)
};

struct NvAddr {   // per-lane LDS byte offsets within a stage buffer
  uint32_t a[2], w[2];  // code fragment of tile 0, chunk kc
  uint32_t sa, sw;      // scale dword of tile 0
};

__device__ __forceinline__ void read_codes(const uint8_t* buf, const NvAddr& ad, int kc, uint4 (&ca)[4], uint4 (&cw)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ca[i] = *(const uint4*)(buf + ad.a[kc] + i * 2048);
    cw[i] = *(const uint4*)(buf + ad.w[kc] + i * 2048);
  }
}

__device__ __forceinline__ void read_scales(const uint8_t* buf, const NvAddr& ad, uint32_t (&ra)[4], uint32_t (&rw)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = *(const uint32_t*)(buf + ad.sa + i * 256);
    rw[i] = *(const uint32_t*)(buf + ad.sw + i * 256);
  }
}

// decode of MFMA step J (0..3) of a chunk: codes word J, scale block J / 2
template <int FA, int FW, int J>
__device__ __forceinline__ void decode_step(const uint4 (&ca)[4], const uint4 (&cw)[4], const uint32_t (&pa)[4],
                                            const uint32_t (&pw)[4], const uint32_t (&xa)[4], const uint32_t (&xw)[4],
                                            half8 (&a)[4], half8 (&b)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = decode8<FA, J / 2>(u4_get(ca[i], J), pa[i], xa[i]);
    b[i] = decode8<FW, J / 2>(u4_get(cw[i], J), pw[i], xw[i]);
  }
}

__device__ __forceinline__ void mfma_step(const half8 (&a)[4], const half8 (&b)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// Placement of the staging work over the 8 MFMA steps of a stage: step t
// stores items [store_at[t], store_at[t+1]) of stage s+1 to LDS and issues
// the global loads of items [load_at[t], load_at[t+1]) of stage s+2 (an item
// is loaded no earlier than the step that stores its register); chunk-1 codes
// are read at step read1 (7: stage s+1's, one stage ahead; 1: stage s's).
struct NvPlan {
  static constexpr int store_at[9] = {0, 6, 10, 10, 10, 10, 10, 10, 10};
  static constexpr int load_at[9] = {0, 0, 2, 4, 6, 8, 10, 10, 10};
  static constexpr int read1 = 7;
};

template <class P>
constexpr int plan_ds_writes(int t) {
  int n = 0;
  for (int i = P::store_at[t]; i < P::store_at[t + 1]; ++i) n += (i < 2 * NCH) ? 1 : 2;
  return n;
}

// every item is reloaded no earlier than the step that stores it, and all
// stores are issued by the first load step (the generic stage loads all items
// there)
template <class P>
constexpr bool plan_valid() {
  int first_load = -1;
  for (int t = 0; t < 8; ++t) {
    if (first_load < 0 && P::load_at[t] < P::load_at[t + 1]) first_load = t;
    for (int i = P::load_at[t]; i < P::load_at[t + 1]; ++i)
      if (!(P::store_at[t + 1] > i)) return false;
  }
  return P::store_at[0] == 0 && P::store_at[8] == kItems && P::load_at[0] == 0 && P::load_at[8] == kItems &&
         first_load >= 0 && P::store_at[first_load + 1] == kItems && (P::read1 == 7 || P::read1 == 1);
}

// The K loop, software-pipelined across stages.  A stage is 128 elements =
// 2 chunks x 4 MFMA steps; stage x lives in LDS buffer x % 2.  While the 16
// MFMAs of step t run, the wave decodes step t + 1 (step 7 decodes the first
// step of the next stage).  Within stage s:
//   steps per NvPlan: store the registers holding stage s+1 into its LDS
//           buffer (last read during stage s-1 or s-2, before an earlier
//           barrier), then reload them with the global loads of stage s+2;
//   steps 0-1: f16 scale pairs of chunk 1;  end of step 2: LDS barrier;
//   step 3: read stage s+1's scale dwords and chunk-0 codes;
//   steps 4-5: f16 scale pairs of stage s+1 chunk 0;
//   step NvPlan::read1: chunk-1 codes.
// Every LDS read is used at least two steps after it is issued.
template <int FA, int FW, class P = NvPlan>
__device__ __forceinline__ void nv_tile(const GemmParams& p, int64_t m0, int64_t n0, uint8_t* smem, int wm, int wn,
                                        int64_t sbeg, int64_t send, f32x16 (&acc)[4][4]) {
  constexpr bool RZ = (FA == RAZER_A || FW == RAZER_A || FW == RAZER_W);  // special values in the decode
  static_assert(plan_valid<P>(), "staging plan");
  Loader<false> L;
  L.init(p, m0, n0);
  // this workgroup's stages [sbeg, send) of the K loop; local stage s starts
  // at element kb + s * BK, and the first nfull local stages lie inside K
  const int64_t kb = sbeg * BK, nstages = send - sbeg, nfull = min(send, p.K / BK) - sbeg;
  const int lane = threadIdx.x & 63, r32 = lane & 31, kh = lane >> 5;
  NvAddr ad;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const int c = 2 * kc + kh;
    const uint32_t o = (uint32_t)(c * 32 + (r32 ^ (c << 2))) * 16;
    ad.a[kc] = o + wm * 4 * 2048;
    ad.w[kc] = o + kCodeBytes + wn * 4 * 2048;
  }
  ad.sa = 2 * kCodeBytes + (wm * 4 * 64 + lane) * 4;
  ad.sw = 2 * kCodeBytes + kScaleBytes + (wn * 4 * 64 + lane) * 4;

  Stage<false> st;
  auto gload = [&](int64_t stg) {
    if (stg < nfull && L.vec_scales) load_fast<false>(L, kb + stg * BK, st);
    else load_any<false>(L, kb + stg * BK, st);
  };
  gload(0);
  store_stage<false>(smem, st);
  if (nstages > 1) gload(1);
  lds_barrier();
  // RaZeR-W specials as f16 (exact: multiples of 1/2 up to 7.5), two per word
  const uint32_t sp_lo = __builtin_bit_cast(uint32_t, (half2v){(_Float16)p.w_special[0], (_Float16)p.w_special[1]});
  const uint32_t sp_hi = __builtin_bit_cast(uint32_t, (half2v){(_Float16)p.w_special[2], (_Float16)p.w_special[3]});
  NvRegs R;
  read_scales(smem, ad, R.ra, R.rw);
  read_codes(smem, ad, 0, R.ca0, R.cw0);
  if constexpr (P::read1 == 7) read_codes(smem, ad, 1, R.ca1, R.cw1);
  // f16 scale (and special) pairs of chunk KC of the dwords in R.ra / R.rw
  auto prep_a = [&](auto kc_tag, uint32_t (&pa)[4], uint32_t (&xa)[4]) {
    constexpr int KC = decltype(kc_tag)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa[i] = scale_pair_f16<FA, KC>(R.ra[i]);
      if constexpr (RZ) xa[i] = special_pair_f16<FA, KC>(R.ra[i], pa[i], sp_lo, sp_hi);
    }
  };
  auto prep_w = [&](auto kc_tag, uint32_t (&pw)[4], uint32_t (&xw)[4]) {
    constexpr int KC = decltype(kc_tag)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = scale_pair_f16<FW, KC>(R.rw[i]);
      if constexpr (RZ) xw[i] = special_pair_f16<FW, KC>(R.rw[i], pw[i], sp_lo, sp_hi);
    }
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  prep_a(K0{}, R.pa0, R.xa0);
  prep_w(K0{}, R.pw0, R.xw0);
  half8 da[2][4], db[2][4];
  decode_step<FA, FW, 0>(R.ca0, R.cw0, R.pa0, R.pw0, R.xa0, R.xw0, da[0], db[0]);

  // FAST: stages s with s + 2 < nfull and word-aligned scales (branch-free);
  // the others check whether stage s+1 / s+2 exist.  On the last stage the
  // reads of the next stage read a stale buffer, which is harmless.
  auto stage = [&](int64_t s, auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    uint8_t* nbuf = smem + ((s + 1) & 1) * kBufBytes;   // stage s+1
    const uint8_t* cbuf = smem + (s & 1) * kBufBytes;   // stage s
    static_for<0, 8>([&](auto tc) {
      constexpr int t = decltype(tc)::value, cur = t & 1;
      constexpr int st0 = P::store_at[t], st1 = P::store_at[t + 1];
      constexpr int ld0 = P::load_at[t], ld1 = P::load_at[t + 1];
      if constexpr (st0 < st1) {
        if (FAST || s + 1 < nstages) store_stage<false, st0, st1>(nbuf, st);
      }
      if constexpr (ld0 < ld1) {
        if constexpr (FAST) load_fast<false, ld0, ld1>(L, kb + (s + 2) * BK, st);
        else if (ld0 == 0 && s + 2 < nstages) gload(s + 2);
      }
      if constexpr (t == 0) prep_a(K1{}, R.pa1, R.xa1);  // chunk-1 pairs, A at step 0, W at step 1
      if constexpr (t == 1) prep_w(K1{}, R.pw1, R.xw1);
      if constexpr (t == P::read1) {
        if constexpr (t == 7) read_codes(nbuf, ad, 1, R.ca1, R.cw1);
        else read_codes(cbuf, ad, 1, R.ca1, R.cw1);
      }
      if constexpr (t == 3) {
        read_scales(nbuf, ad, R.ra, R.rw);
        read_codes(nbuf, ad, 0, R.ca0, R.cw0);
      }
      if constexpr (t == 4) prep_a(K0{}, R.pa0, R.xa0);  // next stage's chunk-0 pairs
      if constexpr (t == 5) prep_w(K0{}, R.pw0, R.xw0);
      // decode of step t + 1
      if constexpr (t < 3)
        decode_step<FA, FW, t + 1>(R.ca0, R.cw0, R.pa0, R.pw0, R.xa0, R.xw0, da[cur ^ 1], db[cur ^ 1]);
      else if constexpr (t < 7)
        decode_step<FA, FW, t - 3>(R.ca1, R.cw1, R.pa1, R.pw1, R.xa1, R.xw1, da[cur ^ 1], db[cur ^ 1]);
      else
        decode_step<FA, FW, 0>(R.ca0, R.cw0, R.pa0, R.pw0, R.xa0, R.xw0, da[cur ^ 1], db[cur ^ 1]);
      mfma_step(da[cur], db[cur], acc);
      if constexpr (FAST) {
        constexpr int ndsr = (t == 3 ? 16 : 0) + (t == P::read1 ? 8 : 0);
        constexpr int extra = (t == 0 || t == 1 || t == 4 || t == 5) || plan_ds_writes<P>(t) > 8 ? 5 : 4;
        sched_step<plan_ds_writes<P>(t), ld1 - ld0, ndsr, extra>();
      }
      if constexpr (t == 2) lds_barrier();
    });
  };
  int64_t s = 0;
  if (L.vec_scales)
    for (; s + 2 < nfull; ++s) stage(s, std::true_type{});
  for (; s < nstages; ++s) stage(s, std::false_type{});
}

// ---------------------------------------------------------------- MXFP4 K loop
// 8 block-scaled MFMAs: chunk KC, A tiles I0 and I0 + 1 x the 4 W tiles; the
// MFMA takes the stage scale dword and selects the chunk's byte
template <int KC, int I0>
__device__ __forceinline__ void mx_mfma_half(const uint4 (&ca)[4], const uint4 (&cw)[4], const uint32_t (&sa)[4],
                                             const uint32_t (&sw)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = I0; i < I0 + 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const i32x8 a = {(int)ca[i].x, (int)ca[i].y, (int)ca[i].z, (int)ca[i].w, 0, 0, 0, 0};
      const i32x8 b = {(int)cw[j].x, (int)cw[j].y, (int)cw[j].z, (int)cw[j].w, 0, 0, 0, 0};
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 4, 4, KC, (int)sa[i], KC, (int)sw[j]);
    }
}

template <int NDSW, int NVMEM, int NDSR>
__device__ __forceinline__ void sched_mx_step() {
  static_for<0, 8>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (k < NDSW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    if constexpr (k < NVMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    if constexpr (k < NDSR) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  });
  __builtin_amdgcn_sched_barrier(0);
}

// global loads of stage s+3 in MXFP4 stage s: items [0, load_at[1]) at step 1,
// [load_at[1], load_at[2]) at step 2, the rest at step 3
struct MxPlan {
  static constexpr int load_at[3] = {0, 5, 10};
};

// The MXFP4 K loop, pipelined across stages like the NVFP4 one.  A stage is
// 2 chunks = 4 steps of 8 MFMAs (a quarter of an NVFP4 stage's time), so the
// global loads run further ahead: two register staging sets alternate by
// stage parity, and stage s stores set s % 2 (stage s+1, loaded during stage
// s-2) and then reloads it with stage s+3.  Stage x lives in LDS buffer x % 2.
// Within stage s:
//   step 0: read stage s's chunk-1 codes; store the first items of stage s+1;
//   step 1: store the rest; issue the first global loads of stage s+3; end
//           of step 1: LDS barrier;
//   step 2: keep stage s's scale dwords for chunk 1, read stage s+1's scale
//           dwords and chunk-0 codes; issue the remaining global loads.
// Chunk-0 and chunk-1 codes are read two steps before use.
__device__ __forceinline__ void mx_tile(const GemmParams& p, int64_t m0, int64_t n0, uint8_t* smem, int wm, int wn,
                                        int64_t sbeg, int64_t send, f32x16 (&acc)[4][4]) {
  Loader<true> L;
  L.init(p, m0, n0);
  const int lane = threadIdx.x & 63, r32 = lane & 31, kh = lane >> 5;
  NvAddr ad;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const int c = 2 * kc + kh;
    const uint32_t o = (uint32_t)(c * 32 + (r32 ^ (c << 2))) * 16;
    ad.a[kc] = o + wm * 4 * 2048;
    ad.w[kc] = o + kCodeBytes + wn * 4 * 2048;
  }
  ad.sa = 2 * kCodeBytes + (wm * 4 * 64 + lane) * 4;
  ad.sw = 2 * kCodeBytes + kScaleBytes + (wn * 4 * 64 + lane) * 4;
  const int64_t kb = sbeg * BK, nstages = send - sbeg, nfull = min(send, p.K / BK) - sbeg;
  Stage<true> st[2];
  auto gload = [&](int64_t stg, Stage<true>& dst) {
    if (stg < nfull && L.vec_scales) load_fast<true>(L, kb + stg * BK, dst);
    else load_any<true>(L, kb + stg * BK, dst);
  };
  gload(0, st[0]);
  store_stage<true>(smem, st[0]);
  if (nstages > 1) gload(1, st[0]);
  if (nstages > 2) gload(2, st[1]);
  lds_barrier();
  uint4 ca0[4], cw0[4], ca1[4], cw1[4];
  uint32_t sa[4], sw[4], qa[4], qw[4];
  read_scales(smem, ad, sa, sw);
  read_codes(smem, ad, 0, ca0, cw0);

  auto stage = [&](int64_t s, auto fast_tag, auto par_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    Stage<true>& sg = st[PAR];
    uint8_t* nbuf = smem + ((s + 1) & 1) * kBufBytes;   // stage s+1
    const uint8_t* cbuf = smem + (s & 1) * kBufBytes;   // stage s
    // step 0
    read_codes(cbuf, ad, 1, ca1, cw1);
    if (FAST || s + 1 < nstages) store_stage<true, 0, 6>(nbuf, sg);
    mx_mfma_half<0, 0>(ca0, cw0, sa, sw, acc);
    if constexpr (FAST) sched_mx_step<6, 0, 4>();
    // step 1
    if (FAST || s + 1 < nstages) store_stage<true, 6, kItems>(nbuf, sg);
    if constexpr (FAST) load_fast<true, 0, MxPlan::load_at[1]>(L, kb + (s + 3) * BK, sg);
    else if (s + 3 < nstages) gload(s + 3, sg);
    mx_mfma_half<0, 2>(ca0, cw0, sa, sw, acc);
    if constexpr (FAST) sched_mx_step<6, MxPlan::load_at[1], 0>();
    lds_barrier();
    // step 2
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qa[i] = sa[i];
      qw[i] = sw[i];
    }
    read_scales(nbuf, ad, sa, sw);
    read_codes(nbuf, ad, 0, ca0, cw0);
    if constexpr (FAST) load_fast<true, MxPlan::load_at[1], MxPlan::load_at[2]>(L, kb + (s + 3) * BK, sg);
    mx_mfma_half<1, 0>(ca1, cw1, qa, qw, acc);
    if constexpr (FAST) sched_mx_step<0, MxPlan::load_at[2] - MxPlan::load_at[1], 8>();
    // step 3
    if constexpr (FAST) load_fast<true, MxPlan::load_at[2], kItems>(L, kb + (s + 3) * BK, sg);
    mx_mfma_half<1, 2>(ca1, cw1, qa, qw, acc);
    if constexpr (FAST) sched_mx_step<0, kItems - MxPlan::load_at[2], 0>();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int64_t s = 0;
  if (L.vec_scales)
    for (; s + 4 < nfull; s += 2) {   // stages s, s+1 load stages s+3, s+4
      stage(s, std::true_type{}, P0{});
      stage(s + 1, std::true_type{}, P1{});
    }
  for (; s < nstages; s += 2) {       // s is even here
    stage(s, std::false_type{}, P0{});
    if (s + 1 < nstages) stage(s + 1, std::false_type{}, P1{});
  }
}

// ---------------------------------------------------------------- MXFP4 K loop, LDS-DMA staging
// For MXFP4 with K % 512 == 0, 16-byte aligned code and scale rows.  Global
// loads write LDS directly (buffer_load ... lds: lane l of a load lands 16 l
// bytes past the wave's LDS address), so staging needs no registers and no
// LDS store instructions.  Codes are loaded per pair of stages (128 bytes,
// one cache line, of each row) into two pair buffers; the loads of pair
// (s + 3) / 2 start right after the barrier of odd stage s.
//   codes: 1 KiB block B holds rows 8 B .. 8 B + 7, 16-byte chunk ch (0-3:
//     the pair's first stage, 4-7: its second) of row 8 B + r7 at slot
//     64 B + 8 r7 + (ch ^ x), x = (r7 / 2) | (B % 2) * 4.  Load unit B (one
//     wave instruction) fills block B: lane l fetches row 8 B + l / 8, chunk
//     (l % 8) ^ x, so each eight lanes read one row's line.  A fragment read
//     of tile g, chunk kc of half h (lane (r32, kh): row 32 g + r32, chunk
//     4 h + 2 kc + kh) covers blocks 4 g .. 4 g + 3, and any 16 consecutive
//     lanes hit 16 distinct slots mod 16.
//   scales: loaded per group of four stages, 16 bytes of each row (the four
//     stages' E8M0 bytes, four per stage) at 16 r, in two group buffers.
//     Lane (r32, kh) reads its row's dword of the stage and shifts it right
//     by 8 kh, so that the MFMA's byte select 2 kc picks block 2 kc + kh.
constexpr int kDlCodes = BM * 2 * KB;                      // 32 KiB per operand per pair of stages
constexpr int kDlBuf = 2 * kDlCodes;                       // 64 KiB
constexpr int kDlNbuf = 2;
constexpr int kDlGroup = 4;                                // stages per scale load
constexpr int kDlScales = 2 * BM * 16;                     // one group's scales, both operands: 8 KiB
constexpr int kDlLds = kDlNbuf * kDlBuf + 2 * kDlScales;   // 144 KiB
constexpr int kDlPairLoads = 16;                           // code loads per wave per pair
typedef __attribute__((address_space(3))) void* lds_ptr;

// Workgroup barrier of the LDS-DMA ring: this wave's LDS reads complete and
// at most N of its loads still in flight (the newest), then all waves meet.
// A release fence would also wait for every load in flight (they write LDS),
// so the wait is explicit; the empty asm statements keep the compiler from
// moving memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void dl_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));  // vmcnt N, lgkmcnt 0
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct DlLoader {
  // per-lane offsets are recomputed from the thread index at each issue (a
  // few VALU per pair), so that they hold no registers across the K loop
  __amdgpu_buffer_rsrc_t ra, rw, rsa, rsw;
  uint32_t lastA, lastW;        // last valid row of the A and W panels (rows past it are clamped)
  uint32_t rowbytes;            // K / 2
  uint32_t nblocks;             // scale bytes per row
  int wv;                       // wave index (uniform)

  int blk;                      // elements per scale byte (32 MXFP4, 16 NVFP4 family)

  __device__ void init(const GemmParams& p, int64_t m0, int64_t n0, int block) {
    const int t = threadIdx.x, lane = t & 63;
    wv = __builtin_amdgcn_readfirstlane(t >> 6);
    blk = block;
    nblocks = (uint32_t)(p.K / block);
    rowbytes = (uint32_t)(p.K / 2);
    lastA = (uint32_t)min(p.M - 1 - m0, (int64_t)255);
    lastW = (uint32_t)min(p.N - 1 - n0, (int64_t)255);
    (void)lane;
    ra = __builtin_amdgcn_make_buffer_rsrc((void*)(p.a_codes + m0 * (int64_t)rowbytes), (short)0, -1,
                                           (int)kRsrcWord3);
    rw = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w_codes + n0 * (int64_t)rowbytes), (short)0, -1,
                                           (int)kRsrcWord3);
    rsa = __builtin_amdgcn_make_buffer_rsrc((void*)(p.a_scales + m0 * (int64_t)nblocks), (short)0, -1,
                                            (int)kRsrcWord3);
    rsw = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w_scales + n0 * (int64_t)nblocks), (short)0, -1,
                                            (int)kRsrcWord3);
  }

  // the kDlPairLoads code loads of the pair of stages at k0 into the pair
  // buffer `buf`: blocks 8 wv .. 8 wv + 7 of each operand
  // (block 8 wv + j: row 8 (8 wv + j) + lane / 8, clamped, chunk bits of the
  // block's parity; offsets below 2^32: at most 255 rows of K / 2 <= 2^23 bytes)
  __device__ __forceinline__ void issue_pair(uint8_t* buf, int64_t k0) const {
    const int kb = (int)(k0 / 2);
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t lrow = 64 * (threadIdx.x >> 6) + (lane >> 3);  // this lane's row in the first block
    const uint32_t chb = 16 * ((lane & 7) ^ (lane >> 4));          // its chunk in even blocks (odd: ^ 64)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t off = __umul24(min(lrow + 8 * j, lastA), rowbytes) + (chb ^ ((j & 1) * 64));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(buf + (8 * wv + j) * 1024), 16, off, kb, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t off = __umul24(min(lrow + 8 * j, lastW), rowbytes) + (chb ^ ((j & 1) * 64));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr)(buf + kDlCodes + (8 * wv + j) * 1024), 16, off, kb,
                                               0, 0);
    }
  }

  // the two scale loads (A, W) of 16 bytes of each row from element k0 into
  // `sbuf`: rows 64 wv + lane, A at 16 row, W at 16 (BM + row)
  __device__ __forceinline__ void issue_scales(uint8_t* sbuf, int64_t k0) const {
    const int b0 = (int)(k0 / blk);
    const uint32_t sa_off = __umul24(min(threadIdx.x, lastA), nblocks);
    const uint32_t sw_off = __umul24(min(threadIdx.x, lastW), nblocks);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr)(sbuf + 1024 * wv), 16, sa_off, b0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_ptr)(sbuf + BM * 16 + 1024 * wv), 16, sw_off, b0, 0, 0);
  }
};

// 8 block-scaled MFMAs of chunk KC, A tiles I0 and I0 + 1 x the 4 W tiles;
// the lane's scale dwords are pre-shifted, byte 2 KC is the chunk's block
template <int KC, int I0>
__device__ __forceinline__ void mx_mfma_half_dl(const uint4 (&ca)[4], const uint4 (&cw)[4], const uint32_t (&sa)[4],
                                                const uint32_t (&sw)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = I0; i < I0 + 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const i32x8 a = {(int)ca[i].x, (int)ca[i].y, (int)ca[i].z, (int)ca[i].w, 0, 0, 0, 0};
      const i32x8 b = {(int)cw[j].x, (int)cw[j].y, (int)cw[j].z, (int)cw[j].w, 0, 0, 0, 0};
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 4, 4, 2 * KC, (int)sa[i], 2 * KC,
                                                                  (int)sw[j]);
    }
}

// LDS addresses of a wave's fragment and scale reads, relative to a pair
// buffer (codes) or a group buffer (scales)
struct DlAddr {
  uint32_t a[2][2], w[2][2];  // code fragment of tile 0, half h, chunk kc
  uint32_t sa, sw;      // 16-byte scale row of tile 0's row
  int sh;               // 8 kh: the lane's scale byte shift
};

struct DlRegs {
  uint4 ca0[4], cw0[4], ca1[4], cw1[4];
  uint32_t sa[4], sw[4], qa[4], qw[4];
};

// the scale dwords of stage PH of a group for the wave's 4 A and 4 W tiles
// (shifted by the stage that uses them, so that the reads are not waited for
// here)
template <int PH>
__device__ __forceinline__ void dl_read_scales(const uint8_t* sbuf, const DlAddr& ad, uint32_t (&ra)[4],
                                               uint32_t (&rw)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = *(const uint32_t*)(sbuf + ad.sa + i * 512 + 4 * PH);
    rw[i] = *(const uint32_t*)(sbuf + ad.sw + i * 512 + 4 * PH);
  }
}

template <int H, int KC>
__device__ __forceinline__ void dl_read_codes(const uint8_t* buf, const DlAddr& ad, uint4 (&ca)[4], uint4 (&cw)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ca[i] = *(const uint4*)(buf + ad.a[H][KC] + i * 4096);
    cw[i] = *(const uint4*)(buf + ad.w[H][KC] + i * 4096);
  }
}

// One stage s, half H of its pair.  cur: the pair buffer of stage s; nxt:
// that of stage s + 1 (half HN); ld: where the code loads of pair (s + 3) / 2
// go (ISSUE, odd s: the buffer of stage s's own pair, whose last read is this
// stage's step 0; that read then goes through ld too, so that no buffer is
// reached through two of the `__restrict__` pointers); srd: the scale group
// buffer of stage s + 1, whose dwords sit at phase PHN; sld: where the next
// group's scales go (SCALES).  The buffers accessed through different
// pointers are distinct, so the compiler orders each LDS read only after the
// loads into its own buffer.  WAITN: this wave's loads left in flight when
// stage s + 1's codes and scales must have landed.
//   step 0: read stage s's chunk-1 codes, shift stage s's scale dwords, chunk
//           0 x tiles 0-1;
//   step 1: chunk 0 x tiles 2-3; wait; barrier;
//   step 2: issue the code loads of pair (s + 3) / 2 and the next group's
//           scale loads, read stage s + 1's chunk-0 codes and scales (NEXT),
//           chunk 1 x tiles 0-1;
//   step 3: chunk 1 x tiles 2-3.
template <bool ISSUE, bool SCALES, int WAITN, bool NEXT, int H, int HN, int PHN>
__device__ __forceinline__ void dl_stage(const uint8_t* __restrict__ cur, const uint8_t* __restrict__ nxt,
                                         uint8_t* __restrict__ ld, const uint8_t* __restrict__ srd,
                                         uint8_t* __restrict__ sld, const DlLoader& L, int64_t k_ld, int64_t k_sc,
                                         const DlAddr& ad, DlRegs& r, f32x16 (&acc)[4][4]) {
  if constexpr (ISSUE) dl_read_codes<H, 1>(ld, ad, r.ca1, r.cw1);  // ld is stage s's buffer
  else dl_read_codes<H, 1>(cur, ad, r.ca1, r.cw1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.sa[i] >>= ad.sh;
    r.sw[i] >>= ad.sh;
  }
  mx_mfma_half_dl<0, 0>(r.ca0, r.cw0, r.sa, r.sw, acc);
  __builtin_amdgcn_sched_barrier(0);
  mx_mfma_half_dl<0, 2>(r.ca0, r.cw0, r.sa, r.sw, acc);
  __builtin_amdgcn_sched_barrier(0);
  dl_barrier<WAITN>();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.qa[i] = r.sa[i];
    r.qw[i] = r.sw[i];
  }
  if constexpr (ISSUE) L.issue_pair(ld, k_ld);
  if constexpr (SCALES) L.issue_scales(sld, k_sc);
  if constexpr (NEXT) {
    dl_read_codes<HN, 0>(nxt, ad, r.ca0, r.cw0);
    dl_read_scales<PHN>(srd, ad, r.sa, r.sw);
  }
  mx_mfma_half_dl<1, 0>(r.ca1, r.cw1, r.qa, r.qw, acc);
  __builtin_amdgcn_sched_barrier(0);
  mx_mfma_half_dl<1, 2>(r.ca1, r.cw1, r.qa, r.qw, acc);
  __builtin_amdgcn_sched_barrier(0);
}

// group 0's scales and the codes of pairs 0 and 1, then stage 0's scales and
// chunk-0 codes once they have landed (pair 1 may stay in flight)
__device__ __forceinline__ void dl_prologue(uint8_t* __restrict__ b0, uint8_t* __restrict__ b1,
                                            uint8_t* __restrict__ sb0, const DlLoader& L, int64_t kb,
                                            const DlAddr& ad, DlRegs& r) {
  L.issue_scales(sb0, kb);
  L.issue_pair(b0, kb);
  L.issue_pair(b1, kb + 2 * BK);
  dl_barrier<kDlPairLoads>();
  dl_read_codes<0, 0>(b0, ad, r.ca0, r.cw0);
  dl_read_scales<0>(sb0, ad, r.sa, r.sw);
}

// ns = send - sbeg is a positive multiple of kDlGroup (whole scale groups).
// Loads in flight per wave, in issue order: odd stage s issues, after its
// barrier, the codes of pair (s + 3) / 2 (16 loads) and, at phase 1 of group
// g, group g + 1's scales (2 loads).  When stage s + 1 must have landed, the
// loads allowed in flight are those issued after the ones it needs: 16 at
// phase 0 (the next pair), none at phase 1, 18 at phase 2 (the next pair and
// group), none at phase 3.  The last group issues nothing.
__device__ __forceinline__ void mx_tile_dl(const GemmParams& p, int64_t m0, int64_t n0, uint8_t* smem, int wm,
                                           int wn, int64_t sbeg, int64_t send, f32x16 (&acc)[4][4]) {
  DlLoader L;
  L.init(p, m0, n0, 32);
  const int lane = threadIdx.x & 63, r32 = lane & 31, kh = lane >> 5;
  DlAddr ad;
  const int r7 = r32 & 7, x = (r7 >> 1) | (((r32 >> 3) & 1) << 2);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int o = (r32 >> 3) * 1024 + 128 * r7 + 16 * ((4 * h + 2 * kc + kh) ^ x);
      ad.a[h][kc] = (uint32_t)(o + wm * 16 * 1024);
      ad.w[h][kc] = (uint32_t)(kDlCodes + o + wn * 16 * 1024);
    }
  ad.sa = (uint32_t)((wm * 128 + r32) * 16);
  ad.sw = (uint32_t)(BM * 16 + (wn * 128 + r32) * 16);
  ad.sh = 8 * kh;
  auto pbuf = [&](int64_t pr) { return smem + (int)(pr & 1) * kDlBuf; };
  auto sbuf = [&](int64_t g) { return smem + kDlNbuf * kDlBuf + (int)(g & 1) * kDlScales; };
  const int64_t kb = sbeg * BK, ns = send - sbeg, ng = ns / kDlGroup;
  DlRegs r;
  dl_prologue(pbuf(0), pbuf(1), sbuf(0), L, kb, ad, r);
  constexpr int P = kDlPairLoads;
  int64_t g = 0;
  for (; g + 1 < ng; ++g) {
    const int64_t pr = 2 * g, s = kDlGroup * g;
    dl_stage<false, false, P, true, 0, 1, 1>(pbuf(pr), pbuf(pr), pbuf(pr + 1), sbuf(g), sbuf(g + 1), L, 0, 0, ad, r,
                                            acc);
    dl_stage<true, true, 0, true, 1, 0, 2>(pbuf(pr), pbuf(pr + 1), pbuf(pr + 2), sbuf(g), sbuf(g + 1), L,
                                           kb + (s + 4) * BK, kb + (s + 4) * BK, ad, r, acc);
    dl_stage<false, false, P + 2, true, 0, 1, 3>(pbuf(pr + 1), pbuf(pr + 1), pbuf(pr + 2), sbuf(g), sbuf(g + 1), L,
                                                0, 0, ad, r, acc);
    dl_stage<true, false, 0, true, 1, 0, 0>(pbuf(pr + 1), pbuf(pr + 2), pbuf(pr + 3), sbuf(g + 1), sbuf(g), L,
                                            kb + (s + 6) * BK, 0, ad, r, acc);
  }
  const int64_t pr = 2 * g;  // the last group
  dl_stage<false, false, P, true, 0, 1, 1>(pbuf(pr), pbuf(pr), pbuf(pr + 1), sbuf(g), sbuf(g + 1), L, 0, 0, ad, r,
                                          acc);
  dl_stage<false, false, 0, true, 1, 0, 2>(pbuf(pr), pbuf(pr + 1), pbuf(pr + 2), sbuf(g), sbuf(g + 1), L, 0, 0, ad,
                                           r, acc);
  dl_stage<false, false, 0, true, 0, 1, 3>(pbuf(pr + 1), pbuf(pr + 1), pbuf(pr + 2), sbuf(g), sbuf(g + 1), L, 0, 0,
                                           ad, r, acc);
  dl_stage<false, false, 0, false, 1, 0, 0>(pbuf(pr + 1), pbuf(pr + 2), pbuf(pr + 3), sbuf(g), sbuf(g + 1), L, 0, 0,
                                            ad, r, acc);
}

// ---------------------------------------------------------------- NVFP4 K loop, LDS-DMA staging
// NVFP4 family with K % 256 == 0 and 16-byte aligned scale rows: the code
// layout and loads of the MXFP4 LDS-DMA path (pairs of stages, 128 bytes of
// each row), plus one 16-byte scale load per row per pair (the pair's 16
// E4M3/E3M3 bytes, stage h at bytes 8 h .. 8 h + 7) into the pair buffer.
// Lane (r32, kh) forms its stage scale dword (blocks 2 kh, 2 kh + 1 of chunk
// 0, 4 + 2 kh, 5 + 2 kh of chunk 1) from the row's 8 stage bytes with one byte
// permute.  The stage is the register path's: 8 MFMA steps, the decode of
// step t + 1 during step t, the barrier after step 2, stage s + 1's scales and
// chunk-0 codes read at step 3 and chunk-1 codes at step 7.
constexpr int kNvPairBuf = 2 * kDlCodes + 2 * BM * 16;  // 72 KiB: codes + scales of a pair
constexpr int kNvPairLoads = 18;                        // per wave per pair: 16 code + 2 scale loads
static_assert(2 * kNvPairBuf <= kDlLds, "two pair buffers fit the ring");

// LDS addresses of the NVFP4 LDS-DMA reads, relative to a pair buffer: the A
// code fragment of tile 0 for chunk kc of the pair's first stage (the second
// stage's is that ^ 64: bit 6 is the stage bit of the chunk slot) and the A
// scale row of tile 0; W's are these plus wave-uniform deltas
struct NvDlAddr {
  uint32_t a[2];
  uint32_t sa;
  int dw, dsw;
};

template <int H, int KC>
__device__ __forceinline__ void nv_dl_read_codes(const uint8_t* buf, const NvDlAddr& ad, uint4 (&ca)[4],
                                                 uint4 (&cw)[4]) {
  const uint32_t o = H ? (ad.a[KC] ^ 64u) : ad.a[KC];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ca[i] = *(const uint4*)(buf + o + i * 4096);
    cw[i] = *(const uint4*)(buf + o + ad.dw + i * 4096);
  }
}

// one NVFP4 stage s (half H of its pair).  nxt: the pair buffer of stage s + 1
// (half HN); ld: where pair (s + 3) / 2 goes (ISSUE: odd s, issued after the
// barrier; nxt and ld are different buffers, and stage s reads only nxt).
// WAITN: this wave's loads left in flight at the barrier (the next pair's at
// even stages, none at odd ones).
template <int FA, int FW, bool ISSUE, int WAITN, int HN, bool NEXT>
__device__ __forceinline__ void nv_stage_dl(const uint8_t* __restrict__ nxt, uint8_t* __restrict__ ld,
                                            const DlLoader& L, int64_t k_ld, const NvDlAddr& ad, uint32_t sel,
                                            uint32_t sp_lo, uint32_t sp_hi, NvRegs& R, half8 (&da)[2][4],
                                            half8 (&db)[2][4], f32x16 (&acc)[4][4]) {
  constexpr bool RZ = (FA == RAZER_A || FW == RAZER_A || FW == RAZER_W);
  uint32_t sa8[4][2], sw8[4][2];
  auto prep_a = [&](auto kc_tag, uint32_t (&pa)[4], uint32_t (&xa)[4]) {
    constexpr int KC = decltype(kc_tag)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa[i] = scale_pair_f16<FA, KC>(R.ra[i]);
      if constexpr (RZ) xa[i] = special_pair_f16<FA, KC>(R.ra[i], pa[i], sp_lo, sp_hi);
    }
  };
  auto prep_w = [&](auto kc_tag, uint32_t (&pw)[4], uint32_t (&xw)[4]) {
    constexpr int KC = decltype(kc_tag)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = scale_pair_f16<FW, KC>(R.rw[i]);
      if constexpr (RZ) xw[i] = special_pair_f16<FW, KC>(R.rw[i], pw[i], sp_lo, sp_hi);
    }
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  static_for<0, 8>([&](auto tc) {
    constexpr int t = decltype(tc)::value, cur = t & 1;
    if constexpr (t == 0) prep_a(K1{}, R.pa1, R.xa1);  // chunk-1 pairs, A at step 0, W at step 1
    if constexpr (t == 1) prep_w(K1{}, R.pw1, R.xw1);
    if constexpr (t == 3) {
      if constexpr (ISSUE) {
        L.issue_pair(ld, k_ld);
        L.issue_scales(ld + 2 * kDlCodes, k_ld);
      }
      if constexpr (NEXT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint2 va = *(const uint2*)(nxt + ad.sa + i * 512 + 8 * HN);
          const uint2 vw = *(const uint2*)(nxt + ad.sa + ad.dsw + i * 512 + 8 * HN);
          sa8[i][0] = va.x; sa8[i][1] = va.y;
          sw8[i][0] = vw.x; sw8[i][1] = vw.y;
        }
        nv_dl_read_codes<HN, 0>(nxt, ad, R.ca0, R.cw0);
      }
    }
    if constexpr (t == 4 && NEXT) prep_a(K0{}, R.pa0, R.xa0);  // next stage's chunk-0 pairs
    if constexpr (t == 5 && NEXT) prep_w(K0{}, R.pw0, R.xw0);
    if constexpr (t == 7 && NEXT) nv_dl_read_codes<HN, 1>(nxt, ad, R.ca1, R.cw1);
    // decode of step t + 1
    if constexpr (t < 3)
      decode_step<FA, FW, t + 1>(R.ca0, R.cw0, R.pa0, R.pw0, R.xa0, R.xw0, da[cur ^ 1], db[cur ^ 1]);
    else if constexpr (t < 7)
      decode_step<FA, FW, t - 3>(R.ca1, R.cw1, R.pa1, R.pw1, R.xa1, R.xw1, da[cur ^ 1], db[cur ^ 1]);
    else if constexpr (NEXT)
      decode_step<FA, FW, 0>(R.ca0, R.cw0, R.pa0, R.pw0, R.xa0, R.xw0, da[cur ^ 1], db[cur ^ 1]);
    mfma_step(da[cur], db[cur], acc);
    constexpr int nvm = (t == 3 && ISSUE) ? 16 : 0;
    constexpr int ndsr = (t == 3 && NEXT) ? 16 : (t == 7 && NEXT) ? 8 : 0;
    constexpr int extra = (t == 0 || t == 1 || t == 4 || t == 5) ? 5 : 4;
    sched_step<0, nvm, ndsr, extra>();
    if constexpr (t == 2) dl_barrier<WAITN>();
    if constexpr (t == 3 && NEXT) {
      const uint32_t sl = 0x05040100u + ((threadIdx.x >> 5) & 1u) * 0x02020202u;  // bytes 2 kh, 2 kh + 1
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        R.ra[i] = __builtin_amdgcn_perm(sa8[i][1], sa8[i][0], sl);
        R.rw[i] = __builtin_amdgcn_perm(sw8[i][1], sw8[i][0], sl);
      }
    }
  });
}

// pairs 0 and 1, then stage 0's scales and codes once pair 0 has landed
template <int FA, int FW, bool TWO>
__device__ __forceinline__ void nv_prologue_dl(uint8_t* __restrict__ b0, uint8_t* __restrict__ b1, const DlLoader& L,
                                               int64_t kb, const NvDlAddr& ad, uint32_t sel, NvRegs& R) {
  L.issue_pair(b0, kb);
  L.issue_scales(b0 + 2 * kDlCodes, kb);
  if constexpr (TWO) {
    L.issue_pair(b1, kb + 2 * BK);
    L.issue_scales(b1 + 2 * kDlCodes, kb + 2 * BK);
  }
  dl_barrier<TWO ? kNvPairLoads : 0>();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint2 va = *(const uint2*)(b0 + ad.sa + i * 512);
    const uint2 vw = *(const uint2*)(b0 + ad.sa + ad.dsw + i * 512);
    R.ra[i] = __builtin_amdgcn_perm(va.y, va.x, sel);
    R.rw[i] = __builtin_amdgcn_perm(vw.y, vw.x, sel);
  }
  nv_dl_read_codes<0, 0>(b0, ad, R.ca0, R.cw0);
  nv_dl_read_codes<0, 1>(b0, ad, R.ca1, R.cw1);
}

// four stages 4g .. 4g + 3 with the pair buffers fixed: B0 holds pairs 2g and
// 2g + 2, B1 pairs 2g + 1 and 2g + 3; k2 is pair 2g + 2's first element.  B0
// and B1 are distinct, so the compiler orders each LDS read only after the
// loads into its own buffer, which the odd stages' waits complete.
template <int FA, int FW>
__device__ __forceinline__ void nv_group_dl(uint8_t* __restrict__ B0, uint8_t* __restrict__ B1, const DlLoader& L,
                                            int64_t k2, const NvDlAddr& ad, uint32_t sel, uint32_t sp_lo,
                                            uint32_t sp_hi, NvRegs& R, half8 (&da)[2][4], half8 (&db)[2][4],
                                            f32x16 (&acc)[4][4]) {
  nv_stage_dl<FA, FW, false, kNvPairLoads, 1, true>(B0, B1, L, 0, ad, sel, sp_lo, sp_hi, R, da, db, acc);
  nv_stage_dl<FA, FW, true, 0, 0, true>(B1, B0, L, k2, ad, sel, sp_lo, sp_hi, R, da, db, acc);
  nv_stage_dl<FA, FW, false, kNvPairLoads, 1, true>(B1, B0, L, 0, ad, sel, sp_lo, sp_hi, R, da, db, acc);
  nv_stage_dl<FA, FW, true, 0, 0, true>(B0, B1, L, k2 + 2 * BK, ad, sel, sp_lo, sp_hi, R, da, db, acc);
}

// ns = send - sbeg is a positive multiple of 2 (whole pairs).  Loads in
// flight per wave: pair q + 1 is issued at odd stage 2 q - 1 (after its
// barrier); stage s + 1 must have landed at stage s's barrier, which leaves
// the next pair in flight at even stages and nothing at odd ones.
template <int FA, int FW>
__device__ __forceinline__ void nv_tile_dl(const GemmParams& p, int64_t m0, int64_t n0, uint8_t* smem, int wm,
                                           int wn, int64_t sbeg, int64_t send, f32x16 (&acc)[4][4]) {
  constexpr bool RZ = (FA == RAZER_A || FW == RAZER_A || FW == RAZER_W);
  DlLoader L;
  L.init(p, m0, n0, 16);
  const int lane = threadIdx.x & 63, r32 = lane & 31, kh = lane >> 5;
  NvDlAddr ad;
  const int r7 = r32 & 7, x = (r7 >> 1) | (((r32 >> 3) & 1) << 2);
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
    ad.a[kc] = (uint32_t)((r32 >> 3) * 1024 + 128 * r7 + 16 * ((2 * kc + kh) ^ x) + wm * 16 * 1024);
  ad.sa = (uint32_t)(2 * kDlCodes + (wm * 128 + r32) * 16);
  ad.dw = __builtin_amdgcn_readfirstlane(kDlCodes + (wn - wm) * 16 * 1024);
  ad.dsw = __builtin_amdgcn_readfirstlane(BM * 16 + (wn - wm) * 128 * 16);
  const uint32_t sel = kh ? 0x07060302u : 0x05040100u;  // bytes 2 kh, 2 kh + 1 of each half
  const uint32_t sp_lo = __builtin_bit_cast(uint32_t, (half2v){(_Float16)p.w_special[0], (_Float16)p.w_special[1]});
  const uint32_t sp_hi = __builtin_bit_cast(uint32_t, (half2v){(_Float16)p.w_special[2], (_Float16)p.w_special[3]});
  auto pbuf = [&](int64_t pr) { return smem + (int)(pr & 1) * kNvPairBuf; };
  const int64_t kb = sbeg * BK, ns = send - sbeg, np = ns / 2;
  NvRegs R;
  if (np > 1) nv_prologue_dl<FA, FW, true>(pbuf(0), pbuf(1), L, kb, ad, sel, R);
  else nv_prologue_dl<FA, FW, false>(pbuf(0), pbuf(1), L, kb, ad, sel, R);
  // the chunk-0 pairs and step-0 decode of stage 0
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    R.pa0[i] = scale_pair_f16<FA, 0>(R.ra[i]);
    R.pw0[i] = scale_pair_f16<FW, 0>(R.rw[i]);
    if constexpr (RZ) {
      R.xa0[i] = special_pair_f16<FA, 0>(R.ra[i], R.pa0[i], sp_lo, sp_hi);
      R.xw0[i] = special_pair_f16<FW, 0>(R.rw[i], R.pw0[i], sp_lo, sp_hi);
    }
  }
  half8 da[2][4], db[2][4];
  decode_step<FA, FW, 0>(R.ca0, R.cw0, R.pa0, R.pw0, R.xa0, R.xw0, da[0], db[0]);
  // groups of two pairs with the buffers fixed (pair 2g in B0, 2g + 1 in B1):
  // the odd stages load pairs 2g + 2 (into B0) and 2g + 3 (into B1)
  int64_t q = 0;
  for (; q + 3 < np; q += 2)
    nv_group_dl<FA, FW>(pbuf(0), pbuf(1), L, kb + (2 * q + 4) * BK, ad, sel, sp_lo, sp_hi, R, da, db, acc);
  // the last one to three pairs (pair r in buffer r % 2), sequenced without
  // alternatives so that register allocation stays as in the loop
  if (np - q == 3) {  // pair q + 2 is still to load
    nv_stage_dl<FA, FW, false, kNvPairLoads, 1, true>(pbuf(q), pbuf(q + 1), L, 0, ad, sel, sp_lo, sp_hi, R, da, db,
                                                       acc);
    nv_stage_dl<FA, FW, true, 0, 0, true>(pbuf(q + 1), pbuf(q), L, kb + (2 * q + 4) * BK, ad, sel, sp_lo, sp_hi, R,
                                          da, db, acc);
    ++q;
  }
  if (np - q == 2) {
    nv_stage_dl<FA, FW, false, kNvPairLoads, 1, true>(pbuf(q), pbuf(q + 1), L, 0, ad, sel, sp_lo, sp_hi, R, da, db,
                                                       acc);
    nv_stage_dl<FA, FW, false, 0, 0, true>(pbuf(q + 1), pbuf(q), L, 0, ad, sel, sp_lo, sp_hi, R, da, db, acc);
    ++q;
  }
  nv_stage_dl<FA, FW, false, kNvPairLoads, 1, true>(pbuf(q), pbuf(q + 1), L, 0, ad, sel, sp_lo, sp_hi, R, da, db, acc);
  nv_stage_dl<FA, FW, false, 0, 0, false>(pbuf(q + 1), pbuf(q), L, 0, ad, sel, sp_lo, sp_hi, R, da, db, acc);
}

// ---------------------------------------------------------------- kernel
// FA, FW: operand formats; FA == MXFP4 selects the block-scaled FP4 MFMA path
template <int FA, int FW, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_tile_kernel(GemmParams p) {
  constexpr bool MX = (FA == MXFP4);
  static_assert(kNbuf * kBufBytes <= kDlLds, "the register-staged layout fits the LDS-DMA ring");
  __shared__ __align__(16) uint8_t smem[kDlLds];
  // workgroup = (tile, K-split); split s owns stages [s * per, (s + 1) * per)
  const int split = (int)(blockIdx.x % (unsigned)p.splits);
  int tm, tn;
  tile_coords(p.M, p.N, (int)(blockIdx.x / (unsigned)p.splits), tm, tn);
  // the LDS-DMA paths take whole groups of stages per split: four (MXFP4
  // scale groups) or two (NVFP4 family pairs)
  constexpr int DLG = MX ? kDlGroup : 2;
  const bool dl = p.K % (DLG * BK) == 0 &&
                  ((((uintptr_t)p.a_codes | (uintptr_t)p.w_codes | (uintptr_t)p.a_scales | (uintptr_t)p.w_scales) &
                    15) == 0);
  const int64_t nst = (p.K + BK - 1) / BK;
  int64_t per = (nst + p.splits - 1) / p.splits;
  if (dl) per = (per + DLG - 1) / DLG * DLG;
  const int64_t sbeg = min(nst, split * per), send = min(nst, sbeg + per);
  if (sbeg >= send) return;  // no stages left for this split (uniform across the workgroup)
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};

  if constexpr (!MX) {
    if (dl) nv_tile_dl<FA, FW>(p, m0, n0, smem, wm, wn, sbeg, send, acc);
    else nv_tile<FA, FW>(p, m0, n0, smem, wm, wn, sbeg, send, acc);
  } else if (dl) mx_tile_dl(p, m0, n0, smem, wm, wn, sbeg, send, acc);
  else mx_tile(p, m0, n0, smem, wm, wn, sbeg, send, acc);

  const float ga = p.a_global ? *p.a_global : 1.0f;
  const float gw = p.w_global ? *p.w_global : 1.0f;
  const int r32 = lane & 31, kh = lane >> 5;
  const int64_t row0 = m0 + wm * 128, col0 = n0 + wn * 128;
  float gg[4];  // the lane's four columns col0 + 32 j + r32
#pragma unroll
  for (int j = 0; j < 4; ++j) gg[j] = ga * col_w_global(p, gw, col0 + 32 * j + r32);
  const bool inside = row0 + 128 <= p.M && col0 + 128 <= p.N;
  constexpr int ES = OUT_BF16 ? 2 : 4;  // output element bytes
  const int64_t pitch = p.ldc * ES;
  if (inside && p.splits == 1 && pitch < (int64_t)1 << 23) {
    // a whole wave tile and plain stores: a buffer view of the wave tile's
    // first element, the lane's column and row quad in the vector offset, the
    // rest of each element's offset (row within the tile, column block) scalar
    // and immediate; 128 rows x pitch < 2^30 bytes keeps every offset in range
    const uint64_t bp = (uint64_t)((uint8_t*)p.c + (row0 * p.ldc + col0) * ES);
    // uniform; each half back to unsigned before widening (the builtin returns int)
    const uint32_t bp_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(bp >> 32));
    const uint32_t bp_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bp);
    uint8_t* base = (uint8_t*)(((uint64_t)bp_hi << 32) | (uint64_t)bp_lo);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, -1, (int)kRsrcWord3);
    const int ld = (int)pitch;
    const int voff = kh * 4 * ld + r32 * ES;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int soff = (32 * i + (r / 4) * 8 + (r % 4)) * ld;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = gg[j] * acc[i][j][r];
          if constexpr (OUT_BF16) {
            uint32_t u = __float_as_uint(v);
            u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)u, rc, voff + 32 * j * ES, soff, 0);
          } else {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rc, voff + 32 * j * ES, soff, 0);
          }
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = col0 + 32 * j + r32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + 32 * i + (r / 4) * 8 + kh * 4 + (r % 4);
        if (!inside && (row >= p.M || col >= p.N)) continue;
        const float v = gg[j] * acc[i][j][r];
        if (p.splits > 1) {
          // this split's RN32(g * acc) into its own dense M x N slice
          p.partials[(split * p.M + row) * p.N + col] = v;
        } else if constexpr (OUT_BF16) {
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

// C = the splits' partial results added in split order, RN32 at each step:
// ((p_0 + p_1) + p_2) + ...; stored fp32, or bf16 rounded to nearest even from
// that FP32 sum.  partials: splits dense M x N slices.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part, int splits, int64_t M,
                                                             int64_t N, void* c, int64_t ldc) {
  const int64_t total = M * N, slice = M * N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    float v = part[i];
    for (int sp = 1; sp < splits; ++sp) v = v + part[sp * slice + i];
    const int64_t row = i / N, col = i - row * N;
    if constexpr (OUT_BF16) {
      uint32_t u = __float_as_uint(v);
      u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
      ((uint16_t*)c)[row * ldc + col] = (uint16_t)u;
    } else {
      ((float*)c)[row * ldc + col] = v;
    }
  }
}

hipError_t launch_reduce(const GemmParams& p, hipStream_t s) {
  const int64_t blocks = std::min<int64_t>((p.M * p.N + 255) / 256, 256 * 8);
  if (p.c_bf16)
    hipLaunchKernelGGL(reduce_splits_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, p.partials, p.splits, p.M,
                       p.N, p.c, p.ldc);
  else
    hipLaunchKernelGGL(reduce_splits_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, p.partials, p.splits,
                       p.M, p.N, p.c, p.ldc);
  return hipGetLastError();
}

// per-device caches of launch facts (0: not yet known); every thread that
// fills an entry writes the same value, so relaxed atomics suffice
constexpr int kMaxDevices = 64;

int current_device() {
  int dev = 0;
  return (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) ? dev : -1;
}

int device_cus() {
  static std::atomic<int> cache[kMaxDevices];
  const int dev = current_device();
  int cus = dev >= 0 ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (cus == 0) {
    int n = 0;
    cus = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) == hipSuccess && n > 0)
              ? n : 256;
    if (dev >= 0) cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

float* ws_pointer(const Workspace& ws, hipStream_t s) { return ws.fixed ? ws.fixed : split_workspace(s); }

// K-splits for a launch with too few tiles to fill the chip: the count that
// minimises (rounds of workgroups over the CUs) x (stages per split), at most
// 4, and only as many as the workspace holds partial results for.  Each split
// writes RN32(g * acc_s) of its stage range to its own slice of the
// workspace; reduce_splits_kernel adds the slices in split order, so the
// result does not depend on which split finishes first.
int choose_splits(const GemmParams& p, int64_t T, size_t ws_bytes) {
  const int cus = device_cus();
  if (T >= cus || ws_bytes == 0) return 1;
  const int64_t nst = (p.K + BK - 1) / BK;
  const int64_t fit = (int64_t)(ws_bytes / ((size_t)p.M * (size_t)p.N * sizeof(float)));
  int best = 1;
  int64_t best_cost = ((T + cus - 1) / cus) * nst;
  for (int sp = 2; sp <= 4 && sp <= nst && sp <= fit; ++sp) {
    const int64_t cost = ((T * sp + cus - 1) / cus) * ((nst + sp - 1) / sp);
    if (cost < best_cost) { best = sp; best_cost = cost; }
  }
  return best;
}

template <int FA, int FW>
hipError_t launch_tile(const GemmParams& p0, hipStream_t s, const Workspace& ws) {
  const int64_t T = ((p0.M + BM - 1) / BM) * ((p0.N + BN - 1) / BN);
  GemmParams p = p0;
  int sp = choose_splits(p0, T, ws.bytes);
  if (sp > 1 && (p.partials = ws_pointer(ws, s)) == nullptr) sp = 1;
  if (sp > 1) {
    // the kernel's stage ranges (whole groups of stages on the LDS-DMA paths):
    // launch only splits that own stages, so that every slice is written
    constexpr int DLG = FA == MXFP4 ? kDlGroup : 2;
    const bool dl = p.K % (DLG * BK) == 0 &&
                    ((((uintptr_t)p.a_codes | (uintptr_t)p.w_codes | (uintptr_t)p.a_scales | (uintptr_t)p.w_scales) &
                      15) == 0);
    const int64_t nst = (p.K + BK - 1) / BK;
    int64_t per = (nst + sp - 1) / sp;
    if (dl) per = (per + DLG - 1) / DLG * DLG;
    sp = (int)((nst + per - 1) / per);
  }
  p.splits = sp;
  const unsigned grid = (unsigned)(T * p.splits);
  if (p.c_bf16) hipLaunchKernelGGL((gemm_tile_kernel<FA, FW, true>), dim3(grid), dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((gemm_tile_kernel<FA, FW, false>), dim3(grid), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && p.splits > 1) e = launch_reduce(p, s);
  return e;
}

// ---------------------------------------------------------------- small M
// M <= 128 (decode shapes), NVFP4 family, K a multiple of 64 windows.  Each
// wave owns 32 output columns and all M rows as MR stacked 32 x 32 MFMA
// accumulators (MR = 1, 2 or 4 row blocks; rows past M are computed from the
// clamped last row and never stored).  A is decoded once per workgroup (4
// waves for one block, 8 for more, so that decoding A stays a small share)
// into LDS in fragment order, a window of WIN 64-element chunks at a time,
// each wave taking a fixed share of the window's (chunk, row block) pieces.
// Each wave streams its 32 weight rows from global memory through a ring of
// two turns of kSmRing chunks in registers (a turn's refills are for the
// chunks two turns on) and decodes each weight fragment once for its MR
// MFMAs; one 16-byte load per lane brings a turn's scales (4 blocks of each
// of 4 chunks of its row), and a window's first turn also loads the wave's
// share of the next window's A.  The decode and the K
// permutation are those of the tile kernel.  K may be split in ranges of
// whole windows; each split writes its partial results to the workspace and
// reduce_splits_kernel adds them in split order (see choose_splits).
//
// No load is conditional: windows are full, the last window is peeled and its
// last turn issues no refills.  Loads complete in issue order, and with the
// same loads on every path the compiler's wait for a ring slot counts exactly
// the loads issued after it, so the ring never drains.
constexpr int kSmallM = 128;
constexpr int kSmRing = 4;  // chunks per ring turn, one scale load each turn

template <int MR>
struct SmCfg {
  static constexpr int WIN = 8;                  // chunks per A window (two turns): LDS of WIN x MR x 4 KiB
  static constexpr int WAVES = MR == 1 ? 4 : 8;  // waves per workgroup: 32 WAVES output columns
  static constexpr int TURNS = WIN / kSmRing;    // ring turns per window
  static constexpr int FPW = WIN * MR / WAVES;   // A pieces (chunk x row block) a wave decodes per window
  static_assert(TURNS == 2 && FPW * WAVES == WIN * MR, "two turns, even shares");
};

// buffer views of one operand for the rows [r0, r0 + 32)
struct SmRows {
  __amdgpu_buffer_rsrc_t codes, scales;
  int voff_c, voff_s;  // byte offsets of this lane's half chunk and scale row
};

__device__ __forceinline__ SmRows sm_rows(const uint8_t* codes, const uint8_t* scales, int64_t r0, int64_t rows,
                                          int64_t K, int r32, int kh) {
  const int64_t rowbytes = K / 2, nblk = K / 16;
  const int64_t r = min((int64_t)r32, rows - 1 - r0);
  SmRows v;
  v.codes = __builtin_amdgcn_make_buffer_rsrc((void*)(codes + r0 * rowbytes), (short)0, -1, (int)kRsrcWord3);
  v.scales = __builtin_amdgcn_make_buffer_rsrc((void*)(scales + r0 * nblk), (short)0, -1, (int)kRsrcWord3);
  v.voff_c = (int)(r * rowbytes + kh * 16);
  v.voff_s = (int)(r * nblk);
  return v;
}

// chunk kc of an A row: 32 codes and the 4 scale bytes of the chunk (the
// lane's two blocks are the half kh of them)
__device__ __forceinline__ void sm_load_a(const SmRows& v, int64_t kc, uint4& c, uint32_t& sc) {
  c = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(v.codes, v.voff_c, (int)(kc * 32), 0));
  sc = __builtin_amdgcn_raw_buffer_load_b32(v.scales, v.voff_s, (int)(kc * 4), 0);
}

// chunk kc of a W row: the lane's 32 codes
__device__ __forceinline__ uint4 sm_codes(const SmRows& v, int64_t kc) {
  return as_uint4(__builtin_amdgcn_raw_buffer_load_b128(v.codes, v.voff_c, (int)(kc * 32), 0));
}

// the 16 scale bytes of chunks kc .. kc + 3 of a W row (kc a multiple of 4)
__device__ __forceinline__ uint4 sm_scales4(const SmRows& v, int64_t kc) {
  return as_uint4(__builtin_amdgcn_raw_buffer_load_b128(v.scales, v.voff_s, (int)(kc * 4), 0));
}

template <int F>
__device__ __forceinline__ void sm_decode(const uint4& c, uint32_t sc, uint32_t sp_lo, uint32_t sp_hi, half8 (&out)[4]) {
  const uint32_t pr = scale_pair_f16<F, 0>(sc);
  uint32_t x = 0;
  if constexpr (F == RAZER_A || F == RAZER_W) x = special_pair_f16<F, 0>(sc, pr, sp_lo, sp_hi);
  static_for<0, 4>([&](auto jc) {
    constexpr int J = decltype(jc)::value;
    out[J] = decode8<F, J / 2>(u4_get(c, J), pr, x);
  });
}

// The weight-only path: the lane's 32 codes of a chunk as bf16 (four words of
// 8), exactly.  value * scale has at most 8 significant bits (E2M1 value 2,
// special value 4, E4M3 / E3M3 scale 4), so the FP32 product is a bf16
// number and its upper half is the bf16 pattern.  RaZeR-W: code 0x8 stands
// for the block's special value; a second convert of a word with +1.0 exactly
// at those codes gives u, and fma(u, special * scale, value * scale) is
// special * scale there (value * scale = -0) and value * scale elsewhere.
// sc: the lane's two scale bytes (blocks of words 0-1 and 2-3).
// E3M3 code k (0..63) as FP32: the E4M3 code with the same bits has the
// value 2^-4 times as large (bias 7 against 3, subnormals alike), so the
// hardware FP8 decode with the exact power-of-two scale 16 gives it in one
// instruction
__device__ __forceinline__ float e3m3_f32(uint32_t k) { return __builtin_amdgcn_cvt_scalef32_f32_fp8(k, 16.0f, 0); }

template <int F>
__device__ __forceinline__ void sm_decode_bf16(const uint4& c, uint32_t sc, const float* special, uint4 (&out)[4]) {
  float s[2], sp[2] = {0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t b = (sc >> (8 * h)) & 0xFFu;
    if constexpr (F == RAZER_W) {
      s[h] = e3m3_f32(b & 0x3Fu);
      sp[h] = special[b >> 6] * s[h];  // exact
    } else {
      s[h] = __builtin_amdgcn_cvt_scalef32_f32_fp8(b & 0x7Fu, 1.0f, 0);
    }
  }
  static_for<0, 4>([&](auto jc) {
    constexpr int J = decltype(jc)::value;
    const uint32_t codes = u4_get(c, J);
    uint32_t t = 0;
    if constexpr (F == RAZER_W) {
      const uint32_t y = codes ^ 0x88888888u;                     // nibble 0 where the code is 0x8
      const uint32_t nz = ((y & 0x77777777u) + 0x77777777u) | y;  // bit 3: nibble != 0
      t = (~nz & 0x88888888u) >> 2;                               // 0x2 (+1.0) where the code is 0x8
    }
    uint32_t w[4];
    static_for<0, 4>([&](auto ic) {
      constexpr int b = decltype(ic)::value;
      const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, b);
      float q0 = v[0] * s[J / 2], q1 = v[1] * s[J / 2];
      if constexpr (F == RAZER_W) {
        const auto u = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(t, 1.0f, b);
        q0 = __builtin_fmaf(u[0], sp[J / 2], q0);
        q1 = __builtin_fmaf(u[1], sp[J / 2], q1);
      }
      w[b] = __builtin_amdgcn_perm(__float_as_uint(q1), __float_as_uint(q0), 0x07060302u);  // upper halves
    });
    out[J] = make_uint4(w[0], w[1], w[2], w[3]);
  });
}

// chunks per split: whole windows, as even as that allows
__host__ __device__ inline int64_t sm_split_len(int64_t nch, int64_t splits, int win) {
  const int64_t q = (nch + splits - 1) / splits;
  return (q + win - 1) / win * win;
}

// Where the A rows come from.  AM_BF16: the weight-only variant (bf16
// activations, p.a_bf16 with pitch p.lda): the activation pieces are copied
// into the fragments as they are, the weight is decoded to bf16 and the MFMA
// is the bf16 one; C = RN32(g_w acc).  AM_Q_*: bf16 activations quantized to
// NVFP4 as they are loaded (abs-max or 4-over-6 under g_a), with the
// quantizer's exact decisions, then decoded as packed A would be: the same
// fragments, so the result is that of quantizing first and multiplying the
// codes.  The workgroups of the first column slab also store the codes and
// scales when p.aq_codes is set.
enum AMode : int { AM_CODES = 0, AM_BF16 = 1, AM_Q_ABSMAX = 2, AM_Q_FOUR6 = 3 };

// NVFP4 quantization of one 16-element block held by one lane (the block
// rule of the 16-element-per-lane quantizer): abs-max E4M3 scale by the
// bracketed hardware convert and one exact midpoint test, codes by the
// bracketed FP4 convert, 4-over-6 by the FP32 block errors (ties keep 6)
struct ActQuant {
  float g, lo6, lo4;
  double inv6, inv4;
  bool fast;
};
__device__ __forceinline__ ActQuant act_quant_setup(float g) {
  ActQuant q;
  q.g = g;
  q.fast = g > 0x1p-100f && g < 0x1p100f;
  q.lo6 = __builtin_amdgcn_rcpf(6.0f * g) * (1.0f - 0x1p-20f);
  q.lo4 = __builtin_amdgcn_rcpf(4.0f * g) * (1.0f - 0x1p-20f);
  q.inv6 = 1.0 / (6.0 * (double)g);
  q.inv4 = 1.0 / (4.0 * (double)g);
  return q;
}
template <bool FOUR_OVER_SIX>
__device__ __forceinline__ void act_quant16(const float* x, const ActQuant& q, uint2& packed, int& sbyte) {
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, fbits(x[i]) & 0x7FFFFFFFu);
  const bool finite = amax < 0x7F800000u;
  int k6 = 0, k4 = 0;
  if (wave_all(q.fast && finite)) {
    typedef short s2v __attribute__((ext_vector_type(2)));
    const float a = bitsf(amax);
    const s2v z = {0, 0};
    const s2v clo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a * q.lo6, a * q.lo4, 1.0f, false);
    const uint32_t wl = (uint16_t)clo[0];
    k6 = e4m3_from_low(wl & 0xFFu, a, 6.0f, q.g);
    if constexpr (FOUR_OVER_SIX) k4 = e4m3_from_low(wl >> 8, a, 4.0f, q.g);
  } else {
    k6 = select_sf_exact<0>(bitsf(amax), q.inv6, 6.0 * (double)q.g);
    if constexpr (FOUR_OVER_SIX) k4 = select_sf_exact<0>(bitsf(amax), q.inv4, 4.0 * (double)q.g);
  }
  const float s6 = sf_f32<0>(k6);
  packed = encode_nv16<1, 0>(x, k6, s6, q.g, finite);
  sbyte = k6;
  if constexpr (FOUR_OVER_SIX) {
    const float s4 = sf_f32<0>(k4);
    const uint2 pk4 = encode_nv16<1, 0>(x, k4, s4, q.g, finite);
    const float e6 = lane_sse16(x, packed, s6, q.g);
    const float e4 = lane_sse16(x, pk4, s4, q.g);
    if (e4 < e6) { packed = pk4; sbyte = k4; }
  }
  packed.x = clear_neg_zero(packed.x);
  packed.y = clear_neg_zero(packed.y);
}

template <int FA, int FW, bool OUT_BF16, int MR, int AM = AM_CODES>
__global__ __launch_bounds__(64 * SmCfg<MR>::WAVES, (MR == 1 ? (AM >= AM_Q_ABSMAX ? 2 : 4) : 1)) void gemm_small_m_kernel(
    GemmParams p) {
  constexpr bool A16 = AM != AM_CODES;      // bf16 rows of A
  constexpr bool ABF = AM == AM_BF16;       // ... fed to the bf16 MFMA as they are
  constexpr bool AQ = AM >= AM_Q_ABSMAX;    // ... quantized on load
  using C = SmCfg<MR>;
  constexpr int WIN = C::WIN, TURNS = C::TURNS, FPW = C::FPW;
  __shared__ __align__(16) uint4 adec[WIN][MR][4][64];
  const int split = (int)(blockIdx.x % (unsigned)p.splits);
  const int64_t slab = blockIdx.x / (unsigned)p.splits;
  // the wave index is uniform: read it into a scalar so that the buffer
  // views built from it stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, r32 = lane & 31, kh = lane >> 5;
  const int64_t n0 = slab * (32 * C::WAVES) + wave * 32;
  const bool live = n0 < p.N;  // waves past N read row N - 1 and decode their share of A
  const int64_t nch = p.K / 64, per = sm_split_len(nch, p.splits, WIN);
  const int64_t cb = split * per, ce = min(nch, cb + per);  // cb < ce: every split is used
  const uint32_t sp_lo = __builtin_bit_cast(uint32_t, (half2v){(_Float16)p.w_special[0], (_Float16)p.w_special[1]});
  const uint32_t sp_hi = __builtin_bit_cast(uint32_t, (half2v){(_Float16)p.w_special[2], (_Float16)p.w_special[3]});
  // the wave's A pieces: piece t is chunk (wave + WAVES t) % WIN of a window,
  // row block (wave + WAVES t) / WIN
  SmRows av[FPW];
  int pc[FPW], pb[FPW];
  static_for<0, FPW>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    const int f = wave + C::WAVES * t;
    pc[t] = f % WIN;
    pb[t] = f / WIN;
    if constexpr (A16) {
      // bf16 rows: the lane's half chunk is 32 consecutive elements, 64 bytes
      const int64_t r0 = min((int64_t)(32 * pb[t]), p.M - 1);
      const int64_t r = min((int64_t)r32, p.M - 1 - r0);
      av[t].codes = __builtin_amdgcn_make_buffer_rsrc((void*)(p.a_bf16 + r0 * p.lda), (short)0, -1, (int)kRsrcWord3);
      av[t].scales = av[t].codes;
      av[t].voff_c = (int)(r * p.lda * 2 + kh * 64);
      av[t].voff_s = 0;
    } else {
      av[t] = sm_rows(p.a_codes, p.a_scales, min((int64_t)(32 * pb[t]), p.M - 1), p.M, p.K, r32, kh);
    }
  });
  const SmRows wv = sm_rows(p.w_codes, p.w_scales, live ? n0 : p.N - 1, p.N, p.K, r32, kh);
  ActQuant aq{};
  if constexpr (AQ) aq = act_quant_setup(p.a_global ? *p.a_global : 1.0f);
  const bool aq_store = AQ && p.aq_codes != nullptr && slab == 0;

  f32x16 acc[MR];
  static_for<0, MR>([&](auto bc) { acc[decltype(bc)::value] = f32x16{}; });
  // ring: turn J of every window holds its chunks in rc[J] and their scales
  // in sc[J]; per >= WIN, so the first two turns are inside the split
  uint4 rc[TURNS][kSmRing], sc[TURNS], ca[FPW][A16 ? 4 : 1];
  uint32_t sa[FPW];
  // A piece t of the window at chunk base wb: codes and scales, or 64 bytes of bf16
  auto load_a = [&](auto tc, int64_t wb) {
    constexpr int t = decltype(tc)::value;
    if constexpr (A16) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ca[t][j] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(av[t].codes, av[t].voff_c,
                                                                  (int)((wb + pc[t]) * 128 + 16 * j), 0));
    } else {
      sm_load_a(av[t], wb + pc[t], ca[t][0], sa[t]);
    }
  };
  const float spw[4] = {p.w_special[0], p.w_special[1], p.w_special[2], p.w_special[3]};
  static_for<0, FPW>([&](auto tc) { load_a(tc, cb); });
  __builtin_amdgcn_sched_barrier(0);  // A first, then the ring in slot order
  static_for<0, TURNS>([&](auto jc) {
    constexpr int J = decltype(jc)::value;
    static_for<0, kSmRing>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      rc[J][u] = sm_codes(wv, cb + kSmRing * J + u);
      __builtin_amdgcn_sched_barrier(0);
    });
    sc[J] = sm_scales4(wv, cb + kSmRing * J);
    __builtin_amdgcn_sched_barrier(0);
  });

  // turn J of the window at wb: chunks g0 .. g0 + 3; with `refill`, loads
  // the same turn of the next window
  auto turn = [&](int64_t wb, auto jc, auto refill, auto next_a) {
    constexpr int J = decltype(jc)::value;
    constexpr bool RF = decltype(refill)::value;
    const int64_t g0 = wb + kSmRing * J;
    if constexpr (decltype(next_a)::value && J == 0) {  // a whole window ahead
      static_for<0, FPW>([&](auto tc) { load_a(tc, wb + WIN); });
      __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t sw[kSmRing];
    static_for<0, kSmRing>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      sw[u] = u4_get(sc[J], u) >> (16 * kh);
      asm volatile("" : "+v"(sw[u]));  // computed here, not sunk into the steps past the reload
    });
    if constexpr (RF) {
      // the words are out before the reload: sc[J] keeps its registers
      __builtin_amdgcn_sched_barrier(0);
      sc[J] = sm_scales4(wv, g0 + WIN);
      __builtin_amdgcn_sched_barrier(0);
    }
    static_for<0, kSmRing>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      // decode the slot, then refill it: the refill's registers are then free
      // and stay the slot's own, with no copies around the loop
      uint4 w[4];
      if (live) {
        if constexpr (ABF) {
          sm_decode_bf16<FW>(rc[J][u], sw[u], spw, w);
        } else {
          half8 wh[4];
          sm_decode<FW>(rc[J][u], sw[u], sp_lo, sp_hi, wh);
          static_for<0, 4>([&](auto ic) { w[decltype(ic)::value] = __builtin_bit_cast(uint4, wh[decltype(ic)::value]); });
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (RF) rc[J][u] = sm_codes(wv, g0 + WIN + u);
      __builtin_amdgcn_sched_barrier(0);
      if (live) {
        static_for<0, 4>([&](auto ic) {
          constexpr int I = decltype(ic)::value;
          static_for<0, MR>([&](auto bc) {
            constexpr int b = decltype(bc)::value;
            const uint4 af = adec[kSmRing * J + u][b][I][lane];
            if constexpr (ABF)
              acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af),
                                                               __builtin_bit_cast(bf16x8, w[I]), acc[b], 0, 0, 0);
            else
              acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, af),
                                                              __builtin_bit_cast(half8, w[I]), acc[b], 0, 0, 0);
          });
        });
      }
    });
  };
  auto window = [&](int64_t wb, auto lastw) {
    constexpr bool LW = decltype(lastw)::value;
    lds_barrier();  // the previous window's fragments have been read
    static_for<0, FPW>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      if constexpr (AQ) {
        // the lane's two 16-element blocks: words 0-3 and 4-7 of the 32 bf16
        uint4 cq;
        uint32_t sq;
        {
          float x[16];
          uint2 pk[2];
          int sb[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const uint4 v = ca[t][2 * h + j];
              const uint32_t wv4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                x[8 * j + 2 * i] = bitsf(wv4[i] << 16);
                x[8 * j + 2 * i + 1] = bitsf(wv4[i] & 0xFFFF0000u);
              }
            }
            act_quant16<AM == AM_Q_FOUR6>(x, aq, pk[h], sb[h]);
          }
          cq = make_uint4(pk[0].x, pk[0].y, pk[1].x, pk[1].y);
          sq = (uint32_t)sb[0] | ((uint32_t)sb[1] << 8);
        }
        if (aq_store) {
          const int64_t row = 32 * (int64_t)pb[t] + r32, kc = wb + pc[t];
          if (row < p.M) {
            *(uint4*)(p.aq_codes + row * (p.K / 2) + kc * 32 + kh * 16) = cq;
            *(uint16_t*)(p.aq_scales + row * (p.K / 16) + kc * 4 + kh * 2) = (uint16_t)sq;
          }
        }
        half8 d[4];
        sm_decode<NVFP4>(cq, sq, 0u, 0u, d);
        static_for<0, 4>([&](auto ic) {
          constexpr int I = decltype(ic)::value;
          adec[pc[t]][pb[t]][I][lane] = __builtin_bit_cast(uint4, d[I]);
        });
      } else if constexpr (A16) {
        static_for<0, 4>([&](auto ic) {
          constexpr int I = decltype(ic)::value;
          adec[pc[t]][pb[t]][I][lane] = ca[t][I];
        });
      } else {
        half8 d[4];
        sm_decode<FA>(ca[t][0], sa[t] >> (16 * kh), sp_lo, sp_hi, d);
        static_for<0, 4>([&](auto ic) {
          constexpr int I = decltype(ic)::value;
          adec[pc[t]][pb[t]][I][lane] = __builtin_bit_cast(uint4, d[I]);
        });
      }
    });
    lds_barrier();
    static_for<0, TURNS>([&](auto jc) {
      turn(wb, jc, std::integral_constant<bool, !LW>{}, std::integral_constant<bool, !LW>{});
    });
  };
  int64_t wb = cb;
  for (; wb + WIN < ce; wb += WIN) window(wb, std::false_type{});
  window(wb, std::true_type{});
  if (!live) return;

  const int64_t col = n0 + r32;
  if (col >= p.N) return;
  const float gw = col_w_global(p, p.w_global ? *p.w_global : 1.0f, col);
  const float gg = ABF ? gw : (p.a_global ? *p.a_global : 1.0f) * gw;
  static_for<0, MR>([&](auto bc) {
    constexpr int b = decltype(bc)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = 32 * b + (r / 4) * 8 + kh * 4 + (r % 4);
      if (row >= p.M) continue;
      const float v = gg * acc[b][r];
      if (p.splits > 1) {
        p.partials[(split * p.M + row) * p.N + col] = v;
      } else if constexpr (OUT_BF16) {
        uint32_t u = __float_as_uint(v);
        u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
        ((uint16_t*)p.c)[row * p.ldc + col] = (uint16_t)u;
      } else {
        ((float*)p.c)[row * p.ldc + col] = v;
      }
    }
  });
}

// ---------------------------------------------------------------- M = 1: matrix-vector product
// One activation row against N weight rows.  A matrix-core tile would use one
// of its 32 rows, and its operand layout reads 16 bytes from each of 32 rows
// per load; here a wave owns whole weight rows and lane l the 16-element
// blocks l, l + 64, ..., so every load instruction reads 512 consecutive code
// bytes (8 per lane) or 64 consecutive scale bytes, and reads past the row
// end return zeros (buffer range).  Elements decode to their E2M1 values in
// f16 (RaZeR's code 0x8 to its special value), exactly; a block's 16
// products meet in v_dot2_f32_f16, exactly (values are multiples of 1/2 of
// at most 8, so every partial sum is a multiple of 1/4 below 2^11), and the
// block sum is then multiplied by the product of the two block scales (at
// most 8 significant bits, exact) into the FP32 sum.  The activation's blocks
// are decoded once per wave.  Each wave keeps two rows' loads in flight
// (fixed ping-pong registers, so no loop-carried moves wait on them); a row
// past N gets a buffer view of no bytes, so its loads are issued but fetch
// nothing.  The lane sums meet in a butterfly and lane 0 writes RN32(g * sum).
constexpr int kGemvWaves = 4096;  // waves per launch (at most), several rows each

// E2M1 values of 8 codes as f16, RaZeR's code 0x8 as the special value sp
// (f16 in both halves of sp2): the convert gives -0 there, and a second
// convert of a word with +1.0 exactly at those codes, times sp, is added
template <int F>
__device__ __forceinline__ half8 gemv_values8(uint32_t codes, uint32_t sp2) {
  uint32_t t = 0;
  if constexpr (F == RAZER_A || F == RAZER_W) {
    const uint32_t y = codes ^ 0x88888888u;                     // nibble 0 where the code is 0x8
    const uint32_t nz = ((y & 0x77777777u) + 0x77777777u) | y;  // bit 3: nibble != 0
    t = (~nz & 0x88888888u) >> 2;                               // 0x2 (+1.0) where the code is 0x8
  }
  half8 out;
  static_for<0, 4>([&](auto ic) {
    constexpr int b = decltype(ic)::value;
    half2v v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, b);
    if constexpr (F == RAZER_A || F == RAZER_W) {
      const half2v u = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(t, 1.0f, b);
      v = __builtin_elementwise_fma(u, __builtin_bit_cast(half2v, sp2), v);
    }
    out[2 * b] = v[0];
    out[2 * b + 1] = v[1];
  });
  return out;
}

// a block's scale as FP32 and its special value (f16, both halves)
template <int F>
__device__ __forceinline__ float gemv_scale(uint32_t sb, uint32_t sp_lo, uint32_t sp_hi, uint32_t& sp2) {
  if constexpr (F == RAZER_W) {
    const uint32_t i = (sb >> 6) & 3u;
    sp2 = __builtin_amdgcn_perm(sp_hi, sp_lo, (2u * i) | ((2u * i + 1u) << 8) | ((2u * i) << 16) | ((2u * i + 1u) << 24));
    return e3m3_f32(sb & 0x3Fu);
  } else {
    if constexpr (F == RAZER_A) sp2 = (sb & 0x80u) ? 0xC500C500u : 0x45004500u;  // -5 or +5
    return __builtin_amdgcn_cvt_scalef32_f32_fp8(sb & 0x7Fu, 1.0f, 0);
  }
}

// sum of the 16 products of a block (exact)
__device__ __forceinline__ float dot16(const half8& a0, const half8& a1, const half8& w0, const half8& w1) {
  const uint4 ua0 = __builtin_bit_cast(uint4, a0), ua1 = __builtin_bit_cast(uint4, a1);
  const uint4 uw0 = __builtin_bit_cast(uint4, w0), uw1 = __builtin_bit_cast(uint4, w1);
  float acc = 0.0f;
  static_for<0, 4>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, u4_get(ua0, i)), __builtin_bit_cast(half2v, u4_get(uw0, i)),
                                 acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, u4_get(ua1, i)), __builtin_bit_cast(half2v, u4_get(uw1, i)),
                                 acc, false);
  });
  return acc;
}

template <int JB>
struct GemvRow {
  uint2 c[JB];
  uint32_t sb[JB];
};

template <int JB>
__device__ __forceinline__ void gemv_load(const GemmParams& p, int64_t n, int lane, GemvRow<JB>& r) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const int rowbytes = (int)(p.K / 2), nblk = (int)(p.K / 16);
  const bool live = n < p.N;
  const int64_t nn = live ? n : 0;
  const auto wc = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w_codes + nn * rowbytes), (short)0,
                                                    live ? rowbytes : 0, (int)kRsrcWord3);
  const auto ws = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w_scales + nn * nblk), (short)0, live ? nblk : 0,
                                                    (int)kRsrcWord3);
  static_for<0, JB>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wc, (lane + 64 * j) * 8, 0, 0);
    r.c[j] = make_uint2((uint32_t)v[0], (uint32_t)v[1]);
    r.sb[j] = __builtin_amdgcn_raw_buffer_load_b8(ws, lane + 64 * j, 0, 0);
  });
}

template <int FW, int JB>
__device__ __forceinline__ void gemv_row(const GemmParams& p, int64_t n, int lane, const GemvRow<JB>& r,
                                         const half8 (&a0)[JB], const half8 (&a1)[JB], const float (&sa)[JB],
                                         uint32_t sp_lo, uint32_t sp_hi, float ga, float gw0) {
  float acc[2] = {0.0f, 0.0f};
  static_for<0, JB>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    uint32_t sp2 = 0;
    const float sw = gemv_scale<FW>(r.sb[j], sp_lo, sp_hi, sp2);
    const half8 w0 = gemv_values8<FW>(r.c[j].x, sp2), w1 = gemv_values8<FW>(r.c[j].y, sp2);
    acc[j & 1] = __builtin_fmaf(dot16(a0[j], a1[j], w0, w1), sa[j] * sw, acc[j & 1]);
  });
  float v = acc[0] + acc[1];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  if (lane == 0 && n < p.N) {
    const float out = ga * col_w_global(p, gw0, n) * v;
    if (p.c_bf16) {
      uint32_t u = __float_as_uint(out);
      u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
      ((uint16_t*)p.c)[n] = (uint16_t)u;
    } else {
      ((float*)p.c)[n] = out;
    }
  }
}

template <int FA, int FW, int JB>
__global__ __launch_bounds__(256) void gemv_kernel(GemmParams p) {
  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; read through a scalar so that the compiler
  // knows it, and the row's buffer views stay in scalar registers (a view it
  // takes for per-lane data is applied by a loop over the distinct values)
  const int64_t wave = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const uint32_t sp_lo = __builtin_bit_cast(uint32_t, (half2v){(_Float16)p.w_special[0], (_Float16)p.w_special[1]});
  const uint32_t sp_hi = __builtin_bit_cast(uint32_t, (half2v){(_Float16)p.w_special[2], (_Float16)p.w_special[3]});
  typedef int i32x2 __attribute__((ext_vector_type(2)));

  // the first weight row's loads go out before the activation's
  int64_t n = wave;
  GemvRow<JB> rx, ry;
  gemv_load<JB>(p, n, lane, rx);

  half8 a0[JB], a1[JB];
  float sa[JB];
  {
    const int rowbytes = (int)(p.K / 2), nblk = (int)(p.K / 16);
    const auto ac = __builtin_amdgcn_make_buffer_rsrc((void*)p.a_codes, (short)0, rowbytes, (int)kRsrcWord3);
    const auto as = __builtin_amdgcn_make_buffer_rsrc((void*)p.a_scales, (short)0, nblk, (int)kRsrcWord3);
    GemvRow<JB> ra;
    static_for<0, JB>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(ac, (lane + 64 * j) * 8, 0, 0);
      ra.c[j] = make_uint2((uint32_t)v[0], (uint32_t)v[1]);
      ra.sb[j] = __builtin_amdgcn_raw_buffer_load_b8(as, lane + 64 * j, 0, 0);
    });
    static_for<0, JB>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      uint32_t sp2 = 0;
      sa[j] = gemv_scale<FA>(ra.sb[j], sp_lo, sp_hi, sp2);
      a0[j] = gemv_values8<FA>(ra.c[j].x, sp2);
      a1[j] = gemv_values8<FA>(ra.c[j].y, sp2);
    });
  }
  const float ga = p.a_global ? *p.a_global : 1.0f;
  const float gw0 = p.w_global ? *p.w_global : 1.0f;

  while (true) {
    gemv_load<JB>(p, n + nwaves, lane, ry);
    gemv_row<FW, JB>(p, n, lane, rx, a0, a1, sa, sp_lo, sp_hi, ga, gw0);
    n += nwaves;
    if (n >= p.N) break;
    gemv_load<JB>(p, n + nwaves, lane, rx);
    gemv_row<FW, JB>(p, n, lane, ry, a0, a1, sa, sp_lo, sp_hi, ga, gw0);
    n += nwaves;
    if (n >= p.N) break;
  }
}

// blocks per lane of the matrix-vector kernel for K, 0 if it does not apply
int gemv_jb(const GemmParams& p) {
  const uintptr_t a = (uintptr_t)p.a_codes | (uintptr_t)p.w_codes;
  if (p.M != 1 || p.K % 16 != 0 || (a & 7u) != 0 || p.K > 64 * 16 * 8) return 0;
  const int64_t per = (p.K / 16 + 63) / 64;
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 3 ? 3 : per <= 5 ? 5 : 8;
}

template <int FA, int FW>
hipError_t launch_gemv(const GemmParams& p, int jb, hipStream_t s) {
  const int64_t waves = std::min<int64_t>(p.N, kGemvWaves);
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  switch (jb) {
    case 1: hipLaunchKernelGGL((gemv_kernel<FA, FW, 1>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<FA, FW, 2>), grid, block, 0, s, p); break;
    case 3: hipLaunchKernelGGL((gemv_kernel<FA, FW, 3>), grid, block, 0, s, p); break;
    case 5: hipLaunchKernelGGL((gemv_kernel<FA, FW, 5>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((gemv_kernel<FA, FW, 8>), grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

int sm_blocks(int64_t M) { return M <= 32 ? 1 : M <= 64 ? 2 : 4; }
int sm_win(int mr) { return mr == 1 ? SmCfg<1>::WIN : mr == 2 ? SmCfg<2>::WIN : SmCfg<4>::WIN; }

// the small-M kernel takes K a multiple of 64 windows and operands aligned
// for its 16-byte code and scale loads
bool small_m_fits(const GemmParams& p) {
  const uintptr_t a = (uintptr_t)p.a_codes | (uintptr_t)p.w_codes | (uintptr_t)p.a_scales | (uintptr_t)p.w_scales;
  return p.M <= kSmallM && p.K % (64 * sm_win(sm_blocks(p.M))) == 0 && (a & 15u) == 0;
}

// The split count minimises an estimate of the time: rounds of resident
// workgroups x chunks per split, plus the partial results the splits write
// and the reduction reads and its launch (measured on MI355X: about 1.1 us
// per chunk and round; about 3.2 us per million partial results and 2 us for
// the reduction launch), among the counts whose partials fit the workspace
int64_t sm_choose_splits(int64_t M, int64_t N, int64_t nch, int64_t slabs, int64_t slots, int win, int64_t fit) {
  int64_t best = 1;
  double best_t = 1e300;
  for (int64_t sp = 1; sp <= nch / win && sp <= std::max<int64_t>(fit, 1); ++sp) {
    const int64_t len = sm_split_len(nch, sp, win), used = (nch + len - 1) / len;
    if (used != sp) continue;
    const double rounds = (double)((slabs * sp + slots - 1) / slots);
    const double t = rounds * (double)len * 1.1 + (sp > 1 ? 3.2e-6 * (double)(sp * M * N) + 2.0 : 0.0);
    if (t < best_t) { best_t = t; best = sp; }
  }
  return best;
}

template <int FA, int FW, int MR, int AM = AM_CODES>
hipError_t launch_small_m_mr(const GemmParams& p0, hipStream_t s, const Workspace& ws) {
  constexpr int WIN = SmCfg<MR>::WIN, WAVES = SmCfg<MR>::WAVES;
  GemmParams p = p0;
  const int64_t slabs = (p.N + 32 * WAVES - 1) / (32 * WAVES), nch = p.K / 64;
  int64_t sp = 1;
  if (ws.bytes > 0) {
    // resident workgroups per CU, as the runtime reports them for this kernel
    static std::atomic<int> cache[kMaxDevices];
    const int dev = current_device();
    int per_cu = dev >= 0 ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (per_cu == 0) {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, gemm_small_m_kernel<FA, FW, false, MR, AM>, 64 * WAVES, 0)
          != hipSuccess || nb < 1)
        nb = 1;
      per_cu = nb;
      if (dev >= 0) cache[dev].store(per_cu, std::memory_order_relaxed);
    }
    const int64_t fit = (int64_t)(ws.bytes / ((size_t)p.M * (size_t)p.N * sizeof(float)));
    sp = sm_choose_splits(p.M, p.N, nch, slabs, (int64_t)per_cu * device_cus(), WIN, fit);
    if (sp > 1 && (p.partials = ws_pointer(ws, s)) == nullptr) sp = 1;
  }
  p.splits = (int)sp;
  const unsigned grid = (unsigned)(slabs * sp);
  const unsigned threads = 64 * WAVES;
  if (p.c_bf16) hipLaunchKernelGGL((gemm_small_m_kernel<FA, FW, true, MR, AM>), dim3(grid), dim3(threads), 0, s, p);
  else hipLaunchKernelGGL((gemm_small_m_kernel<FA, FW, false, MR, AM>), dim3(grid), dim3(threads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && p.splits > 1) e = launch_reduce(p, s);
  return e;
}

template <int FA, int FW, int AM = AM_CODES>
hipError_t launch_small_m(const GemmParams& p, hipStream_t s, const Workspace& ws) {
  switch (sm_blocks(p.M)) {
    case 1: return launch_small_m_mr<FA, FW, 1, AM>(p, s, ws);
    case 2: return launch_small_m_mr<FA, FW, 2, AM>(p, s, ws);
    default: return launch_small_m_mr<FA, FW, 4, AM>(p, s, ws);
  }
}

template <int FA, int FW>
hipError_t launch_nv(const GemmParams& p, hipStream_t s, const Workspace& ws) {
  if (const int jb = gemv_jb(p)) return launch_gemv<FA, FW>(p, jb, s);
  if (small_m_fits(p)) return launch_small_m<FA, FW>(p, s, ws);
  return launch_tile<FA, FW>(p, s, ws);
}

template <int FA>
hipError_t launch_nv_a(int fw, const GemmParams& p, hipStream_t s, const Workspace& ws) {
  switch (fw) {
    case RAZER_A: return launch_nv<FA, RAZER_A>(p, s, ws);
    case RAZER_W: return launch_nv<FA, RAZER_W>(p, s, ws);
    default: return launch_nv<FA, NVFP4>(p, s, ws);
  }
}

}  // namespace

// Split-K workspace of one stream: allocated on the stream's first matmul
// and kept until the process ends.  Work on one stream runs in order, so the
// launches of one stream can share it; different streams (and devices) get
// their own.  nullptr if the allocation failed: that stream runs unsplit.
float* split_workspace(hipStream_t s) {
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, void*> cache;
  const std::pair<int, hipStream_t> key(current_device(), s);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return (float*)it->second;
  void* ptr = nullptr;
  if (hipMalloc(&ptr, kSplitWorkspaceBytes) != hipSuccess) {
    (void)hipGetLastError();  // clear the error: the launches below must not report it
    ptr = nullptr;
  }
  cache[key] = ptr;
  return (float*)ptr;
}

// Split-K scratch of the non-allocating matmul entry point: one array per
// device, part of the loaded code object, held until the process ends and
// shared by every call of that entry point on the device (calls that overlap
// on one device race on it).  Host code never uses the name itself, which on
// the host is only a stand-in: it uses the device address looked up below.
__device__ __align__(256) uint8_t scratch[kSplitWorkspaceBytes];

float* noalloc_scratch() {
  static std::mutex mu;
  static void* addr[kMaxDevices];
  static bool looked_up[kMaxDevices];
  const int dev = current_device();
  if (dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!looked_up[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      ptr = nullptr;
    }
    addr[dev] = ptr;
    looked_up[dev] = true;
  }
  return (float*)addr[dev];
}

// Weight-only matmul: the small-M kernel with bf16 activations, 128 rows of A
// per launch (the weight is streamed once per launch)
hipError_t launch_gemm_w4a16(int fw, const GemmParams& p0, hipStream_t s, const Workspace& ws) {
  if (p0.M == 0 || p0.N == 0) return hipSuccess;
  const int es = p0.c_bf16 ? 2 : 4;
  for (int64_t m0 = 0; m0 < p0.M; m0 += kSmallM) {
    GemmParams p = p0;
    p.partials = nullptr;
    p.splits = 1;
    p.M = std::min<int64_t>(kSmallM, p0.M - m0);
    p.a_bf16 = p0.a_bf16 + m0 * p0.lda;
    p.c = (uint8_t*)p0.c + m0 * p0.ldc * es;
    const hipError_t e = fw == RAZER_W ? launch_small_m<NVFP4, RAZER_W, AM_BF16>(p, s, ws)
                                       : launch_small_m<NVFP4, NVFP4, AM_BF16>(p, s, ws);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// W4A4 with activations quantized on load: the small-M kernel, 128 rows of A
// per launch (each launch streams the weight once)
template <int AM>
hipError_t launch_act_bf16_fw(int fw, const GemmParams& p, hipStream_t s, const Workspace& ws) {
  switch (fw) {
    case RAZER_A: return launch_small_m<NVFP4, RAZER_A, AM>(p, s, ws);
    case RAZER_W: return launch_small_m<NVFP4, RAZER_W, AM>(p, s, ws);
    default: return launch_small_m<NVFP4, NVFP4, AM>(p, s, ws);
  }
}

hipError_t launch_gemm_act_bf16(int rule, int fw, const GemmParams& p0, hipStream_t s, const Workspace& ws) {
  if (p0.M == 0 || p0.N == 0) return hipSuccess;
  const int es = p0.c_bf16 ? 2 : 4;
  for (int64_t m0 = 0; m0 < p0.M; m0 += kSmallM) {
    GemmParams p = p0;
    p.partials = nullptr;
    p.splits = 1;
    p.M = std::min<int64_t>(kSmallM, p0.M - m0);
    p.a_bf16 = p0.a_bf16 + m0 * p0.lda;
    p.c = (uint8_t*)p0.c + m0 * p0.ldc * es;
    if (p0.aq_codes) {
      p.aq_codes = p0.aq_codes + m0 * (p0.K / 2);
      p.aq_scales = p0.aq_scales + m0 * (p0.K / 16);
    }
    const hipError_t e = rule == FOUR6 ? launch_act_bf16_fw<AM_Q_FOUR6>(fw, p, s, ws)
                                       : launch_act_bf16_fw<AM_Q_ABSMAX>(fw, p, s, ws);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm(int fa, int fw, const GemmParams& p0, hipStream_t s, const Workspace& ws) {
  if (p0.M == 0 || p0.N == 0) return hipSuccess;
  GemmParams p = p0;
  p.partials = nullptr;
  p.splits = 1;
  if (fa == MXFP4) return launch_tile<MXFP4, MXFP4>(p, s, ws);
  if (fa == RAZER_A) return launch_nv_a<RAZER_A>(fw, p, s, ws);
  return launch_nv_a<NVFP4>(fw, p, s, ws);
}

}  // namespace fp4q
