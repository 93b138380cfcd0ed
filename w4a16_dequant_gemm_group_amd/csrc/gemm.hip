// Fused W4A16 GEMM for prefill-sized M on gfx950 bf16 MFMA.
//
// Same product as the GEMV ("vLLM 量化与推测解码" section 2: Y = X W^T with a
// fused dequantizing kernel), for the compute-bound prefill shape
// ("量化：为何加速推理与精度权衡", follow-up questions: weight-only INT4 leaves the
// matmul FLOPs unchanged; prefill is compute-bound).
//
// Precision: the dequantized weight S(q - z) is never rounded to bf16.  The
// MFMA B operand is the exact small integer q - z (|q - z| <= 15 is exact in
// bf16), so every product is exact in fp32, and the fp16 group scale is applied
// in fp32.  To keep a single accumulator per output element, the accumulator
// holds the running sum divided by the current group's scale,
//   U_g = T_g / c_g,   T_g = sum_{g' <= g} S_g' P_g'   (P = unscaled group sum),
// so the MFMAs of group g+1 accumulate P_{g+1} straight into it after one
// rescale U <- U * (c_g / c_{g+1}) at the group boundary; at the end
// T = U * c_last.  c_g is the group's scale, or the previous c when a scale is
// 0 (that group's B operand is then zeroed).  Ratios of fp16 scales stay far
// inside fp32 range, and each rescale adds one fp32 rounding.  The output is
// rounded once to bf16 (nearest-even).
//
// Two kernels share this arithmetic.
//
// w4a16_gemm_lds_kernel (K % 64 == 0 and group size 32, 64, 128 or a multiple
// of 256): a workgroup of 8 wavefronts computes a 256 x 256 tile of Y; wavefront
// (wm, wn) owns rows 128 wm .. +128 and columns 64 wn .. +64 as 4 x 2
// v_mfma_f32_32x32x16_bf16 tiles.  K advances in 64-wide tiles through two LDS
// stages.  The activation tile goes from memory straight into LDS (16-byte
// buffer loads with the LDS destination), 16-byte chunks XOR-swizzled by row so
// the MFMA operand reads are free of bank conflicts with 32 or 64 banks.  The
// packed weights are loaded into registers one tile ahead and expanded into
// exact bf16 (q - z) in the other LDS stage while the current tile's MFMAs run:
// one 8-nibble word per 16-k step, scheduled between the MFMAs, and the group
// rescale of each accumulator tile is placed right before its first MFMA of the
// new group.  Vector work and MFMAs then overlap instead of alternating, which
// matters because on this GPU only a few vector instructions per MFMA hide
// behind its execution.  Group boundaries fall on fixed k steps for the
// supported group sizes, so the boundary pattern is a template argument.
//
// w4a16_gemm_kernel (any other shape): a workgroup computes a (128 WM) x 256
// tile with WM x 4 wavefronts, each owning a 128 x 64 block as 4 x 2 MFMA tiles.
// K advances in 64-wide tiles through two LDS stages: the activation tile is
// copied in (bf16, 144-byte padded rows), the packed weight tile is expanded
// once per workgroup into exact bf16 (q - z), and the tile's column scales are
// stored beside it.  Global loads run two tiles ahead in registers; they are
// unconditional raw buffer loads (anything outside the matrices reads as zero),
// so the compiler's wait counts stay exact.  When K is a multiple of 64 the
// per-lane offsets are fixed and the k step (or the past-the-end marker) is a
// wave-uniform scalar offset, which the hardware range check includes.
//
// In both, workgroups are dealt round-robin to the 8 XCDs with the M tile
// varying fastest, so each XCD keeps the same activation rows in its L2.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <type_traits>

#include "gq_internal.h"

namespace gq {
namespace {

constexpr int kBK = 64;
constexpr int kLdsRow = kBK + 8;  // bf16 elements per LDS row (+16 B pad)
constexpr int kBN = 256;
constexpr uint32_t kOob = 0x80000000u;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane((uint32_t)std::min<uint64_t>(bytes, 0xFFFFFFFFull));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                           0x00020000);
}

// voff: per-lane byte offset; soff: wave-uniform byte offset.  The range check
// covers voff + soff, so soff = kOob makes the whole load read zeros.
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint16_t bload2(rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// two fp32 holding small integers -> packed bf16 pair (exact)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Byte B of x as fp32 (one v_cvt_f32_ubyteB; written out because the compiler
// turns the masked shift into a bit-field extract plus a conversion).
template <int B>
__device__ __forceinline__ float ubyte_f32(uint32_t x) {
  float r;
  if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
  if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
  if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
  if constexpr (B == 3) asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// two fp32 holding small integers -> packed fp16 pair (exact)
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// 8 nibbles (k = 0..7 at bits 4p) -> 8 bf16 (XF16: fp16) values q - z in k
// order (4 dwords); |q - z| <= 15 is exact in both.
template <bool XF16>
__device__ __forceinline__ uint4 expand8(uint32_t d, float z) {
  const uint32_t e = d & 0x0F0F0F0Fu, o = (d >> 4) & 0x0F0F0F0Fu;
  const float q0 = ubyte_f32<0>(e) - z, q2 = ubyte_f32<1>(e) - z;
  const float q4 = ubyte_f32<2>(e) - z, q6 = ubyte_f32<3>(e) - z;
  const float q1 = ubyte_f32<0>(o) - z, q3 = ubyte_f32<1>(o) - z;
  const float q5 = ubyte_f32<2>(o) - z, q7 = ubyte_f32<3>(o) - z;
  if (XF16) return make_uint4(pack_f16(q0, q1), pack_f16(q2, q3), pack_f16(q4, q5), pack_f16(q6, q7));
  return make_uint4(pack_bf16(q0, q1), pack_bf16(q2, q3), pack_bf16(q4, q5), pack_bf16(q6, q7));
}

// 32 x 32 x 16 MFMA on 8-element operand registers of bf16 or fp16
template <bool XF16>
using opnd8_t = typename std::conditional<XF16, f16x8_t, bf16x8_t>::type;

template <bool XF16>
__device__ __forceinline__ f32x16_t mfma32(const opnd8_t<XF16>& a, const opnd8_t<XF16>& b,
                                           const f32x16_t& c) {
  if constexpr (XF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The output element: bf16 (XF16: fp16), nearest-even.
template <bool XF16>
__device__ __forceinline__ uint16_t out16(float v) {
  if constexpr (XF16) return __builtin_bit_cast(uint16_t, (_Float16)v);
  else return f32_to_bf16_rne(v);
}

// XF16: fp16 activations, fp16 MFMA and fp16 output; otherwise bf16.
template <int WM, bool SYM, bool TAIL, bool XF16 = false>
__global__ __launch_bounds__(256 * WM, 2) void w4a16_gemm_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int N, int G,
    uint16_t* __restrict__ y) {
  constexpr int BM = 128 * WM;
  constexpr int NT = 256 * WM;
  constexpr int A_CH = BM * kBK / 8 / NT;  // 16-byte activation chunks per thread (4)
  constexpr int B_HALF = kBN * 2 / NT;     // 32-k column halves expanded per thread
  extern __shared__ uint4 lds_raw[];
  uint16_t* As = (uint16_t*)lds_raw;          // [2][BM][kLdsRow]
  uint16_t* Bs = As + 2 * BM * kLdsRow;       // [2][kBN][kLdsRow]
  float* Cs = (float*)(Bs + 2 * kBN * kLdsRow);  // [2][2][kBN] scales of the tile's groups

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int ntm = (M + BM - 1) / BM;
  const int m0 = (blockIdx.x % ntm) * BM;
  const int n0 = (blockIdx.x / ntm) * kBN;
  const int ng = K / G;
  const uint32_t rb = (uint32_t)K / 2;

  const rsrc_t rA = make_rsrc(x + (size_t)m0 * K, (uint64_t)(M - m0) * K * 2);
  const rsrc_t rB = make_rsrc(qw + (size_t)n0 * rb, (uint64_t)(N - n0) * rb);
  const rsrc_t rS = make_rsrc(scales + (size_t)n0 * ng, (uint64_t)(N - n0) * ng * 2);
  const rsrc_t rZ = make_rsrc(SYM ? (const void*)scales : (const void*)(zeros + (size_t)n0 * ng),
                              (uint64_t)(N - n0) * ng * 2);

  const int lcol[2] = {wn * 64 + (lane & 31), wn * 64 + 32 + (lane & 31)};  // tile-local columns
  struct Stage {
    uint4 a[A_CH];
    uint4 b[B_HALF];
    uint16_t z[B_HALF], s[B_HALF];
    uint16_t cs[2];  // scales of this lane's MFMA columns for the tile's first group
  };
  // Per-lane offsets that do not depend on k (K % 64 == 0: the k step and the
  // past-the-end marker travel in the wave-uniform soffset).
  uint32_t voa[A_CH], vob[B_HALF], vos[B_HALF], vocs[2];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int id = tid + i * NT;
    voa[i] = (uint32_t)((id >> 3) * K + (id & 7) * 8) * 2u;
  }
#pragma unroll
  for (int h = 0; h < B_HALF; ++h) {
    const int id = tid + h * NT;
    vob[h] = (uint32_t)(id >> 1) * rb + (uint32_t)(id & 1) * 16u;
    vos[h] = (uint32_t)((id >> 1) * ng) * 2u;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) vocs[j] = (uint32_t)(lcol[j] * ng) * 2u;
  auto load_tile = [&](Stage& S, int k0) {
    const int g0 = __builtin_amdgcn_readfirstlane(k0 / G);
    const int g1 = __builtin_amdgcn_readfirstlane((k0 + 32) / G);
    if (!TAIL) {
      // readfirstlane keeps the offsets in scalar registers: a buffer load whose
      // soffset the compiler cannot prove uniform becomes a loop over lanes
      const bool kin = k0 < K;
      const uint32_t sa = __builtin_amdgcn_readfirstlane(kin ? (uint32_t)k0 * 2u : kOob);
      const uint32_t sb = __builtin_amdgcn_readfirstlane(kin ? (uint32_t)k0 / 2u : kOob);
      const uint32_t sg = __builtin_amdgcn_readfirstlane(kin ? (uint32_t)g0 * 2u : kOob);
#pragma unroll
      for (int i = 0; i < A_CH; ++i) S.a[i] = bload16(rA, voa[i], sa);
#pragma unroll
      for (int j = 0; j < 2; ++j) S.cs[j] = bload2(rS, vocs[j], sg);
#pragma unroll
      for (int h = 0; h < B_HALF; ++h) {
        S.b[h] = bload16(rB, vob[h], sb);
        // column half 1 may start the next group (g1 = g0 + 1)
        const uint32_t vg = vos[h] + (((tid + h * NT) & 1) && g1 != g0 ? 2u : 0u);
        S.s[h] = bload2(rS, vg, sg);
        if (!SYM) S.z[h] = bload2(rZ, vg, sg);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int id = tid + i * NT;
      const int gk = k0 + (id & 7) * 8;
      S.a[i] = bload16(rA, gk < K ? voa[i] + (uint32_t)k0 * 2u : kOob);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) S.cs[j] = bload2(rS, k0 < K ? vocs[j] + (uint32_t)g0 * 2u : kOob);
#pragma unroll
    for (int h = 0; h < B_HALF; ++h) {
      const int id = tid + h * NT;
      const int half = id & 1;
      const bool kin = k0 + half * 32 < K;
      S.b[h] = bload16(rB, kin ? vob[h] + (uint32_t)k0 / 2u : kOob);
      const uint32_t go = kin ? vos[h] + (uint32_t)(half ? g1 : g0) * 2u : kOob;
      S.s[h] = bload2(rS, go);
      if (!SYM) S.z[h] = bload2(rZ, go);
    }
  };
  auto store_tile = [&](const Stage& S, int buf) {
    uint16_t* as = As + buf * BM * kLdsRow;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int id = tid + i * NT;
      const int r = id >> 3, c = id & 7;
      *(uint4*)&as[r * kLdsRow + c * 8] = S.a[i];
    }
#pragma unroll
    for (int h = 0; h < B_HALF; ++h) {
      const int id = tid + h * NT;
      const int col = id >> 1, half = id & 1;
      uint16_t* bs = Bs + (buf * kBN + col) * kLdsRow + half * 32;
      const float zf = SYM ? 8.f : h2f(S.z[h]);
      uint4 e0 = expand8<XF16>(S.b[h].x, zf), e1 = expand8<XF16>(S.b[h].y, zf);
      uint4 e2 = expand8<XF16>(S.b[h].z, zf), e3 = expand8<XF16>(S.b[h].w, zf);
      if ((S.s[h] & 0x7FFF) == 0) e0 = e1 = e2 = e3 = make_uint4(0, 0, 0, 0);  // S = 0: no contribution
      *(uint4*)(bs + 0) = e0;
      *(uint4*)(bs + 8) = e1;
      *(uint4*)(bs + 16) = e2;
      *(uint4*)(bs + 24) = e3;
      Cs[(buf * 2 + half) * kBN + col] = h2f(S.s[h]);
    }
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  float cref[2] = {1.f, 1.f};

  // Rescale the running sum from the current group scale cref to scale s of
  // the group that starts next (s = 0: that group is skipped, keep cref).
  auto rescale = [&](const float (&s)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float cn = s[j] != 0.f ? s[j] : cref[j];
      const float r = cref[j] * __builtin_amdgcn_rcpf(cn);  // within 1 ulp of the quotient
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] *= r;
      cref[j] = cn;
    }
  };

  // nxt: the stage of tile t+1 (its first group's scales, for a boundary at the tile end)
  auto compute_tile = [&](int t, const Stage& nxt) {
    const int k0 = t * kBK;
    const int cur = t & 1;
    const uint16_t* as = As + (cur * BM + wm * 128 + (lane & 31)) * kLdsRow;
    const uint16_t* bs = Bs + (cur * kBN + wn * 64 + (lane & 31)) * kLdsRow;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kk = ks * 16 + 8 * (lane >> 5);
      opnd8_t<XF16> a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = __builtin_bit_cast(opnd8_t<XF16>, *(const uint4*)&as[i * 32 * kLdsRow + kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = __builtin_bit_cast(opnd8_t<XF16>, *(const uint4*)&bs[j * 32 * kLdsRow + kk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = mfma32<XF16>(a[i], b[j], acc[i][j]);
      const int kend = k0 + (ks + 1) * 16;
      if ((ks == 1 || ks == 3) && kend % G == 0 && kend < K) {
        float s[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          s[j] = ks == 1 ? Cs[(cur * 2 + 1) * kBN + lcol[j]] : h2f(nxt.cs[j]);
        rescale(s);
      }
    }
  };

  const int ntiles = (K + kBK - 1) / kBK;
  Stage s0, s1;
  load_tile(s0, 0);
  load_tile(s1, kBK);
  store_tile(s0, 0);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float c0 = Cs[lcol[j]];
    cref[j] = c0 != 0.f ? c0 : 1.f;
  }
  // Tile t sits in LDS; the stage holding tile t+1 is in flight; tile t+2 is
  // issued into the stage just drained.  Loads past the end read zeros.
  for (int t = 0; t < ntiles; t += 2) {
    load_tile(s0, (t + 2) * kBK);
    compute_tile(t, s1);
    if (t + 1 < ntiles) store_tile(s1, 1);
    __syncthreads();
    if (t + 1 >= ntiles) break;
    load_tile(s1, (t + 3) * kBK);
    compute_tile(t + 1, s0);
    if (t + 2 < ntiles) store_tile(s0, 0);
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*(v/4) + 4*(lane/32) + v%4
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gn = n0 + lcol[j];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int gm = m0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (gm < M && gn < N) y[(size_t)gm * N + gn] = out16<XF16>(acc[i][j][v] * cref[j]);
      }
    }
}

// ---------------------------------------------------------------------------
// 256 x 256 tile kernel with direct-to-LDS activations (K % 64 == 0)
// ---------------------------------------------------------------------------

constexpr int kLM = 256, kLN = 256, kLT = 512;  // tile rows, columns, threads
constexpr int kLBRow = kBK + 8;                  // bf16 per expanded weight column (+16 B)

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt that bounds only the outstanding vector-memory operations
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 8 nibbles (k = 0..7 at bits 4p) -> 8 exact bf16 (or, XF16, fp16) values
// m (q - z) in k order, with nz = -z m and m = 1, or m = 0 for a group whose
// scale is 0.
template <bool XF16>
__device__ __forceinline__ uint4 expand8m(uint32_t d, float m, float nz) {
  const uint32_t e = d & 0x0F0F0F0Fu, o = (d >> 4) & 0x0F0F0F0Fu;
  const float q0 = fmaf(ubyte_f32<0>(e), m, nz), q2 = fmaf(ubyte_f32<1>(e), m, nz);
  const float q4 = fmaf(ubyte_f32<2>(e), m, nz), q6 = fmaf(ubyte_f32<3>(e), m, nz);
  const float q1 = fmaf(ubyte_f32<0>(o), m, nz), q3 = fmaf(ubyte_f32<1>(o), m, nz);
  const float q5 = fmaf(ubyte_f32<2>(o), m, nz), q7 = fmaf(ubyte_f32<3>(o), m, nz);
  if (XF16) return make_uint4(pack_f16(q0, q1), pack_f16(q2, q3), pack_f16(q4, q5), pack_f16(q6, q7));
  return make_uint4(pack_bf16(q0, q1), pack_bf16(q2, q3), pack_bf16(q4, q5), pack_bf16(q6, q7));
}

// Activation LDS tile: 16-byte chunk c of row r sits at position c ^ swz(r) of
// the row's 128 bytes.  Sixteen consecutive rows read at one chunk touch 16
// distinct 16-byte bank groups, eight consecutive rows 8 distinct ones.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

struct WStage {
  uint4 b;        // 32 nibbles: one column, one 32-k half of a tile
  uint16_t s, z;  // its group's scale and zero (fp16 bits)
};

// MODE: where groups start.  0: G = 32 (k steps 0 and 2 of every tile);
// 1: G = 64 (every tile); 2: G = 128 (even tiles); 3: G a multiple of 256
// (even tiles whose k0 is a multiple of G).
//
// The launch covers output tiles [tile0, tile0 + nt) in the M-fastest order.
// SPLIT: the grid holds two workgroups per output tile, the first covering
// 64-k tiles [0, tsplit), the second [tsplit, K/64) (tsplit keeps whole
// groups).  Each converts its running sum to the true scale; the first to finish
// publishes it in `part` and raises the tile's flag, the second adds it to its
// own (a sum of two terms, so the result does not depend on which finishes
// first) and writes Y.  `sync` holds two 64-bit words per tile (arrival,
// flag) in caller memory of unknown content: each workgroup swaps the launch's
// id into the arrival word, and the one that gets the id back is second (an id
// is unique per call and random per process, so stale words never match it);
// the second clears both words, so a graph that replays the same id finds
// them clear.
// XF16: fp16 activations and output (fp16 MFMA), otherwise bf16.
template <bool SYM, int MODE, bool SPLIT, bool XF16 = false, bool NARROW = false>
__global__ __launch_bounds__(kLT, 1) void w4a16_gemm_lds_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int N, int G,
    uint16_t* __restrict__ y, uint64_t* __restrict__ sync, float* __restrict__ part, int tsplit,
    int tile0, int nt, uint64_t launch_id, int poll_limit) {
  __shared__ uint4 sA0[kLM * 8], sA1[kLM * 8];                        // 2 x 32 KiB
  __shared__ uint4 sB0[kLN * kLBRow / 8], sB1[kLN * kLBRow / 8];      // 2 x 36 KiB
  __shared__ float sC0[2 * kLN], sC1[2 * kLN];                        // scales per column half

  // NARROW: 256 x 192 tiles, waves 4 (rows) x 2 (columns) of 64 x 96 (2 x 3
  // MFMA tiles); otherwise 256 x 256 tiles, waves 2 x 4 of 128 x 64 (4 x 2).
  // The weight stages keep 256 columns; the threads of columns >= 192 load
  // zeros (range check) and expand them into columns no wave reads.
  constexpr int TN = NARROW ? 192 : kLN;
  constexpr int TI = NARROW ? 2 : 4, TJ = NARROW ? 3 : 2;
  constexpr int WMW = NARROW ? 4 : 2;  // waves along M
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WMW, wn = wave / WMW;
  const int ntm = (M + kLM - 1) / kLM;
  const int split = SPLIT && (int)blockIdx.x >= nt;
  const int lt = (int)blockIdx.x - split * nt;  // tile within the launch: its sync and partial slot
  const int tile_id = tile0 + lt;
  const int m0 = (tile_id % ntm) * kLM;
  const int n0 = (tile_id / ntm) * TN;
  const int ng = K / G;
  const uint32_t rb = (uint32_t)K / 2;
  // this workgroup's 64-k tiles: [kt0, kt0 + T)
  const int kt0 = SPLIT && split ? tsplit : 0;
  const int T = SPLIT ? (split ? K / kBK - tsplit : tsplit) : K / kBK;
  const int kb = kt0 * kBK;  // first k

  const rsrc_t rA = make_rsrc(x + (size_t)m0 * K, (uint64_t)(M - m0) * K * 2);
  const rsrc_t rB = make_rsrc(qw + (size_t)n0 * rb, (uint64_t)(N - n0) * rb);
  const rsrc_t rS = make_rsrc(scales + (size_t)n0 * ng, (uint64_t)(N - n0) * ng * 2);
  const rsrc_t rZ = make_rsrc(SYM ? (const void*)scales : (const void*)(zeros + (size_t)n0 * ng),
                              (uint64_t)(N - n0) * ng * 2);

  // Activation DMA: LDS slot i*512 + tid (16 bytes) holds row slot/8 at
  // position slot%8; a wavefront's load fills 1 KiB (8 rows) contiguously.
  uint32_t voA[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = i * kLT + tid;
    const int r = slot >> 3, p = slot & 7;
    voA[i] = (uint32_t)r * (uint32_t)K * 2u + (uint32_t)((p ^ swz(r)) * 16);
  }
  // Weights: a thread expands column tid/2, k half tid%2 of each tile.
  const int bcol = tid >> 1, bhalf = tid & 1;
  const uint32_t voB = bcol < TN ? (uint32_t)bcol * rb + (uint32_t)bhalf * 16u : kOob;
  const uint32_t voS = bcol < TN ? (uint32_t)(bcol * ng) * 2u + (MODE == 0 && bhalf ? 2u : 0u) : kOob;

  auto issueA = [&](uint4* sA, int k0) {
    // scalar offsets stay in SGPRs (a non-uniform soffset turns into a lane loop)
    const uint32_t so = __builtin_amdgcn_readfirstlane(k0 < K ? (uint32_t)k0 * 2u : kOob);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(sA + i * kLT + wave * 64), 16, voA[i],
                                               so, 0, 0);
  };
  auto loadW = [&](WStage& S, int k0) {
    const bool kin = k0 < K;
    const uint32_t sb = __builtin_amdgcn_readfirstlane(kin ? (uint32_t)k0 / 2u : kOob);
    const uint32_t sg = __builtin_amdgcn_readfirstlane(kin ? (uint32_t)(k0 / G) * 2u : kOob);
    S.b = bload16(rB, voB, sb);
    S.s = bload2(rS, voS, sg);
    if (!SYM) S.z = bload2(rZ, voS, sg);
  };
  auto mult = [&](const WStage& S) { return (S.s & 0x7FFF) ? 1.f : 0.f; };
  auto negz = [&](const WStage& S, float m) { return -(SYM ? 8.f : h2f(S.z)) * m; };
  auto expand_all = [&](const WStage& S, uint4* sB, float* sC) {
    const float m = mult(S), nz = negz(S, m);
    uint4* d = sB + (bcol * kLBRow + bhalf * 32) / 8;
    d[0] = expand8m<XF16>(S.b.x, m, nz);
    d[1] = expand8m<XF16>(S.b.y, m, nz);
    d[2] = expand8m<XF16>(S.b.z, m, nz);
    d[3] = expand8m<XF16>(S.b.w, m, nz);
    sC[bhalf * kLN + bcol] = h2f(S.s);
  };

  f32x16_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  float cref[TJ];
  const int lcol0 = wn * 32 * TJ + (lane & 31);

  // factors moving the running sum from scale cref to the next group's scale
  // (exactly 1 when no group starts here: use = false)
  auto factors = [&](const float* sC, int half, float (&r)[TJ], bool use) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const float sn = use ? sC[half * kLN + lcol0 + 32 * j] : cref[j];
      const float cn = sn != 0.f ? sn : cref[j];
      r[j] = cref[j] * __builtin_amdgcn_rcpf(cn);  // within 1 ulp of the quotient
      cref[j] = cn;
    }
  };

  // per-lane LDS offsets (uint4 units) of the MFMA operands
  const int fl = swz(lane & 31);
  const int arow = wm * 32 * TI + (lane & 31);
  int aoff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) aoff[ks] = arow * 8 + ((2 * ks + (lane >> 5)) ^ fl);
  const int boff = (lcol0 * kLBRow + 8 * (lane >> 5)) / 8;

  // One 64-k tile from (sA, sB, sC) while the next tile's weights Wn are expanded
  // into (sBn, sCn).  R0 / R2: a group starts at k step 0 / 2.
  auto tile = [&](auto R0c, auto R2c, const uint4* sA, const uint4* sB, const float* sC,
                  const WStage& Wn, uint4* sBn, float* sCn, bool start) {
    constexpr bool R0 = decltype(R0c)::value, R2 = decltype(R2c)::value;
    float r0[TJ], r2[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) r0[j] = r2[j] = 1.f;
    if (R0) factors(sC, 0, r0, start);
    const float m = mult(Wn), nz = negz(Wn, m);
    uint4* dn = sBn + (bcol * kLBRow + bhalf * 32) / 8;
    opnd8_t<XF16> a[2][TI], b[2][TJ];
    auto ld = [&](int ks, int buf) {
#pragma unroll
      for (int i = 0; i < TI; ++i) a[buf][i] = __builtin_bit_cast(opnd8_t<XF16>, sA[aoff[ks] + i * 32 * 8]);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        b[buf][j] = __builtin_bit_cast(opnd8_t<XF16>, sB[boff + ks * 2 + j * 32 * kLBRow / 8]);
    };
    ld(0, 0);
    auto step = [&](auto KSc) {
      constexpr int ks = decltype(KSc)::value;
      constexpr bool RS = (R0 && ks == 0) || (R2 && ks == 2);
      if (ks < 3) ld(ks + 1, (ks + 1) & 1);
      if (R2 && ks == 2) factors(sC, 1, r2, true);
      const uint32_t word = ks == 0 ? Wn.b.x : ks == 1 ? Wn.b.y : ks == 2 ? Wn.b.z : Wn.b.w;
      const uint4 e = expand8m<XF16>(word, m, nz);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          if (R0 && ks == 0) acc[i][j] *= r0[j];
          if (R2 && ks == 2) acc[i][j] *= r2[j];
          acc[i][j] = mfma32<XF16>(a[ks & 1][i], b[ks & 1][j], acc[i][j]);
        }
      dn[ks] = e;
      // the next step's LDS reads first, then every MFMA behind its share of the
      // vector work (its accumulator's rescale, the expansion)
      constexpr int kX = (24 + TI * TJ - 1) / (TI * TJ);  // expansion instructions per MFMA
      if (ks < 3) __builtin_amdgcn_sched_group_barrier(0x100, TI + TJ, 0);
#pragma unroll
      for (int q = 0; q < TI * TJ; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x2, RS ? 16 + kX : kX, 0);
        __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    sCn[bhalf * kLN + bcol] = h2f(Wn.s);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // Even tiles of modes 2 and 3 run the rescale step; in mode 3 its factors are
  // exactly 1 unless a group starts (one code path keeps the registers in place).
  auto tile_even = [&](int k0, const uint4* sA, const uint4* sB, const float* sC, const WStage& Wn,
                       uint4* sBn, float* sCn) {
    if constexpr (MODE == 0) tile(T_{}, T_{}, sA, sB, sC, Wn, sBn, sCn, true);
    else tile(T_{}, F_{}, sA, sB, sC, Wn, sBn, sCn, MODE != 3 || k0 % G == 0);
  };
  auto tile_odd = [&](const uint4* sA, const uint4* sB, const float* sC, const WStage& Wn,
                      uint4* sBn, float* sCn) {
    if constexpr (MODE == 0) tile(T_{}, T_{}, sA, sB, sC, Wn, sBn, sCn, true);
    else if constexpr (MODE == 1) tile(T_{}, F_{}, sA, sB, sC, Wn, sBn, sCn, true);
    else tile(F_{}, F_{}, sA, sB, sC, Wn, sBn, sCn, false);
  };

  constexpr int nW = SYM ? 2 : 3;  // vector-memory loads per weight stage
  WStage w0, w1;
  issueA(sA0, kb);
  loadW(w0, kb);
  loadW(w1, kb + kBK);
  wait_vm<nW>();
  expand_all(w0, sB0, sC0);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const float c0 = sC0[lcol0 + 32 * j];
    cref[j] = c0 != 0.f ? c0 : 1.f;  // the first tile's factors are then 1
  }
  // Tile t computes from stage t%2 while the DMA fills the other activation
  // stage with tile t+1, the weights of tile t+1 (in registers since tile t-1)
  // are expanded into the other weight stage, and tile t+2's weights load into
  // the register stage just drained.  Pairs of tiles keep the stages static and
  // the loop single-exit; an odd last tile runs after it.
  // (kb is a multiple of the group size in tiles, so even/odd keep their roles)
  int t = 0;
  for (; t + 1 < T; t += 2) {
    issueA(sA1, kb + (t + 1) * kBK);
    wait_vm<4 + nW>();
    tile_even(kb + t * kBK, sA0, sB0, sC0, w1, sB1, sC1);
    loadW(w0, kb + (t + 2) * kBK);
    wait_vm<nW>();
    __syncthreads();
    issueA(sA0, kb + (t + 2) * kBK);
    wait_vm<4 + nW>();
    tile_odd(sA1, sB1, sC1, w0, sB0, sC0);
    loadW(w1, kb + (t + 3) * kBK);
    wait_vm<nW>();
    __syncthreads();
  }
  if (t < T) tile_even(kb + t * kBK, sA0, sB0, sC0, w1, sB1, sC1);

  if constexpr (SPLIT) {
    // Partial sums in the accumulator layout [tile][wave][128][lane], written
    // and read as relaxed agent-scope atomics: those are coherent across the
    // XCDs' L2 caches without the whole-cache write-back and invalidation that
    // release/acquire fences would cost every other workgroup on the XCD.  The
    // writer drains its stores (vmcnt 0: acknowledged by the coherent level)
    // before any thread raises the flag; the reader issues its loads only after
    // it has seen the flag (the loads are issued after the poll's value
    // returned, and they bypass the non-coherent caches).
    float* slot = part + ((size_t)lt * 8 + wave) * 128 * 64 + lane;
    uint64_t* arrive = sync + 2 * lt;
    uint64_t* flag = arrive + 1;
    // 1: first to arrive; 2: second, the partner's sums are published;
    // 3: second, the partner never published them (the poll bound expired)
    __shared__ uint32_t s_role;
    if (tid == 0) {
      uint32_t role = 1;
      if (__hip_atomic_exchange(arrive, launch_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == launch_id) {
        // the partner has swapped its id in, so it is running and publishes
        // after its stores; the bound only guards against a lost workgroup
        role = 3;
        for (int n = 0; n < poll_limit; ++n) {
          if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == launch_id) {
            role = 2;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      s_role = role;
    }
    __syncthreads();
    const uint32_t role = s_role;
    if (role == 1) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            __hip_atomic_store(&slot[((i * TJ + j) * 16 + v) * 64], acc[i][j][v] * cref[j],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait_vm<0>();
      __syncthreads();
      if (tid == 0) __hip_atomic_store(flag, launch_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (tid == 0) {
      __hip_atomic_store(arrive, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(flag, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (role == 2) {
#pragma clang fp contract(off)
      // One accumulator tile (16 values) at a time: add the partner's 16
      // partial sums and store that tile's outputs right away, with the next
      // tile's partial sums already in flight.  (Adding all 128 first and
      // storing after kept every sum live across the stores, spilled, and made
      // the stores ten times slower than in the unsplit kernel.)
      float o[2][16];
      auto ld = [&](int q, float* d) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          d[v] = __hip_atomic_load(&slot[(q * 16 + v) * 64], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      };
      ld(0, o[0]);
#pragma unroll
      for (int q = 0; q < TI * TJ; ++q) {  // q = i TJ + j
        const int i = q / TJ, j = q % TJ;
        if (q < TI * TJ - 1) ld(q + 1, o[(q + 1) & 1]);
        const int gn = n0 + lcol0 + 32 * j;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // round(a c) + round(a' c'): each half's product is rounded on its
          // own (contraction off), so the sum does not depend on which half
          // came first
          const float s_ = acc[i][j][v] * cref[j] + o[q & 1][v];
          const int gm = m0 + wm * 32 * TI + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (gm < M && gn < N) y[(size_t)gm * N + gn] = out16<XF16>(s_);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    // never silently wrong: a tile whose other half never arrived is NaN
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_nanf("");
        cref[j] = 1.f;
      }
  }

  // lane holds column (lane & 31) and rows 8*(v/4) + 4*(lane/32) + v%4 of each MFMA tile
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int gn = n0 + lcol0 + 32 * j;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int gm = m0 + wm * 32 * TI + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (gm < M && gn < N) {
          const float v_ = acc[i][j][v] * cref[j];
          y[(size_t)gm * N + gn] = out16<XF16>(v_);
        }
      }
    }
}

// Tile width of the 256-row kernel: 192 when 256-wide tiles would run more
// than half of the compute units but leave part of a round idle (too many to
// split in two) while 192-wide tiles fill whole rounds exactly (qkv at
// M = 2048: 192 tiles of 256 columns, 256 of 192); else 256.
int lds_tile_n(int M, int N) {
  const int64_t ntm = (M + kLM - 1) / kLM, cus = num_cus();
  const int64_t t256 = ntm * ((N + kLN - 1) / kLN), t192 = ntm * ((N + 191) / 192);
  if (N % 192 == 0 && 2 * t256 > cus && t256 % cus != 0 && t192 % cus == 0) return 192;
  return kLN;
}

// Split K in two for the tiles of a round that fills at most half of the
// compute units: all tiles when there are at most half as many as compute
// units, else the last partial round (launched after the full rounds, so its
// 2r half-tile workgroups run side by side).  Each half keeps at least two
// groups' worth of 64-k tiles.  Returns the number of split tiles (0: no split).
int64_t split_tail(int M, int K, int N, int G, int64_t cus, int* tsplit) {
  const int tn = lds_tile_n(M, N);
  const int64_t tiles = (int64_t)((M + kLM - 1) / kLM) * ((N + tn - 1) / tn);
  const int T = K / kBK;
  const int tpg = G >= kBK ? G / kBK : 1;  // 64-k tiles per group
  *tsplit = (T / 2) / std::max(tpg, 2) * std::max(tpg, 2);
  const int64_t tail = tiles <= cus ? tiles : tiles % cus;  // tiles of the last round
  if (tail > 0 && 2 * tail <= cus && *tsplit >= 2 * tpg && T - *tsplit >= 2 * tpg) return tail;
  return 0;
}

// Scratch of a split: per split tile two 64-bit words (padded to 256 bytes
// in all), then a 256 x 256 fp32 partial tile.
size_t split_sync_bytes(int64_t tail) { return ((size_t)tail * 16 + 255) / 256 * 256; }
size_t split_bytes(int64_t tail) { return tail ? split_sync_bytes(tail) + (size_t)tail * kLM * kLN * 4 : 0; }

// Polls of the second half of a split tile before it gives up on the first
// and writes NaN: 2^24 (each poll sleeps about 128 cycles, so about a second),
// or GQ_SPLIT_POLL_LIMIT from the environment (a test sets 0 to take the
// timeout path on purpose; every workgroup still exits normally).
int split_poll_limit() {
  const char* e = std::getenv("GQ_SPLIT_POLL_LIMIT");
  if (!e || !*e) return 1 << 24;
  const long v = std::strtol(e, nullptr, 10);
  return (int)std::min<long>(std::max<long>(v, 0), 1 << 24);
}

// ws: scratch of at least split_bytes(split_tail(...)) bytes, or NULL: the
// tiles then all run unsplit.
template <bool SYM, int MODE, bool XF16, bool NARROW>
hipError_t launch_lds_t(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                      const uint16_t* zr, int N, int G, uint16_t* y, void* ws, hipStream_t s) {
  constexpr int TN = NARROW ? 192 : kLN;
  const int64_t tiles = (int64_t)((M + kLM - 1) / kLM) * ((N + TN - 1) / TN);
  int tsplit = 0;
  const int64_t tail = ws ? split_tail(M, K, N, G, num_cus(), &tsplit) : 0;
  if (tail > 0) {
    uint64_t* sync = (uint64_t*)ws;
    float* part = (float*)((char*)ws + split_sync_bytes(tail));
    const int64_t full = tiles - tail;  // a multiple of the CU count: whole rounds
    if (full > 0) {
      hipLaunchKernelGGL((w4a16_gemm_lds_kernel<SYM, MODE, false, XF16, NARROW>), dim3((unsigned)full),
                         dim3(kLT), 0, s, x, M, K, qw, sc, zr, N, G, y, nullptr, nullptr, 0, 0,
                         (int)full, (uint64_t)0, 0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((w4a16_gemm_lds_kernel<SYM, MODE, true, XF16, NARROW>), dim3((unsigned)(2 * tail)),
                       dim3(kLT), 0, s, x, M, K, qw, sc, zr, N, G, y, sync, part, tsplit,
                       (int)full, (int)tail, next_launch_id(), split_poll_limit());
    return hipGetLastError();
  }
  hipLaunchKernelGGL((w4a16_gemm_lds_kernel<SYM, MODE, false, XF16, NARROW>), dim3((unsigned)tiles), dim3(kLT), 0,
                     s, x, M, K, qw, sc, zr, N, G, y, nullptr, nullptr, 0, 0, (int)tiles, (uint64_t)0, 0);
  return hipGetLastError();
}

template <bool SYM, int MODE, bool XF16 = false>
hipError_t launch_lds(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                      const uint16_t* zr, int N, int G, uint16_t* y, void* ws, hipStream_t s) {
  if (lds_tile_n(M, N) == 192) return launch_lds_t<SYM, MODE, XF16, true>(x, M, K, qw, sc, zr, N, G, y, ws, s);
  return launch_lds_t<SYM, MODE, XF16, false>(x, M, K, qw, sc, zr, N, G, y, ws, s);
}

// Boundary pattern of the 256 x 256 kernel for this group size, or -1.
int lds_mode(int K, int G) {
  if (K % kBK != 0) return -1;
  if (G == 32) return -1;  // two rescales per tile exceed the register budget
  if (G == 64) return 1;
  if (G == 128) return 2;
  if (G % 256 == 0) return 3;
  return -1;
}

template <int WM, bool SYM, bool XF16>
hipError_t launch_t(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                    const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  constexpr int BM = 128 * WM;
  const int64_t grid = (int64_t)((M + BM - 1) / BM) * ((N + kBN - 1) / kBN);
  const size_t lds = (size_t)2 * (BM + kBN) * kLdsRow * 2 + (size_t)2 * 2 * kBN * 4;
  if (K % kBK == 0)
    hipLaunchKernelGGL((w4a16_gemm_kernel<WM, SYM, false, XF16>), dim3((unsigned)grid), dim3(256 * WM),
                       lds, s, x, M, K, qw, sc, zr, N, G, y);
  else
    hipLaunchKernelGGL((w4a16_gemm_kernel<WM, SYM, true, XF16>), dim3((unsigned)grid), dim3(256 * WM),
                       lds, s, x, M, K, qw, sc, zr, N, G, y);
  return hipGetLastError();
}

template <bool SYM, bool XF16>
hipError_t dispatch(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                    const uint16_t* zr, int N, int G, uint16_t* y, void* ws, hipStream_t s) {
  switch (lds_mode(K, G)) {
    case 1: return launch_lds<SYM, 1, XF16>(x, M, K, qw, sc, zr, N, G, y, ws, s);
    case 2: return launch_lds<SYM, 2, XF16>(x, M, K, qw, sc, zr, N, G, y, ws, s);
    case 3: return launch_lds<SYM, 3, XF16>(x, M, K, qw, sc, zr, N, G, y, ws, s);
    default: break;
  }
  // 256-row tiles run two waves per SIMD and are faster per compute unit; the
  // 128-row tile (one wave per SIMD) wins when its tiles exactly fill the GPU
  // once while the 256-row tiles would leave compute units idle (measured on
  // 2048 x 4096 x 4096 and 2048 x 4096 x 14336: +11 %).
  const int64_t tiles256 = (int64_t)((M + 255) / 256) * ((N + kBN - 1) / kBN);
  if (tiles256 < num_cus() && 2 * tiles256 <= num_cus())
    return launch_t<1, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
  return launch_t<2, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
}

}  // namespace

// Scratch of gq_w4a16_gemm_noalloc: a fixed array in device memory, one per
// GPU (each device's copy at its own address), held until the process ends.
// It holds the split handshake words and partial sums of one call at a time;
// nothing in it needs to start at zero (the handshake tells stale words from
// this call's by the launch id).  Host code uses the per-device address from
// hipGetSymbolAddress, never the array's name.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

void* noalloc_scratch(hipError_t* err) {
  constexpr int kMaxDev = 64;
  static std::atomic<void*> addr[kMaxDev];
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDev) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N, int G) {
  if (lds_mode((int)K, G) < 0) return 0;
  int tsplit = 0;
  return split_bytes(split_tail((int)M, (int)K, (int)N, G, num_cus(), &tsplit));
}

hipError_t launch_w4a16_gemm(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                             const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                             int symmetric, uint16_t* y, void* workspace, bool xf16, hipStream_t s) {
  const int m = (int)M, k = (int)K, n = (int)N;
  if (xf16)
    return symmetric ? dispatch<true, true>(x, m, k, qweight, scales, zeros, n, G, y, workspace, s)
                     : dispatch<false, true>(x, m, k, qweight, scales, zeros, n, G, y, workspace, s);
  return symmetric ? dispatch<true, false>(x, m, k, qweight, scales, zeros, n, G, y, workspace, s)
                   : dispatch<false, false>(x, m, k, qweight, scales, zeros, n, G, y, workspace, s);
}

}  // namespace gq
