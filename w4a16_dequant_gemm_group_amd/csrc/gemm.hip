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
// Tiling: a workgroup computes a (128 WM) x 256 tile of Y with WM x 4
// wavefronts; each wavefront owns a 128 x 64 block as 4 x 2
// v_mfma_f32_32x32x16_bf16 tiles.  K advances in 64-wide tiles through two LDS
// stages: the activation tile is copied in (bf16, 144-byte padded rows), the
// packed weight tile is expanded once per workgroup into exact bf16 (q - z), and
// the tile's column scales are stored beside it.  Global loads run two tiles
// ahead in registers; they are unconditional raw buffer loads (anything outside
// the matrices reads as zero), so the compiler's wait counts stay exact.  When
// K is a multiple of 64 the per-lane offsets are fixed and the k step (or the
// past-the-end marker) is a wave-uniform scalar offset, which the hardware
// range check includes; this keeps address arithmetic off the vector ALU,
// which on this GPU barely overlaps with MFMA execution.  With
// workgroups dealt round-robin to the 8 XCDs and the M tile varying fastest,
// each XCD keeps the same activation rows in its L2.
#include <algorithm>

#include "gq_internal.h"

namespace gq {
namespace {

constexpr int kBK = 64;
constexpr int kLdsRow = kBK + 8;  // bf16 elements per LDS row (+16 B pad)
constexpr int kBN = 256;
constexpr uint32_t kOob = 0x80000000u;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
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

// 8 nibbles (k = 0..7 at bits 4p) -> 8 bf16 values q - z in k order (4 dwords).
__device__ __forceinline__ uint4 expand8(uint32_t d, float z) {
  const uint32_t e = d & 0x0F0F0F0Fu, o = (d >> 4) & 0x0F0F0F0Fu;
  const float q0 = ubyte_f32<0>(e) - z, q2 = ubyte_f32<1>(e) - z;
  const float q4 = ubyte_f32<2>(e) - z, q6 = ubyte_f32<3>(e) - z;
  const float q1 = ubyte_f32<0>(o) - z, q3 = ubyte_f32<1>(o) - z;
  const float q5 = ubyte_f32<2>(o) - z, q7 = ubyte_f32<3>(o) - z;
  return make_uint4(pack_bf16(q0, q1), pack_bf16(q2, q3), pack_bf16(q4, q5), pack_bf16(q6, q7));
}

template <int WM, bool SYM, bool TAIL>
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
      uint4 e0 = expand8(S.b[h].x, zf), e1 = expand8(S.b[h].y, zf);
      uint4 e2 = expand8(S.b[h].z, zf), e3 = expand8(S.b[h].w, zf);
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
      bf16x8_t a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)&as[i * 32 * kLdsRow + kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = __builtin_bit_cast(bf16x8_t, *(const uint4*)&bs[j * 32 * kLdsRow + kk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
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
        if (gm < M && gn < N) y[(size_t)gm * N + gn] = f32_to_bf16_rne(acc[i][j][v] * cref[j]);
      }
    }
}

template <int WM, bool SYM>
hipError_t launch_t(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                    const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  constexpr int BM = 128 * WM;
  const int64_t grid = (int64_t)((M + BM - 1) / BM) * ((N + kBN - 1) / kBN);
  const size_t lds = (size_t)2 * (BM + kBN) * kLdsRow * 2 + (size_t)2 * 2 * kBN * 4;
  if (K % kBK == 0)
    hipLaunchKernelGGL((w4a16_gemm_kernel<WM, SYM, false>), dim3((unsigned)grid), dim3(256 * WM), lds,
                       s, x, M, K, qw, sc, zr, N, G, y);
  else
    hipLaunchKernelGGL((w4a16_gemm_kernel<WM, SYM, true>), dim3((unsigned)grid), dim3(256 * WM), lds,
                       s, x, M, K, qw, sc, zr, N, G, y);
  return hipGetLastError();
}

template <bool SYM>
hipError_t dispatch(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                    const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  // 256-row tiles run two waves per SIMD and are faster per compute unit; the
  // 128-row tile (one wave per SIMD) wins when its tiles exactly fill the GPU
  // once while the 256-row tiles would leave compute units idle (measured on
  // 2048 x 4096 x 4096 and 2048 x 4096 x 14336: +11 %).
  const int64_t tiles256 = (int64_t)((M + 255) / 256) * ((N + kBN - 1) / kBN);
  if (tiles256 < num_cus() && 2 * tiles256 <= num_cus())
    return launch_t<1, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
  return launch_t<2, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
}

}  // namespace

hipError_t launch_w4a16_gemm(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                             const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                             int symmetric, uint16_t* y, hipStream_t s) {
  if (symmetric)
    return dispatch<true>(x, (int)M, (int)K, qweight, scales, zeros, (int)N, G, y, s);
  return dispatch<false>(x, (int)M, (int)K, qweight, scales, zeros, (int)N, G, y, s);
}

}  // namespace gq
