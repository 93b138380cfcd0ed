// Fused W4A16 GEMV for decode (M <= 16) on gfx950.
//
// What is computed ("vLLM 量化与推测解码" section 2, fused W4A16 paragraph; the
// S08 "量化" page, "工作原理" figure right panel and "亲手实现"):
//   y[m, n] = bf16( sum_g S[n,g] * sum_{k in g} x[m,k] * (q[n,k] - z[n,g]) )
// reading only packed nibbles and the fp16 group scale/zero from HBM; the
// dequantized weight exists only in registers.
//
// Decode is bound by HBM bandwidth (S08 "为什么重要": latency = bytes /
// bandwidth), so the kernel is shaped around the weight stream:
//   * a wavefront owns RPW rows; lane l of the wave reads 16 contiguous bytes
//     (32 nibbles) of a row at k = 2048 t + 32 l, so one wave load instruction
//     covers 1 KiB of a row contiguously (global_load_dwordx4, fully coalesced);
//     every weight load of the wave's rows is issued before any arithmetic;
//   * x is staged once per workgroup into LDS, pre-permuted so that each
//     dword holds the bf16 pair (x[k+p], x[k+p+4]) that matches the nibble pair
//     (k+p, k+p+4) extracted below, plus the sum of every 32-element chunk;
//   * a nibble pair becomes two exact bf16 values 128+q with one AND-OR
//     (0x4300 is bf16 128.0; the nibble fills the low mantissa bits), and
//     v_dot2c_f32_bf16 multiplies both by x and accumulates in fp32:
//     11 VALU ops per 8 weights;
//   * per 32-chunk the offset and zero point are removed with the chunk sum:
//     sum x (q - z) = sum x (128 + q) - (128 + z) sum x, then scaled by S;
//   * the fp32 partials are summed across the wave with cross-lane adds and
//     rounded once to bf16 (nearest-even).
#include "gq_internal.h"

namespace gq {
namespace {

constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kWaves = kThreads / 64;
constexpr int kStepK = 2048;   // k covered by one wave load (64 lanes x 32)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// 8 nibbles of one dword (k offsets 0..7 at bits 4p) against the permuted
// activation dwords (x0,x4) (x1,x5) (x2,x6) (x3,x7).
__device__ __forceinline__ float dot8(uint32_t d, const uint4& xp, float a) {
  constexpr uint32_t kMask = 0x000F000Fu, kMagic = 0x43004300u;
  a = dot2((d & kMask) | kMagic, xp.x, a);
  a = dot2(((d >> 4) & kMask) | kMagic, xp.y, a);
  a = dot2(((d >> 8) & kMask) | kMagic, xp.z, a);
  a = dot2(((d >> 12) & kMask) | kMagic, xp.w, a);
  return a;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Stage x[:, kc0 : kc0 + KC) into LDS as permuted pairs plus 32-chunk sums.
template <int MT, int KC>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, int M, int K, int kc0,
                                        uint4 (*xs)[KC / 8], float (*sx)[KC / 32]) {
  static_assert((KC / 8) % kThreads == 0, "chunk must be a multiple of 2048");
  for (int idx = threadIdx.x; idx < MT * (KC / 8); idx += kThreads) {
    const int m = idx / (KC / 8);
    const int c = idx - m * (KC / 8);
    const int k = kc0 + c * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < M && k < K) v = *(const uint4*)(x + (size_t)m * K + k);
    uint4 p;
    p.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // (x0, x4)
    p.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // (x1, x5)
    p.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // (x2, x6)
    p.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // (x3, x7)
    xs[m][c] = p;
    float s = bf16_to_f32(v.x & 0xFFFFu) + bf16_to_f32(v.x >> 16);
    s += bf16_to_f32(v.y & 0xFFFFu) + bf16_to_f32(v.y >> 16);
    s += bf16_to_f32(v.z & 0xFFFFu) + bf16_to_f32(v.z >> 16);
    s += bf16_to_f32(v.w & 0xFFFFu) + bf16_to_f32(v.w >> 16);
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if ((c & 3) == 0) sx[m][c >> 2] = s;
  }
}

// MT: activation rows handled together (M <= MT), RPW: weight rows per wave,
// T: 2048-wide steps per LDS chunk.  Each workgroup owns 4*RPW rows.
template <int MT, int RPW, int T, bool SYM>
__global__ __launch_bounds__(kThreads) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int N, int G,
    uint16_t* __restrict__ y) {
  constexpr int KC = T * kStepK;
  __shared__ uint4 xs[MT][KC / 8];
  __shared__ float sx[MT][KC / 32];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * kWaves + wave) * RPW;
  const int ng = K / G;
  const size_t row_bytes = (size_t)K / 2;

  float acc[MT][RPW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[m][r] = 0.f;

  for (int kc0 = 0; kc0 < K; kc0 += KC) {
    if (kc0) __syncthreads();
    stage_x<MT, KC>(x, M, K, kc0, xs, sx);
    __syncthreads();

    // Phase 1: issue every weight/scale load of this chunk.
    uint4 wv[T][RPW];
    float sc[T][RPW], zo[T][RPW];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int k = kc0 + t * kStepK + lane * 32;
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int row = row0 + r;
        wv[t][r] = make_uint4(0, 0, 0, 0);
        sc[t][r] = 0.f;
        zo[t][r] = 0.f;
        if (k < K && row < N) {
          wv[t][r] = load_nt16(qw + row * row_bytes + k / 2);
          const int gi = row * ng + k / G;
          sc[t][r] = f16_to_f32(scales[gi]);
          zo[t][r] = SYM ? 136.f : 128.f + f16_to_f32(zeros[gi]);
        }
      }
    }
    // Phase 2: unpack, dot, correct per 32-chunk.
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int kl = t * kStepK + lane * 32;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint4* xp = &xs[m][kl / 8];
        const uint4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
        const float sxm = sx[m][kl / 32];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          float a = dot8(wv[t][r].x, x0, 0.f);
          a = dot8(wv[t][r].y, x1, a);
          a = dot8(wv[t][r].z, x2, a);
          a = dot8(wv[t][r].w, x3, a);
          acc[m][r] = fmaf(sc[t][r], fmaf(-zo[t][r], sxm, a), acc[m][r]);
        }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const float v = wave_sum(acc[m][r]);
      const int row = row0 + r;
      if (lane == 0 && m < M && row < N) y[(size_t)m * N + row] = f32_to_bf16_rne(v);
    }
}

template <int MT, int RPW, int T, bool SYM>
hipError_t launch_t(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                    const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  const int rows_per_block = kWaves * RPW;
  const unsigned grid = (unsigned)((N + rows_per_block - 1) / rows_per_block);
  hipLaunchKernelGGL((w4a16_gemv_kernel<MT, RPW, T, SYM>), dim3(grid), dim3(kThreads), 0, s, x,
                     M, K, qw, sc, zr, N, G, y);
  return hipGetLastError();
}

template <bool SYM>
hipError_t dispatch(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                    const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  const int steps = (K + kStepK - 1) / kStepK;
  if (M == 1) {
    switch (steps) {
      case 1: return launch_t<1, 2, 1, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
      case 2: return launch_t<1, 2, 2, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
      case 3: return launch_t<1, 2, 3, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
      case 4: return launch_t<1, 2, 4, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
      case 5: return launch_t<1, 2, 5, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
      case 6: return launch_t<1, 2, 6, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
      case 7: return launch_t<1, 2, 7, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
      default: return launch_t<1, 2, 8, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
    }
  }
  if (M == 2) return launch_t<2, 2, 2, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
  if (M <= 4) return launch_t<4, 2, 1, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
  if (M <= 8) return launch_t<8, 2, 1, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
  return launch_t<16, 2, 1, SYM>(x, M, K, qw, sc, zr, N, G, y, s);
}

}  // namespace

hipError_t launch_w4a16_gemv(const uint16_t* x, int M, int64_t K, const uint8_t* qweight,
                             const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                             int symmetric, uint16_t* y, hipStream_t s) {
  if (symmetric) return dispatch<true>(x, M, (int)K, qweight, scales, zeros, (int)N, G, y, s);
  return dispatch<false>(x, M, (int)K, qweight, scales, zeros, (int)N, G, y, s);
}

}  // namespace gq
