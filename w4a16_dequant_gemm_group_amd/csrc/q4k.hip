// Nested 4-bit super-block format: quantize and fused GEMV on gfx950.
//
// Format (S08 "量化" page, "工作原理" figure, middle panel): 256 weights form a
// super-block of 8 sub-blocks of 32; each sub-block has a 6-bit scale and a
// 6-bit min, each super-block an fp16 scale-of-scales d and min-of-mins dmin,
// 4.5 bits per weight in all.  Bytes of one block (144, a multiple of 16):
//   [0] d fp16  [2] dmin fp16  [4] sc_0..7 (48-bit little-endian, 6 bits each)
//   [10] mn_0..7 likewise  [16] 128 nibble bytes, sub-block j at 16+16j.
// x^ = d*sc_j*q - dmin*mn_j.
//
// The GEMV uses the layout of the plain INT4 GEMV: lane l of a wave owns the
// 32 weights at k = 2048 t + 32 l, which here is sub-block l%8 of block
// 8t + l/8; it loads the block's 16-byte header (the eight lanes of one block
// share one address) and its 16 nibble bytes, both as dwordx4.
#include "gq_internal.h"

namespace gq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kStepK = 2048;
constexpr int kBlockBytes = 144;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float dot8(uint32_t d, const uint4& xp, float a) {
  constexpr uint32_t kMask = 0x000F000Fu, kMagic = 0x43004300u;  // bf16 128 + q
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

// One thread quantizes one 256-weight block (offline; binary64 decisions).
__global__ __launch_bounds__(kThreads) void q4k_quantize_kernel(const void* __restrict__ w,
                                                                gq_dtype dt, int64_t N,
                                                                int64_t K,
                                                                uint8_t* __restrict__ blocks) {
#pragma clang fp contract(off)
  const int64_t nb = K / 256;
  const int64_t bid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (bid >= N * nb) return;
  const int64_t base = (bid / nb) * K + (bid % nb) * 256;

  double s[8], m[8], smax = 0.0, mmax = 0.0;
  for (int j = 0; j < 8; ++j) {
    double lo = 0.0, hi = 0.0;
    for (int i = 0; i < 32; ++i) {
      const double v = load_elem_f64(w, base + 32 * j + i, dt);
      lo = fmin(lo, v);
      hi = fmax(hi, v);
    }
    s[j] = (hi != lo) ? (hi - lo) / 15.0 : 0.0;
    m[j] = 0.0 - lo;
    smax = fmax(smax, s[j]);
    mmax = fmax(mmax, m[j]);
  }
  const uint16_t dh = scale_to_f16(smax / 63.0);
  const uint16_t mh = scale_to_f16(mmax / 63.0);
  const double D = f16_to_f64(dh), Dm = f16_to_f64(mh);

  uint64_t scbits = 0, mnbits = 0;
  double S[8], Mn[8];
  for (int j = 0; j < 8; ++j) {
    const double sc = D > 0.0 ? fmin(fmax(rint(s[j] / D), 0.0), 63.0) : 0.0;
    const double mn = Dm > 0.0 ? fmin(fmax(rint(m[j] / Dm), 0.0), 63.0) : 0.0;
    scbits |= (uint64_t)sc << (6 * j);
    mnbits |= (uint64_t)mn << (6 * j);
    S[j] = D * sc;
    Mn[j] = Dm * mn;
  }

  uint8_t* out = blocks + bid * kBlockBytes;
  out[0] = (uint8_t)dh; out[1] = (uint8_t)(dh >> 8);
  out[2] = (uint8_t)mh; out[3] = (uint8_t)(mh >> 8);
  for (int b = 0; b < 6; ++b) {
    out[4 + b] = (uint8_t)(scbits >> (8 * b));
    out[10 + b] = (uint8_t)(mnbits >> (8 * b));
  }
  for (int j = 0; j < 8; ++j) {
    for (int i = 0; i < 32; i += 2) {
      uint32_t q2[2];
      for (int h = 0; h < 2; ++h) {
        const double v = load_elem_f64(w, base + 32 * j + i + h, dt);
        q2[h] = S[j] > 0.0 ? (uint32_t)fmin(fmax(rint((v + Mn[j]) / S[j]), 0.0), 15.0) : 0u;
      }
      out[16 + 16 * j + i / 2] = (uint8_t)(q2[0] | (q2[1] << 4));
    }
  }
}

template <int MT, int KC>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, int M, int K, int kc0,
                                        uint4 (*xs)[KC / 8], float (*sx)[KC / 32]) {
  for (int idx = threadIdx.x; idx < MT * (KC / 8); idx += kThreads) {
    const int m = idx / (KC / 8);
    const int c = idx - m * (KC / 8);
    const int k = kc0 + c * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < M && k < K) v = *(const uint4*)(x + (size_t)m * K + k);
    uint4 p;
    p.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
    p.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
    p.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
    p.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
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

template <int MT, int RPW, int T>
__global__ __launch_bounds__(kThreads) void q4k_gemv_kernel(const uint16_t* __restrict__ x, int M,
                                                            int K,
                                                            const uint8_t* __restrict__ blocks,
                                                            int N, uint16_t* __restrict__ y) {
  constexpr int KC = T * kStepK;
  __shared__ uint4 xs[MT][KC / 8];
  __shared__ float sx[MT][KC / 32];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * kWaves + wave) * RPW;
  const size_t row_bytes = (size_t)(K / 256) * kBlockBytes;
  const int sub = lane & 7;

  float acc[MT][RPW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[m][r] = 0.f;

  for (int kc0 = 0; kc0 < K; kc0 += KC) {
    if (kc0) __syncthreads();
    stage_x<MT, KC>(x, M, K, kc0, xs, sx);
    __syncthreads();

    uint4 hd[T][RPW], wv[T][RPW];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int k = kc0 + t * kStepK + lane * 32;
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int row = row0 + r;
        hd[t][r] = make_uint4(0, 0, 0, 0);
        wv[t][r] = make_uint4(0, 0, 0, 0);
        if (k < K && row < N) {
          const uint8_t* blk = blocks + row * row_bytes + (size_t)(k / 256) * kBlockBytes;
          hd[t][r] = *(const uint4*)blk;
          wv[t][r] = load_nt16(blk + 16 + 16 * sub);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int kl = t * kStepK + lane * 32;
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const uint4 h = hd[t][r];
        const float d = f16_to_f32((uint16_t)(h.x & 0xFFFFu));
        const float dmin = f16_to_f32((uint16_t)(h.x >> 16));
        const uint64_t scb = (uint64_t)h.y | ((uint64_t)(h.z & 0xFFFFu) << 32);
        const uint64_t mnb = (uint64_t)(h.z >> 16) | ((uint64_t)h.w << 16);
        const float S = d * (float)(uint32_t)((scb >> (6 * sub)) & 63u);
        const float Mn = dmin * (float)(uint32_t)((mnb >> (6 * sub)) & 63u);
        // contribution S*(sum x (128+q) - 128 sum x) - Mn sum x
        const float off = fmaf(128.f, S, Mn);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint4* xp = &xs[m][kl / 8];
          float a = dot8(wv[t][r].x, xp[0], 0.f);
          a = dot8(wv[t][r].y, xp[1], a);
          a = dot8(wv[t][r].z, xp[2], a);
          a = dot8(wv[t][r].w, xp[3], a);
          acc[m][r] = fmaf(S, a, fmaf(-off, sx[m][kl / 32], acc[m][r]));
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

template <int MT, int RPW, int T>
hipError_t launch_t(const uint16_t* x, int M, int K, const uint8_t* b, int N, uint16_t* y,
                    hipStream_t s) {
  const int rows_per_block = kWaves * RPW;
  const unsigned grid = (unsigned)((N + rows_per_block - 1) / rows_per_block);
  hipLaunchKernelGGL((q4k_gemv_kernel<MT, RPW, T>), dim3(grid), dim3(kThreads), 0, s, x, M, K, b,
                     N, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q4k_quantize(const void* w, gq_dtype dt, int64_t N, int64_t K, uint8_t* blocks,
                               hipStream_t s) {
  const int64_t nblk = N * (K / 256);
  hipLaunchKernelGGL(q4k_quantize_kernel, dim3((unsigned)((nblk + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, w, dt, N, K, blocks);
  return hipGetLastError();
}

hipError_t launch_q4k_gemv(const uint16_t* x, int M, int64_t K, const uint8_t* blocks, int64_t N,
                           uint16_t* y, hipStream_t s) {
  const int steps = (int)((K + kStepK - 1) / kStepK);
  const int k = (int)K, n = (int)N;
  if (M == 1) {
    switch (steps) {
      case 1: return launch_t<1, 2, 1>(x, M, k, blocks, n, y, s);
      case 2: return launch_t<1, 2, 2>(x, M, k, blocks, n, y, s);
      case 3: return launch_t<1, 2, 3>(x, M, k, blocks, n, y, s);
      case 4: return launch_t<1, 2, 4>(x, M, k, blocks, n, y, s);
      case 5: return launch_t<1, 2, 5>(x, M, k, blocks, n, y, s);
      case 6: return launch_t<1, 2, 6>(x, M, k, blocks, n, y, s);
      case 7: return launch_t<1, 2, 7>(x, M, k, blocks, n, y, s);
      default: return launch_t<1, 2, 8>(x, M, k, blocks, n, y, s);
    }
  }
  if (M == 2) return launch_t<2, 2, 2>(x, M, k, blocks, n, y, s);
  if (M <= 4) return launch_t<4, 2, 1>(x, M, k, blocks, n, y, s);
  if (M <= 8) return launch_t<8, 2, 1>(x, M, k, blocks, n, y, s);
  return launch_t<16, 2, 1>(x, M, k, blocks, n, y, s);
}

}  // namespace gq
