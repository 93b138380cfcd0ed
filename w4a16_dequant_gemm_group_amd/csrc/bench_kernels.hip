// Comparators and probes that the 4-bit kernels are measured against, with no
// quantization in them:
//   - a plain bf16 GEMV over an unquantized [N, K] weight: the 16-bit baseline
//     the fused W4A16 kernel is compared with ("vLLM 量化与推测解码", section 2:
//     decode reads every weight once per token, so the weight bytes set the
//     time), and the second half of the unfused path "dequantize to a bf16
//     weight in HBM, then multiply" ("量化" chapter, "亲手实现", the paragraph
//     on the common pitfall of materializing the weight);
//   - an HBM stream read: the read bandwidth one kernel reaches on this GPU,
//     the practical ceiling for every weight-streaming kernel.
#include "gq_internal.h"

namespace gq {
namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr uint32_t kOob = 0x80000000u;  // past every buffer's range: loads read zero
constexpr int kWaves = 4;               // waves per workgroup
constexpr int kRowsPerWave = 2;
constexpr int kUnroll = 4;              // 16-byte loads in flight per row per wave
constexpr int kStep = 512;              // k covered by one wave-wide 16-byte load

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                           0x00020000);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float dot8(const uint4& w, const uint4& x, float a) {
  a = dot2(w.x, x.x, a);
  a = dot2(w.y, x.y, a);
  a = dot2(w.z, x.z, a);
  return dot2(w.w, x.w, a);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// y[m, n] = bf16(sum_k x[m, k] w[n, k]), fp32 accumulation.  A wave owns two
// rows; lane l reads the 8 weights at k = 512 j + 8 l of each, 16 bytes per
// load, with kUnroll loads per row in flight.  x is staged in LDS, zero-padded
// to a multiple of kStep * kUnroll; weight loads past a row's end or past the
// last row read zero through the buffer range check or the out-of-range
// offset, so no lane branches.
template <int M>
__global__ __launch_bounds__(256) void bf16_gemv_kernel(const uint16_t* __restrict__ x, int K,
                                                        int Kpad, const uint16_t* __restrict__ w,
                                                        int N, uint16_t* __restrict__ y) {
  extern __shared__ uint4 xs[];  // [M][Kpad / 8]
  const int tid = threadIdx.x;
  const int kq = Kpad / 8;
  for (int i = tid; i < M * kq; i += 256) {
    const int m = i / kq, c = i - m * kq;
    uint4 v = {0u, 0u, 0u, 0u};
    if (c * 8 < K) v = *(const uint4*)(x + (size_t)m * K + (size_t)c * 8);
    xs[i] = v;
  }
  __syncthreads();

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row0 = (blockIdx.x * kWaves + wave) * kRowsPerWave;
  const rsrc_t rw = make_rsrc(w, (uint32_t)((size_t)N * K * 2));
  uint32_t roff[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
    roff[r] = row0 + r < N ? (uint32_t)(row0 + r) * (uint32_t)K * 2u : kOob;

  float acc[kRowsPerWave][M];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  for (int k0 = 0; k0 < K; k0 += kStep * kUnroll) {
    uint4 wv[kUnroll][kRowsPerWave];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k = k0 + kStep * u + 8 * lane;
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        const uint32_t off = (k < K && roff[r] != kOob) ? roff[r] + 2u * (uint32_t)k : kOob;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 2);
        wv[u][r] = __builtin_bit_cast(uint4, v);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = (k0 + kStep * u) / 8 + lane;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4 xv = xs[m * kq + c];
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) acc[r][m] = dot8(wv[u][r], xv, acc[r][m]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[r][m];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0 && row0 + r < N) y[(size_t)m * N + row0 + r] = to_bf16(v);
    }
}

constexpr int kReadUnroll = 8;  // 16-byte loads per lane per workgroup

// Reads every 16-byte word of buf once (nontemporal) and folds them with xor.
// The fold is stored only when it equals a fixed constant, so the loads cannot
// be optimized away and the kernel writes (almost) nothing.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ buf,
                                                          int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * (256 * kReadUnroll) + threadIdx.x;
  u32x4_t v[kReadUnroll];
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) {
    const int64_t i = base + 256 * u;
    v[u] = i < n16 ? __builtin_nontemporal_load(buf + i) : u32x4_t{0u, 0u, 0u, 0u};
  }
  uint32_t a = 0;
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) a ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (a == 0x2545F491u) sink[0] = a;
}

}  // namespace

int bf16_gemv_kpad(int64_t K) {
  const int64_t c = (int64_t)kStep * kUnroll;
  return (int)((K + c - 1) / c * c);
}

hipError_t launch_bf16_gemv(const uint16_t* x, int M, int64_t K, const uint16_t* w, int64_t N,
                            uint16_t* y, hipStream_t s) {
  const int kpad = bf16_gemv_kpad(K);
  const size_t lds = (size_t)M * kpad * 2;
  const int rows_per_wg = kWaves * kRowsPerWave;
  const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg));
  switch (M) {
    case 1: bf16_gemv_kernel<1><<<grid, 256, lds, s>>>(x, (int)K, kpad, w, (int)N, y); break;
    case 2: bf16_gemv_kernel<2><<<grid, 256, lds, s>>>(x, (int)K, kpad, w, (int)N, y); break;
    case 3: bf16_gemv_kernel<3><<<grid, 256, lds, s>>>(x, (int)K, kpad, w, (int)N, y); break;
    case 4: bf16_gemv_kernel<4><<<grid, 256, lds, s>>>(x, (int)K, kpad, w, (int)N, y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t per_wg = 256 * kReadUnroll;
  const int64_t blocks = (n16 + per_wg - 1) / per_wg;
  stream_read_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>((const u32x4_t*)buf, n16, sink);
  return hipGetLastError();
}

}  // namespace gq
