// Group-wise affine quantization, INT4 packing and dequantization kernels.
//
// Quantization follows "vLLM 量化与推测解码" section 1 (q = clamp(round(x/s)+z),
// x^ = s(q - z); min-max scale and zero over a zero-inclusive range; per-group
// along the last axis) and the symmetric max-abs quantizer of the S08 "量化"
// page ("核心思路").  The decisions are taken in binary64 with the stored fp16
// scale, so every output is a deterministic function of the input bits.  None
// of this runs on the decode path: it is the offline step that produces the
// packed weight the fused kernels read.
#include "gq_internal.h"

namespace gq {
namespace {

constexpr int kThreads = 256;

// One thread quantizes one (row, group).  Offline work: simple and exact.
__global__ __launch_bounds__(kThreads) void quantize_groups_kernel(
    const void* __restrict__ w, gq_dtype dt, int64_t N, int64_t K, int bits, int G,
    int symmetric, uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
    uint16_t* __restrict__ zeros) {
#pragma clang fp contract(off)
  const int64_t ng = K / G;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= N * ng) return;
  const int64_t row = gid / ng;
  const int64_t g = gid - row * ng;
  const int64_t base = row * K + g * G;

  if (symmetric) {
    const double qmax = (double)((1 << (bits - 1)) - 1);
    const double qmin = -(double)(1 << (bits - 1));
    double amax = 0.0;
    for (int i = 0; i < G; ++i) amax = fmax(amax, fabs(load_elem_f64(w, base + i, dt)));
    const double s = amax > 0.0 ? amax / qmax : 1.0;
    const uint16_t sh = scale_to_f16(s);
    const double S = f16_to_f64(sh);
    for (int i = 0; i < G; ++i) {
      const double q = fmin(fmax(rint(load_elem_f64(w, base + i, dt) / S), qmin), qmax);
      codes[base + i] = (uint8_t)(int8_t)(int)q;
    }
    scales[gid] = sh;
  } else {
    const double qmax = (double)((1 << bits) - 1);
    double lo = 0.0, hi = 0.0;  // the range always holds 0
    for (int i = 0; i < G; ++i) {
      const double v = load_elem_f64(w, base + i, dt);
      lo = fmin(lo, v);
      hi = fmax(hi, v);
    }
    const double s = (hi != lo) ? (hi - lo) / qmax : 1.0;
    const uint16_t sh = scale_to_f16(s);
    const double S = f16_to_f64(sh);
    const double z = fmin(fmax(rint(0.0 - lo / S), 0.0), qmax);
    for (int i = 0; i < G; ++i) {
      const double q = fmin(fmax(rint(load_elem_f64(w, base + i, dt) / S) + z, 0.0), qmax);
      codes[base + i] = (uint8_t)(int)q;
    }
    scales[gid] = sh;
    zeros[gid] = f64_to_f16_rne(z);
  }
}

// One thread writes one packed byte (two codes along K).
__global__ __launch_bounds__(kThreads) void pack_int4_kernel(const uint8_t* __restrict__ codes,
                                                           int64_t total_bytes, int symmetric,
                                                           uint8_t* __restrict__ qweight) {
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= total_bytes) return;
  const uint32_t off = symmetric ? 8u : 0u;
  const uint32_t lo = ((uint32_t)codes[2 * j] + off) & 15u;
  const uint32_t hi = ((uint32_t)codes[2 * j + 1] + off) & 15u;
  qweight[j] = (uint8_t)(lo | (hi << 4));
}

// One thread expands one packed byte into two weights: S (nibble - z), exact
// in float32 (11-bit scale times a 5-bit integer).
__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    const uint8_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ zeros, int64_t N, int64_t K, int G, int symmetric,
    void* __restrict__ out, gq_dtype odt) {
  const int64_t half = K / 2;
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= N * half) return;
  const int64_t row = j / half;
  const int64_t k = 2 * (j - row * half);
  const int64_t gi = row * (K / G) + k / G;
  const float S = f16_to_f32(scales[gi]);
  const float z = symmetric ? 8.0f : f16_to_f32(zeros[gi]);
  const uint32_t b = qweight[j];
  const float v0 = S * ((float)(b & 15u) - z);
  const float v1 = S * ((float)(b >> 4) - z);
  const int64_t o = row * K + k;
  if (odt == GQ_F32) {
    ((float*)out)[o] = v0;
    ((float*)out)[o + 1] = v1;
  } else if (odt == GQ_BF16) {
    ((uint16_t*)out)[o] = f32_to_bf16_rne(v0);
    ((uint16_t*)out)[o + 1] = f32_to_bf16_rne(v1);
  } else {
    ((_Float16*)out)[o] = (_Float16)v0;
    ((_Float16*)out)[o + 1] = (_Float16)v1;
  }
}

// Ingest of the group-major layout of the "量化" chapter's fused_matmul (codes
// [n_groups, group, N], i.e. K-major with N contiguous): a 128 (k) x 64 (n) tile
// is read row by row (64 consecutive bytes per wave load), transposed through
// LDS, and written as 64 packed rows of 64 bytes (16-byte stores; K % 32 == 0,
// so every 32-k chunk of a row is wholly inside or outside K).
constexpr int kIngK = 128, kIngN = 64;

__global__ __launch_bounds__(kThreads) void ingest_codes_kernel(const int8_t* __restrict__ codes,
                                                              int64_t K, int64_t N,
                                                              uint8_t* __restrict__ qweight) {
  __shared__ int8_t tile[kIngK][kIngN + 4];
  const int64_t ntn = (N + kIngN - 1) / kIngN;
  const int64_t k0 = (int64_t)blockIdx.x / ntn * kIngK;
  const int64_t n0 = (int64_t)blockIdx.x % ntn * kIngN;
  const int t = threadIdx.x;
  {
    const int nc = t & (kIngN - 1);
    const int64_t n = n0 + nc;
    for (int kr = t / kIngN; kr < kIngK; kr += kThreads / kIngN) {
      const int64_t k = k0 + kr;
      tile[kr][nc] = (k < K && n < N) ? codes[k * N + n] : (int8_t)0;
    }
  }
  __syncthreads();
  const int nr = t >> 2;             // output row within the tile
  const int jb = (t & 3) * 16;       // first packed byte (32 k values)
  const int64_t n = n0 + nr;
  if (n >= N || k0 + 2 * jb >= K) return;
  uint32_t w[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int kk = 2 * (jb + 4 * d + b);
      const uint32_t lo = ((uint32_t)(int)tile[kk][nr] + 8u) & 15u;
      const uint32_t hi = ((uint32_t)(int)tile[kk + 1][nr] + 8u) & 15u;
      v |= (lo | (hi << 4)) << (8 * b);
    }
    w[d] = v;
  }
  *(uint4*)(qweight + n * (K / 2) + k0 / 2 + jb) = make_uint4(w[0], w[1], w[2], w[3]);
}

// scales [n_groups, N] -> [N, n_groups]: one thread per element.
__global__ __launch_bounds__(kThreads) void transpose_scales_kernel(const uint16_t* __restrict__ in,
                                                                  int64_t ng, int64_t N,
                                                                  uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= ng * N) return;
  const int64_t n = i / ng, g = i - n * ng;
  out[i] = in[g * N + n];
}

// One thread expands 8 consecutive weights of a row (4 packed bytes, one group:
// G is a multiple of 32) and writes them with 16-byte stores.  Needs qweight
// 4-byte and the output 16-byte aligned; the per-byte kernel serves the rest.
__global__ __launch_bounds__(kThreads) void dequantize8_kernel(
    const uint8_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ zeros, int64_t N, int64_t K, int G, int symmetric,
    void* __restrict__ out, gq_dtype odt) {
  const int64_t per_row = K / 8;
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= N * per_row) return;
  const int64_t row = j / per_row;
  const int64_t k = 8 * (j - row * per_row);
  const int64_t gi = row * (K / G) + k / G;
  const float S = f16_to_f32(scales[gi]);
  const float z = symmetric ? 8.0f : f16_to_f32(zeros[gi]);
  const uint32_t d = *(const uint32_t*)(qweight + row * (K / 2) + k / 2);
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = S * ((float)((d >> (4 * i)) & 15u) - z);  // exact in fp32
  const int64_t o = row * K + k;
  if (odt == GQ_F32) {
    float4* p = (float4*)((float*)out + o);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = odt == GQ_BF16 ? f32_to_bf16_rne(v[2 * i])
                                          : __builtin_bit_cast(uint16_t, (_Float16)v[2 * i]);
      const uint32_t hi = odt == GQ_BF16 ? f32_to_bf16_rne(v[2 * i + 1])
                                          : __builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]);
      h[i] = lo | (hi << 16);
    }
    *(uint4*)((uint16_t*)out + o) = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_quantize_groups(const void* w, gq_dtype dt, int64_t N, int64_t K, int bits,
                                  int G, int symmetric, void* codes, uint16_t* scales,
                                  uint16_t* zeros, hipStream_t s) {
  const int64_t groups = N * (K / G);
  hipLaunchKernelGGL(quantize_groups_kernel, dim3(blocks_for(groups)), dim3(kThreads), 0, s, w,
                     dt, N, K, bits, G, symmetric, (uint8_t*)codes, scales, zeros);
  return hipGetLastError();
}

hipError_t launch_pack_int4(const void* codes, int64_t N, int64_t K, int symmetric,
                            uint8_t* qweight, hipStream_t s) {
  const int64_t total = N * (K / 2);
  hipLaunchKernelGGL(pack_int4_kernel, dim3(blocks_for(total)), dim3(kThreads), 0, s,
                     (const uint8_t*)codes, total, symmetric, qweight);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* qweight, const uint16_t* scales,
                             const uint16_t* zeros, int64_t N, int64_t K, int G, int symmetric,
                             void* out, gq_dtype odt, hipStream_t s) {
  if (((uintptr_t)qweight & 3u) == 0 && ((uintptr_t)out & 15u) == 0 && K % 8 == 0 && G % 8 == 0) {
    const int64_t total8 = N * (K / 8);
    hipLaunchKernelGGL(dequantize8_kernel, dim3(blocks_for(total8)), dim3(kThreads), 0, s, qweight,
                       scales, zeros, N, K, G, symmetric, out, odt);
    return hipGetLastError();
  }
  const int64_t total = N * (K / 2);
  hipLaunchKernelGGL(dequantize_kernel, dim3(blocks_for(total)), dim3(kThreads), 0, s, qweight,
                     scales, zeros, N, K, G, symmetric, out, odt);
  return hipGetLastError();
}

hipError_t launch_ingest_group_major(const int8_t* codes, const uint16_t* scales, int64_t ng,
                                     int64_t group, int64_t N, uint8_t* qweight,
                                     uint16_t* scales_out, hipStream_t s) {
  const int64_t K = ng * group;
  const int64_t tiles = ((N + kIngN - 1) / kIngN) * ((K + kIngK - 1) / kIngK);
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ingest_codes_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, s, codes, K, N,
                     qweight);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(transpose_scales_kernel, dim3(blocks_for(ng * N)), dim3(kThreads), 0, s, scales,
                     ng, N, scales_out);
  return hipGetLastError();
}

}  // namespace gq
