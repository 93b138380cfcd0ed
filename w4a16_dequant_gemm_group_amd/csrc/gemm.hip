// Fused W4A16 GEMM for prefill-sized M on gfx950 bf16 MFMA.
//
// Same product as the GEMV ("vLLM 量化与推测解码" section 2: Y = X W^T with a
// fused dequantizing kernel), for the compute-bound prefill shape
// ("量化：为何加速推理与精度权衡", follow-up questions: weight-only INT4 leaves the
// matmul FLOPs unchanged; prefill is compute-bound).
//
// Precision: the dequantized weight S(q - z) is *not* rounded to bf16.  The
// MFMA B operand is the exact small integer q - z (|q - z| <= 15 is exact in
// bf16), products are exact in fp32, and each group's partial sum is scaled by
// its fp16 scale in fp32: C += S[n,g] * (A_g . (q - z)_g).  The output is
// rounded once to bf16 (nearest-even).
//
// Tiling: a 512-thread workgroup (8 wavefronts, 4 x 2) computes a 256 x 128
// tile of Y; each wavefront a 64 x 64 block as 2 x 2 v_mfma_f32_32x32x16_bf16
// tiles.  K advances in 64-wide tiles: the activation tile is copied to LDS,
// the packed weight tile is expanded once per workgroup to exact bf16 (q - z)
// in LDS (so 256 rows of X share each expansion), and global loads of the next
// tile are in flight while the current one is multiplied.  With M = 2048 the 8
// row tiles of a column of workgroups land on the 8 XCDs (workgroups are
// dealt round-robin), so every XCD keeps one activation row-tile in its L2.
#include "gq_internal.h"

namespace gq {
namespace {

constexpr int kBM = 256, kBN = 128, kKT = 64;
constexpr int kThreads = 512;
constexpr int kLdsStride = kKT + 8;  // bf16 elements per LDS row (+16 B pad)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 8 nibbles (k = 0..7 at bits 4p) -> 8 exact bf16 values (q - z) in k order,
// as 4 dwords.  Bytes are biased by 128 so the per-byte subtraction never
// borrows, flipped back to two's complement, widened to fp32 (exact), and the
// upper halves of consecutive k are paired.
__device__ __forceinline__ uint4 expand8(uint32_t d, uint32_t zb) {
  uint32_t lo = ((d & 0x0F0F0F0Fu) | 0x80808080u) - zb;  // k = 0,2,4,6
  uint32_t hi = (((d >> 4) & 0x0F0F0F0Fu) | 0x80808080u) - zb;  // k = 1,3,5,7
  lo ^= 0x80808080u;
  hi ^= 0x80808080u;
  uint32_t f[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f[2 * b] = __float_as_uint((float)(int8_t)(lo >> (8 * b)));
    f[2 * b + 1] = __float_as_uint((float)(int8_t)(hi >> (8 * b)));
  }
  uint4 r;
  r.x = __builtin_amdgcn_perm(f[1], f[0], 0x07060302u);
  r.y = __builtin_amdgcn_perm(f[3], f[2], 0x07060302u);
  r.z = __builtin_amdgcn_perm(f[5], f[4], 0x07060302u);
  r.w = __builtin_amdgcn_perm(f[7], f[6], 0x07060302u);
  return r;
}

template <bool SYM>
__global__ __launch_bounds__(kThreads) void w4a16_gemm_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int N, int G,
    uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLdsStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // 4 x 2 wavefronts
  const int ntm = (M + kBM - 1) / kBM;
  const int m0 = (blockIdx.x % ntm) * kBM;
  const int n0 = (blockIdx.x / ntm) * kBN;
  const int ng = K / G;
  const size_t row_bytes = (size_t)K / 2;

  // --- global -> register prefetch of one K tile ---------------------------
  // A: 256 rows x 128 B = 2048 chunks of 16 B, 4 per thread.
  // B: 128 rows x 32 B packed, 8 B per thread (row tid/4, k-part tid%4).
  uint4 ra[4];
  uint2 rb;
  uint32_t rz;
  const int b_row = tid >> 2, b_part = tid & 3;

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + i * kThreads;
      const int r = id >> 3, c = id & 7;
      const int gm = m0 + r, gk = k0 + c * 8;
      ra[i] = make_uint4(0, 0, 0, 0);
      if (gm < M && gk < K) ra[i] = *(const uint4*)(x + (size_t)gm * K + gk);
    }
    const int gn = n0 + b_row, gk = k0 + b_part * 16;
    rb = make_uint2(0, 0);
    rz = 0;
    if (gn < N && gk < K) {
      rb = *(const uint2*)(qw + gn * row_bytes + gk / 2);
      const uint32_t z = SYM ? 8u : (uint32_t)f16_to_f32(zeros[(size_t)gn * ng + gk / G]);
      rz = z * 0x01010101u;
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + i * kThreads;
      const int r = id >> 3, c = id & 7;
      *(uint4*)&As[r * kLdsStride + c * 8] = ra[i];
    }
    uint4 e0 = expand8(rb.x, rz);
    uint4 e1 = expand8(rb.y, rz);
    uint16_t* dst = &Bs[b_row * kLdsStride + b_part * 16];
    *(uint4*)dst = e0;
    *(uint4*)(dst + 8) = e1;
  };

  f32x16_t acc[2][2], part[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) { acc[i][j][v] = 0.f; part[i][j][v] = 0.f; }

  const int ntiles = (K + kKT - 1) / kKT;
  load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * kKT;
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(k0 + kKT);

    // scales of the (at most two) groups this tile touches, per column block
    float s_lo[2], s_hi[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gn = n0 + wn * 64 + j * 32 + (lane & 31);
      const int g0 = k0 / G, g1 = (k0 + 32) / G;
      s_lo[j] = 0.f;
      s_hi[j] = 0.f;
      if (gn < N) {
        s_lo[j] = f16_to_f32(scales[(size_t)gn * ng + g0]);
        if (k0 + 32 < K) s_hi[j] = f16_to_f32(scales[(size_t)gn * ng + g1]);
      }
    }

#pragma unroll
    for (int ks = 0; ks < kKT / 16; ++ks) {
      const int kk = ks * 16 + 8 * (lane >> 5);
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4 v = *(const uint4*)&As[(wm * 64 + i * 32 + (lane & 31)) * kLdsStride + kk];
        a[i] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 v = *(const uint4*)&Bs[(wn * 64 + j * 32 + (lane & 31)) * kLdsStride + kk];
        b[j] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], part[i][j], 0, 0, 0);

      // end of a group (or of K): fold the group's partial into the output
      const int kend = k0 + (ks + 1) * 16;
      if ((kend % G) == 0 || kend >= K) {
        const bool upper = (ks >= 2);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float s = upper ? s_hi[j] : s_lo[j];
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              acc[i][j][v] = fmaf(s, part[i][j][v], acc[i][j][v]);
              part[i][j][v] = 0.f;
            }
        }
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*(v/4) + 4*(lane/32) + v%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gn = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int gm = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (gm < M && gn < N) y[(size_t)gm * N + gn] = f32_to_bf16_rne(acc[i][j][v]);
      }
    }
}

}  // namespace

hipError_t launch_w4a16_gemm(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                             const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                             int symmetric, uint16_t* y, hipStream_t s) {
  const int64_t ntm = (M + kBM - 1) / kBM, ntn = (N + kBN - 1) / kBN;
  const dim3 grid((unsigned)(ntm * ntn));
  if (symmetric)
    hipLaunchKernelGGL(w4a16_gemm_kernel<true>, grid, dim3(kThreads), 0, s, x, (int)M, (int)K,
                       qweight, scales, zeros, (int)N, G, y);
  else
    hipLaunchKernelGGL(w4a16_gemm_kernel<false>, grid, dim3(kThreads), 0, s, x, (int)M, (int)K,
                       qweight, scales, zeros, (int)N, G, y);
  return hipGetLastError();
}

}  // namespace gq
