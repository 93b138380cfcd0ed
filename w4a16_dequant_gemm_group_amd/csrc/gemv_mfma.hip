// Small-batch W4A16 GEMV (4 <= M <= 16) on the matrix cores: a streaming
// kernel without scratch (every activation row in LDS, K split over the waves
// of a workgroup; bf16 or fp16 activations) where x fits, and a tile kernel
// split along K with partial sums in scratch otherwise.
//
// Same product as the streaming GEMV ("vLLM 量化与推测解码" section 2, fused
// W4A16 paragraph; "量化" page, "工作原理" figure right panel):
//   y[m, n] = bf16( sum_g S[n,g] * sum_{k in g} x[m,k] * (q[n,k] - z[n,g]) ).
// With M activation rows the dot-product form costs M times the vector ALU work
// per weight, so here the weights become the B operand of
// v_mfma_f32_16x16x32_bf16 and the activations its A operand: the matrix core
// multiplies all M rows at the cost of one.
//
// Operand construction (per 16-row block of W and 128-wide step of K):
//  * lane (n, g) = (lane & 15, lane >> 4) loads 16 bytes of weight row n at
//    k = k0 + 32 g, i.e. the four 8-nibble dwords of one 32-wide chunk;
//  * a 4 x 4 transpose across the lane rows (v_permlane16/32_swap) gives lane
//    (n, g) dword g of every chunk c, so MFMA c covers exactly the 32-wide
//    chunk c, which lies in one quantization group for any group size that is
//    a multiple of 32;
//  * each dword becomes four bf16 pairs 128 + q (the nibble under exponent
//    byte 0x43, exact) in the order (0,2)(4,6)(1,3)(5,7); the activations are
//    staged in LDS permuted the same way;
//  * per group segment, the offset and zero point are removed with the chunk
//    sums of x and the scale applied in fp32:
//      acc[m][n] += S * (D[m][n] - (128 + z) * sum_{k in segment} x[m][k]).
// Tile kernel: a workgroup (4 waves, 64 rows) covers a 1024-wide slice of K
// and writes fp32 partial sums to the caller's workspace; a second kernel adds
// the slices in slice order (so the result does not depend on scheduling) and
// rounds once to bf16 (fp16 for fp16 activations), nearest-even.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "gq_internal.h"

namespace gq {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kKC = 1024;            // K covered by one workgroup
constexpr int kXRow = kKC / 8 + 1;   // 16-byte chunks per staged x row (+1 pad: no bank conflicts)
constexpr uint32_t kOob = 0x80000000u;

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

// x0..x7 (bf16) -> pairs (x0,x2) (x4,x6) (x1,x3) (x5,x7)
__device__ __forceinline__ uint4 perm_x(uint4 v) {
  return make_uint4(__builtin_amdgcn_perm(v.y, v.x, 0x05040100u),
                    __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                    __builtin_amdgcn_perm(v.y, v.x, 0x07060302u),
                    __builtin_amdgcn_perm(v.w, v.z, 0x07060302u));
}

// a + the two 16-bit values of v (bf16 pairs, or fp16 pairs if XF16)
template <bool XF16>
__device__ __forceinline__ float dot2x(uint32_t v, float a) {
  if constexpr (XF16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, v),
                                  __builtin_bit_cast(f16x2_t, 0x3C003C00u), a, false);
  return dot2(v, 0x3F803F80u, a);
}

// 8 nibbles -> bf16 128 + q in the same pair order
__device__ __forceinline__ uint4 unpack8(uint32_t e, uint32_t magic) {
  const uint32_t ev = e & 0x0F0F0F0Fu, od = (e >> 4) & 0x0F0F0F0Fu;
  return make_uint4(__builtin_amdgcn_perm(ev, magic, 0x01050104u),
                    __builtin_amdgcn_perm(ev, magic, 0x01070106u),
                    __builtin_amdgcn_perm(od, magic, 0x01050104u),
                    __builtin_amdgcn_perm(od, magic, 0x01070106u));
}

// out[c] at lane row g = in[g] at lane row c (rows of 16 lanes)
__device__ __forceinline__ void transpose4(uint32_t& d0, uint32_t& d1, uint32_t& d2, uint32_t& d3) {
  const auto a = __builtin_amdgcn_permlane32_swap(d0, d2, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(d1, d3, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  d0 = c[0];
  d1 = c[1];
  d2 = d[0];
  d3 = d[1];
}

// CPG: 32-wide chunks per correction segment (1: G = 32, 2: G = 64, 4: G a
// multiple of 128).  MR: activation rows staged (>= M; 4, 8 or 16).  Requires
// N * K / 2 and M * K * 2 below 2^31 (byte offsets of the buffer loads).
// G = 32 needs about 400 registers per lane without spilling: one wave per SIMD.
// XF16: fp16 activations (nibbles as fp16 1024 + q, fp16 MFMA).
template <int CPG, bool SYM, int MR, bool XF16>
__global__ __launch_bounds__(256, CPG == 1 ? 1 : 2) void gemv_mfma_tile_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int N, int G,
    float* __restrict__ part) {
  __shared__ uint4 xs[MR * kXRow];     // x[m][k0 .. k0 + 1024) as permuted 8-chunks
  __shared__ float sxs[kKC / 32][16];  // per 32-chunk and row m: sum of x (0 for m >= MR)
  // G = 32: per wave, scale | zero << 16 of its 16 rows x 32 groups (registers would spill)
  __shared__ uint32_t meta[CPG == 1 ? 4 : 1][16][32];
  constexpr int GPS = 4 / CPG;         // groups per 128-wide step
  constexpr int XJ = MR * 128 / 256;   // x chunks staged per thread
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.y;
  const int k0 = split * kKC;
  const int row = blockIdx.x * 64 + w * 16 + n;  // this lane's weight row
  const bool rin = row < N;
  const int NG = K / G;
  const uint32_t rb = (uint32_t)K / 2;
  const rsrc_t rx = make_rsrc(x, (uint32_t)M * K * 2);
  const rsrc_t rw = make_rsrc(qw, (uint32_t)N * rb);
  const rsrc_t rs = make_rsrc(scales, (uint32_t)N * NG * 2);
  const rsrc_t rz = make_rsrc(SYM ? (const void*)scales : (const void*)zeros, (uint32_t)N * NG * 2);

  // 1. activations (rows >= M and k >= K read zero)
  uint4 xv[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int id = threadIdx.x + 256 * j;
    const int m = id >> 7, c = id & 127;
    const int k = k0 + c * 8;
    const uint32_t off = (m < M && k < K) ? (uint32_t)(m * K + k) * 2u : kOob;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
    xv[j] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  // 2. scales and zeros of row `row` for the 8 steps (GPS consecutive groups
  //    each); for G = 32 one 16-byte load per lane covers the wave's 16 rows x 32
  //    groups (lane l: row l / 4, groups 8 (l % 4) ..) and goes through LDS
  uint32_t ms[8], mz[8];
  uint4 gs4 = make_uint4(0, 0, 0, 0), gz4 = make_uint4(0, 0, 0, 0);
  if (GPS == 4) {
    const int mrow = blockIdx.x * 64 + w * 16 + (lane >> 2);
    const int gq = k0 / 32 + 8 * (lane & 3);
    const uint32_t off = (mrow < N && gq < NG) ? ((uint32_t)mrow * NG + gq) * 2u : kOob;
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    gs4 = make_uint4(a[0], a[1], a[2], a[3]);
    if (!SYM) {
      const auto b = __builtin_amdgcn_raw_buffer_load_b128(rz, off, 0, 0);
      gz4 = make_uint4(b[0], b[1], b[2], b[3]);
    }
  } else {
#pragma unroll
    for (int L = 0; L < 8; ++L) {
      const int k = k0 + 128 * L;
      const uint32_t off = (rin && k < K) ? ((uint32_t)row * NG + k / G) * 2u : kOob;
      mz[L] = 0u;
      if (GPS == 1) {
        ms[L] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
        if (!SYM) mz[L] = __builtin_amdgcn_raw_buffer_load_b16(rz, off, 0, 0);
      } else {
        ms[L] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
        if (!SYM) mz[L] = __builtin_amdgcn_raw_buffer_load_b32(rz, off, 0, 0);
      }
    }
  }
  // 3. weights: lane (n, g) reads 16 bytes of row `row` at k = k0 + 128 L + 32 g
  uint4 wv[8];
  const uint32_t wrow = (uint32_t)row * rb + (uint32_t)(k0 + 32 * g) / 2;
#pragma unroll
  for (int L = 0; L < 8; ++L) {
    const bool ok = rin && k0 + 128 * L + 32 * g < K;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? wrow + 64 * L : kOob, 0, 2);
    wv[L] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  // 4. stage x and its 32-chunk sums (the 4 chunks of a 32-chunk sit in
  //    consecutive lanes: two quad-permute adds)
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int id = threadIdx.x + 256 * j;
    const int m = id >> 7, c = id & 127;
    const uint4 v = xv[j];
    xs[m * kXRow + c] = perm_x(v);
    float s = dot2x<XF16>(v.x, 0.f);  // against 1.0 pairs
    s = dot2x<XF16>(v.y, s);
    s = dot2x<XF16>(v.z, s);
    s = dot2x<XF16>(v.w, s);
    s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0xB1,
                                                               0xF, 0xF, true));
    s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x4E,
                                                               0xF, 0xF, true));
    if ((c & 3) == 0) sxs[c >> 2][m] = s;
  }
  if (MR < 16) {
    for (int i = threadIdx.x; i < (kKC / 32) * (16 - MR); i += 256)
      sxs[i / (16 - MR)][MR + i % (16 - MR)] = 0.f;
  }
  if (GPS == 4) {
    const uint32_t sv[4] = {gs4.x, gs4.y, gs4.z, gs4.w}, zv[4] = {gz4.x, gz4.y, gz4.z, gz4.w};
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[2 * j] = __builtin_amdgcn_perm(zv[j], sv[j], 0x05040100u);      // (s, z) of group 2j
      o[2 * j + 1] = __builtin_amdgcn_perm(zv[j], sv[j], 0x07060302u);  // (s, z) of group 2j + 1
    }
    uint32_t* dst = &meta[GPS == 4 ? w : 0][lane >> 2][8 * (lane & 3)];
    *(uint4*)dst = make_uint4(o[0], o[1], o[2], o[3]);
    *(uint4*)(dst + 4) = make_uint4(o[4], o[5], o[6], o[7]);
  }
  __syncthreads();

  // 5. MFMAs and per-segment corrections; lane (n, g) accumulates rows m = 4g + r
  const uint32_t magic = XF16 ? 0x64006400u : 0x43004300u;  // 1024 + q (fp16) / 128 + q (bf16)
  constexpr float kOff = XF16 ? 1024.f : 128.f;
  const int xrow = (n % MR) * kXRow;  // A row of this lane (rows >= M are dropped at the end)
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4_t D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int L = 0; L < 8; ++L) {
    uint32_t e0 = wv[L].x, e1 = wv[L].y, e2 = wv[L].z, e3 = wv[L].w;
    transpose4(e0, e1, e2, e3);
    const uint32_t ev[4] = {e0, e1, e2, e3};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 A = xs[xrow + 16 * L + 4 * c + g];
      const uint4 B = unpack8(ev[c], magic);
      const f32x4_t Cin = (c % CPG == 0) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : D;
      if constexpr (XF16)
        D = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, A),
                                                   __builtin_bit_cast(f16x8_t, B), Cin, 0, 0, 0);
      else
        D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A),
                                                    __builtin_bit_cast(bf16x8_t, B), Cin, 0, 0, 0);
      if (c % CPG == CPG - 1) {
        uint32_t sb, zb;
        if (GPS == 1) {
          sb = ms[L];
          zb = mz[L];
        } else if (GPS == 2) {
          sb = ms[L] >> (16 * (c / 2));
          zb = mz[L] >> (16 * (c / 2));
        } else {
          sb = meta[GPS == 4 ? w : 0][n][4 * L + c];
          zb = sb >> 16;
        }
        const float s = f16_to_f32((uint16_t)sb);
        const float zc = kOff + (SYM ? 8.f : f16_to_f32((uint16_t)zb));
        const int ch = 4 * L + c;  // last 32-chunk of the segment
        float4 sx = *(const float4*)&sxs[ch][4 * g];
#pragma unroll
        for (int q = 1; q < CPG; ++q) {
          const float4 t = *(const float4*)&sxs[ch - q][4 * g];
          sx.x += t.x;
          sx.y += t.y;
          sx.z += t.z;
          sx.w += t.w;
        }
        acc[0] = fmaf(s, fmaf(-zc, sx.x, D[0]), acc[0]);
        acc[1] = fmaf(s, fmaf(-zc, sx.y, D[1]), acc[1]);
        acc[2] = fmaf(s, fmaf(-zc, sx.z, D[2]), acc[2]);
        acc[3] = fmaf(s, fmaf(-zc, sx.w, D[3]), acc[3]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep each step's fragments short-lived
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * g + r;
    if (m < M && rin) part[((size_t)split * M + m) * N + row] = acc[r];
  }
}

// y = bf16 (XF16: fp16) of the sum of the K slices, in slice order
template <bool XF16>
__global__ __launch_bounds__(256) void gemv_split_finalize_kernel(const float* __restrict__ part,
                                                                  int splits, int64_t MN,
                                                                  uint16_t* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= MN) return;
  float s = 0.f;
  for (int j = 0; j < splits; ++j) s += part[(size_t)j * MN + i];
  y[i] = XF16 ? __builtin_bit_cast(uint16_t, (_Float16)s) : f32_to_bf16_rne(s);
}


// ---------------------------------------------------------------------------
// Streaming variant (no scratch): every activation row in LDS, K split over the
// waves of a workgroup, partial tiles added in LDS
// ---------------------------------------------------------------------------
//
// A workgroup of NW waves owns a 16-row block of W at a time (persistent over
// row blocks); wave w covers k in [w K/NW, (w+1) K/NW) in items of 512: lane
// (n, g) loads 16 bytes of row n at k = k0 + 128 L + 32 g (L = 0..3) and the
// scales (and zeros) of row n for the item, two items ahead of the one it
// multiplies.  The operands, MFMAs and per-segment corrections are those of the
// tile kernel above.  At the end of a row block each wave writes its 16 x 16
// partial tile to LDS and, after a barrier, 16 M threads add the NW tiles in
// wave order (deterministic) and store y rounded once to bf16 (fp16 when the
// activations are fp16).
//
// When x is too long for LDS, K runs in chunks of KC (a multiple of NW 512):
// the workgroup stages x[:, chunk] before each chunk's items (a barrier on
// either side) and the tiles keep accumulating until the row block ends; items
// at or past K (a partial last chunk) load zeros.
//
// GQ: group size 32 << GQ (GQ = 4: 512 or any multiple of 512).  MR: staged
// activation rows (8 or 16, >= M).  Requires K % 512 == 0, KC % (NW * 512) ==
// 0 and the LDS of mfma_stream_lds_bytes(MR, NW, KC, chunked).
constexpr int kMSItem = 512;  // k per item
constexpr size_t kMSTeamLds = 160 * 1024;  // LDS of one compute unit

// Chunk sums are stored for the MR staged rows plus a zeroed slot read by the
// lanes of rows >= MR; the chunked form keeps 16 rows per chunk (rows >= MR
// zero), which measured faster there.
size_t mfma_stream_lds_bytes(int MR, int NW, int64_t KC, bool chunked) {
  const size_t sums = chunked ? (size_t)(KC / 32) * 16 * 4 : (size_t)(KC / 32) * MR * 4 + 16;
  return (size_t)MR * (size_t)(KC / 8 + 1) * 16 + sums + (size_t)NW * 64 * 16;
}

template <int GQ, bool SYM>
struct MsBuf {
  static constexpr int kHalves = GQ >= 4 ? 1 : (16 >> GQ);  // scale halves per item and lane
  static constexpr int kWords = (kHalves + 1) / 2;
  uint4 w[4];
  uint32_t s[kWords], z[SYM ? 1 : kWords];
};

// LINES: load j brings rows 8 (j % 2) .. + 8 of the row block, 128 whole bytes
// (a cache line of each) per row: lane (n, g) the 16 bytes at 128 (j / 2) +
// 64 (n / 8) + 16 g of row 8 (j % 2) + n % 8, so step 2 (j / 2) + n / 8 of that
// row; ms_rows_to_steps then swaps the pieces between lanes n and n ^ 8.
// Otherwise load L brings step L of row n (64 bytes of each of 16 rows).
template <int GQ, bool SYM, bool LINES = false>
__device__ __forceinline__ void ms_load(MsBuf<GQ, SYM>& B, int rb, int k0, int n, int g, int N, int K,
                                        int G, rsrc_t rw, rsrc_t rs, rsrc_t rz) {
  const int row = rb * 16 + n;
  const bool rin = row < N && k0 < K;  // k0 >= K: an item past a partial last chunk
  const uint32_t rbytes = (uint32_t)K / 2;
  if constexpr (LINES) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rb * 16 + (n & 7) + 8 * (j & 1);
      const uint32_t o = r < N && k0 < K
                             ? (uint32_t)r * rbytes + (uint32_t)k0 / 2 +
                                   (uint32_t)(128 * (j >> 1) + 64 * (n >> 3) + 16 * g)
                             : kOob;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, o, 0, 2);
      B.w[j] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  } else {
    const uint32_t wo = rin ? (uint32_t)row * rbytes + (uint32_t)(k0 + 32 * g) / 2 : kOob;
#pragma unroll
    for (int L = 0; L < 4; ++L) {
      // the step in the lane offset (kOob + 192 is still out of range); a
      // lane-dependent scalar offset would need a waterfall loop per load
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, wo + 64u * L, 0, 2);
      B.w[L] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
  const uint32_t so = rin ? ((uint32_t)row * (uint32_t)(K / G) + (uint32_t)(k0 / G)) * 2u : kOob;
  auto ld = [&](rsrc_t r, uint32_t* d) {
    if constexpr (GQ == 0) {
      const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, so, 0, 0);
      const auto b = __builtin_amdgcn_raw_buffer_load_b128(r, so + 16u, 0, 0);
      d[0] = a[0]; d[1] = a[1]; d[2] = a[2]; d[3] = a[3];
      d[4] = b[0]; d[5] = b[1]; d[6] = b[2]; d[7] = b[3];
    } else if constexpr (GQ == 1) {
      const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, so, 0, 0);
      d[0] = a[0]; d[1] = a[1]; d[2] = a[2]; d[3] = a[3];
    } else if constexpr (GQ == 2) {
      const auto a = __builtin_amdgcn_raw_buffer_load_b64(r, so, 0, 0);
      d[0] = a[0]; d[1] = a[1];
    } else if constexpr (GQ == 3) {
      d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, so, 0, 0);
    } else {
      d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, so, 0, 0);
    }
  };
  ld(rs, B.s);
  if (!SYM) ld(rz, B.z);
}

// scale/zero half of 32-chunk j (0..15) of the item
template <int GQ>
__device__ __forceinline__ uint16_t ms_half(const uint32_t* v, int j) {
  const int h = GQ >= 4 ? 0 : (j >> GQ);
  return (uint16_t)(v[h >> 1] >> (16 * (h & 1)));
}

// XF16: fp16 activations and output (fp16 MFMA, nibbles as fp16 1024 + q).
// TM teams of NW waves share one workgroup and its staged x: each team works
// as a workgroup of its own on its row blocks (K split over its waves), and
// every team runs the same number of items (a team short of row blocks runs
// empty ones: zero weights, no stores) so that all meet at the same barriers.
// One team with 8 staged rows and 8 waves runs two workgroups per compute
// unit: the launch bounds then ask for four waves per SIMD (at most 128
// registers) — except with asymmetric group-32 weights, whose register stages
// (16 scale and 16 zero halves per item) would spill there: one workgroup.
template <int MR, int NW, int GQ, bool SYM, bool CHUNKED, bool XF16, int TM>
constexpr bool ms_two_per_cu() {
  return TM == 1 && MR == 8 && NW == 8 && !CHUNKED && !(GQ == 0 && !SYM);
}
template <int MR, int NW, int GQ, bool SYM, bool CHUNKED, bool XF16, int TM>
__global__ __launch_bounds__(NW * 64 * TM, (ms_two_per_cu<MR, NW, GQ, SYM, CHUNKED, XF16, TM>() ? 4 : 1)) void
gemv_mfma_stream_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int N, int G,
    uint16_t* __restrict__ y, int KC) {
  constexpr int CPG = GQ >= 2 ? 4 : (1 << GQ);  // 32-chunks per correction segment
  extern __shared__ uint4 lds4[];
  const int XR = KC / 8 + 1;                     // uint4 per staged x row (+1: no bank conflicts)
  uint4* xs = lds4;                              // [MR][XR] permuted pairs of the chunk
  constexpr int SXW = CHUNKED ? 16 : MR;         // chunk-sum rows stored per 32-chunk
  float* sxs = (float*)(xs + MR * XR);           // [KC / 32][SXW] chunk sums (+ 4 zeros)
  const int zslot = (KC / 32) * SXW;             // the zero slot (SXW == MR)
  constexpr int NT = NW * 64 * TM;              // threads per workgroup
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int team = TM == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / (NW * 64));
  float* red = sxs + zslot + (CHUNKED ? 0 : 4) + team * NW * 256;  // [TM][NW][64][4] partial tiles
  const int tl = (int)threadIdx.x - team * NW * 64;  // thread within the team
  const int w = __builtin_amdgcn_readfirstlane(tl >> 6);
  const int vb = (int)blockIdx.x * TM + team, vgrid = (int)gridDim.x * TM;  // the team's place
  const int NB = (N + 15) / 16;
  const int NCH = (K + KC - 1) / KC;             // K chunks
  const int kw = KC / NW;                        // k per wave and chunk
  const int IPC = kw / kMSItem;                  // items per wave and chunk
  const int IPW = NCH * IPC;                     // items per wave and row block
  const rsrc_t rw = make_rsrc(qw, (uint32_t)N * (uint32_t)(K / 2));
  const rsrc_t rs = make_rsrc(scales, (uint32_t)N * (uint32_t)(K / G) * 2);
  const rsrc_t rz = make_rsrc(SYM ? (const void*)scales : (const void*)zeros, (uint32_t)N * (uint32_t)(K / G) * 2);
  // row blocks of the workgroup's first team (the others have as many or one fewer)
  const int b0 = (int)blockIdx.x * TM;
  const int nrb = b0 < NB ? (NB - 1 - b0) / vgrid + 1 : 0;
  const int items = nrb * IPW;                   // the same for every wave of the workgroup

  // item i -> (row block, k0); row blocks >= NB read zeros and store nothing
  auto item_rb = [&](int i) { return vb + (i / IPW) * vgrid; };
  auto item_k0 = [&](int i) {
    const int j = i % IPW;
    return (j / IPC) * KC + w * kw + (j % IPC) * kMSItem;
  };

  // stage x[:, kb .. kb + KC) (rows >= M, k >= K and the chunk sums of rows
  // >= MR are zero) in batches of kUX 16-byte loads per thread, all in flight
  // before any is used; MR KC / 8 is a multiple of kUX NT, so every lane runs
  // every batch (the quad shuffles)
  constexpr int kUX = TM == 1 ? 8 : 4;
  const int CC = KC / 8;  // 16-byte chunks per row
  auto stage_load = [&](int kb, int f0, uint4 (&v)[kUX]) {
#pragma unroll
    for (int u = 0; u < kUX; ++u) {
      const int f = f0 + u * NT + (int)threadIdx.x;
      const int m = f / CC, c = f - m * CC;
      v[u] = make_uint4(0, 0, 0, 0);
      if (m < M && kb + c * 8 < K) v[u] = *(const uint4*)(x + (size_t)m * K + (size_t)(kb + c * 8));
    }
  };
  auto stage_store = [&](int f0, const uint4 (&v)[kUX]) {
#pragma unroll
    for (int u = 0; u < kUX; ++u) {
      const int f = f0 + u * NT + (int)threadIdx.x;
      const int m = f / CC, c = f - m * CC;
      xs[m * XR + c] = perm_x(v[u]);
      float sm = dot2x<XF16>(v[u].x, 0.f);  // against 1.0 pairs
      sm = dot2x<XF16>(v[u].y, sm);
      sm = dot2x<XF16>(v[u].z, sm);
      sm = dot2x<XF16>(v[u].w, sm);
      sm += __shfl_xor(sm, 1, 64);
      sm += __shfl_xor(sm, 2, 64);
      if ((c & 3) == 0) sxs[(c >> 2) * SXW + m] = sm;
    }
  };
  auto stage = [&](int kb, int from) {
    for (int f0 = from; f0 < MR * CC; f0 += kUX * NT) {
      uint4 v[kUX];
      stage_load(kb, f0, v);
      stage_store(f0, v);
    }
  };

  // the first x batch is issued before the weight prefetch, so staging it
  // does not wait for the weights (loads retire in order)
  uint4 xv0[kUX];
  stage_load(0, 0, xv0);
  // every prefetch is issued, also past the last item (row blocks >= NB read
  // zeros), so the compiler's waits before each item count exactly the items
  // in flight; a prefetch that may be skipped would make it wait for every
  // outstanding load
  MsBuf<GQ, SYM> buf[3];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    ms_load<GQ, SYM>(buf[j], item_rb(j), item_k0(j), n, g, N, K, G, rw, rs, rz);
  stage_store(0, xv0);
  stage(0, kUX * NT);
  if (SXW == MR) {
    if (threadIdx.x < 4) sxs[zslot + threadIdx.x] = 0.f;
  } else {
    for (int i = threadIdx.x; i < (KC / 32) * (16 - MR); i += NT)
      sxs[(i / (16 - MR)) * 16 + MR + i % (16 - MR)] = 0.f;
  }
  __syncthreads();

  const uint32_t magic = XF16 ? 0x64006400u : 0x43004300u;  // 1024 + q or 128 + q
  constexpr float kOff = XF16 ? 1024.f : 128.f;
  const int xrow = (n % MR) * XR;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const MsBuf<GQ, SYM>& B, int i) {
    const int k0 = item_k0(i);
    const int kb = (i % IPW) / IPC * KC;  // the item's chunk
    if (CHUNKED && i > 0 && i % IPC == 0) {  // a new chunk: every wave is done with the last one
      __syncthreads();
      stage(kb, 0);
      __syncthreads();
    }
    const int xc0 = (k0 - kb) / 8, ch0 = (k0 - kb) / 32;
#pragma unroll
    for (int L = 0; L < 4; ++L) {
      uint32_t e0 = B.w[L].x, e1 = B.w[L].y, e2 = B.w[L].z, e3 = B.w[L].w;
      transpose4(e0, e1, e2, e3);
      const uint32_t ev[4] = {e0, e1, e2, e3};
      // the step's MFMAs first (one accumulation chain per correction
      // segment), then the segments' corrections: with one segment per chunk
      // (G = 32) no correction waits for the MFMA just issued
      f32x4_t Dq[4 / CPG];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 A = xs[xrow + xc0 + 16 * L + 4 * c + g];
        const uint4 Bv = unpack8(ev[c], magic);
        const int sg = c / CPG;
        const f32x4_t Cin = (c % CPG == 0) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : Dq[sg];
        if constexpr (XF16)
          Dq[sg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, A),
                                                          __builtin_bit_cast(f16x8_t, Bv), Cin, 0, 0, 0);
        else
          Dq[sg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A),
                                                           __builtin_bit_cast(bf16x8_t, Bv), Cin, 0, 0, 0);
      }
#pragma unroll
      for (int sg = 0; sg < 4 / CPG; ++sg) {
        const f32x4_t D = Dq[sg];
        const int j = 4 * L + sg * CPG + CPG - 1;  // last 32-chunk of the segment
        const float sc = f16_to_f32(ms_half<GQ>(B.s, j));
        const float zc = kOff + (SYM ? 8.f : f16_to_f32(ms_half<GQ>(B.z, j)));
        // rows 4 g .. 4 g + 3; lanes whose rows are >= MR (no activations)
        // read a zeroed slot
        float4 sx = *(const float4*)&sxs[SXW == 16 || 4 * g < MR ? (ch0 + j) * SXW + 4 * g : zslot];
#pragma unroll
        for (int q = 1; q < CPG; ++q) {
          const float4 t =
              *(const float4*)&sxs[SXW == 16 || 4 * g < MR ? (ch0 + j - q) * SXW + 4 * g : zslot];
          sx.x += t.x;
          sx.y += t.y;
          sx.z += t.z;
          sx.w += t.w;
        }
        acc[0] = fmaf(sc, fmaf(-zc, sx.x, D[0]), acc[0]);
        acc[1] = fmaf(sc, fmaf(-zc, sx.y, D[1]), acc[1]);
        acc[2] = fmaf(sc, fmaf(-zc, sx.z, D[2]), acc[2]);
        acc[3] = fmaf(sc, fmaf(-zc, sx.w, D[3]), acc[3]);
      }
    }
    if (i % IPW == IPW - 1) {  // the row block is done: add the waves' tiles
      *(float4*)&red[(w * 64 + lane) * 4] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      acc[0] = acc[1] = acc[2] = acc[3] = 0.f;
      __syncthreads();
      const int t = tl;
      if (t < 16 * M) {
        const int m = t >> 4, nn = t & 15, rb = item_rb(i);
        const int src = (nn + 16 * (m >> 2)) * 4 + (m & 3);
        float v = 0.f;
        for (int u = 0; u < NW; ++u) v += red[u * 256 + src];
        const int row = rb * 16 + nn;
        if (row < N)
          y[(size_t)m * N + row] = XF16 ? __builtin_bit_cast(uint16_t, (_Float16)v) : f32_to_bf16_rne(v);
      }
      __syncthreads();
    }
  };

  // three register buffers: item i + 2 loads while item i is multiplied; whole
  // rounds in the loop, the last 0-2 items after it
  const int rounds = items / 3, rest = items % 3;
  int i = 0;
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      ms_load<GQ, SYM>(buf[(j + 2) % 3], item_rb(i + 2), item_k0(i + 2), n, g, N, K, G, rw, rs, rz);
      __builtin_amdgcn_sched_barrier(0);
      compute(buf[j], i);
      ++i;
    }
  }
  if (rest > 0) compute(buf[0], i++);
  if (rest > 1) compute(buf[1], i++);
}

constexpr int kXrGroup = 8;  // row blocks per group (the waves meet once per group)

// Lane n of a 16-lane row exchanges with lane n ^ 8 (row_ror:8).
__device__ __forceinline__ uint32_t ror8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
}
__device__ __forceinline__ uint4 ror8(const uint4& v) {
  return make_uint4(ror8(v.x), ror8(v.y), ror8(v.z), ror8(v.w));
}

// The pieces of a LINES load (ms_load) in step order: W[L] = step L of row n.
// Lanes n < 8 hold steps 0 and 2 of row n and steps 0 and 2 of row n + 8;
// lanes n >= 8 steps 1 and 3 of row n - 8 and of row n.
__device__ __forceinline__ void ms_rows_to_steps2(const uint4 (&w)[2], int n, uint4 (&W)[2]) {
  // the same for two steps: load j brings rows 8 j .. + 8, step n / 8
  const bool lo = n < 8;
  const uint4 a = ror8(lo ? w[1] : w[0]);
  W[0] = lo ? w[0] : a;
  W[1] = lo ? a : w[1];
}
__device__ __forceinline__ void ms_rows_to_steps(const uint4 (&w)[4], int n, uint4 (&W)[4]) {
  const bool lo = n < 8;
  const uint4 a = ror8(lo ? w[1] : w[0]);
  const uint4 b = ror8(lo ? w[3] : w[2]);
  W[0] = lo ? w[0] : a;
  W[1] = lo ? a : w[1];
  W[2] = lo ? w[2] : b;
  W[3] = lo ? b : w[3];
}

// The activation operands of a register-x wave, xa[L][c] = x[n][k0 + 128 L +
// 32 c + 8 g .. + 8) for lane (n, g) (rows >= M zero), loaded with whole-wave
// contiguous 16-byte loads (lane l takes x[r][k0 + 8 l .. + 8) of row r: 1 KiB
// per instruction, all rows issued at once) and moved into operand order
// through the wave's own 8 KiB of LDS, eight rows at a time (16-byte units
// XOR-swizzled by row, so the writes and the operand reads are free of bank
// conflicts).  The region is private to the wave: no barrier.  Loading the
// operands directly took 16 instructions per wave of sixteen 64-byte pieces
// each; loading the second eight rows only after the first eight had passed
// through the region cost a second memory round trip at M > 8.
__device__ __forceinline__ void xreg_load_x(rsrc_t rx, int M, int K, int k0, int lane, uint4* region,
                                            uint4 (&xa)[4][4]) {
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int L = 0; L < 4; ++L)
#pragma unroll
    for (int c = 0; c < 4; ++c) xa[L][c] = make_uint4(0, 0, 0, 0);
  uint4 v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r == 8 && M <= 8) break;
    const uint32_t off = r < M ? ((uint32_t)r * (uint32_t)K + (uint32_t)(k0 + 8 * lane)) * 2u : kOob;
    const auto t = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
    v[r] = make_uint4(t[0], t[1], t[2], t[3]);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (8 * h >= M) break;
    if (h == 1) {
      // every lane's reads of the first half are done before it is overwritten
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) region[r * 64 + (lane ^ r)] = v[8 * h + r];
    // other lanes' writes: ordered within the wavefront
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if ((n >> 3) == h) {
      const int rr = n & 7;
#pragma unroll
      for (int L = 0; L < 4; ++L)
#pragma unroll
        for (int c = 0; c < 4; ++c) xa[L][c] = region[rr * 64 + ((16 * L + 4 * c + g) ^ rr)];
    }
  }
}

// Small-batch GEMV with the activations in registers (5 <= M <= 16, K = 512 NW
// for NW = 1..8 waves): the product, operands and MFMAs of
// gemv_mfma_stream_kernel, but wave w always covers the same 512 columns
// [512 w, 512 w + 512) of every row block, so the A operands of its 16
// 32-wide chunks (16 bytes per lane and chunk, 64 registers) are loaded from x
// once, permuted into the pair order of the nibble unpack, and kept for the
// whole launch: no x in LDS, no LDS reads or address arithmetic per MFMA, no
// staging barrier.  The zero-point term goes to the matrix cores as in the
// super-block kernel:
//   acc[m][n] = sum_c S_c (D_c[m][n] - (128 + z_c) sx[m][c])
//             = sum_c S_c D_c[m][n]  +  sum_c sx[m][c] T[c][n],   T = -S (128 + z),
// the second sum over the four chunks of a 128-wide step being one
// v_mfma_f32_16x16x4f32 (fp32): lane (n, g) supplies the sum over chunk g of
// activation row n (kept in a register with the operands) and T of weight row
// n, chunk g.  Each row block is one item per wave (16 rows x 512 columns,
// 4 KiB), two items in flight; each wave leaves its 16 x 16 tile of a row
// block in an LDS slot, and only once per group of eight row blocks do the
// waves meet at a barrier, after which the workgroup adds each row block's
// tiles in wave order and stores y, rounded once (two sets of slots, so the
// next group's tiles cannot meet this group's reads).  A barrier per row
// block made every row block wait for the workgroup's slowest wave.
template <int NW, int GQ, bool SYM, bool XF16>
__global__ __launch_bounds__(NW * 64, 2) void gemv_mfma_xreg_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int N, int G,
    uint16_t* __restrict__ y) {
  constexpr int CPG = GQ >= 2 ? 4 : (1 << GQ);  // 32-chunks per correction segment
  // partial tiles [slot][wave][lane][4]: two sets of kXrGroup item slots
  __shared__ float red[2 * kXrGroup * NW * 256];
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int NB = (N + 15) / 16;
  const int k0 = w * kMSItem;  // K == NW * 512
  const rsrc_t rw = make_rsrc(qw, (uint32_t)N * (uint32_t)(K / 2));
  const rsrc_t rs = make_rsrc(scales, (uint32_t)N * (uint32_t)(K / G) * 2);
  const rsrc_t rz = make_rsrc(SYM ? (const void*)scales : (const void*)zeros, (uint32_t)N * (uint32_t)(K / G) * 2);
  const int items = (int)blockIdx.x < NB ? (NB - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  auto item_rb = [&](int i) { return (int)blockIdx.x + i * (int)gridDim.x; };

  // x first (loads retire in order: the weight prefetch behind them does not
  // hold up the operand set-up); rows >= M read zero.  (Staging x through LDS
  // with coalesced loads and a barrier measured slower: every wave then waits
  // for the slowest one's loads.)
  const rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  uint4 xa[4][4];  // [step L][chunk c]: x[n][k0 + 128 L + 32 c + 8 g .. + 8), permuted
  // the second set of tile slots is first written after the first group's
  // barrier, when every wave holds its operands
  xreg_load_x(rx, M, K, k0, lane, (uint4*)(red + kXrGroup * NW * 256) + w * 512, xa);
  MsBuf<GQ, SYM> buf[3];
  // chunk sums of row n: lane (n, g) holds 8 of each chunk's 32 values (a
  // partial sum p_c per chunk c); the 4 x 4 transpose across the lane rows
  // gives lane (n, g) the four partials of chunk g, whose sum it keeps
  float sxa[4];
  auto x_sums = [&]() {
#pragma unroll
  for (int L = 0; L < 4; ++L) {
    uint32_t p[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 v = xa[L][c];
      float s = dot2x<XF16>(v.x, 0.f);
      s = dot2x<XF16>(v.y, s);
      s = dot2x<XF16>(v.z, s);
      s = dot2x<XF16>(v.w, s);
      p[c] = __builtin_bit_cast(uint32_t, s);
      xa[L][c] = perm_x(v);
    }
    transpose4(p[0], p[1], p[2], p[3]);
    sxa[L] = (__builtin_bit_cast(float, p[0]) + __builtin_bit_cast(float, p[1])) +
             (__builtin_bit_cast(float, p[2]) + __builtin_bit_cast(float, p[3]));
  }
  };

  const uint32_t magic = XF16 ? 0x64006400u : 0x43004300u;  // 1024 + q or 128 + q
  constexpr float kOff = XF16 ? 1024.f : 128.f;
  // byte selector of the scale (and zero) half of chunk g of a step within
  // its two words (group 32: word 2L + g / 2; group 64: word L, half g / 2)
  const uint32_t hsel = GQ == 0 ? (uint32_t)(2 * g) | ((uint32_t)(2 * g + 1) << 8) | 0x0C0C0000u
                                : (uint32_t)(2 * (g >> 1)) | ((uint32_t)(2 * (g >> 1) + 1) << 8) | 0x0C0C0000u;
  auto lane_half = [&](const uint32_t* v, int L) -> uint16_t {
    if constexpr (GQ == 0) return (uint16_t)__builtin_amdgcn_perm(v[2 * L + 1], v[2 * L], hsel);
    else if constexpr (GQ == 1) return (uint16_t)__builtin_amdgcn_perm(v[L], v[L], hsel);
    else return ms_half<GQ>(v, 4 * L);
  };

  auto compute = [&](const MsBuf<GQ, SYM>& B, int i) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4_t accz = {0.f, 0.f, 0.f, 0.f};
    uint4 W[4];
    ms_rows_to_steps(B.w, n, W);
#pragma unroll
    for (int L = 0; L < 4; ++L) {
      uint32_t e0 = W[L].x, e1 = W[L].y, e2 = W[L].z, e3 = W[L].w;
      transpose4(e0, e1, e2, e3);
      const uint32_t ev[4] = {e0, e1, e2, e3};
      f32x4_t Dq[4 / CPG];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 Bv = unpack8(ev[c], magic);
        const int sg = c / CPG;
        const f32x4_t Cin = (c % CPG == 0) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : Dq[sg];
        if constexpr (XF16)
          Dq[sg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, xa[L][c]),
                                                          __builtin_bit_cast(f16x8_t, Bv), Cin, 0, 0, 0);
        else
          Dq[sg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[L][c]),
                                                           __builtin_bit_cast(bf16x8_t, Bv), Cin, 0, 0, 0);
      }
      // x-sum term of the step: T of chunk g of weight row n
      const float sg_ = f16_to_f32(lane_half(B.s, L));
      const float zg = kOff + (SYM ? 8.f : f16_to_f32(lane_half(B.z, L)));
      accz = __builtin_amdgcn_mfma_f32_16x16x4f32(sxa[L], -sg_ * zg, accz, 0, 0, 0);
#pragma unroll
      for (int sg = 0; sg < 4 / CPG; ++sg) {
        const float sc = f16_to_f32(ms_half<GQ>(B.s, 4 * L + sg * CPG));
        acc[0] = fmaf(sc, Dq[sg][0], acc[0]);
        acc[1] = fmaf(sc, Dq[sg][1], acc[1]);
        acc[2] = fmaf(sc, Dq[sg][2], acc[2]);
        acc[3] = fmaf(sc, Dq[sg][3], acc[3]);
      }
    }
    // the wave's tile of this row block waits in its slot until the group's
    // barrier
    const int grp = i / kXrGroup;
    *(float4*)&red[((grp & 1) * kXrGroup + i % kXrGroup) * NW * 256 + (w * 64 + lane) * 4] =
        make_float4(acc[0] + accz[0], acc[1] + accz[1], acc[2] + accz[2], acc[3] + accz[3]);
    if (i % kXrGroup != kXrGroup - 1 && i != items - 1) return;
    // a group of row blocks is done (the waves meet once per group, not per
    // row block): add the waves' tiles of each in wave order and store y; the
    // next group writes the other set of slots
    __syncthreads();
    const int i0g = grp * kXrGroup, nrb = i - i0g + 1;
    for (int t = threadIdx.x; t < nrb * 16 * M; t += NW * 64) {
      const int j = t / (16 * M), r = t - j * (16 * M);
      const int m = r >> 4, nn = r & 15;
      const float* rd = red + ((grp & 1) * kXrGroup + j) * NW * 256;
      const int src = (nn + 16 * (m >> 2)) * 4 + (m & 3);
      float v = 0.f;
#pragma unroll
      for (int u = 0; u < NW; ++u) v += rd[u * 256 + src];
      const int row = item_rb(i0g + j) * 16 + nn;
      if (row < N)
        y[(size_t)m * N + row] = XF16 ? __builtin_bit_cast(uint16_t, (_Float16)v) : f32_to_bf16_rne(v);
    }
  };

  // With two or more row blocks every prefetch is issued, also past the last
  // row block (those read zeros), so the compiler's waits before each item
  // count exactly the items in flight; a prefetch that may be skipped would
  // make it wait for every outstanding load.  With one row block the second
  // prefetch is skipped (an extra load that only costs).
  auto run = [&](auto all_tag) {
    constexpr bool kAll = decltype(all_tag)::value;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (kAll || j < items) ms_load<GQ, SYM, true>(buf[j], item_rb(j), k0, n, g, N, K, G, rw, rs, rz);
    x_sums();
    const int rounds = items / 3, rest = items % 3;
    int i = 0;
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (kAll || i + 2 < items)
          ms_load<GQ, SYM, true>(buf[(j + 2) % 3], item_rb(i + 2), k0, n, g, N, K, G, rw, rs, rz);
        __builtin_amdgcn_sched_barrier(0);
        compute(buf[j], i);
        ++i;
      }
    }
    if (rest > 0) compute(buf[0], i++);
    if (rest > 1) compute(buf[1], i++);
  };
  if (items >= 2) run(std::true_type{});
  else run(std::false_type{});
}

// Small-batch GEMV for long K (5 <= M <= 16, K a multiple of 256 beyond the
// register-resident kernel's range): the operands, MFMAs and fp32 zero-point
// MFMA of gemv_mfma_xreg_kernel, but x is too long to stay in registers, so
// each 256-wide item brings its own activation rows, loaded with the item's
// weights two items ahead as whole-wave contiguous pieces (two rows of 512
// bytes per load; 8 or 16 rows, MR, a compile-time count) and moved into
// operand order through the wave's own LDS region when the item is
// multiplied (rows >= M read zero).  Every compute unit reads all of x once per
// row block from L2 (no staging shared by the waves, no scratch).  Wave w
// takes items w, w + NW, ... of each row block (items at or past K load
// zeros); the tiles meet in LDS once per group of four row blocks (the LDS
// also holds the waves' x regions).
template <int GQ, bool SYM, int MR>
struct XsBuf {
  static constexpr int kHalves = GQ >= 3 ? 1 : (8 >> GQ);  // scale halves per item and lane
  static constexpr int kWords = (kHalves + 1) / 2;
  uint4 w[2];       // sub-chunk g of each 128-wide step
  uint4 x[MR / 2];  // the item's activation rows, two per load (xs_load_x)
  uint32_t s[kWords], z[SYM ? 1 : kWords];
};

constexpr int kXsItem = 256;  // k per item
constexpr int kXsGroup = 4;   // row blocks per group of the streamed-x kernels (LDS: tiles + x)

// The activation rows of a 256-wide item, loaded whole-wave contiguous: v[j]
// of lane l is x[2 j + l / 32][k0 + 8 (l % 32) .. + 8) (rows >= M and items at
// or past K read zero): MR / 2 loads of two 512-byte row pieces each.
template <int MR>
__device__ __forceinline__ void xs_load_x(rsrc_t rx, int M, int K, int k0, bool kin, int lane,
                                          uint4 (&v)[MR / 2]) {
#pragma unroll
  for (int j = 0; j < MR / 2; ++j) {
    const int row = 2 * j + (lane >> 5);
    const uint32_t off = row < M && kin ? ((uint32_t)row * (uint32_t)K + (uint32_t)(k0 + 8 * (lane & 31))) * 2u : kOob;
    const auto t = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
    v[j] = make_uint4(t[0], t[1], t[2], t[3]);
  }
}

// Those rows in operand order through the wave's own LDS region (16-byte
// units XOR-swizzled by row: no bank conflicts): A[4 L + c] of lane (n, g) is
// x[n][k0 + 128 L + 32 c + 8 g .. + 8) in natural order, zero for n >= MR.
template <int MR>
__device__ __forceinline__ void xs_operands(const uint4 (&v)[MR / 2], int lane, uint4* region,
                                            uint4 (&A)[8]) {
#pragma unroll
  for (int j = 0; j < MR / 2; ++j) {
    const int row = 2 * j + (lane >> 5), u = lane & 31;
    region[row * 32 + (u ^ (row & 7))] = v[j];
  }
  // other lanes' writes: ordered within the wavefront
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < 8; ++q) A[q] = make_uint4(0, 0, 0, 0);
  if (MR == 16 || n < MR) {
#pragma unroll
    for (int q = 0; q < 8; ++q) A[q] = region[n * 32 + ((4 * q + g) ^ (n & 7))];
  }
  // the next item's writes to the region must follow these reads (same wave)
  __builtin_amdgcn_wave_barrier();
}

template <int GQ, bool SYM, int MR>
__device__ __forceinline__ void xs_load(XsBuf<GQ, SYM, MR>& B, int rb, int k0, int n, int g, int M, int N,
                                        int K, int G, rsrc_t rx, rsrc_t rw, rsrc_t rs, rsrc_t rz) {
  const int row = rb * 16 + n;
  const bool kin = k0 < K && rb * 16 < N;  // else an item past K or past the last row block: zeros
  const bool rin = row < N && kin;
  // load j: the item's 128 bytes of rows 8 j .. + 8 (whole lines; lane (n, g)
  // the 16 bytes at 64 (n / 8) + 16 g, step n / 8), reordered by
  // ms_rows_to_steps2
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = rb * 16 + (n & 7) + 8 * j;
    const uint32_t o = r < N && kin ? (uint32_t)r * (uint32_t)(K / 2) + (uint32_t)k0 / 2 +
                                          (uint32_t)(64 * (n >> 3) + 16 * g)
                                    : kOob;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, o, 0, 2);
    B.w[j] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  xs_load_x<MR>(rx, M, K, k0, kin, (int)(threadIdx.x & 63), B.x);
  const uint32_t so = rin ? ((uint32_t)row * (uint32_t)(K / G) + (uint32_t)(k0 / G)) * 2u : kOob;
  auto ld = [&](rsrc_t r, uint32_t* d) {
    if constexpr (GQ == 0) {
      const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, so, 0, 0);
      d[0] = a[0]; d[1] = a[1]; d[2] = a[2]; d[3] = a[3];
    } else if constexpr (GQ == 1) {
      const auto a = __builtin_amdgcn_raw_buffer_load_b64(r, so, 0, 0);
      d[0] = a[0]; d[1] = a[1];
    } else if constexpr (GQ == 2) {
      d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, so, 0, 0);
    } else {
      d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, so, 0, 0);
    }
  };
  ld(rs, B.s);
  if (!SYM) ld(rz, B.z);
}

template <int NW, int GQ, bool SYM, bool XF16, int MR>
__global__ __launch_bounds__(NW * 64, 2) void gemv_mfma_xs_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int N, int G,
    uint16_t* __restrict__ y) {
  constexpr int CPG = GQ >= 2 ? 4 : (1 << GQ);  // 32-chunks per correction segment
  __shared__ float red[2 * kXsGroup * NW * 256];  // [slot][wave][lane][4] partial tiles
  __shared__ uint4 xlds[NW][MR * 32];            // each wave's item rows in operand order
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int NB = (N + 15) / 16;
  const int NI = K / kXsItem;                 // items per row block
  const int IPW = (NI + NW - 1) / NW;         // of them per wave (the last ones may lie past K)
  const rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const rsrc_t rw = make_rsrc(qw, (uint32_t)N * (uint32_t)(K / 2));
  const rsrc_t rs = make_rsrc(scales, (uint32_t)N * (uint32_t)(K / G) * 2);
  const rsrc_t rz = make_rsrc(SYM ? (const void*)scales : (const void*)zeros, (uint32_t)N * (uint32_t)(K / G) * 2);
  const int nrb = (int)blockIdx.x < NB ? (NB - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int items = nrb * IPW;
  auto item_rb = [&](int i) { return (int)blockIdx.x + (i / IPW) * (int)gridDim.x; };
  auto item_k0 = [&](int i) { return ((i % IPW) * NW + w) * kXsItem; };

  // At 8 rows every prefetch is issued, also past the last item (those read
  // zeros), so the compiler's waits before each item count exactly the two
  // items in flight (a prefetch that may be skipped makes it wait for every
  // outstanding load); at 16 rows that measured slower and the loads past the
  // end are skipped.
  XsBuf<GQ, SYM, MR> buf[3];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (MR == 8 || j < items)
      xs_load<GQ, SYM, MR>(buf[j], item_rb(j), item_k0(j), n, g, M, N, K, G, rx, rw, rs, rz);

  const uint32_t magic = XF16 ? 0x64006400u : 0x43004300u;  // 1024 + q or 128 + q
  constexpr float kOff = XF16 ? 1024.f : 128.f;
  const uint32_t hsel = GQ == 0 ? (uint32_t)(2 * g) | ((uint32_t)(2 * g + 1) << 8) | 0x0C0C0000u
                                : (uint32_t)(2 * (g >> 1)) | ((uint32_t)(2 * (g >> 1) + 1) << 8) | 0x0C0C0000u;
  // scale (zero) half of chunk g of step L of the item, and of the segment
  // starting at chunk 4 L + c0
  auto lane_half = [&](const uint32_t* v, int L) -> uint16_t {
    if constexpr (GQ == 0) return (uint16_t)__builtin_amdgcn_perm(v[2 * L + 1], v[2 * L], hsel);
    else if constexpr (GQ == 1) return (uint16_t)__builtin_amdgcn_perm(v[L], v[L], hsel);
    else if constexpr (GQ == 2) return (uint16_t)(v[0] >> (16 * L));
    else return (uint16_t)v[0];
  };
  auto seg_half = [&](const uint32_t* v, int L, int c0) -> uint16_t {
    if constexpr (GQ <= 2) {
      const int h = (4 * L + c0) >> GQ;
      return (uint16_t)(v[h >> 1] >> (16 * (h & 1)));
    } else {
      return (uint16_t)v[0];
    }
  };

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4_t accz = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const XsBuf<GQ, SYM, MR>& B, int i) {
    uint4 X[8], W[2];
    xs_operands<MR>(B.x, lane, xlds[w], X);
    ms_rows_to_steps2(B.w, n, W);
#pragma unroll
    for (int L = 0; L < 2; ++L) {
      // the step's activation operands and chunk sums (row n, chunk g)
      uint4 A[4];
      uint32_t p[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 v = X[4 * L + c];
        float s = dot2x<XF16>(v.x, 0.f);
        s = dot2x<XF16>(v.y, s);
        s = dot2x<XF16>(v.z, s);
        s = dot2x<XF16>(v.w, s);
        p[c] = __builtin_bit_cast(uint32_t, s);
        A[c] = perm_x(v);
      }
      transpose4(p[0], p[1], p[2], p[3]);
      const float sx = (__builtin_bit_cast(float, p[0]) + __builtin_bit_cast(float, p[1])) +
                       (__builtin_bit_cast(float, p[2]) + __builtin_bit_cast(float, p[3]));
      uint32_t e0 = W[L].x, e1 = W[L].y, e2 = W[L].z, e3 = W[L].w;
      transpose4(e0, e1, e2, e3);
      const uint32_t ev[4] = {e0, e1, e2, e3};
      f32x4_t Dq[4 / CPG];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 Bv = unpack8(ev[c], magic);
        const int sg = c / CPG;
        const f32x4_t Cin = (c % CPG == 0) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : Dq[sg];
        if constexpr (XF16)
          Dq[sg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, A[c]),
                                                          __builtin_bit_cast(f16x8_t, Bv), Cin, 0, 0, 0);
        else
          Dq[sg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A[c]),
                                                           __builtin_bit_cast(bf16x8_t, Bv), Cin, 0, 0, 0);
      }
      const float sg_ = f16_to_f32(lane_half(B.s, L));
      const float zg = kOff + (SYM ? 8.f : f16_to_f32(lane_half(B.z, L)));
      accz = __builtin_amdgcn_mfma_f32_16x16x4f32(sx, -sg_ * zg, accz, 0, 0, 0);
#pragma unroll
      for (int sg = 0; sg < 4 / CPG; ++sg) {
        const float sc = f16_to_f32(seg_half(B.s, L, sg * CPG));
        acc[0] = fmaf(sc, Dq[sg][0], acc[0]);
        acc[1] = fmaf(sc, Dq[sg][1], acc[1]);
        acc[2] = fmaf(sc, Dq[sg][2], acc[2]);
        acc[3] = fmaf(sc, Dq[sg][3], acc[3]);
      }
    }
    if (i % IPW != IPW - 1) return;
    // the wave's part of the row block is done: its tile waits in the row
    // block's slot until the group's barrier
    const int r = i / IPW;  // the workgroup's row block index
    const int grp = r / kXsGroup;
    *(float4*)&red[((grp & 1) * kXsGroup + r % kXsGroup) * NW * 256 + (w * 64 + lane) * 4] =
        make_float4(acc[0] + accz[0], acc[1] + accz[1], acc[2] + accz[2], acc[3] + accz[3]);
    acc[0] = acc[1] = acc[2] = acc[3] = 0.f;
    accz = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (r % kXsGroup != kXsGroup - 1 && r != nrb - 1) return;
    __syncthreads();
    const int r0 = grp * kXsGroup, nr = r - r0 + 1;
    for (int t = threadIdx.x; t < nr * 16 * M; t += NW * 64) {
      const int j = t / (16 * M), q = t - j * (16 * M);
      const int m = q >> 4, nn = q & 15;
      const float* rd = red + ((grp & 1) * kXsGroup + j) * NW * 256;
      const int src = (nn + 16 * (m >> 2)) * 4 + (m & 3);
      float v = 0.f;
#pragma unroll
      for (int u = 0; u < NW; ++u) v += rd[u * 256 + src];
      const int row = ((int)blockIdx.x + (r0 + j) * (int)gridDim.x) * 16 + nn;
      if (row < N)
        y[(size_t)m * N + row] = XF16 ? __builtin_bit_cast(uint16_t, (_Float16)v) : f32_to_bf16_rne(v);
    }
  };

  const int rounds = items / 3, rest = items % 3;
  int i = 0;
  for (int rr = 0; rr < rounds; ++rr) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (MR == 8 || i + 2 < items)
        xs_load<GQ, SYM, MR>(buf[(j + 2) % 3], item_rb(i + 2), item_k0(i + 2), n, g, M, N, K, G, rx, rw, rs, rz);
      __builtin_amdgcn_sched_barrier(0);
      compute(buf[j], i);
      ++i;
    }
  }
  if (rest > 0) compute(buf[0], i++);
  if (rest > 1) compute(buf[1], i++);
}

// Super-block (Q4_K-style) GEMV on the matrix cores, 5 <= M <= 16 ("量化" page,
// "工作原理" figure, middle panel): the structure of gemv_mfma_stream_kernel
// with the 144-byte blocks as the weight operand.  A 32-wide chunk of K is one
// sub-block, so MFMA c of a 128-wide step covers sub-block c: lane (n, g)
// loads the 16 nibble bytes of sub-block g of each step of its row (the same
// nibble order as the packed INT4 rows) and both block headers of its row per
// 512-wide item; after the 4 x 4 transpose MFMA c takes the scale and min of
// sub-block c:
//   acc[m][n] += S D[m][n] - (128 S + Mn) sum_{k in sub-block} x[m][k],
//   S = d sc_j, Mn = dmin mn_j  (products of an fp16 and a 6-bit field: exact),
// D being sum x (128 + q) from the bf16 magic-number unpack.  The second term
// is itself a product over the sub-blocks of a step, [16 rows of x sums] x
// [4 sub-blocks x 16 weight rows], so it runs on one fp32 MFMA
// (v_mfma_f32_16x16x4f32, fp32 products and sums) per step into an
// accumulator of its own: lane (n, g) supplies the x sum of row n and the
// -(128 S + Mn) of weight row n, both for sub-block g, and decodes the min of
// that one sub-block only (per-lane byte selectors as in the M = 1 kernel).
struct QkBuf {
  uint4 w[4];  // sub-block g of each 128-wide step
  uint4 h[2];  // the headers of the item's two blocks
};

// 6-bit field at bit P of the 96-bit {h.w : h.z : h.y} (compile-time P)
template <int P>
__device__ __forceinline__ uint32_t q4k_field(const uint4& h) {
  constexpr int wd = P / 32, sh = P % 32;
  const uint32_t lo = wd == 0 ? h.y : wd == 1 ? h.z : h.w;
  if constexpr (sh <= 26) {
    return (lo >> sh) & 63u;
  } else {
    const uint32_t hi = wd == 0 ? h.z : h.w;
    return __builtin_amdgcn_alignbit(hi, lo, sh) & 63u;
  }
}

template <int MR, bool CHUNKED>
__global__ __launch_bounds__(512, 1) void q4k_mfma_stream_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ blocks, int N,
    uint16_t* __restrict__ y, int KC) {
  constexpr int NW = 8, NT = NW * 64;
  extern __shared__ uint4 lds4[];
  const int XR = KC / 8 + 1;                     // uint4 per staged x row (+1: no bank conflicts)
  uint4* xs = lds4;                              // [MR][XR] permuted pairs of the chunk
  constexpr int SXW = CHUNKED ? 16 : MR;         // chunk-sum rows stored per 32-chunk
  float* sxs = (float*)(xs + MR * XR);           // [KC / 32][SXW] chunk sums (+ 4 zeros)
  const int zslot = (KC / 32) * SXW;             // the zero slot (SXW == MR)
  float* red = sxs + zslot + (CHUNKED ? 0 : 4);  // [NW][64][4] partial tiles
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NB = (N + 15) / 16;
  const int NCH = (K + KC - 1) / KC;             // K chunks
  const int kw = KC / NW;                        // k per wave and chunk
  const int IPC = kw / kMSItem;                  // items per wave and chunk
  const int IPW = NCH * IPC;                     // items per wave and row block
  const uint32_t row_bytes = (uint32_t)(K / 256) * 144u;
  const rsrc_t rb = make_rsrc(blocks, (uint32_t)N * row_bytes);
  const int nrb = (int)blockIdx.x < NB ? (NB - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int items = nrb * IPW;                   // the same for every wave of the workgroup

  auto item_rb = [&](int i) { return (int)blockIdx.x + (i / IPW) * (int)gridDim.x; };
  auto item_k0 = [&](int i) {
    const int j = i % IPW;
    return (j / IPC) * KC + w * kw + (j % IPC) * kMSItem;
  };
  auto load = [&](QkBuf& B, int rbk, int k0) {
    const int row = rbk * 16 + n;
    const bool rin = row < N && k0 < K;  // k0 >= K: an item past a partial last chunk
    const uint32_t base = rin ? (uint32_t)row * row_bytes + (uint32_t)(k0 / 256) * 144u : kOob;
#pragma unroll
    for (int L = 0; L < 4; ++L) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(
          rb, base + (uint32_t)((L >> 1) * 144 + 16 + 16 * ((L & 1) * 4 + g)), 0, 2);
      B.w[L] = make_uint4(v[0], v[1], v[2], v[3]);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rb, base + 144u * b, 0, 0);
      B.h[b] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };

  // x staging as in gemv_mfma_stream_kernel (MR KC / 8 is a multiple of 8 NT)
  constexpr int kUX = 8;
  const int CC = KC / 8;  // 16-byte chunks per row
  auto stage_load = [&](int kb, int f0, uint4 (&v)[kUX]) {
#pragma unroll
    for (int u = 0; u < kUX; ++u) {
      const int f = f0 + u * NT + (int)threadIdx.x;
      const int m = f / CC, c = f - m * CC;
      v[u] = make_uint4(0, 0, 0, 0);
      if (m < M && kb + c * 8 < K) v[u] = *(const uint4*)(x + (size_t)m * K + (size_t)(kb + c * 8));
    }
  };
  auto stage_store = [&](int f0, const uint4 (&v)[kUX]) {
#pragma unroll
    for (int u = 0; u < kUX; ++u) {
      const int f = f0 + u * NT + (int)threadIdx.x;
      const int m = f / CC, c = f - m * CC;
      xs[m * XR + c] = perm_x(v[u]);
      float sm = dot2x<false>(v[u].x, 0.f);  // against 1.0 pairs
      sm = dot2x<false>(v[u].y, sm);
      sm = dot2x<false>(v[u].z, sm);
      sm = dot2x<false>(v[u].w, sm);
      sm += __shfl_xor(sm, 1, 64);
      sm += __shfl_xor(sm, 2, 64);
      if ((c & 3) == 0) sxs[(c >> 2) * SXW + m] = sm;
    }
  };
  auto stage = [&](int kb, int from) {
    for (int f0 = from; f0 < MR * CC; f0 += kUX * NT) {
      uint4 v[kUX];
      stage_load(kb, f0, v);
      stage_store(f0, v);
    }
  };

  uint4 xv0[kUX];
  stage_load(0, 0, xv0);
  QkBuf buf[3];  // every prefetch issued (exact waits), as in gemv_mfma_stream_kernel
#pragma unroll
  for (int j = 0; j < 2; ++j)
    load(buf[j], item_rb(j), item_k0(j));
  stage_store(0, xv0);
  stage(0, kUX * NT);
  if (SXW == MR) {
    if (threadIdx.x < 4) sxs[zslot + threadIdx.x] = 0.f;
  } else {
    for (int i = threadIdx.x; i < (KC / 32) * (16 - MR); i += NT)
      sxs[(i / (16 - MR)) * 16 + MR + i % (16 - MR)] = 0.f;
  }
  __syncthreads();

  const int xrow = (n % MR) * XR;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4_t accz = {0.f, 0.f, 0.f, 0.f};  // the x-sum terms, from the fp32 MFMAs
  // byte selectors and bit offset of the 6-bit scale and min of sub-block g
  // (even steps) and 4 + g (odd steps) of a block, as in q4k_stream_kernel
  uint32_t sel_sc[2], sel_mn[2], fbit[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t o6 = 6u * (uint32_t)(4 * e + g);
    const uint32_t sb = o6 >> 3, mb = 2u + (o6 >> 3);
    fbit[e] = o6 & 7u;
    sel_sc[e] = sb | ((sb + 1u) << 8) | 0x0C0C0000u;
    sel_mn[e] = mb | ((mb < 7u ? mb + 1u : 12u) << 8) | 0x0C0C0000u;
  }

  auto compute = [&](const QkBuf& B, int i) {
    const int k0 = item_k0(i);
    const int kb = (i % IPW) / IPC * KC;  // the item's chunk
    if (CHUNKED && i > 0 && i % IPC == 0) {  // a new chunk: every wave is done with the last one
      __syncthreads();
      stage(kb, 0);
      __syncthreads();
    }
    const int xc0 = (k0 - kb) / 8, ch0 = (k0 - kb) / 32;
    auto step = [&](auto Lc) {
      constexpr int L = decltype(Lc)::value;
      uint32_t e0 = B.w[L].x, e1 = B.w[L].y, e2 = B.w[L].z, e3 = B.w[L].w;
      transpose4(e0, e1, e2, e3);
      const uint32_t ev[4] = {e0, e1, e2, e3};
      f32x4_t D[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 A = xs[xrow + xc0 + 16 * L + 4 * c + g];
        D[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A),
                                                       __builtin_bit_cast(bf16x8_t, unpack8(ev[c], 0x43004300u)),
                                                       f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      }
      const uint4 h = B.h[L >> 1];
      const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(h.x & 0xFFFFu));
      const _Float16 dmin = __builtin_bit_cast(_Float16, (uint16_t)(h.x >> 16));
      auto corr = [&](auto Cc) {
        constexpr int c = decltype(Cc)::value;
        constexpr int j = (L & 1) * 4 + c;  // the sub-block of the block
        const float S = __builtin_fmaf((float)d, (float)q4k_field<6 * j>(h), 0.f);
        acc[0] = fmaf(S, D[c][0], acc[0]);
        acc[1] = fmaf(S, D[c][1], acc[1]);
        acc[2] = fmaf(S, D[c][2], acc[2]);
        acc[3] = fmaf(S, D[c][3], acc[3]);
      };
      corr(std::integral_constant<int, 0>{});
      corr(std::integral_constant<int, 1>{});
      corr(std::integral_constant<int, 2>{});
      corr(std::integral_constant<int, 3>{});
      // sub-block g of the step: -(128 S + Mn) of weight row n against the x
      // sum of activation row n (0 for rows >= MR)
      constexpr int e = L & 1;
      const uint32_t sc6 = __builtin_amdgcn_ubfe(__builtin_amdgcn_perm(h.z, h.y, sel_sc[e]), fbit[e], 6);
      const uint32_t mn6 = __builtin_amdgcn_ubfe(__builtin_amdgcn_perm(h.w, h.z, sel_mn[e]), fbit[e], 6);
      const float Sg = __builtin_fmaf((float)d, (float)sc6, 0.f);
      const float Mg = __builtin_fmaf((float)dmin, (float)mn6, 0.f);
      const float Tg = -__builtin_fmaf(128.f, Sg, Mg);
      const float sxg = SXW == 16 || n < MR ? sxs[(ch0 + 4 * L + g) * SXW + n] : 0.f;
      accz = __builtin_amdgcn_mfma_f32_16x16x4f32(sxg, Tg, accz, 0, 0, 0);
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    if (i % IPW == IPW - 1) {  // the row block is done: add the waves' tiles
      *(float4*)&red[(w * 64 + lane) * 4] =
          make_float4(acc[0] + accz[0], acc[1] + accz[1], acc[2] + accz[2], acc[3] + accz[3]);
      acc[0] = acc[1] = acc[2] = acc[3] = 0.f;
      accz = f32x4_t{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      const int t = threadIdx.x;
      if (t < 16 * M) {
        const int m = t >> 4, nn = t & 15, rbk = item_rb(i);
        const int src = (nn + 16 * (m >> 2)) * 4 + (m & 3);
        float v = 0.f;
        for (int u = 0; u < NW; ++u) v += red[u * 256 + src];
        const int row = rbk * 16 + nn;
        if (row < N) y[(size_t)m * N + row] = f32_to_bf16_rne(v);
      }
      __syncthreads();
    }
  };

  // three register buffers: item i + 2 loads while item i is multiplied; whole
  // rounds in the loop, the last 0-2 items after it
  const int rounds = items / 3, rest = items % 3;
  int i = 0;
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      load(buf[(j + 2) % 3], item_rb(i + 2), item_k0(i + 2));
      __builtin_amdgcn_sched_barrier(0);
      compute(buf[j], i);
      ++i;
    }
  }
  if (rest > 0) compute(buf[0], i++);
  if (rest > 1) compute(buf[1], i++);
}

// Super-block GEMV on the matrix cores with x in registers (K = 512 NW,
// q4k_mfma_xreg_kernel) or streamed with each 256-wide item (longer K,
// q4k_mfma_xs_kernel), 5 <= M <= 16: the structures of gemv_mfma_xreg_kernel
// and gemv_mfma_xs_kernel with the operands and per-step scale and min terms
// of q4k_mfma_stream_kernel (one bf16 MFMA per sub-block and 16 rows, the
// x-sum term -(128 S + Mn) on one fp32 MFMA per step).

// per-lane byte selectors and bit offset of the 6-bit scale and min of
// sub-block 4 e + g of a block (e = 0, 1)
struct QkSel {
  uint32_t sc[2], mn[2], fbit[2];
};
__device__ __forceinline__ QkSel qk_sel(int g) {
  QkSel q;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t o6 = 6u * (uint32_t)(4 * e + g);
    const uint32_t sb = o6 >> 3, mb = 2u + (o6 >> 3);
    q.fbit[e] = o6 & 7u;
    q.sc[e] = sb | ((sb + 1u) << 8) | 0x0C0C0000u;
    q.mn[e] = mb | ((mb < 7u ? mb + 1u : 12u) << 8) | 0x0C0C0000u;
  }
  return q;
}

// One 128-wide step covering sub-blocks 4 E .. 4 E + 3 of the block with
// header h: lane (n, g) holds sub-block g's 16 nibble bytes of row n (before
// the transpose), A[c] the activation operands of chunk c and sx the sum of
// row n over chunk g.
template <int E>
__device__ __forceinline__ void qk_step(const uint4& wv, const uint4 (&A)[4], float sx, const uint4& h,
                                        const QkSel& q, float (&acc)[4], f32x4_t& accz) {
  uint32_t e0 = wv.x, e1 = wv.y, e2 = wv.z, e3 = wv.w;
  transpose4(e0, e1, e2, e3);
  const uint32_t ev[4] = {e0, e1, e2, e3};
  f32x4_t D[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    D[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A[c]),
                                                   __builtin_bit_cast(bf16x8_t, unpack8(ev[c], 0x43004300u)),
                                                   f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(h.x & 0xFFFFu));
  const _Float16 dmin = __builtin_bit_cast(_Float16, (uint16_t)(h.x >> 16));
  auto corr = [&](auto Cc) {
    constexpr int c = decltype(Cc)::value;
    const float S = __builtin_fmaf((float)d, (float)q4k_field<6 * (4 * E + c)>(h), 0.f);
    acc[0] = fmaf(S, D[c][0], acc[0]);
    acc[1] = fmaf(S, D[c][1], acc[1]);
    acc[2] = fmaf(S, D[c][2], acc[2]);
    acc[3] = fmaf(S, D[c][3], acc[3]);
  };
  corr(std::integral_constant<int, 0>{});
  corr(std::integral_constant<int, 1>{});
  corr(std::integral_constant<int, 2>{});
  corr(std::integral_constant<int, 3>{});
  const uint32_t sc6 = __builtin_amdgcn_ubfe(__builtin_amdgcn_perm(h.z, h.y, q.sc[E]), q.fbit[E], 6);
  const uint32_t mn6 = __builtin_amdgcn_ubfe(__builtin_amdgcn_perm(h.w, h.z, q.mn[E]), q.fbit[E], 6);
  const float Sg = __builtin_fmaf((float)d, (float)sc6, 0.f);
  const float Mg = __builtin_fmaf((float)dmin, (float)mn6, 0.f);
  accz = __builtin_amdgcn_mfma_f32_16x16x4f32(sx, -__builtin_fmaf(128.f, Sg, Mg), accz, 0, 0, 0);
}

// x operands of four chunks (natural order in v) -> permuted operands and the
// sum of row n over chunk g (4 x 4 lane-row transpose of the partial sums)
__device__ __forceinline__ float qk_operands(const uint4* v, uint4 (&A)[4]) {
  uint32_t p[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float s = dot2x<false>(v[c].x, 0.f);
    s = dot2x<false>(v[c].y, s);
    s = dot2x<false>(v[c].z, s);
    s = dot2x<false>(v[c].w, s);
    p[c] = __builtin_bit_cast(uint32_t, s);
    A[c] = perm_x(v[c]);
  }
  transpose4(p[0], p[1], p[2], p[3]);
  return (__builtin_bit_cast(float, p[0]) + __builtin_bit_cast(float, p[1])) +
         (__builtin_bit_cast(float, p[2]) + __builtin_bit_cast(float, p[3]));
}

// the workgroup's row block r is done for this wave: its tile waits in the
// row block's slot; at the end of a group of kXrGroup row blocks (or of the
// workgroup's last) the waves meet and add each row block's tiles in wave
// order
template <int NW, int GRP>
__device__ __forceinline__ void qk_tile_done(float* red, int r, int nrb, int w, int lane, int M, int N,
                                             float (&acc)[4], f32x4_t& accz, uint16_t* __restrict__ y) {
  const int grp = r / GRP;
  *(float4*)&red[((grp & 1) * GRP + r % GRP) * NW * 256 + (w * 64 + lane) * 4] =
      make_float4(acc[0] + accz[0], acc[1] + accz[1], acc[2] + accz[2], acc[3] + accz[3]);
  acc[0] = acc[1] = acc[2] = acc[3] = 0.f;
  accz = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (r % GRP != GRP - 1 && r != nrb - 1) return;
  __syncthreads();
  const int r0 = grp * GRP, nr = r - r0 + 1;
  for (int t = threadIdx.x; t < nr * 16 * M; t += NW * 64) {
    const int j = t / (16 * M), q = t - j * (16 * M);
    const int m = q >> 4, nn = q & 15;
    const float* rd = red + ((grp & 1) * GRP + j) * NW * 256;
    const int src = (nn + 16 * (m >> 2)) * 4 + (m & 3);
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < NW; ++u) v += rd[u * 256 + src];
    const int row = ((int)blockIdx.x + (r0 + j) * (int)gridDim.x) * 16 + nn;
    if (row < N) y[(size_t)m * N + row] = f32_to_bf16_rne(v);
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 2) void q4k_mfma_xreg_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ blocks, int N,
    uint16_t* __restrict__ y) {
  __shared__ float red[2 * kXrGroup * NW * 256];
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int NB = (N + 15) / 16;
  const int k0 = w * kMSItem;  // K == NW * 512
  const uint32_t row_bytes = (uint32_t)(K / 256) * 144u;
  const rsrc_t rb = make_rsrc(blocks, (uint32_t)N * row_bytes);
  const rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const int items = (int)blockIdx.x < NB ? (NB - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  auto item_rb = [&](int i) { return (int)blockIdx.x + i * (int)gridDim.x; };
  // nibbles as in ms_load's LINES form: load j brings the 128 nibble bytes of
  // block j / 2 of rows 8 (j % 2) .. + 8 (two cache lines per row at most,
  // against up to two per 64 bytes with a row's 4 lanes per load), the
  // headers of row n as they are
  auto load = [&](QkBuf& B, int rbk) {
    const int row = rbk * 16 + n;
    const uint32_t base = row < N ? (uint32_t)row * row_bytes + (uint32_t)(k0 / 256) * 144u : kOob;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rbk * 16 + (n & 7) + 8 * (j & 1);
      const uint32_t bj = r < N ? (uint32_t)r * row_bytes + (uint32_t)(k0 / 256) * 144u : kOob;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(
          rb, bj + (uint32_t)((j >> 1) * 144 + 16 + 64 * (n >> 3) + 16 * g), 0, 2);
      B.w[j] = make_uint4(v[0], v[1], v[2], v[3]);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rb, base + 144u * b, 0, 0);
      B.h[b] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  // x first (loads retire in order), then the weight prefetch; the second
  // set of tile slots holds no tile before the first group's barrier
  uint4 xa[4][4];  // [step L][chunk c]: x[n][k0 + 128 L + 32 c + 8 g .. + 8)
  xreg_load_x(rx, M, K, k0, lane, (uint4*)(red + kXrGroup * NW * 256) + w * 512, xa);
  QkBuf buf[3];
  float sxa[4];
  auto x_sums = [&]() {
#pragma unroll
    for (int L = 0; L < 4; ++L) {
      const uint4 v[4] = {xa[L][0], xa[L][1], xa[L][2], xa[L][3]};
      sxa[L] = qk_operands(v, xa[L]);
    }
  };
  const QkSel q = qk_sel(g);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4_t accz = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const QkBuf& B, int i) {
    uint4 W[4];
    ms_rows_to_steps(B.w, n, W);
    qk_step<0>(W[0], xa[0], sxa[0], B.h[0], q, acc, accz);
    qk_step<1>(W[1], xa[1], sxa[1], B.h[0], q, acc, accz);
    qk_step<0>(W[2], xa[2], sxa[2], B.h[1], q, acc, accz);
    qk_step<1>(W[3], xa[3], sxa[3], B.h[1], q, acc, accz);
    qk_tile_done<NW, kXrGroup>(red, i, items, w, lane, M, N, acc, accz, y);
  };
  // every prefetch issued with two or more row blocks (exact waits), the
  // second skipped with one, as in gemv_mfma_xreg_kernel
  auto run = [&](auto all_tag) {
    constexpr bool kAll = decltype(all_tag)::value;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (kAll || j < items) load(buf[j], item_rb(j));
    x_sums();
    const int rounds = items / 3, rest = items % 3;
    int i = 0;
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (kAll || i + 2 < items) load(buf[(j + 2) % 3], item_rb(i + 2));
        __builtin_amdgcn_sched_barrier(0);
        compute(buf[j], i);
        ++i;
      }
    }
    if (rest > 0) compute(buf[0], i++);
    if (rest > 1) compute(buf[1], i++);
  };
  if (items >= 2) run(std::true_type{});
  else run(std::false_type{});
}

// one 256-wide item of q4k_mfma_xs_kernel: sub-block g of both steps, the
// block header, the activation operands of both steps
template <int MR>
struct QxBuf {
  uint4 w[2], h, x[MR / 2];
};

template <int NW, int MR>
__global__ __launch_bounds__(NW * 64, 2) void q4k_mfma_xs_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ blocks, int N,
    uint16_t* __restrict__ y) {
  __shared__ float red[2 * kXsGroup * NW * 256];
  __shared__ uint4 xlds[NW][MR * 32];  // each wave's item rows in operand order
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int NB = (N + 15) / 16;
  const int NI = K / 256;               // blocks (items) per row
  const int IPW = (NI + NW - 1) / NW;   // of them per wave (the last ones may lie past K)
  const uint32_t row_bytes = (uint32_t)(K / 256) * 144u;
  const rsrc_t rb = make_rsrc(blocks, (uint32_t)N * row_bytes);
  const rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const int nrb = (int)blockIdx.x < NB ? (NB - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int items = nrb * IPW;
  auto item_rb = [&](int i) { return (int)blockIdx.x + (i / IPW) * (int)gridDim.x; };
  auto item_blk = [&](int i) { return (i % IPW) * NW + w; };
  auto load = [&](QxBuf<MR>& B, int i) {
    const int row = item_rb(i) * 16 + n, blk = item_blk(i);
    const bool kin = blk < NI && item_rb(i) * 16 < N;  // else past K or past the last row block: zeros
    const uint32_t base = row < N && kin ? (uint32_t)row * row_bytes + (uint32_t)blk * 144u : kOob;
    // load j: the block's 128 nibble bytes of rows 8 j .. + 8 (ms_rows_to_steps2)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = item_rb(i) * 16 + (n & 7) + 8 * j;
      const uint32_t bj = r < N && kin ? (uint32_t)r * row_bytes + (uint32_t)blk * 144u : kOob;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(
          rb, bj + (uint32_t)(16 + 64 * (n >> 3) + 16 * g), 0, 2);
      B.w[j] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    const auto hv = __builtin_amdgcn_raw_buffer_load_b128(rb, base, 0, 0);
    B.h = make_uint4(hv[0], hv[1], hv[2], hv[3]);
    xs_load_x<MR>(rx, M, K, blk * 256, kin, lane, B.x);
  };
  QxBuf<MR> buf[3];
  // prefetches as in gemv_mfma_xs_kernel: all issued at 8 rows (exact waits)
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (MR == 8 || j < items) load(buf[j], j);
  const QkSel q = qk_sel(g);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4_t accz = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const QxBuf<MR>& B, int i) {
    uint4 X[8], A[4], W[2];
    xs_operands<MR>(B.x, lane, xlds[w], X);
    ms_rows_to_steps2(B.w, n, W);
    float sx = qk_operands(&X[0], A);
    qk_step<0>(W[0], A, sx, B.h, q, acc, accz);
    sx = qk_operands(&X[4], A);
    qk_step<1>(W[1], A, sx, B.h, q, acc, accz);
    if (i % IPW == IPW - 1) qk_tile_done<NW, kXsGroup>(red, i / IPW, nrb, w, lane, M, N, acc, accz, y);
  };
  const int rounds = items / 3, rest = items % 3;
  int i = 0;
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (MR == 8 || i + 2 < items) load(buf[(j + 2) % 3], i + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(buf[j], i);
      ++i;
    }
  }
  if (rest > 0) compute(buf[0], i++);
  if (rest > 1) compute(buf[1], i++);
}

// Two teams per workgroup with 16 staged rows when x is staged whole, both
// teams' partial tiles fit beside it, and there are row blocks for two teams
// on every compute unit: the 16 waves of a compute unit then share one x stage
// (one 8-wave workgroup per compute unit otherwise, as x takes most of LDS).
// gate_up at M = 16: 26.7-26.8 -> 25.3-25.5 us.  With 8 staged rows, two
// 8-wave workgroups per compute unit stay faster (gate_up at M = 8: 23.0 -> 25.2
// us with one of 16 waves).  Not for asymmetric group-32 weights, which would
// spill at the four waves per SIMD a 1024-thread workgroup implies.
template <int MR, int NW, bool SYM, bool XF16>
hipError_t launch_ms(const uint16_t* x, int M, int K, int KC, const uint8_t* qw, const uint16_t* sc,
                     const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  const size_t lds = mfma_stream_lds_bytes(MR, NW, KC, KC < K);
  const size_t lds2 = lds + (size_t)NW * 64 * 16;
  const int nb = (N + 15) / 16;
  const bool teams = MR == 16 && KC >= K && lds2 <= kMSTeamLds && nb >= 2 * num_cus() &&
                     !(!SYM && G == 32);
  const int per_cu = lds <= 80 * 1024 && !(!SYM && G == 32) ? 2 : 1;
  const int grid = teams ? std::max(1, std::min((nb + 1) / 2, num_cus()))
                         : std::max(1, std::min(nb, per_cu * num_cus()));
#define GQ_MS_LAUNCH(GQ_)                                                                         \
  if (KC < K)                                                                                     \
    hipLaunchKernelGGL((gemv_mfma_stream_kernel<MR, NW, GQ_, SYM, true, XF16, 1>), dim3(grid),    \
                       dim3(NW * 64), lds, s, x, M, K, qw, sc, zr, N, G, y, KC);                  \
  else if (MR == 16 && teams)                                                                     \
    hipLaunchKernelGGL((gemv_mfma_stream_kernel<MR, NW, GQ_, SYM, false, XF16, MR == 16 && (SYM || GQ_ != 0) ? 2 : 1>),\
                       dim3(grid), dim3(NW * 128), lds2, s, x, M, K, qw, sc, zr, N, G, y, KC);    \
  else                                                                                            \
    hipLaunchKernelGGL((gemv_mfma_stream_kernel<MR, NW, GQ_, SYM, false, XF16, 1>), dim3(grid),   \
                       dim3(NW * 64), lds, s, x, M, K, qw, sc, zr, N, G, y, KC)
  switch (G) {
    case 32: GQ_MS_LAUNCH(0); break;
    case 64: GQ_MS_LAUNCH(1); break;
    case 128: GQ_MS_LAUNCH(2); break;
    case 256: GQ_MS_LAUNCH(3); break;
    default: GQ_MS_LAUNCH(4); break;
  }
#undef GQ_MS_LAUNCH
  return hipGetLastError();
}

// One workgroup of K / 512 waves per row-block stream; as many workgroups per
// compute unit as make 8 waves (two per SIMD, the launch bounds' register cap).
template <int NW, bool SYM, bool XF16>
hipError_t launch_xreg(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                       const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  const int nb = (N + 15) / 16;
  const int grid = std::max(1, std::min(nb, num_cus() * (8 / NW)));
#define GQ_XR_LAUNCH(GQ_)                                                                       \
  hipLaunchKernelGGL((gemv_mfma_xreg_kernel<NW, GQ_, SYM, XF16>), dim3(grid), dim3(NW * 64), 0, s, \
                     x, M, K, qw, sc, zr, N, G, y)
  switch (G) {
    case 32: GQ_XR_LAUNCH(0); break;
    case 64: GQ_XR_LAUNCH(1); break;
    case 128: GQ_XR_LAUNCH(2); break;
    case 256: GQ_XR_LAUNCH(3); break;
    default: GQ_XR_LAUNCH(4); break;
  }
#undef GQ_XR_LAUNCH
  return hipGetLastError();
}

template <bool SYM, bool XF16>
hipError_t xreg_nw(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                   const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  switch (K / kMSItem) {
    case 1: return launch_xreg<1, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
    case 2: return launch_xreg<2, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
    case 4: return launch_xreg<4, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
    case 8: return launch_xreg<8, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
    default: return hipErrorInvalidValue;
  }
}

// One workgroup of 8 waves per compute unit (its tile slots and x rows take
// 64 + 32 or 64 KiB of LDS); 8 activation rows per item when M <= 8.
template <bool SYM, bool XF16>
hipError_t launch_xs(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                     const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  const int nb = (N + 15) / 16;
  const int grid = std::max(1, std::min(nb, num_cus()));
#define GQ_XS_LAUNCH(GQ_)                                                                            \
  if (M <= 8)                                                                                          \
    hipLaunchKernelGGL((gemv_mfma_xs_kernel<8, GQ_, SYM, XF16, 8>), dim3(grid), dim3(512), 0, s, x, M, K, \
                       qw, sc, zr, N, G, y);                                                           \
  else                                                                                                 \
    hipLaunchKernelGGL((gemv_mfma_xs_kernel<8, GQ_, SYM, XF16, 16>), dim3(grid), dim3(512), 0, s, x, M, K, \
                       qw, sc, zr, N, G, y)
  switch (G) {
    case 32: GQ_XS_LAUNCH(0); break;
    case 64: GQ_XS_LAUNCH(1); break;
    case 128: GQ_XS_LAUNCH(2); break;
    case 256: GQ_XS_LAUNCH(3); break;
    default: GQ_XS_LAUNCH(4); break;
  }
#undef GQ_XS_LAUNCH
  return hipGetLastError();
}

template <int CPG, bool SYM, bool XF16>
hipError_t launch_cpg(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                      const uint16_t* zr, int N, int G, float* part, int splits, hipStream_t s) {
  const dim3 grid((unsigned)((N + 63) / 64), (unsigned)splits);
  if (M <= 4)
    hipLaunchKernelGGL((gemv_mfma_tile_kernel<CPG, SYM, 4, XF16>), grid, dim3(256), 0, s, x, M, K, qw,
                       sc, zr, N, G, part);
  else if (M <= 8)
    hipLaunchKernelGGL((gemv_mfma_tile_kernel<CPG, SYM, 8, XF16>), grid, dim3(256), 0, s, x, M, K, qw,
                       sc, zr, N, G, part);
  else
    hipLaunchKernelGGL((gemv_mfma_tile_kernel<CPG, SYM, 16, XF16>), grid, dim3(256), 0, s, x, M, K, qw,
                       sc, zr, N, G, part);
  return hipGetLastError();
}

template <bool SYM, bool XF16>
hipError_t launch_all(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                      const uint16_t* zr, int N, int G, float* part, int splits, hipStream_t s) {
  if (G == 32) return launch_cpg<1, SYM, XF16>(x, M, K, qw, sc, zr, N, G, part, splits, s);
  if (G == 64) return launch_cpg<2, SYM, XF16>(x, M, K, qw, sc, zr, N, G, part, splits, s);
  return launch_cpg<4, SYM, XF16>(x, M, K, qw, sc, zr, N, G, part, splits, s);
}

}  // namespace

// The streaming matrix-core GEMV: 8 or 16 staged rows and 8 waves per
// workgroup (two workgroups per compute unit when x fits 80 KiB of LDS: 8 rows
// of 4096 columns; the launch bounds then hold each wave to 128 registers),
// or with 8 staged rows and K = 2048 4 waves (one 512-wide item each).  K
// runs in chunks of KC (the largest multiple of 4096 whose x fits LDS: 8192
// columns of 8 rows, 4096 of 16); chunks only with 8 staged rows: with 16 the
// split-K kernel is faster on [4096, 14336] (24 against 30 us at M = 16).
// Measured at M = 8 against 4-wave workgroups: qkv 10.75 -> 10.3 us, gate_up
// 24.8 -> 23.9 us.  False if K or G do not fit.
static bool mfma_stream_config(int M, int64_t K, int64_t N, int* MR, int* NW, int* KC) {
  (void)N;
  if (K % kMSItem != 0 || K > ((int64_t)1 << 24)) return false;
  *MR = M <= 8 ? 8 : 16;
  if (*MR == 8 && K % 4096 != 0 && K % 2048 == 0 &&
      mfma_stream_lds_bytes(8, 4, K, false) <= 80 * 1024) {
    *NW = 4;
    *KC = (int)K;
    return true;
  }
  *NW = 8;
  const int kcmax = *MR == 8 ? 8192 : 4096;
  *KC = (int)std::min<int64_t>(kcmax, (K + 4095) / 4096 * 4096);
  if (*MR == 16 && *KC < K) return false;
  return mfma_stream_lds_bytes(*MR, 8, *KC, *KC < K) <= 156 * 1024;
}

bool gemv_mfma_stream_supported(int M, int64_t K, int64_t N, int G) {
  if (M < 4 || M > 16) return false;
  if (G % 32 != 0 || (G < 512 && 512 % G != 0) || (G >= 512 && G % 512 != 0)) return false;
  int MR, NW, KC;
  if (!mfma_stream_config(M, K, N, &MR, &NW, &KC)) return false;
  if (N * (K / 2) >= ((int64_t)1 << 31) || (int64_t)M * K * 2 >= ((int64_t)1 << 31)) return false;
  return true;
}

hipError_t launch_w4a16_gemv_mfma_stream(const uint16_t* x, int M, int64_t K, const uint8_t* qweight,
                                         const uint16_t* scales, const uint16_t* zeros, int64_t N,
                                         int G, int symmetric, uint16_t* y, hipStream_t s, bool xf16) {
  int MR, NW, KC;
  if (!mfma_stream_config(M, K, N, &MR, &NW, &KC)) return hipErrorInvalidValue;
  const int k = (int)K, n = (int)N;
#define GQ_MS_ROWS(MR_, NW_)                                                                       \
  (xf16 ? (symmetric ? launch_ms<MR_, NW_, true, true>(x, M, k, KC, qweight, scales, zeros, n, G, y, s)   \
                     : launch_ms<MR_, NW_, false, true>(x, M, k, KC, qweight, scales, zeros, n, G, y, s)) \
        : (symmetric ? launch_ms<MR_, NW_, true, false>(x, M, k, KC, qweight, scales, zeros, n, G, y, s)  \
                     : launch_ms<MR_, NW_, false, false>(x, M, k, KC, qweight, scales, zeros, n, G, y, s)))
  if (MR == 8 && NW == 4) return GQ_MS_ROWS(8, 4);
  if (MR == 8) return GQ_MS_ROWS(8, 8);
  return GQ_MS_ROWS(16, 8);
#undef GQ_MS_ROWS
}

// The register-resident small-batch GEMV: K of 512, 1024, 2048 or 4096 (one
// 512-wide column range per wave), 4 <= M <= 16, group sizes as for the
// streaming matrix-core kernel.
bool gemv_xreg_supported(int M, int64_t K, int64_t N, int G) {
  if (M < 4 || M > 16) return false;
  if (K != 512 && K != 1024 && K != 2048 && K != 4096) return false;
  if (G % 32 != 0 || (G < 512 && 512 % G != 0) || (G >= 512 && G % 512 != 0)) return false;
  if (N * (K / 2) >= ((int64_t)1 << 31) || (int64_t)M * K * 2 >= ((int64_t)1 << 31)) return false;
  return true;
}

hipError_t launch_w4a16_gemv_xreg(const uint16_t* x, int M, int64_t K, const uint8_t* qweight,
                                  const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                                  int symmetric, uint16_t* y, hipStream_t s, bool xf16) {
  if (!gemv_xreg_supported(M, K, N, G)) return hipErrorInvalidValue;
  const int k = (int)K, n = (int)N;
  if (xf16)
    return symmetric ? xreg_nw<true, true>(x, M, k, qweight, scales, zeros, n, G, y, s)
                     : xreg_nw<false, true>(x, M, k, qweight, scales, zeros, n, G, y, s);
  return symmetric ? xreg_nw<true, false>(x, M, k, qweight, scales, zeros, n, G, y, s)
                   : xreg_nw<false, false>(x, M, k, qweight, scales, zeros, n, G, y, s);
}

// The long-K small-batch GEMV with x streamed from L2 (5 <= M <= 16, K a
// multiple of 256 beyond 4096, groups that divide 256 or are multiples of it).
bool gemv_xs_supported(int M, int64_t K, int64_t N, int G) {
  if (M < 5 || M > 16) return false;
  if (K <= 4096 || K % kXsItem != 0 || K > ((int64_t)1 << 24)) return false;
  if (G % 32 != 0 || (G <= kXsItem && kXsItem % G != 0) || (G > kXsItem && G % kXsItem != 0)) return false;
  if (N * (K / 2) >= ((int64_t)1 << 31) || (int64_t)M * K * 2 >= ((int64_t)1 << 31)) return false;
  return true;
}

hipError_t launch_w4a16_gemv_xs(const uint16_t* x, int M, int64_t K, const uint8_t* qweight,
                                const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                                int symmetric, uint16_t* y, hipStream_t s, bool xf16) {
  if (!gemv_xs_supported(M, K, N, G)) return hipErrorInvalidValue;
  const int k = (int)K, n = (int)N;
  if (xf16)
    return symmetric ? launch_xs<true, true>(x, M, k, qweight, scales, zeros, n, G, y, s)
                     : launch_xs<false, true>(x, M, k, qweight, scales, zeros, n, G, y, s);
  return symmetric ? launch_xs<true, false>(x, M, k, qweight, scales, zeros, n, G, y, s)
                   : launch_xs<false, false>(x, M, k, qweight, scales, zeros, n, G, y, s);
}

bool gemv_mfma_supported(int M, int64_t K, int64_t N, int G) {
  if (M < 4 || M > 16) return false;
  if (G != 32 && G != 64 && G % 128 != 0) return false;
  if (K % 256 != 0) return false;  // keeps the 4-, 8- and 16-byte scale loads aligned
  if (N * (K / 2) >= ((int64_t)1 << 31) || (int64_t)M * K * 2 >= ((int64_t)1 << 31)) return false;
  if (N > ((int64_t)1 << 30) / 64) return false;
  return true;
}

size_t gemv_workspace_bytes(int M, int64_t K, int64_t N, int G) {
  if (gemv_stream_supported(M, K) || gemv_xreg_supported(M, K, N, G) || gemv_xs_supported(M, K, N, G) ||
      gemv_mfma_stream_supported(M, K, N, G) || !gemv_mfma_supported(M, K, N, G))
    return 0;
  return (size_t)((K + kKC - 1) / kKC) * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_w4a16_gemv_mfma(const uint16_t* x, int M, int64_t K, const uint8_t* qweight,
                                  const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                                  int symmetric, uint16_t* y, void* workspace, bool xf16,
                                  hipStream_t s) {
  const int splits = (int)((K + kKC - 1) / kKC);
  const int k = (int)K, n = (int)N;
  float* part = (float*)workspace;
  hipError_t e;
  if (xf16)
    e = symmetric ? launch_all<true, true>(x, M, k, qweight, scales, zeros, n, G, part, splits, s)
                  : launch_all<false, true>(x, M, k, qweight, scales, zeros, n, G, part, splits, s);
  else
    e = symmetric ? launch_all<true, false>(x, M, k, qweight, scales, zeros, n, G, part, splits, s)
                  : launch_all<false, false>(x, M, k, qweight, scales, zeros, n, G, part, splits, s);
  if (e != hipSuccess) return e;
  const int64_t mn = (int64_t)M * N;
  if (xf16)
    hipLaunchKernelGGL(gemv_split_finalize_kernel<true>, dim3((unsigned)((mn + 255) / 256)), dim3(256),
                       0, s, (const float*)part, splits, mn, y);
  else
    hipLaunchKernelGGL(gemv_split_finalize_kernel<false>, dim3((unsigned)((mn + 255) / 256)), dim3(256),
                       0, s, (const float*)part, splits, mn, y);
  return hipGetLastError();
}

// The super-block matrix-core GEMV with x staged in LDS: 8 staged rows (M <=
// 8) or 16, one workgroup of 8 waves per compute unit, K in 512-wide items, x
// staged whole (K up to 4096; longer K streams x per block instead, see
// q4k_xs_ok).  False if K is not a multiple of 512 or a byte offset would not
// fit 32 bits.
static bool q4k_mfma_config(int M, int64_t K, int64_t N, int* MR, int* KC) {
  if (M < 5 || M > 16 || K % kMSItem != 0 || K > 4096) return false;
  if (N * (K / 256) * 144 >= ((int64_t)1 << 31) || (int64_t)M * K * 2 >= ((int64_t)1 << 31)) return false;
  *MR = M <= 8 ? 8 : 16;
  *KC = 4096;  // a multiple of 8 waves x 512 columns; items at or past K load zeros
  return mfma_stream_lds_bytes(*MR, 8, *KC, false) <= 156 * 1024;
}

// x in registers: K of 512 .. 4096 (one 512-wide column range per wave); x
// streamed per block: longer K.
static bool q4k_xreg_ok(int M, int64_t K, int64_t N) {
  if (M < 5 || M > 16 || (K != 512 && K != 1024 && K != 2048 && K != 4096)) return false;
  return N * (K / 256) * 144 < ((int64_t)1 << 31) && (int64_t)M * K * 2 < ((int64_t)1 << 31);
}
static bool q4k_xs_ok(int M, int64_t K, int64_t N) {
  if (M < 5 || M > 16 || K <= 4096 || K % 256 != 0 || K > ((int64_t)1 << 24)) return false;
  return N * (K / 256) * 144 < ((int64_t)1 << 31) && (int64_t)M * K * 2 < ((int64_t)1 << 31);
}

bool q4k_mfma_stream_supported(int M, int64_t K, int64_t N) {
  int MR, KC;
  return q4k_xreg_ok(M, K, N) || q4k_xs_ok(M, K, N) || q4k_mfma_config(M, K, N, &MR, &KC);
}

hipError_t launch_q4k_gemv_mfma_stream(const uint16_t* x, int M, int64_t K, const uint8_t* blocks,
                                       int64_t N, uint16_t* y, hipStream_t s) {
  const int k = (int)K, n = (int)N;
  const int nb = (n + 15) / 16;
  if (q4k_xreg_ok(M, K, N)) {  // as many workgroups per compute unit as make 8 waves
#define GQ_QX_LAUNCH(NW_)                                                                          \
  hipLaunchKernelGGL((q4k_mfma_xreg_kernel<NW_>), dim3(std::max(1, std::min(nb, num_cus() * (8 / NW_)))), \
                     dim3(NW_ * 64), 0, s, x, M, k, blocks, n, y)
    switch (k / kMSItem) {
      case 1: GQ_QX_LAUNCH(1); break;
      case 2: GQ_QX_LAUNCH(2); break;
      case 4: GQ_QX_LAUNCH(4); break;
      default: GQ_QX_LAUNCH(8); break;
    }
#undef GQ_QX_LAUNCH
    return hipGetLastError();
  }
  if (q4k_xs_ok(M, K, N)) {  // one workgroup of 8 waves per compute unit
    const dim3 grid(std::max(1, std::min(nb, num_cus())));
    if (M <= 8)
      hipLaunchKernelGGL((q4k_mfma_xs_kernel<8, 8>), grid, dim3(512), 0, s, x, M, k, blocks, n, y);
    else
      hipLaunchKernelGGL((q4k_mfma_xs_kernel<8, 16>), grid, dim3(512), 0, s, x, M, k, blocks, n, y);
    return hipGetLastError();
  }
  int MR, KC;
  if (!q4k_mfma_config(M, K, N, &MR, &KC)) return hipErrorInvalidValue;
  const size_t lds = mfma_stream_lds_bytes(MR, 8, KC, false);
  const int grid = std::max(1, std::min((n + 15) / 16, num_cus()));
  if (MR == 8)
    hipLaunchKernelGGL((q4k_mfma_stream_kernel<8, false>), dim3(grid), dim3(512), lds, s, x, M, k, blocks,
                       n, y, KC);
  else
    hipLaunchKernelGGL((q4k_mfma_stream_kernel<16, false>), dim3(grid), dim3(512), lds, s, x, M, k, blocks,
                       n, y, KC);
  return hipGetLastError();
}

}  // namespace gq
