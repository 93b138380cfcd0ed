// Fused W4A16 GEMV for decode (M <= 16) on gfx950.
//
// What is computed ("vLLM 量化与推测解码" section 2, fused W4A16 paragraph; the
// S08 "量化" page, "工作原理" figure right panel and "亲手实现"):
//   y[m, n] = bf16( sum_g S[n,g] * sum_{k in g} x[m,k] * (q[n,k] - z[n,g]) )
// reading only packed nibbles and the fp16 group scale/zero from HBM; the
// dequantized weight exists only in registers.
//
// Decode is bound by HBM bandwidth (S08 "为什么重要": latency = bytes /
// bandwidth), so both kernels are shaped around the weight stream.  Lane l of a
// wavefront owns the 32 weights at k = 2048 t + 32 l of a row (one 16-byte
// load; a wave load covers 1 KiB of a row contiguously).  A nibble becomes the
// exact bf16 value 128 + q by placing it under the exponent byte 0x43 (bf16
// 128.0, whose low mantissa bits the nibble fills), v_dot2_f32_bf16 multiplies
// a pair of them by the matching activation pair with fp32 accumulation, and
// per 32-element chunk the offset and zero point are removed with the chunk's
// sum of x:  sum x (q - z) = sum x (128 + q) - (128 + z) sum x,  then scaled by
// S.  The row's 64 lane partials are summed across the wave and rounded once
// to bf16 (nearest-even).
//
// gemv_stream_kernel (M = 1..4): persistent workgroups; x is staged once per
// workgroup into LDS (pre-permuted into the pairs the nibble extraction yields,
// plus every chunk sum).  Each wave walks a sequence of work items (a pair of
// rows x one 2048-wide k step) with three register buffers, so two items' loads
// are in flight while one is multiplied.  With M > 1 activation rows each
// weight is unpacked once and multiplied against every row, so the vector work
// per weight grows by the dot products only and the weights stream once.  Loads are raw buffer loads with the
// nontemporal hint against whole-matrix descriptors; anything past the matrix
// (rows beyond N, lanes beyond a ragged K) reads as zero from the hardware's
// range check, so the loads are unconditional and the compiler's wait counts
// stay exact.  Row sums are reduced with DPP (quad_perm, row_ror, row_bcast).
//
// gemv_chunked_kernel (M = 2..16, or K too long for x to sit in LDS): x staged
// per K chunk for all M rows; one workgroup per 4*RPW rows.
#include <algorithm>

#include "gq_internal.h"
#include "stream_util.h"

namespace gq {
namespace {

using namespace stream_util;

constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kWaves = kThreads / 64;
constexpr int kStepK = 2048;   // k covered by one wave load (64 lanes x 32)

// 8 nibbles of one dword (k offsets 0..7 at bits 4p) against the permuted
// activation dwords (x0,x4) (x1,x5) (x2,x6) (x3,x7): bf16 128 + q, or (XF16)
// fp16 1024 + q against fp16 activations.
template <bool XF16>
__device__ __forceinline__ float dot8(uint32_t d, const uint4& xp, float a) {
  constexpr uint32_t kMask = 0x000F000Fu, kMagic = XF16 ? 0x64006400u : 0x43004300u;
  if (XF16) {
    a = dot2h((d & kMask) | kMagic, xp.x, a);
    a = dot2h(((d >> 4) & kMask) | kMagic, xp.y, a);
    a = dot2h(((d >> 8) & kMask) | kMagic, xp.z, a);
    return dot2h(((d >> 12) & kMask) | kMagic, xp.w, a);
  }
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

// Stage x[:, kc0 : kc0 + KC) into LDS as permuted pairs plus 32-chunk sums
// (XF16: fp16 activations).
template <int MT, int KC, bool XF16>
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
    float s = XF16 ? sum_f16x8(v) : sum_bf16x8(v);
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if ((c & 3) == 0) sx[m][c >> 2] = s;
  }
}

// MT: activation rows handled together (M <= MT), RPW: weight rows per wave,
// T: 2048-wide steps per LDS chunk.  Each workgroup owns 4*RPW rows.  XF16:
// fp16 activations and output.
template <int MT, int RPW, int T, bool SYM, bool XF16>
__global__ __launch_bounds__(kThreads) void gemv_chunked_kernel(
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
    stage_x<MT, KC, XF16>(x, M, K, kc0, xs, sx);
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
          zo[t][r] = (XF16 ? 1024.f : 128.f) + (SYM ? 8.f : f16_to_f32(zeros[gi]));
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
          float a = dot8<XF16>(wv[t][r].x, x0, 0.f);
          a = dot8<XF16>(wv[t][r].y, x1, a);
          a = dot8<XF16>(wv[t][r].z, x2, a);
          a = dot8<XF16>(wv[t][r].w, x3, a);
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
      if (lane == 0 && m < M && row < N)
        y[(size_t)m * N + row] = XF16 ? f32_to_f16_rne(v) : f32_to_bf16_rne(v);
    }
}

template <int MT, int RPW, int T, bool SYM, bool XF16>
hipError_t launch_t(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                    const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  const int rows_per_block = kWaves * RPW;
  const unsigned grid = (unsigned)((N + rows_per_block - 1) / rows_per_block);
  hipLaunchKernelGGL((gemv_chunked_kernel<MT, RPW, T, SYM, XF16>), dim3(grid), dim3(kThreads), 0, s,
                     x, M, K, qw, sc, zr, N, G, y);
  return hipGetLastError();
}

template <bool SYM, bool XF16>
hipError_t dispatch(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                    const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  const int steps = (K + kStepK - 1) / kStepK;
  if (M == 1) {
    switch (steps) {
      case 1: return launch_t<1, 2, 1, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
      case 2: return launch_t<1, 2, 2, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
      case 3: return launch_t<1, 2, 3, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
      case 4: return launch_t<1, 2, 4, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
      case 5: return launch_t<1, 2, 5, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
      case 6: return launch_t<1, 2, 6, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
      case 7: return launch_t<1, 2, 7, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
      default: return launch_t<1, 2, 8, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
    }
  }
  if (M == 2) return launch_t<2, 2, 2, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
  if (M <= 4) return launch_t<4, 2, 1, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
  if (M <= 8) return launch_t<8, 2, 1, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
  return launch_t<16, 2, 1, SYM, XF16>(x, M, K, qw, sc, zr, N, G, y, s);
}


// ---------------------------------------------------------------------------
// Streaming kernel, M = 1..4
// ---------------------------------------------------------------------------

constexpr int kSNbuf = 3;   // register buffers (items in flight + 1)
constexpr int kSMaxM = 4;   // activation rows the streaming kernel takes
constexpr size_t kSLdsMulti = 80 * 1024;  // LDS of each of two workgroups per compute unit
constexpr size_t kSLdsOne = 156 * 1024;   // LDS of one workgroup per compute unit

// LDS bytes of the streaming kernel: per activation row and 2048-step 4 KiB of
// permuted pairs and 64 chunk sums; per step 512 B of offset tables (TAB).
size_t stream_lds_bytes(int M, int64_t K, bool tab) {
  const int64_t T = (K + kStepK - 1) / kStepK;
  return (size_t)(M * T * (256 * 16 + 64 * 4) + (tab ? T * 64 * 8 : 0));
}
// Scale and zero stay 16-bit in registers: widening them where the loop
// carries them would force a wait on every outstanding load.
template <int RPW>
struct StreamBuf {
  uint4 w[RPW];
  uint16_t s[RPW], z[RPW];
};

struct Cursor {
  int b, p;  // row block (RPW rows), k step
};

__device__ __forceinline__ void advance(Cursor& c, int T, int W) {
  if (++c.p == T) {
    c.p = 0;
    c.b += W;
  }
}

// TAB: per-(step, lane) byte offsets come from LDS tables (ragged K or a group
// size that does not divide 2048); otherwise they are lane constants plus a
// uniform per-step term.
template <int RPW, bool SYM, bool TAB>
__device__ __forceinline__ void stream_load(StreamBuf<RPW>& B, Cursor c, int N, uint32_t rb, uint32_t ngb,
                                            uint32_t sgs, uint32_t vw, uint32_t vs,
                                            const uint32_t* wtab, const uint32_t* stab, int lane,
                                            rsrc_t rw, rsrc_t rs, rsrc_t rz) {
  uint32_t ow = vw, os = vs, uw = (uint32_t)c.p * 1024u, us = (uint32_t)c.p * sgs;
  if (TAB) {
    ow = wtab[c.p * 64 + lane];
    os = stab[c.p * 64 + lane];
    uw = 0;
    us = 0;
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const uint32_t row = (uint32_t)min(c.b * RPW + r, N);  // row N reads out of range
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, ow, row * rb + uw, 2);
    B.w[r] = make_uint4(v[0], v[1], v[2], v[3]);
    B.s[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, os, row * ngb + us, 2);
    if (!SYM) B.z[r] = __builtin_amdgcn_raw_buffer_load_b16(rz, os, row * ngb + us, 2);
  }
}

template <int MT, int RPW, bool SYM, bool XF16>
__device__ __forceinline__ void stream_compute(const StreamBuf<RPW>& B, Cursor c, int T, int N, int ldy,
                                               int lane, const uint4* xs, const float* sxs,
                                               uint16_t* __restrict__ y, uint32_t magic,
                                               float (&acc)[MT][RPW]) {
  if (c.p == 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < RPW; ++r) acc[m][r] = 0.f;
  }
  constexpr float kOff = XF16 ? -1024.f : -128.f;  // the magic offset of every weight
  if constexpr (MT == 1) {
    const uint4* xp = xs + c.p * 256 + lane;
    const uint4 x0 = xp[0], x1 = xp[64], x2 = xp[128], x3 = xp[192];
    const float sx = sxs[c.p * 64 + lane];
    const float init = kOff * sx;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      float a = dot8_perm<XF16>(B.w[r].x, x0, init, magic);
      a = dot8_perm<XF16>(B.w[r].y, x1, a, magic);
      a = dot8_perm<XF16>(B.w[r].z, x2, a, magic);
      a = dot8_perm<XF16>(B.w[r].w, x3, a, magic);
      const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)B.s[r]);
      const float z = SYM ? 8.f : (float)__builtin_bit_cast(_Float16, (uint16_t)B.z[r]);
      acc[0][r] = fmaf(sc, fmaf(-z, sx, a), acc[0][r]);
    }
  } else {
    // activation row m: permuted pairs at xs[m T 256 ..], chunk sums at sxs[m T 64 ..]
    uint4 xq[MT][4];
    float sx[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint4* xp = xs + (m * T + c.p) * 256 + lane;
      xq[m][0] = xp[0];
      xq[m][1] = xp[64];
      xq[m][2] = xp[128];
      xq[m][3] = xp[192];
      sx[m] = sxs[(m * T + c.p) * 64 + lane];
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const uint4 u0 = unpack8_words(B.w[r].x, magic), u1 = unpack8_words(B.w[r].y, magic);
      const uint4 u2 = unpack8_words(B.w[r].z, magic), u3 = unpack8_words(B.w[r].w, magic);
      const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)B.s[r]);
      const float z = SYM ? 8.f : (float)__builtin_bit_cast(_Float16, (uint16_t)B.z[r]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float a = dot8_words<XF16>(u0, xq[m][0], kOff * sx[m]);
        a = dot8_words<XF16>(u1, xq[m][1], a);
        a = dot8_words<XF16>(u2, xq[m][2], a);
        a = dot8_words<XF16>(u3, xq[m][3], a);
        acc[m][r] = fmaf(sc, fmaf(-z, sx[m], a), acc[m][r]);
      }
    }
  }
  if (c.p == T - 1) {
    if constexpr (MT == 1 && RPW == 2) {
      // both rows' sums together: row 0's in lane 31, row 1's in lane 63
      const float v = wave_sums_pair(acc[0][0], acc[0][1]);
      const int row = c.b * 2 + (lane >> 5);
      if ((lane & 31) == 31 && row < N) y[row] = XF16 ? f32_to_f16_rne(v) : f32_to_bf16_rne(v);
    } else if constexpr (MT == 1) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float v = wave_sum_to_lane63(acc[0][r]);
        const int row = c.b * RPW + r;
        if (lane == 63 && row < N) y[row] = XF16 ? f32_to_f16_rne(v) : f32_to_bf16_rne(v);
      }
    } else {
      // all (m, r) sums together, four per register (padded with zeros); the
      // last lane of each 16-lane row stores the one its row holds
      constexpr int V = MT * RPW;
      constexpr int VP = V <= 4 ? 4 : V <= 8 ? 8 : 16;
      static_assert(V <= 16, "at most sixteen sums per row block");
      float v[VP], u[VP / 4];
#pragma unroll
      for (int i = 0; i < VP; ++i) v[i] = i < V ? acc[i / RPW][i % RPW] : 0.f;
      wave_sums_by_row<VP>(v, u);
      const int q = lane >> 4;
      const int qi = (q & 1) * 2 + (q >> 1);
      if ((lane & 15) == 15) {
#pragma unroll
        for (int j = 0; j < VP / 4; ++j) {
          const int idx = 4 * j + qi;
          const int m = idx / RPW, row = c.b * RPW + idx % RPW;
          if (idx < V && row < N)
            y[(size_t)m * ldy + row] = XF16 ? f32_to_f16_rne(u[j]) : f32_to_bf16_rne(u[j]);
        }
      }
    }
  }
}

// MT activation rows (x [MT, K]); y row m at y + m * ldy.  RPW weight rows
// per work item (more rows reuse each activation read from LDS more often);
// NT threads per workgroup.
// Requires N * K/2 < 2^32 and N * (K/G) * 2 < 2^32 (the launcher splits N).
template <int MT, int RPW, int NT, bool SYM, bool TAB, bool XF16>
__global__ __launch_bounds__(NT) void gemv_stream_kernel(
    const uint16_t* __restrict__ x, int K, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int N, int G,
    uint16_t* __restrict__ y, int ldy) {
  extern __shared__ uint4 lds[];
  const int T = (K + kStepK - 1) / kStepK;
  uint4* xs = lds;                                      // [MT][T][4][64] permuted x pairs
  float* sxs = (float*)(xs + MT * T * 256);             // [MT][T * 64] chunk sums
  uint32_t* wtab = (uint32_t*)(sxs + MT * T * 64);      // [T * 64] (TAB only)
  uint32_t* stab = wtab + T * 64;                       // [T * 64] (TAB only)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int NW = NT / 64;  // waves per workgroup
  const int nb = (N + RPW - 1) / RPW;
  const int W = gridDim.x * NW;
  const uint32_t rb = (uint32_t)K / 2;
  const uint32_t ngb = (uint32_t)(K / G) * 2;
  const uint32_t sgs = TAB ? 0u : (uint32_t)(kStepK / G) * 2;
  const uint32_t vw = (uint32_t)lane * 16;
  const uint32_t vs = TAB ? 0u : (uint32_t)((lane * 32) / G) * 2;
  const uint32_t magic = XF16 ? 0x64006400u : 0x43004300u;
  const rsrc_t rw = make_rsrc(qw, (uint32_t)N * rb);
  const rsrc_t rs = make_rsrc(scales, (uint32_t)N * ngb);
  const rsrc_t rz = make_rsrc(SYM ? (const void*)scales : (const void*)zeros, (uint32_t)N * ngb);

  if (TAB) {  // byte offsets per (step, lane); lanes past K read out of range
    for (int i = threadIdx.x; i < T * 64; i += NT) {
      const int k = (i >> 6) * kStepK + (i & 63) * 32;
      wtab[i] = k < K ? (uint32_t)k / 2 : kOob;
      stab[i] = k < K ? (uint32_t)(k / G) * 2 : kOob;
    }
    __syncthreads();
  }

  // x: issue the first loads before the weight prefetch, stage after it.
  // Flat chunk f = m T 256 + c holds x[m, 8c .. 8c + 8); a quad of lanes holds
  // one 32-chunk of one row (T 256 is a multiple of 4).
  constexpr int kXr = 8;
  const int TC = T * 256;  // chunks per activation row
  uint4 xv[kXr];
#pragma unroll
  for (int i = 0; i < kXr; ++i) {
    const int f = threadIdx.x + NT * i;
    const int m = MT == 1 ? 0 : f / TC, c = f - m * TC;
    xv[i] = make_uint4(0, 0, 0, 0);
    if (f < MT * TC && c * 8 < K) xv[i] = *(const uint4*)(x + (size_t)m * K + c * 8);
  }

  StreamBuf<RPW> buf[kSNbuf];
  float acc[MT][RPW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[m][r] = 0.f;
  Cursor lc{(int)blockIdx.x * NW + wave, 0};
  Cursor cc = lc;
#pragma unroll
  for (int j = 0; j < kSNbuf - 1; ++j) {
    stream_load<RPW, SYM, TAB>(buf[j], lc, N, rb, ngb, sgs, vw, vs, wtab, stab, lane, rw, rs, rz);
    // keep the loads in item order: the loop's waits assume it
    __builtin_amdgcn_sched_barrier(0);
    advance(lc, T, W);
  }

  for (int c0 = 0; c0 < MT * TC; c0 += kXr * NT) {
#pragma unroll
    for (int i = 0; i < kXr; ++i) {
      const int f = c0 + threadIdx.x + NT * i;
      const int m = MT == 1 ? 0 : f / TC, c = f - m * TC;
      // every load issued here is consumed here: a load left in flight on
      // some path would make the main loop wait for all loads at its head
      if (f < MT * TC) {
        uint4 v = xv[i];
        if (c0 > 0) {
          v = make_uint4(0, 0, 0, 0);
          if (c * 8 < K) v = *(const uint4*)(x + (size_t)m * K + c * 8);
        }
        // chunk c = 8 x values; lane l of step p reads its four chunks at
        // p*256 + j*64 + l (j = 0..3), so the 16-byte LDS reads of a wave are
        // consecutive and free of bank conflicts
        xs[m * TC + ((c & ~255) | ((c & 3) << 6) | ((c >> 2) & 63))] = perm_x_pairs(v);
        float sm = XF16 ? sum_f16x8(v) : sum_bf16x8(v);
        sm += __shfl_xor(sm, 1, 64);
        sm += __shfl_xor(sm, 2, 64);
        if ((c & 3) == 0) sxs[m * T * 64 + (c >> 2)] = sm;
      }
    }
  }
  __syncthreads();

  // Whole buffer rounds in the loop, the last 0-2 items (already loaded) after
  // it: with its only exit at the bottom, the loop head waits for exactly the
  // item it multiplies (an exit in the middle would merge just-issued loads
  // into the head's wait), and no item is computed twice or padded.
  const int b0 = (int)blockIdx.x * NW + wave;
  const int items = b0 < nb ? ((nb - 1 - b0) / W + 1) * T : 0;
  const int rounds = items / kSNbuf, rest = items % kSNbuf;
  for (int it = 0; it < rounds; ++it) {
#pragma unroll
    for (int j = 0; j < kSNbuf; ++j) {
      stream_load<RPW, SYM, TAB>(buf[(j + kSNbuf - 1) % kSNbuf], lc, N, rb, ngb, sgs, vw, vs, wtab, stab,
                            lane, rw, rs, rz);
      __builtin_amdgcn_sched_barrier(0);  // issue the loads before this item's wait
      advance(lc, T, W);
      stream_compute<MT, RPW, SYM, XF16>(buf[j], cc, T, N, ldy, lane, xs, sxs, y, magic, acc);
      advance(cc, T, W);
    }
  }
  static_assert(kSNbuf == 3, "the tail below finishes at most two prefetched items");
  if (rest > 0) {
    stream_compute<MT, RPW, SYM, XF16>(buf[0], cc, T, N, ldy, lane, xs, sxs, y, magic, acc);
    advance(cc, T, W);
  }
  if (rest > 1) stream_compute<MT, RPW, SYM, XF16>(buf[1], cc, T, N, ldy, lane, xs, sxs, y, magic, acc);
}

template <int MT, int RPW, bool SYM, bool TAB, bool XF16>
hipError_t launch_stream_rpw(const uint16_t* x, int K, const uint8_t* qw, const uint16_t* sc,
                             const uint16_t* zr, int N, int G, uint16_t* y, int ldy, hipStream_t s) {
  const size_t lds = stream_lds_bytes(MT, K, TAB);
  const int nb = (N + RPW - 1) / RPW;
  // One workgroup of 8 waves per compute unit (x staged once per compute unit)
  // when x needs more LDS than two workgroups can have, and once K spans four
  // or more 2048-steps ([4096, 14336]: M = 1 8.6 -> 8.0 us, M = 2 13.2 ->
  // 10.2 us; the K = 4096 shapes are faster with two workgroups of 4 waves:
  // qkv 4.8 against 5.3 us at M = 1).
  const int T = (K + kStepK - 1) / kStepK;
  if (lds > kSLdsMulti || T >= 4) {
    const int grid = std::max(1, std::min((nb + 7) / 8, num_cus()));
    hipLaunchKernelGGL((gemv_stream_kernel<MT, RPW, 512, SYM, TAB, XF16>), dim3(grid), dim3(512),
                       lds, s, x, K, qw, sc, zr, N, G, y, ldy);
    return hipGetLastError();
  }
  const int grid = std::max(1, std::min((nb + 3) / 4, 2 * num_cus()));
  hipLaunchKernelGGL((gemv_stream_kernel<MT, RPW, 256, SYM, TAB, XF16>), dim3(grid), dim3(256), lds,
                     s, x, K, qw, sc, zr, N, G, y, ldy);
  return hipGetLastError();
}

// Two weight rows per item; with three or more activation rows four, when
// every wave still gets about four items (each activation read from LDS then
// serves four rows; with fewer items per wave the tail costs more than that
// saves: measured on the Llama-3-8B shapes, four rows win on [28672, 4096]
// only).
template <int MT, bool SYM, bool TAB, bool XF16>
hipError_t launch_stream(const uint16_t* x, int K, const uint8_t* qw, const uint16_t* sc,
                         const uint16_t* zr, int N, int G, uint16_t* y, int ldy, hipStream_t s) {
  if constexpr (MT >= 3) {
    const int64_t T = (K + kStepK - 1) / kStepK;
    const int64_t waves = (int64_t)num_cus() * 8;
    if ((int64_t)((N + 3) / 4) * T >= 4 * waves)
      return launch_stream_rpw<MT, 4, SYM, TAB, XF16>(x, K, qw, sc, zr, N, G, y, ldy, s);
  }
  return launch_stream_rpw<MT, 2, SYM, TAB, XF16>(x, K, qw, sc, zr, N, G, y, ldy, s);
}

template <int MT, bool SYM, bool XF16 = false>
hipError_t stream_m(const uint16_t* x, int K, const uint8_t* qw, const uint16_t* sc,
                    const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  // Rows per launch so that every byte offset fits 32 bits.
  const uint64_t rb = (uint64_t)K / 2, ngb = (uint64_t)(K / G) * 2;
  const int64_t cap = (int64_t)std::min<uint64_t>(((uint64_t)1 << 31) / rb, ((uint64_t)1 << 31) / ngb);
  const bool tab = (K % kStepK) != 0 || (kStepK % G) != 0;
  for (int64_t n0 = 0; n0 < N; n0 += cap) {
    const int n = (int)std::min<int64_t>(cap, N - n0);
    const uint8_t* q = qw + n0 * rb;
    const uint16_t* a = sc + n0 * (K / G);
    const uint16_t* b = SYM ? zr : zr + n0 * (K / G);
    hipError_t e = tab ? launch_stream<MT, SYM, true, XF16>(x, K, q, a, b, n, G, y + n0, N, s)
                       : launch_stream<MT, SYM, false, XF16>(x, K, q, a, b, n, G, y + n0, N, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool SYM, bool XF16 = false>
hipError_t stream_any(const uint16_t* x, int M, int K, const uint8_t* qw, const uint16_t* sc,
                      const uint16_t* zr, int N, int G, uint16_t* y, hipStream_t s) {
  switch (M) {
    case 1: return stream_m<1, SYM, XF16>(x, K, qw, sc, zr, N, G, y, s);
    case 2: return stream_m<2, SYM, XF16>(x, K, qw, sc, zr, N, G, y, s);
    case 3: return stream_m<3, SYM, XF16>(x, K, qw, sc, zr, N, G, y, s);
    default: return stream_m<4, SYM, XF16>(x, K, qw, sc, zr, N, G, y, s);
  }
}
}  // namespace

bool gemv_stream_supported(int M, int64_t K) {
  // every activation row (and the offset tables) in one compute unit's LDS
  return M >= 1 && M <= kSMaxM && stream_lds_bytes(M, K, true) <= kSLdsOne;
}

// Kernel choice: the streaming kernel (M = 1..4 while x fits its LDS stage),
// the matrix-core kernels with x in registers (M = 4..16, K <= 4096), x
// streamed per item (M = 5..16, longer K) or x staged in LDS (the other K
// where it takes the shape), the split-K matrix-core kernel when the caller
// gives a workspace for it, and the per-row dot-product kernel for everything
// else; none of them allocates.
hipError_t launch_w4a16_gemv(const uint16_t* x, int M, int64_t K, const uint8_t* qweight,
                             const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                             int symmetric, uint16_t* y, void* workspace, bool xf16, hipStream_t s) {
  const int k = (int)K, n = (int)N;
  // M = 4 at K <= 4096: the register-x matrix-core kernel (same-box o 7.05 ->
  // 6.04 us, gate_up 22.3 -> 19.9 us, qkv level); the dot-product kernel
  // keeps M = 1..3 and M = 4 on longer K (down level)
  if (M == 4 && gemv_xreg_supported(M, K, N, G))
    return launch_w4a16_gemv_xreg(x, M, K, qweight, scales, zeros, N, G, symmetric, y, s, xf16);
  if (gemv_stream_supported(M, K)) {
    if (xf16)
      return symmetric ? stream_any<true, true>(x, M, k, qweight, scales, zeros, n, G, y, s)
                       : stream_any<false, true>(x, M, k, qweight, scales, zeros, n, G, y, s);
    return symmetric ? stream_any<true>(x, M, k, qweight, scales, zeros, n, G, y, s)
                     : stream_any<false>(x, M, k, qweight, scales, zeros, n, G, y, s);
  }
  if (gemv_xreg_supported(M, K, N, G))
    return launch_w4a16_gemv_xreg(x, M, K, qweight, scales, zeros, N, G, symmetric, y, s, xf16);
  if (gemv_xs_supported(M, K, N, G))
    return launch_w4a16_gemv_xs(x, M, K, qweight, scales, zeros, N, G, symmetric, y, s, xf16);
  if (gemv_mfma_stream_supported(M, K, N, G))
    return launch_w4a16_gemv_mfma_stream(x, M, K, qweight, scales, zeros, N, G, symmetric, y, s, xf16);
  if (workspace && gemv_workspace_bytes(M, K, N, G) > 0)
    return launch_w4a16_gemv_mfma(x, M, K, qweight, scales, zeros, N, G, symmetric, y, workspace, xf16, s);
  if (xf16)
    return symmetric ? dispatch<true, true>(x, M, k, qweight, scales, zeros, n, G, y, s)
                     : dispatch<false, true>(x, M, k, qweight, scales, zeros, n, G, y, s);
  return symmetric ? dispatch<true, false>(x, M, k, qweight, scales, zeros, n, G, y, s)
                   : dispatch<false, false>(x, M, k, qweight, scales, zeros, n, G, y, s);
}

}  // namespace gq
