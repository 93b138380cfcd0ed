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
// The GEMVs use the layout of the plain INT4 GEMV: lane l of a wave owns the
// 32 weights at k = 2048 t + 32 l, which here is sub-block l%8 of block
// 8t + l/8; it loads the block's 16-byte header (the eight lanes of one block
// share one address) and its 16 nibble bytes, both as dwordx4.  M = 1..4 with
// every activation row in one compute unit's LDS run the persistent streaming
// kernel of the INT4 GEMV; larger M and longer K run a per-workgroup kernel
// that stages x in k chunks.
#include <algorithm>

#include "gq_internal.h"
#include "stream_util.h"

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

// ---------------------------------------------------------------------------
// M = 1..4: the streaming structure of the packed INT4 GEMV.  Persistent
// workgroups stage every activation row once (permuted pairs + chunk sums) and
// each wave walks (row pair, 2048-wide k step) items with three register
// buffers, two items' loads in flight.  Lane l loads, per row, the 16-byte
// header of block 8t + l/8 and the 16 nibble bytes of its sub-block l % 8 with
// raw buffer loads (the header address is shared by 8 lanes); lanes past K and
// rows past N read zero from the range check.  With MT > 1 activation rows
// each nibble word is unpacked once and multiplied against every row.
// ---------------------------------------------------------------------------
constexpr int kQRpw = 2;    // rows per item
constexpr int kQNbuf = 3;   // register buffers
constexpr int kQMaxM = 4;   // activation rows the streaming kernel takes
constexpr size_t kQLdsTwo = 80 * 1024;   // LDS of each of two workgroups per compute unit
constexpr size_t kQLdsOne = 156 * 1024;  // LDS of one workgroup per compute unit

// LDS bytes of the streaming kernel: per activation row and 2048-step 4 KiB of
// permuted pairs and 64 chunk sums.
size_t q4k_stream_lds(int M, int64_t K) { return (size_t)M * (size_t)((K + kStepK - 1) / kStepK) * (256 * 16 + 64 * 4); }

struct QBuf {
  uint4 h[kQRpw], w[kQRpw];
};

// x [MT, K]; y row m at y + m * ldy.
template <int NT, int MT>
__global__ __launch_bounds__(NT) void q4k_stream_kernel(const uint16_t* __restrict__ x, int K,
                                                              const uint8_t* __restrict__ blocks,
                                                              int N, uint16_t* __restrict__ y, int ldy) {
  namespace su = stream_util;
  extern __shared__ uint4 lds[];
  const int T = (K + kStepK - 1) / kStepK;
  uint4* xs = lds;                           // [MT][T][4][64] permuted x pairs
  float* sxs = (float*)(xs + MT * T * 256);  // [MT][T * 64] chunk sums
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = (N + kQRpw - 1) / kQRpw;
  constexpr int NW = NT / 64;  // waves per workgroup
  const int W = gridDim.x * NW;
  const uint32_t row_bytes = (uint32_t)(K / 256) * kBlockBytes;
  const su::rsrc_t rb = su::make_rsrc(blocks, (uint32_t)N * row_bytes);
  const uint32_t hoff = (uint32_t)(lane >> 3) * kBlockBytes;
  const uint32_t woff = hoff + 16u + 16u * (uint32_t)(lane & 7);
  // This lane's sub-block fields: the 6-bit scale at bit o6 = 6 sub of the
  // header's bytes 4..9 ({h.z : h.y}), the 6-bit min at bit o6 + 16 of bytes
  // 8..15 ({h.w : h.z}).  Each lies within two bytes, which one v_perm with a
  // per-lane selector brings to the bottom (selector byte 12 reads 0x00), so
  // one bit-field extract at o6 & 7 finishes it.
  const uint32_t o6 = 6u * (uint32_t)(lane & 7);
  const uint32_t fbit = o6 & 7u, sbyte = o6 >> 3, mbyte = 2u + (o6 >> 3);
  const uint32_t sel_sc = sbyte | ((sbyte + 1u) << 8) | 0x0C0C0000u;
  const uint32_t sel_mn = mbyte | ((mbyte < 7u ? mbyte + 1u : 12u) << 8) | 0x0C0C0000u;

  auto load = [&](QBuf& B, int b, int t) {
    const bool kin = t * kStepK + lane * 32 < K;
    const uint32_t step = (uint32_t)t * 8u * kBlockBytes;
    const uint32_t vh = kin ? hoff + step : su::kOob, vw = kin ? woff + step : su::kOob;
#pragma unroll
    for (int r = 0; r < kQRpw; ++r) {
      const uint32_t row = (uint32_t)min(b * kQRpw + r, N);  // row N reads out of range
      const auto h = __builtin_amdgcn_raw_buffer_load_b128(rb, vh, row * row_bytes, 0);
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(rb, vw, row * row_bytes, 2);
      B.h[r] = make_uint4(h[0], h[1], h[2], h[3]);
      B.w[r] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };

  // x: first loads before the weight prefetch, staged after it.  Flat chunk
  // f = m T 256 + c holds x[m, 8c .. 8c + 8).
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
  QBuf buf[kQNbuf];
  float acc[MT][kQRpw];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < kQRpw; ++r) acc[m][r] = 0.f;
  int lb = (int)blockIdx.x * NW + wave, lt = 0;  // next item to load
  int cb = lb, ct = 0;                               // next item to compute
  auto advance = [&](int& b, int& t) {
    if (++t == T) {
      t = 0;
      b += W;
    }
  };
#pragma unroll
  for (int j = 0; j < kQNbuf - 1; ++j) {
    load(buf[j], lb, lt);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads in item order: the loop's waits assume it
    advance(lb, lt);
  }
  for (int c0 = 0; c0 < MT * TC; c0 += kXr * NT) {
#pragma unroll
    for (int i = 0; i < kXr; ++i) {
      const int f = c0 + threadIdx.x + NT * i;
      const int m = MT == 1 ? 0 : f / TC, c = f - m * TC;
      // every load issued here is consumed here: a load left in flight on
      // some path would make the main loop wait for all loads at its head
      if (f < MT * TC) {  // uniform over each wave (T * 256 is a multiple of 64)
        uint4 v = xv[i];
        if (c0 > 0) {
          v = make_uint4(0, 0, 0, 0);
          if (c * 8 < K) v = *(const uint4*)(x + (size_t)m * K + c * 8);
        }
        // lane l of step p reads its four chunks at p*256 + j*64 + l
        xs[m * TC + ((c & ~255) | ((c & 3) << 6) | ((c >> 2) & 63))] = su::perm_x_pairs(v);
        float sm = su::sum_bf16x8(v);
        sm += __shfl_xor(sm, 1, 64);
        sm += __shfl_xor(sm, 2, 64);
        if ((c & 3) == 0) sxs[m * T * 64 + (c >> 2)] = sm;
      }
    }
  }
  __syncthreads();

  // the sub-block scale S = d sc and min Mn = dmin mn of row r's header
  auto fields = [&](const uint4& h, float& S, float& Mn) {
    const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(h.x & 0xFFFFu));
    const _Float16 dmin = __builtin_bit_cast(_Float16, (uint16_t)(h.x >> 16));
    const uint32_t sc6 = __builtin_amdgcn_ubfe(__builtin_amdgcn_perm(h.z, h.y, sel_sc), fbit, 6);
    const uint32_t mn6 = __builtin_amdgcn_ubfe(__builtin_amdgcn_perm(h.w, h.z, sel_mn), fbit, 6);
    // exact products (11 x 6 significant bits) in one mixed-precision fma each
    S = __builtin_fmaf((float)d, (float)sc6, 0.f);
    Mn = __builtin_fmaf((float)dmin, (float)mn6, 0.f);
  };
  // the row block's sums start at zero and are cleared after its last k step
  // (in the branch that stores them, so no other item pays for the reset)
  auto compute = [&](const QBuf& B, int b, int t) {
    if constexpr (MT == 1) {
    const uint4* xp = xs + t * 256 + lane;
    const uint4 x0 = xp[0], x1 = xp[64], x2 = xp[128], x3 = xp[192];
    const float sx = sxs[t * 64 + lane];
    const float init = -128.f * sx;  // bf16 128 + q: remove the offset of the 32 weights
#pragma unroll
    for (int r = 0; r < kQRpw; ++r) {
      float a = su::dot8_perm(B.w[r].x, x0, init, 0x43004300u);
      a = su::dot8_perm(B.w[r].y, x1, a, 0x43004300u);
      a = su::dot8_perm(B.w[r].z, x2, a, 0x43004300u);
      a = su::dot8_perm(B.w[r].w, x3, a, 0x43004300u);
      const uint4 h = B.h[r];
      const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(h.x & 0xFFFFu));
      const _Float16 dmin = __builtin_bit_cast(_Float16, (uint16_t)(h.x >> 16));
      const uint32_t sc6 = __builtin_amdgcn_ubfe(__builtin_amdgcn_perm(h.z, h.y, sel_sc), fbit, 6);
      const uint32_t mn6 = __builtin_amdgcn_ubfe(__builtin_amdgcn_perm(h.w, h.z, sel_mn), fbit, 6);
      // exact products (11 x 6 significant bits) in one mixed-precision fma each
      const float S = __builtin_fmaf((float)d, (float)sc6, 0.f);
      const float Mn = __builtin_fmaf((float)dmin, (float)mn6, 0.f);
      acc[0][r] = fmaf(S, a, fmaf(-Mn, sx, acc[0][r]));
    }
    } else {
      // activation row m: permuted pairs at xs[m T 256 ..], chunk sums at sxs[m T 64 ..]
      uint4 xq[MT][4];
      float sx[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint4* xp = xs + (m * T + t) * 256 + lane;
        xq[m][0] = xp[0];
        xq[m][1] = xp[64];
        xq[m][2] = xp[128];
        xq[m][3] = xp[192];
        sx[m] = sxs[(m * T + t) * 64 + lane];
      }
#pragma unroll
      for (int r = 0; r < kQRpw; ++r) {
        const uint4 u0 = su::unpack8_words(B.w[r].x, 0x43004300u);
        const uint4 u1 = su::unpack8_words(B.w[r].y, 0x43004300u);
        const uint4 u2 = su::unpack8_words(B.w[r].z, 0x43004300u);
        const uint4 u3 = su::unpack8_words(B.w[r].w, 0x43004300u);
        float S, Mn;
        fields(B.h[r], S, Mn);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float a = su::dot8_words(u0, xq[m][0], -128.f * sx[m]);
          a = su::dot8_words(u1, xq[m][1], a);
          a = su::dot8_words(u2, xq[m][2], a);
          a = su::dot8_words(u3, xq[m][3], a);
          acc[m][r] = fmaf(S, a, fmaf(-Mn, sx[m], acc[m][r]));
        }
      }
    }
    if (t == T - 1) {
      static_assert(kQRpw == 2, "the paired reduction takes two rows");
      if constexpr (MT == 1) {
        // both rows' sums together: row 0's in lane 31, row 1's in lane 63
        const float v = su::wave_sums_pair(acc[0][0], acc[0][1]);
        const int row = b * kQRpw + (lane >> 5);
        if ((lane & 31) == 31 && row < N) y[row] = f32_to_bf16_rne(v);
      } else {
        // all (m, r) sums together, four per register (padded with zeros); the
        // last lane of each 16-lane row stores the one its row holds
        constexpr int V = MT * kQRpw;
        constexpr int VP = V <= 4 ? 4 : 8;
        float v[VP], u[VP / 4];
#pragma unroll
        for (int i = 0; i < VP; ++i) v[i] = i < V ? acc[i / kQRpw][i % kQRpw] : 0.f;
        su::wave_sums_by_row<VP>(v, u);
        const int q = lane >> 4;
        const int qi = (q & 1) * 2 + (q >> 1);
        if ((lane & 15) == 15) {
#pragma unroll
          for (int j = 0; j < VP / 4; ++j) {
            const int idx = 4 * j + qi;
            const int m = idx / kQRpw, row = b * kQRpw + idx % kQRpw;
            if (idx < V && row < N) y[(size_t)m * ldy + row] = f32_to_bf16_rne(u[j]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < kQRpw; ++r) acc[m][r] = 0.f;
    }
  };
  // Whole buffer rounds in the loop, the last 0-2 items (already loaded) after
  // it: with its only exit at the bottom, the loop head waits for exactly the
  // item it multiplies, and no item is computed twice or padded.
  const int b0 = (int)blockIdx.x * NW + wave;
  const int items = b0 < nb ? ((nb - 1 - b0) / W + 1) * T : 0;
  const int rounds = items / kQNbuf, rest = items % kQNbuf;
  for (int it = 0; it < rounds; ++it) {
#pragma unroll
    for (int j = 0; j < kQNbuf; ++j) {
      load(buf[(j + kQNbuf - 1) % kQNbuf], lb, lt);
      __builtin_amdgcn_sched_barrier(0);  // issue the loads before this item's wait
      advance(lb, lt);
      compute(buf[j], cb, ct);
      advance(cb, ct);
    }
  }
  static_assert(kQNbuf == 3, "the tail below finishes at most two prefetched items");
  if (rest > 0) {
    compute(buf[0], cb, ct);
    advance(cb, ct);
  }
  if (rest > 1) compute(buf[1], cb, ct);
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

template <int MT>
hipError_t q4k_stream(const uint16_t* x, int K, const uint8_t* blocks, int N, uint16_t* y, hipStream_t s) {
  const int steps = (K + kStepK - 1) / kStepK;
  // rows per launch so that every byte offset fits 32 bits
  const uint64_t row_bytes = (uint64_t)(K / 256) * kBlockBytes;
  const int64_t cap = (int64_t)(((uint64_t)1 << 31) / row_bytes);
  const size_t lds = q4k_stream_lds(MT, K);
  for (int64_t n0 = 0; n0 < N; n0 += cap) {
    const int nn = (int)std::min<int64_t>(cap, N - n0);
    const int nb = (nn + kQRpw - 1) / kQRpw;
    // one workgroup of 8 waves per compute unit once K spans four or more
    // 2048-steps or x needs more than two workgroups' LDS (x staged once per
    // compute unit), else two of 4 waves
    if (steps >= 4 || lds > kQLdsTwo) {
      const int grid = std::max(1, std::min((nb + 7) / 8, num_cus()));
      hipLaunchKernelGGL((q4k_stream_kernel<512, MT>), dim3(grid), dim3(512), lds, s, x, K,
                         blocks + n0 * row_bytes, nn, y + n0, N);
    } else {
      const int grid = std::max(1, std::min((nb + kWaves - 1) / kWaves, 2 * num_cus()));
      hipLaunchKernelGGL((q4k_stream_kernel<kThreads, MT>), dim3(grid), dim3(kThreads), lds, s, x, K,
                         blocks + n0 * row_bytes, nn, y + n0, N);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_q4k_gemv(const uint16_t* x, int M, int64_t K, const uint8_t* blocks, int64_t N,
                           uint16_t* y, hipStream_t s) {
  const int steps = (int)((K + kStepK - 1) / kStepK);
  const int k = (int)K, n = (int)N;
  // the streaming kernel while every activation row fits one compute unit's LDS
  if (M <= kQMaxM && q4k_stream_lds(M, K) <= kQLdsOne) {
    switch (M) {
      case 1: return q4k_stream<1>(x, k, blocks, n, y, s);
      case 2: return q4k_stream<2>(x, k, blocks, n, y, s);
      case 3: return q4k_stream<3>(x, k, blocks, n, y, s);
      default: return q4k_stream<4>(x, k, blocks, n, y, s);
    }
  }
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
  // M = 5..16: the matrix cores (one MFMA per sub-block and 16 rows)
  if (M >= 5 && q4k_mfma_stream_supported(M, K, N))
    return launch_q4k_gemv_mfma_stream(x, M, K, blocks, N, y, s);
  if (M == 2) return launch_t<2, 2, 2>(x, M, k, blocks, n, y, s);
  if (M <= 4) return launch_t<4, 2, 1>(x, M, k, blocks, n, y, s);
  if (M <= 8) return launch_t<8, 2, 1>(x, M, k, blocks, n, y, s);
  return launch_t<16, 2, 1>(x, M, k, blocks, n, y, s);
}

}  // namespace gq
