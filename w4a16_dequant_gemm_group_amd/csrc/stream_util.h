// Helpers shared by the weight-streaming GEMV kernels (the packed INT4 GEMV and
// the super-block GEMV): raw buffer descriptors, the exact nibble-to-16-bit
// unpack with v_perm and the packed dot products, activation pair permutation
// and chunk sums, and the DPP wave reduction.
#pragma once

#include "gq_internal.h"

namespace gq {
namespace stream_util {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// fp16 pairs: v_dot2_f32_f16 (fp32 accumulation)
__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                false);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOob = 0x80000000u;  // an offset past every buffer's range

// Raw buffer descriptor over [base, base + bytes); every field wave-uniform.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                           0x00020000);
}

// 8 nibbles (k = 0..7 at bits 4p) against activation pairs (x0,x2) (x4,x6)
// (x1,x3) (x5,x7): the even and odd nibbles are split into bytes, and each
// byte pair gets an exponent byte from `magic` by v_perm: 0x43 makes the bf16
// value 128 + q (magic 0x43004300), 0x64 the fp16 value 1024 + q (0x64006400);
// both are exact.  XF16: fp16 activations.
template <bool XF16 = false>
__device__ __forceinline__ float dot8_perm(uint32_t d, const uint4& xp, float a, uint32_t magic) {
  const uint32_t ev = d & 0x0F0F0F0Fu;
  const uint32_t od = (d >> 4) & 0x0F0F0F0Fu;
  if (XF16) {
    a = dot2h(__builtin_amdgcn_perm(ev, magic, 0x01050104u), xp.x, a);
    a = dot2h(__builtin_amdgcn_perm(ev, magic, 0x01070106u), xp.y, a);
    a = dot2h(__builtin_amdgcn_perm(od, magic, 0x01050104u), xp.z, a);
    return dot2h(__builtin_amdgcn_perm(od, magic, 0x01070106u), xp.w, a);
  }
  a = dot2(__builtin_amdgcn_perm(ev, magic, 0x01050104u), xp.x, a);
  a = dot2(__builtin_amdgcn_perm(ev, magic, 0x01070106u), xp.y, a);
  a = dot2(__builtin_amdgcn_perm(od, magic, 0x01050104u), xp.z, a);
  a = dot2(__builtin_amdgcn_perm(od, magic, 0x01070106u), xp.w, a);
  return a;
}

// The four 16-bit pair words of dot8_perm (same order), for reuse against
// several activation rows.
__device__ __forceinline__ uint4 unpack8_words(uint32_t d, uint32_t magic) {
  const uint32_t ev = d & 0x0F0F0F0Fu;
  const uint32_t od = (d >> 4) & 0x0F0F0F0Fu;
  return make_uint4(__builtin_amdgcn_perm(ev, magic, 0x01050104u),
                    __builtin_amdgcn_perm(ev, magic, 0x01070106u),
                    __builtin_amdgcn_perm(od, magic, 0x01050104u),
                    __builtin_amdgcn_perm(od, magic, 0x01070106u));
}

// a + u . xp over four pair words (bf16 pairs, or fp16 pairs if XF16)
template <bool XF16 = false>
__device__ __forceinline__ float dot8_words(const uint4& u, const uint4& xp, float a) {
  if (XF16) {
    a = dot2h(u.x, xp.x, a);
    a = dot2h(u.y, xp.y, a);
    a = dot2h(u.z, xp.z, a);
    return dot2h(u.w, xp.w, a);
  }
  a = dot2(u.x, xp.x, a);
  a = dot2(u.y, xp.y, a);
  a = dot2(u.z, xp.z, a);
  return dot2(u.w, xp.w, a);
}

// x0..x7 (bf16, natural order in v) -> pairs (x0,x2) (x4,x6) (x1,x3) (x5,x7).
__device__ __forceinline__ uint4 perm_x_pairs(uint4 v) {
  uint4 p;
  p.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
  p.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
  p.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
  p.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
  return p;
}

__device__ __forceinline__ float sum_f16x8(uint4 v) {
  auto h = [](uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); };
  float s = h(v.x & 0xFFFFu) + h(v.x >> 16);
  s += h(v.y & 0xFFFFu) + h(v.y >> 16);
  s += h(v.z & 0xFFFFu) + h(v.z >> 16);
  s += h(v.w & 0xFFFFu) + h(v.w >> 16);
  return s;
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float sum_bf16x8(uint4 v) {
  float s = bf16_to_f32(v.x & 0xFFFFu) + bf16_to_f32(v.x >> 16);
  s += bf16_to_f32(v.y & 0xFFFFu) + bf16_to_f32(v.y >> 16);
  s += bf16_to_f32(v.z & 0xFFFFu) + bf16_to_f32(v.z >> 16);
  s += bf16_to_f32(v.w & 0xFFFFu) + bf16_to_f32(v.w >> 16);
  return s;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, ROW_MASK == 0xF));
}

// Sums over the 64 lanes of VP values (VP = 4, 8 or 16) at once, four per
// register.  v32 = permlane32_swap pairs v[2i] and v[2i+1] (one add halves
// both), v16 = permlane16_swap pairs the results (one add halves four), and
// four row-local DPP adds finish each 16-lane row: every lane of row q of u[j]
// then holds the sum of v[4j + (q & 1) * 2 + (q >> 1)].  10 instructions per
// four values, against 8 per value for wave_sum_to_lane63.
template <int VP>
__device__ __forceinline__ void wave_sums_by_row(const float (&v)[VP], float (&u)[VP / 4]) {
  static_assert(VP == 4 || VP == 8 || VP == 16, "four, eight or sixteen values");
  float s[VP / 2];
#pragma unroll
  for (int i = 0; i < VP / 2; ++i) {
    const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v[2 * i]),
                                                    __builtin_bit_cast(uint32_t, v[2 * i + 1]), false, false);
    const uint32_t lo = p[0], hi = p[1];  // bit-casting p[1] in place reads p[0]
    s[i] = __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
  }
#pragma unroll
  for (int j = 0; j < VP / 4; ++j) {
    const auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, s[2 * j]),
                                                    __builtin_bit_cast(uint32_t, s[2 * j + 1]), false, false);
    const uint32_t lo = p[0], hi = p[1];
    float t = __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
    t += dpp_f32<0xB1, 0xF>(t);   // quad_perm [1,0,3,2]
    t += dpp_f32<0x4E, 0xF>(t);   // quad_perm [2,3,0,1]
    t += dpp_f32<0x124, 0xF>(t);  // row_ror:4
    t += dpp_f32<0x128, 0xF>(t);  // row_ror:8
    u[j] = t;
  }
}

// Sums over the 64 lanes of two values: a's lands in lane 31, b's in lane 63.
// One permlane32_swap and add halve both, four row-local DPP adds give every
// row its 16-lane sum, and a row_bcast:15 into rows 1 and 3 adds rows 0 and 2
// to them (8 instructions, against 8 per value for wave_sum_to_lane63).
__device__ __forceinline__ float wave_sums_pair(float a, float b) {
  const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                  __builtin_bit_cast(uint32_t, b), false, false);
  const uint32_t lo = p[0], hi = p[1];  // bit-casting p[1] in place reads p[0]
  float t = __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
  t += dpp_f32<0xB1, 0xF>(t);   // quad_perm [1,0,3,2]
  t += dpp_f32<0x4E, 0xF>(t);   // quad_perm [2,3,0,1]
  t += dpp_f32<0x124, 0xF>(t);  // row_ror:4
  t += dpp_f32<0x128, 0xF>(t);  // row_ror:8
  t += dpp_f32<0x142, 0xA>(t);  // row_bcast:15 into rows 1 and 3
  return t;
}

// Sum over the 64 lanes; the total lands in lane 63.
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v += dpp_f32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x124, 0xF>(v);  // row_ror:4
  v += dpp_f32<0x128, 0xF>(v);  // row_ror:8  (every lane holds its row's sum)
  v += dpp_f32<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f32<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}


}  // namespace stream_util
}  // namespace gq
