// device.h -- small device helpers: bf16 packing, OCP E4M3 decode/encode,
// cross-lane reductions.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qln {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Value of a non-negative OCP E4M3FN code (0x00..0x7E): exponent bias 7, three
// mantissa bits, exponent 0 subnormal (m/8 * 2^-6).
__device__ __forceinline__ float e4m3_decode(uint32_t q) {
  uint32_t e = (q >> 3) & 15u, m = q & 7u;
  float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
  float sub = (float)m * 0x1p-9f;
  return e ? normal : sub;
}

// Round a non-negative float to the nearest E4M3FN code, ties to even,
// saturating at 448 (code 0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  uint32_t bits = __float_as_uint(v);
  int ex = (int)(bits >> 23) - 127;
  if (ex < -6) {
    // subnormal range: multiples of 2^-9; v * 512 is exact, rintf rounds half to even
    float m = __builtin_rintf(v * 512.0f);
    return (uint32_t)m;  // 8 becomes 0x08 = the smallest normal, as it should
  }
  uint32_t m23 = bits & 0x7FFFFFu;
  uint32_t keep = m23 >> 20, rem = m23 & 0xFFFFFu;
  uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (keep & 1u));
  uint32_t code = (((uint32_t)(ex + 7)) << 3) + keep + up;  // a mantissa carry bumps the exponent
  return code > 0x7Eu ? 0x7Eu : code;
}

// DPP cross-lane moves (gfx9 encodings).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;

// max over each aligned group of 8 lanes
__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, dpp_f32<DPP_QUAD_XOR1>(x));
  x = fmaxf(x, dpp_f32<DPP_QUAD_XOR2>(x));
  x = fmaxf(x, dpp_f32<DPP_ROW_HALF_MIRROR>(x));
  return x;
}

// max over each aligned group of 16 lanes (one DPP row)
__device__ __forceinline__ float max16(float x) {
  x = max8(x);
  return fmaxf(x, dpp_f32<DPP_ROW_MIRROR>(x));
}

// max over the whole wave (result valid in every lane)
__device__ __forceinline__ float wave_max(float x) {
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

}  // namespace qln
