// Number formats on the gfx950 decode path.
//
// Formats (monolith page, "Design decisions"; e2m1 grid from the TSCT
// super-kernel note, section 3b):
//   bf16  the upper half of an IEEE binary32, rounded to nearest even
//   e4m3  OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits, no
//         infinities, largest finite 448 (code 0x7E)
//   e2m1  sign, 2 exponent bits (bias 1), 1 mantissa bit: {0,.5,1,1.5,2,3,4,6}
//
// Decoding uses gfx950's converters: v_cvt_pk_f32_fp8 reads OCP E4M3 and
// v_cvt_scalef32_pk_f32_fp4 with scale 1.0 reads E2M1 exactly; the GEMVs use
// v_cvt_scalef32_pk_bf16_fp8 / _fp4, which turn two codes into a bf16 pair
// (exact: every E4M3 and E2M1 value is a bf16 value) for v_dot2_f32_bf16.
// All four are checked against every code.  Encoding, used only by the packer, is written from
// the format definition: round to nearest, ties to even, saturate to the
// largest finite magnitude, keep the sign (so tiny negatives become -0).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// acc + a.lo*b.lo + a.hi*b.hi for two packed bf16 pairs (products exact in fp32).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, a), __builtin_bit_cast(bf2, b), acc, false);
}
// Bytes 0,1 (HI=false) or 2,3 (HI=true) of `w`, E4M3, as a bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Nibbles of byte SEL of `w`, E2M1 (low nibble first), as a bf16 pair.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (no NaN on this path).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> one bf16 pair (lo in bits 0..15), round to nearest even, with
// gfx950's v_cvt_pk_bf16_f32 (checked against the bit formula above).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, bf2));
}

// Four e4m3 bytes of `w` -> four floats.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* o) {
  f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
}

// Eight e2m1 nibbles of `w` (element 2j in the low nibble of byte j) -> eight floats.
__device__ __forceinline__ void e2m1x8_to_f32(uint32_t w, float* o) {
  f2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  f2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  f2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  f2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
  o[4] = c[0]; o[5] = c[1]; o[6] = d[0]; o[7] = d[1];
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)(byte & 0xFFu), false)[0];
}

// Unbiased exponent of a positive normal float.
__device__ __forceinline__ int exp_of(float a) { return (int)((__float_as_uint(a) >> 23) & 0xFF) - 127; }

// fp32 -> e4m3 byte: nearest even, saturating at 448, sign kept.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t s = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a < 448.0f)) return s | 0x7Eu;              // saturate (NaN is not expected)
  if (a < 0.015625f) {                               // below 2^-6: subnormal step 2^-9
    return s | (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8; 8 is the smallest normal, 0x08
  }
  const int e = exp_of(a);                           // -6..8
  const float q = __builtin_rintf(a * __builtin_ldexpf(1.0f, 3 - e));  // 8..16, exact scaling
  return s | (uint32_t)(((e + 7) << 3) + (int)q - 8);  // q == 16 rolls into the next exponent
}

// fp32 -> e2m1 nibble: nearest even, saturating at 6, sign kept.
__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
  const uint32_t s = (__float_as_uint(x) >> 28) & 0x8u;
  const float a = fabsf(x);
  if (!(a < 6.0f)) return s | 0x7u;
  if (a < 1.0f) return s | (uint32_t)__builtin_rintf(a * 2.0f);   // 0, 0.5, 1 -> codes 0..2
  const int e = exp_of(a);                                           // 0..2
  const float q = __builtin_rintf(a * __builtin_ldexpf(1.0f, 1 - e));  // 2..4
  return s | (uint32_t)(((e + 1) << 1) + (int)q - 2);
}

}  // namespace mk
