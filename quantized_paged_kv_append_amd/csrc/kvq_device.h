// kvq_device.h -- device-side building blocks shared by the library's HIP
// kernels (gfx950 / CDNA4, wave64). Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

typedef _Float16 half_t;
typedef half_t half2v __attribute__((ext_vector_type(2)));
typedef half_t half4v __attribute__((ext_vector_type(4)));
typedef half_t half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---- 16-bit float inputs -------------------------------------------------
// bf16 is the upper half of a binary32; fp16 converts exactly to binary32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(half_t, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(half_t, (uint16_t)(w >> 16));
}
template <bool kBf16>
__device__ __forceinline__ void unpack2(uint32_t w, float& a, float& b) {
  if (kBf16) {
    a = bf16_lo(w);
    b = bf16_hi(w);
  } else {
    a = f16_lo(w);
    b = f16_hi(w);
  }
}

// ---- lane reductions within aligned groups of N lanes (N | 64) ----------
template <int N>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = N / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
template <int N>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
  for (int m = N / 2; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, kWave));
  return v;
}

// ---- IEEE binary32 division, correctly rounded ---------------------------
// The library is built without fast-math, so '/' on float is the correctly
// rounded IEEE quotient; this wrapper only documents the intent.
__device__ __forceinline__ float div_rn(float a, float b) { return a / b; }

// Round half to even to an integral float (v_rndne_f32).
__device__ __forceinline__ float rne(float x) { return __builtin_rintf(x); }

// Fast quotient y = x * inv (inv = 1/b rounded) with a check that y is far
// enough from every rounding boundary of rne(): |y - fl(x/b)| <= 3 * 2^-24 *
// |x/b|, i.e. below 2^-15 for |x/b| <= 256, so rne(y) == rne(fl(x/b)) unless
// y lies within 2^-14 of a half-integer. r = rne(y), hence |y - r| <= 1/2 and
// the test is one comparison. Callers then recompute with div_rn.
__device__ __forceinline__ bool near_half(float y, float r) {
  return fabsf(y - r) > 0.5f - 6.103515625e-05f;  // 1/2 - 2^-14
}

// The bound above needs inv = fl(1/s) to be a normal number with relative
// error 2^-24, i.e. s in [2^-126, 2^126]. Outside that range (scales of
// near-denormal rows, where 1/s overflows) the exact quotient is used.
__device__ __forceinline__ bool recip_unsafe(float s) {
  return !(s >= 1.17549435e-38f && s <= 8.50705917e+37f);
}

// ---- OCP E4M3 encoding of a binary32 value ------------------------------
// Nearest E4M3 value, ties to even mantissa, magnitudes above 448 saturate to
// 448, sign kept (0x80 for -0 and for negatives that round to zero).
// With e = max(floor(log2|y|), -6) the code is ((e + 7) << 3) + rne(|y| *
// 2^(3 - e)) - 8: the scaled magnitude lies in [8, 16) for normals and in
// [0, 8) below 2^-6, where the same formula yields the subnormal codes. A
// result of 16 carries into the next exponent; codes above 0x7E saturate.
// `m` returns the scaled magnitude so callers can test for near-ties.
__device__ __forceinline__ uint32_t e4m3_encode(float y, float& m, float& rm) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(y);
  int e = (int)((bits >> 23) & 0xFFu) - 127;  // floor(log2 a) for normal a
  e = e < -6 ? -6 : e;
  e = e > 8 ? 8 : e;
  const float p = __uint_as_float((uint32_t)(127 + 3 - e) << 23);  // 2^(3-e)
  m = a * p;                                                        // exact
  rm = rne(m);
  int code = ((e + 7) << 3) + (int)rm - 8;
  code = code > 0x7E ? 0x7E : code;
  return sign | (uint32_t)code;
}

// ---- FP8 / INT8 / INT4 codes to fp16, exactly ---------------------------
// Two E4M3 bytes (byte 2*sel and 2*sel+1 of w) to two fp16 (hardware
// conversion with unit scale; every finite E4M3 value is an fp16 value).
template <bool HI>
__device__ __forceinline__ half2v fp8x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Two's-complement int8 codes are biased (XOR 0x80 = code + 128) and placed in
// the low byte of an fp16 whose high byte is 0x64: the value is 1024 + code +
// 128 exactly; subtracting 1152 leaves the code. `wx` already holds the XORed
// bytes; sel picks which two bytes (perm selector built by the caller).
__device__ __forceinline__ half2v i8x2_to_h2(uint32_t wx, uint32_t sel) {
  uint32_t packed = __builtin_amdgcn_perm(0x64646464u, wx, sel);
  half2v h = __builtin_bit_cast(half2v, packed);
  const half2v bias = {(half_t)1152.0f, (half_t)1152.0f};
  return h - bias;
}

}  // namespace kvq
