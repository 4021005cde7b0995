// kvq_encode.h -- the byte coder of one new K or V row, shared by the append
// kernels and the decode kernel that appends the step's token itself.
// Internal to the library.
//
// What is coded ("Dynamic KV Cache Quantization for Fast LLM Inference",
// section "Understanding Dynamic Quantization Techniques for KV Caches"): the
// row's scale from its own range when it enters the cache, s = amax / qmax in
// fp32 with correctly rounded division (or a static scale given in advance),
// then codes rne(x / s): INT8 within [-127, 127], E4M3 by the hardware's
// round to nearest even. Codes use the reciprocal with a near-tie check that
// falls back to the exact quotient, so the stored bytes equal those of the
// exact quotient.
#pragma once

#include "kvq_device.h"

namespace kvq {
namespace {

// max over the four lanes of a quad (DPP quad permutations, no LDS)
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true)));
  return v;
}

__device__ __forceinline__ uint32_t pack_bytes(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) |
         ((uint32_t)(c & 0xFF) << 16) | ((uint32_t)(d & 0xFF) << 24);
}

// E4M3 codes of four binary32 values with the hardware converter (round to
// nearest even). Every input here is below 464 in magnitude: dynamic scales
// bound it, static ones are clamped to +-448 first, so no saturation occurs.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Saturation to the largest finite E4M3 magnitude. Every y in (448, 464)
// rounds to 448 anyway, so clamping first leaves the rounding of in-range
// values unchanged and sends the rest to +-448.
__device__ __forceinline__ float sat448(float y) { return fminf(fmaxf(y, -448.0f), 448.0f); }

// True when the E4M3 rounding of y might differ from that of the exact
// quotient. With the E4M3 step of y's binade scaled to 1, y lies within 2^-14
// of a midpoint between neighbouring codes exactly when the low 20 bits of its
// binary32 mantissa are within 64 of 0x80000 (the scaled magnitude is
// 8 + (mantissa bits) / 2^20). Magnitudes below 2^-6 (subnormal codes, other
// midpoints) always take the exact path.
__device__ __forceinline__ bool fp8_near_tie(float y) {
  const uint32_t low = __float_as_uint(y) & 0xFFFFFu;
  return (low - 0x80000u + 64u) < 128u || fabsf(y) < 0.015625f;
}

// Eight 16-bit inputs (one 16-byte piece) as floats, exactly.
template <bool BF16>
__device__ __forceinline__ void unpack8(const u32x4& w, float* x) {
  unpack2<BF16>(w.x, x[0], x[1]);
  unpack2<BF16>(w.y, x[2], x[3]);
  unpack2<BF16>(w.z, x[4], x[5]);
  unpack2<BF16>(w.w, x[6], x[7]);
}

// One row of d 16-bit inputs to byte codes and its scale. The four lanes of
// a quad share the row: lane k holds elements 32 u + 8 k + e (u < d/32,
// e < 8) as d/32 16-byte pieces `w`, writes their codes to `codes` (the
// row's first byte) and, for k = 0, the scale to `*scale`; nothing is
// written unless `live`. STATIC takes `st_scale` as the scale and saturates
// the codes; otherwise the scale comes from the quad's absmax.
template <int CODE, int D, bool BF16, bool STATIC>
__device__ __forceinline__ void code_row8(const u32x4* w, int k, float st_scale, uint8_t* codes,
                                          float* scale, bool live) {
  constexpr int NV = D / 32;
  float x[NV][8];
#pragma unroll
  for (int u = 0; u < NV; ++u) unpack8<BF16>(w[u], x[u]);
  constexpr float kQmax = CODE == KVQ_CODE_INT8 ? 127.0f : 448.0f;
  float s;
  if constexpr (STATIC) {
    s = st_scale;
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < NV; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[u][e]));
    amax = quad_max(amax);
    s = amax == 0.0f ? 1.0f : div_rn(amax, kQmax);
  }
  const float inv = __builtin_amdgcn_rcpf(s);   // within 1 ulp of 1/s
  uint32_t o[NV][2];
  // an element near a rounding boundary (rare) takes the exact quotient on
  // its own, so a wave redoes only the elements some lane needs
  const bool unsafe = recip_unsafe(s);
  if constexpr (CODE == KVQ_CODE_INT8) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      int c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = x[u][e] * inv;
        float q = rne(y);
        if (unsafe || near_half(y, q)) q = rne(div_rn(x[u][e], s));
        c[e] = (int)fminf(fmaxf(q, -127.0f), 127.0f);
      }
      o[u][0] = pack_bytes(c[0], c[1], c[2], c[3]);
      o[u][1] = pack_bytes(c[4], c[5], c[6], c[7]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = x[u][e] * inv;
        if (unsafe || fp8_near_tie(y[e])) y[e] = div_rn(x[u][e], s);
        if constexpr (STATIC) y[e] = sat448(y[e]);
      }
      o[u][0] = fp8x4(y[0], y[1], y[2], y[3]);
      o[u][1] = fp8x4(y[4], y[5], y[6], y[7]);
    }
  }
  if (live) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      u32x2 v2 = {o[u][0], o[u][1]};
      *reinterpret_cast<u32x2*>(codes + 32 * u + 8 * k) = v2;
    }
    if (k == 0) *scale = s;
  }
}

}  // namespace
}  // namespace kvq
