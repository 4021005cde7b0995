// kvq_attn_tiles.h -- the attention tile machinery shared by decode
// (kvq_decode.hip) and multi-query attention (kvq_prefill.hip): cache-tile
// loads, exact code-to-fp16 conversion, the 16-token MFMA tile step with
// online softmax, per-channel query folding, and small wave reductions.
// Device code for gfx950, internal to the library.
#pragma once

#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const uint16_t* q;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_scale;
  const float* v_scale;
  const uint8_t* k_zero;
  const uint8_t* v_zero;
  const uint16_t* k_stage;  // per-channel keys: raw rows of partial blocks
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;
  float* ws_ml;
  int64_t num_blocks;
  int32_t q_bf16;
  int32_t stage_bf16;
  int32_t Hq;
  int32_t H;
  int32_t G;
  int32_t max_blocks;
  int32_t batch;
  int32_t max_len;       // every context length is cut to this
  int32_t split_blocks;  // 0: planned from the lengths
  float sm_log2;  // sm_scale * log2(e)
  // Append before attending (kvq_append_decode_attention): row b of new_k /
  // new_v (16-bit, H*d per token, strides in elements) is coded into position
  // context_lens[b] - 1 of sequence b, through the writable views of the
  // planes. new_k == nullptr: decode only.
  const uint16_t* new_k = nullptr;
  const uint16_t* new_v = nullptr;
  int64_t new_k_stride = 0;
  int64_t new_v_stride = 0;
  uint8_t* k_codes_w = nullptr;
  uint8_t* v_codes_w = nullptr;
  float* k_scale_w = nullptr;
  float* v_scale_w = nullptr;
  int32_t new_bf16 = 0;
};

// Max and sum of a float over the wave by the same DPP pattern, with -inf
// (max) or 0 (sum) in lanes that have no source; the result is lane 63's.
template <bool MAX>
__device__ __forceinline__ float wave_reduce_f(float x) {
  const int idle = MAX ? __float_as_int(-INFINITY) : 0;
  auto step = [&](float v, float w) { return MAX ? fmaxf(v, w) : v + w; };
#define KVQ_DPP_STEP(ctrl, rmask)                                                       \
  x = step(x, __int_as_float(__builtin_amdgcn_update_dpp(idle, __float_as_int(x), ctrl, \
                                                          rmask, 0xF, false)))
  KVQ_DPP_STEP(0x111, 0xF);
  KVQ_DPP_STEP(0x112, 0xF);
  KVQ_DPP_STEP(0x114, 0xF);
  KVQ_DPP_STEP(0x118, 0xF);
  KVQ_DPP_STEP(0x142, 0xA);
  KVQ_DPP_STEP(0x143, 0xC);
#undef KVQ_DPP_STEP
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
}

template <int D, int BS>
struct Tile8 {
  static constexpr int NT = BS / 16;     // 16-token MFMA tiles per block
  static constexpr int KV = D / 64;      // 16-byte key vectors per lane per tile
  static constexpr int VB = D / 16;      // value bytes per token per lane
  u32x4 k[NT][KV];
  uint32_t v[NT][4][VB / 4];             // [tile][token i][dword]
  float4v sk[NT];
  float4v sv[NT];
  float kc[D / 64];                      // per-channel key scales, lane's slice
};

// A load of code bytes that are read once: with NT the load is
// non-temporal (the `nt` cache policy), so the streamed codes do not displace
// what is reused from the caches (scales shared by neighbouring heads, block
// tables, queries, the other half of a key line).
template <bool NT, class T>
__device__ __forceinline__ T load_codes(const T* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// KCH: keys carry one scale per channel for the whole block
// (CHANNEL_BLOCK_SYM), loaded as D/64 consecutive floats per lane. NT: value
// code loads are non-temporal (see load_codes). Each value load instruction
// reads whole 128-byte rows; each key load reads half of every line it
// touches and the lane's next load the other half, so key loads stay cached
// (made non-temporal too, the decode of the 70B and 8B shapes ran 2-5%
// slower than with values alone; values alone are 6-12% faster than neither).
template <int D, int BS, bool KCH, bool NT = false>
__device__ __forceinline__ void load_tile8(Tile8<D, BS>& t, const DecodeArgs& a,
                                           int64_t bh, int lane) {
  const int r = lane & 15, j = lane >> 4;
  const uint8_t* kb = a.k_codes + bh * BS * D;
  const uint8_t* vb = a.v_codes + bh * BS * D;
#pragma unroll
  for (int nt = 0; nt < Tile8<D, BS>::NT; ++nt) {
    const uint8_t* kr = kb + (nt * 16 + r) * D + j * (D / 4);
#pragma unroll
    for (int u = 0; u < Tile8<D, BS>::KV; ++u)
      t.k[nt][u] = *reinterpret_cast<const u32x4*>(kr + 16 * u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint8_t* vr = vb + (nt * 16 + 4 * j + i) * D + r * (D / 16);
      if constexpr (D == 128) {
        u32x2 w = load_codes<NT>(reinterpret_cast<const u32x2*>(vr));
        t.v[nt][i][0] = w.x;
        t.v[nt][i][1] = w.y;
      } else {
        t.v[nt][i][0] = load_codes<NT>(reinterpret_cast<const uint32_t*>(vr));
      }
    }
    if constexpr (!KCH)
      t.sk[nt] = *reinterpret_cast<const float4v*>(a.k_scale + bh * BS + nt * 16 + 4 * j);
    t.sv[nt] = *reinterpret_cast<const float4v*>(a.v_scale + bh * BS + nt * 16 + 4 * j);
  }
  if constexpr (KCH) {
    const float* kc = a.k_scale + bh * D + lane * (D / 64);
    if constexpr (D == 128) {
      const float2 w = *reinterpret_cast<const float2*>(kc);
      t.kc[0] = w.x;
      t.kc[1] = w.y;
    } else {
      t.kc[0] = *kc;
    }
  }
}

// 8 code bytes (two dwords) to 8 fp16 values, in byte order.
template <int CODE>
__device__ __forceinline__ half8v codes8_to_h8(uint32_t lo, uint32_t hi) {
  half2v p0, p1, p2, p3;
  if constexpr (CODE == KVQ_CODE_FP8_E4M3) {
    p0 = fp8x2_to_h2<false>(lo);
    p1 = fp8x2_to_h2<true>(lo);
    p2 = fp8x2_to_h2<false>(hi);
    p3 = fp8x2_to_h2<true>(hi);
  } else {
    const uint32_t xl = lo ^ 0x80808080u, xh = hi ^ 0x80808080u;
    p0 = i8x2_to_h2(xl, 0x04010400u);
    p1 = i8x2_to_h2(xl, 0x04030402u);
    p2 = i8x2_to_h2(xh, 0x04010400u);
    p3 = i8x2_to_h2(xh, 0x04030402u);
  }
  half8v o;
  o[0] = p0[0]; o[1] = p0[1]; o[2] = p1[0]; o[3] = p1[1];
  o[4] = p2[0]; o[5] = p2[1]; o[6] = p3[0]; o[7] = p3[1];
  return o;
}

// Value operand of MFMA c: bytes c of the lane's four token words, as fp16.
// a01 = [t0.bX, t1.bX, t0.bY, t1.bY], a23 likewise for tokens 2, 3.
template <int CODE, bool HI>
__device__ __forceinline__ half4v vpair_to_h4(uint32_t a01, uint32_t a23) {
  half2v x, y;
  if constexpr (CODE == KVQ_CODE_FP8_E4M3) {
    x = fp8x2_to_h2<HI>(a01);
    y = fp8x2_to_h2<HI>(a23);
  } else {
    const uint32_t sel = HI ? 0x04030402u : 0x04010400u;
    x = i8x2_to_h2(a01 ^ 0x80808080u, sel);
    y = i8x2_to_h2(a23 ^ 0x80808080u, sel);
  }
  half4v o;
  o[0] = x[0]; o[1] = x[1]; o[2] = y[0]; o[3] = y[1];
  return o;
}

// max over the four lanes {l, l^16, l^32, l^48} (one head column), with
// the gfx950 lane-swap instructions instead of LDS permutes. The NaN-
// propagating maximum is one v_maximum3_f32 per level; the IEEE maxNum
// would first quiet both swapped operands (two more instructions per
// level). The callers' masked entries are -inf, never NaN.
__device__ __forceinline__ float colmax4(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(p[0]), __uint_as_float(p[1]));
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
// colmax4 of two values at once. The first swap trades a's upper 32 lanes
// for b's lower 32, so one maximum leaves a reduced over the lane pairs
// {l, l^32} in lanes 0..31 and b in lanes 32..63; the row swap finishes
// both; a last swap gives every lane both results. Seven instructions
// instead of two colmax4 (twelve, with their copies).
__device__ __forceinline__ void colmax4x2(float a, float b, float& ma, float& mb) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  float x = __builtin_elementwise_maximum(__uint_as_float(p[0]), __uint_as_float(p[1]));
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(q[0]), __uint_as_float(q[1]));
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  ma = __uint_as_float(t[0]);
  mb = __uint_as_float(t[1]);
}
__device__ __forceinline__ float colsum4(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <int D>
struct SoftmaxState {
  float m;                 // running max (log2 units) of head r
  float l;                 // this lane's part of the running sum
  float4v acc[D / 16];     // O^T accumulators
};

// Raw 16-bit rows (the passthrough cache, staged per-channel key rows) enter
// the MFMA in their own format: fp16 rows through the f16 instructions, bf16
// rows through the bf16 ones, so that no element is rounded or leaves its
// range on the way. The other operand (the power-of-two-scaled query, the
// softmax weights) is fp32 and goes to the bf16 instructions as a pair
// hi + lo of bf16 values: hi = x rounded to bf16, lo = (x - hi) rounded to
// bf16 (x - hi is exact in fp32), which holds x to a relative 2^-17.
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void bf16_split8(const float* x, half8v& hi, half8v& lo) {
  bf16x8v h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (__bf16)x[e];
    l[e] = (__bf16)(x[e] - (float)h[e]);
  }
  hi = __builtin_bit_cast(half8v, h);
  lo = __builtin_bit_cast(half8v, l);
}

// S += rows (eight raw 16-bit elements per lane) x query. bf16: the query is
// the pair qhi + qlo of bf16_split8; fp16: qhi is the fp16 query.
__device__ __forceinline__ float4v raw_scores(const u32x4& rows, const half8v& qhi,
                                              const half8v& qlo, float4v S, bool bf16) {
  if (bf16) {
    const bf16x8v k = __builtin_bit_cast(bf16x8v, rows);
    S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, __builtin_bit_cast(bf16x8v, qhi), S, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, __builtin_bit_cast(bf16x8v, qlo), S, 0, 0,
                                                   0);
  }
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8v, rows), qhi, S, 0, 0, 0);
}

// Where the keys of a tile come from.
enum KeySource {
  kKeyTokenScale = 0,  // codes; the score takes the token's key scale
  kKeyChannel = 1,     // codes; per-channel scales are already in the query
  kKeyRaw = 2,         // raw staged rows, kraw[c] = elements of chunk c
};

// One 16-token tile: scores, online softmax, PV. TAIL handles a tile with
// masked tokens: the lane's column sees token t only if t < L and (t >= lo
// or t < sk) -- L its causal limit, lo the start of its window and sk the
// number of sink tokens (lo = 0: no window) -- and value codes of tokens at
// or past Lv (the rows that hold data; Lv < 0 means L) are zeroed, since
// they may hold NaN bytes. In decode L is the length for every column; the
// columns of multi-query attention differ in L and lo while sharing the
// value operand, so only rows past the data are zeroed.
template <int CODE, int D, int BS, bool TAIL, int KSRC = kKeyTokenScale>
__device__ __forceinline__ void tile_step(const Tile8<D, BS>& t, int nt, int pos0, int L,
                                          const half8v* qop, float cscore, int j,
                                          SoftmaxState<D>& st, const u32x4* kraw = nullptr,
                                          bool raw_bf16 = false, const half8v* qlo = nullptr,
                                          int Lv = -1, int lo = 0, int sk = 0) {
  constexpr int NCH = D / 32;
  constexpr int NPV = D / 16;
  const int Ld = Lv < 0 ? L : Lv;
  float4v S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if constexpr (KSRC == kKeyRaw) {   // bf16 rows: qop/qlo are the bf16 pair
      S = raw_scores(kraw[c], qop[c], raw_bf16 ? qlo[c] : qop[c], S, raw_bf16);
      continue;
    }
    const u32x4& kw = t.k[nt][c / 2];
    const uint32_t lo = (c & 1) ? kw.z : kw.x;
    const uint32_t hi = (c & 1) ? kw.w : kw.y;
    const half8v kop = codes8_to_h8<CODE>(lo, hi);
    S = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[c], S, 0, 0, 0);
    if constexpr (KSRC == kKeyChannel)  // low half of the split query
      S = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qlo[c], S, 0, 0, 0);
  }
  bool ok[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int tk = pos0 + 4 * j + e;
    ok[e] = !TAIL || (tk < L && (tk >= lo || tk < sk));
  }
  float s[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s[e] = KSRC == kKeyTokenScale ? S[e] * t.sk[nt][e] * cscore : S[e] * cscore;
    if (TAIL && !ok[e]) s[e] = -INFINITY;
  }
  const float mt = colmax4(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
  const float mn = fmaxf(st.m, mt);
  const float msafe = mn == -INFINITY ? 0.0f : mn;
  if (__any(mn > st.m)) {  // a running max grew: rescale (rare after warm-up)
    const float alpha = __builtin_amdgcn_exp2f(st.m - msafe);
    st.l *= alpha;
#pragma unroll
    for (int c = 0; c < NPV; ++c) st.acc[c] *= alpha;
  }
  st.m = mn;
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(s[e] - msafe);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
  half4v pop;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float pv = p[e] * t.sv[nt][e];
    if (TAIL && !ok[e]) pv = 0.0f;
    pop[e] = (half_t)pv;
  }
#pragma unroll
  for (int w = 0; w < D / 64; ++w) {
    uint32_t t0 = t.v[nt][0][w], t1 = t.v[nt][1][w];
    uint32_t t2 = t.v[nt][2][w], t3 = t.v[nt][3][w];
    if (TAIL) {  // zero the codes of rows past the data (E4M3 NaN bytes)
      const int pv0 = pos0 + 4 * j;
      t0 = pv0 + 0 < Ld ? t0 : 0u;
      t1 = pv0 + 1 < Ld ? t1 : 0u;
      t2 = pv0 + 2 < Ld ? t2 : 0u;
      t3 = pv0 + 3 < Ld ? t3 : 0u;
    }
    // [t0.b0 t1.b0 t0.b1 t1.b1], [t0.b2 t1.b2 t0.b3 t1.b3]
    const uint32_t a01l = __builtin_amdgcn_perm(t1, t0, 0x05010400u);
    const uint32_t a01h = __builtin_amdgcn_perm(t1, t0, 0x07030602u);
    const uint32_t a23l = __builtin_amdgcn_perm(t3, t2, 0x05010400u);
    const uint32_t a23h = __builtin_amdgcn_perm(t3, t2, 0x07030602u);
    const int c0 = 4 * w;
    st.acc[c0 + 0] = __builtin_amdgcn_mfma_f32_16x16x16f16(vpair_to_h4<CODE, false>(a01l, a23l), pop, st.acc[c0 + 0], 0, 0, 0);
    st.acc[c0 + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(vpair_to_h4<CODE, true>(a01l, a23l), pop, st.acc[c0 + 1], 0, 0, 0);
    st.acc[c0 + 2] = __builtin_amdgcn_mfma_f32_16x16x16f16(vpair_to_h4<CODE, false>(a01h, a23h), pop, st.acc[c0 + 2], 0, 0, 0);
    st.acc[c0 + 3] = __builtin_amdgcn_mfma_f32_16x16x16f16(vpair_to_h4<CODE, true>(a01h, a23h), pop, st.acc[c0 + 3], 0, 0, 0);
  }
}

// Two whole 16-token tiles of 8-bit codes with per-token scales (tile na of
// ta, then tile nb of tb: consecutive tokens of one block, or the tiles of
// two consecutive blocks) in one step: their scores, one softmax update for
// the 32 tokens, and the PV products on 16x16x32 MFMAs whose contraction
// runs over both tiles (k = 8 j + 4 T + e for tile T, token 4 j + e; the
// value and probability operands are each tile's 16x16x16 operands side by
// side), half the MFMAs and one cross-lane max and rescale test per 32
// tokens instead of per 16.
template <int CODE, int D, int BS>
__device__ __forceinline__ void tile_pair_step(const Tile8<D, BS>& ta, int na,
                                               const Tile8<D, BS>& tb, int nb,
                                               const half8v* qop, float cscore,
                                               SoftmaxState<D>& st) {
  constexpr int NCH = D / 32;
  constexpr int NPV = D / 16;
  float4v Sa = {0.0f, 0.0f, 0.0f, 0.0f}, Sb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const u32x4& ka = ta.k[na][c / 2];
    const u32x4& kb = tb.k[nb][c / 2];
    const half8v opa = codes8_to_h8<CODE>((c & 1) ? ka.z : ka.x, (c & 1) ? ka.w : ka.y);
    const half8v opb = codes8_to_h8<CODE>((c & 1) ? kb.z : kb.x, (c & 1) ? kb.w : kb.y);
    Sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(opa, qop[c], Sa, 0, 0, 0);
    Sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(opb, qop[c], Sb, 0, 0, 0);
  }
  float s[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s[e] = Sa[e] * ta.sk[na][e] * cscore;
    s[4 + e] = Sb[e] * tb.sk[nb][e] * cscore;
  }
  const float mt = colmax4(fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                                 fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]))));
  const float mn = fmaxf(st.m, mt);
  const float msafe = mn == -INFINITY ? 0.0f : mn;
  if (__any(mn > st.m)) {  // a running max grew: rescale (rare after warm-up)
    const float alpha = __builtin_amdgcn_exp2f(st.m - msafe);
    st.l *= alpha;
#pragma unroll
    for (int c = 0; c < NPV; ++c) st.acc[c] *= alpha;
  }
  st.m = mn;
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(s[e] - msafe);
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  half8v pop;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pop[e] = (half_t)(p[e] * ta.sv[na][e]);
    pop[4 + e] = (half_t)(p[4 + e] * tb.sv[nb][e]);
  }
#pragma unroll
  for (int w = 0; w < D / 64; ++w) {
    const uint32_t a0 = ta.v[na][0][w], a1 = ta.v[na][1][w];
    const uint32_t a2 = ta.v[na][2][w], a3 = ta.v[na][3][w];
    const uint32_t b0 = tb.v[nb][0][w], b1 = tb.v[nb][1][w];
    const uint32_t b2 = tb.v[nb][2][w], b3 = tb.v[nb][3][w];
    // per tile: [t0.b0 t1.b0 t0.b1 t1.b1], [t0.b2 t1.b2 t0.b3 t1.b3]
    const uint32_t a01l = __builtin_amdgcn_perm(a1, a0, 0x05010400u);
    const uint32_t a01h = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
    const uint32_t a23l = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
    const uint32_t a23h = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
    const uint32_t b01l = __builtin_amdgcn_perm(b1, b0, 0x05010400u);
    const uint32_t b01h = __builtin_amdgcn_perm(b1, b0, 0x07030602u);
    const uint32_t b23l = __builtin_amdgcn_perm(b3, b2, 0x05010400u);
    const uint32_t b23h = __builtin_amdgcn_perm(b3, b2, 0x07030602u);
    auto cat = [](half4v x, half4v y) {
      return (half8v){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    };
    const int c0 = 4 * w;
    st.acc[c0 + 0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        cat(vpair_to_h4<CODE, false>(a01l, a23l), vpair_to_h4<CODE, false>(b01l, b23l)), pop,
        st.acc[c0 + 0], 0, 0, 0);
    st.acc[c0 + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        cat(vpair_to_h4<CODE, true>(a01l, a23l), vpair_to_h4<CODE, true>(b01l, b23l)), pop,
        st.acc[c0 + 1], 0, 0, 0);
    st.acc[c0 + 2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        cat(vpair_to_h4<CODE, false>(a01h, a23h), vpair_to_h4<CODE, false>(b01h, b23h)), pop,
        st.acc[c0 + 2], 0, 0, 0);
    st.acc[c0 + 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        cat(vpair_to_h4<CODE, true>(a01h, a23h), vpair_to_h4<CODE, true>(b01h, b23h)), pop,
        st.acc[c0 + 3], 0, 0, 0);
  }
}

// A block whose BS tokens all lie before the sequence end.
template <int CODE, int D, int BS, int KSRC = kKeyTokenScale>
__device__ __forceinline__ void full_block_step(const Tile8<D, BS>& t, int i, int L,
                                                const half8v* qop, float cscore, int j,
                                                SoftmaxState<D>& st,
                                                const half8v* qlo = nullptr) {
#pragma unroll
  for (int nt = 0; nt < BS / 16; ++nt)
    tile_step<CODE, D, BS, false, KSRC>(t, nt, i * BS + nt * 16, L, qop, cscore, j, st,
                                        nullptr, false, qlo);
}

// Per-channel keys: the block's scales fold into the query,
// q'[c] = (q[c] 2^-e) sK[c] in fp32, which enters the MFMA as the sum of two
// fp16 operands, hi = fp16(q') and lo = fp16(q' - hi): one fp16 rounding of
// q' would cost 2^-12 relative per term, as much as the whole error budget
// when a few outlier channels dominate the score. Each lane holds D/64
// scales of the block; the wave trades them through its own LDS slice `x`
// (D floats) so that lane (r, j) gets channels [j D/4, (j+1) D/4). The fences
// only keep the compiler from moving LDS accesses across them: a wave's LDS
// operations complete in issue order.
template <int D, int BS>
__device__ __forceinline__ void channel_query(const Tile8<D, BS>& t, float* x, const float* qs,
                                              int lane, half8v* qop, half8v* qlo) {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  if constexpr (D == 128)
    *reinterpret_cast<float2*>(x + 2 * lane) = make_float2(t.kc[0], t.kc[1]);
  else
    x[lane] = t.kc[0];
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const float* src = x + (lane >> 4) * (D / 4);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const float4v s0 = *reinterpret_cast<const float4v*>(src + 8 * c);
    const float4v s1 = *reinterpret_cast<const float4v*>(src + 8 * c + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // hi and lo each in one mixed-precision FMA from the exact product
      const float q = qs[8 * c + e], sc = e < 4 ? s0[e] : s1[e - 4];
      const half_t hi = (half_t)__builtin_fmaf(q, sc, 0.0f);
      qop[c][e] = hi;
      qlo[c][e] = (half_t)__builtin_fmaf(q, sc, -(float)hi);
    }
  }
}

// The sequence's last block when it is only partly filled. With KRAW the
// keys come from the staged rows kraw[tile][chunk] instead of the codes.
template <int CODE, int D, int BS, bool KRAW = false>
__device__ __forceinline__ void last_block_step(const Tile8<D, BS>& t, int i, int L,
                                                const half8v* qop, float cscore, int j,
                                                SoftmaxState<D>& st,
                                                const u32x4 (*kraw)[D / 32] = nullptr,
                                                bool raw_bf16 = false,
                                                const half8v* qlo = nullptr) {
  constexpr int KS = KRAW ? kKeyRaw : kKeyTokenScale;
#pragma unroll
  for (int nt = 0; nt < BS / 16; ++nt) {
    const int pos0 = i * BS + nt * 16;
    const u32x4* kr = KRAW ? kraw[nt] : nullptr;
    if (pos0 + 16 <= L)
      tile_step<CODE, D, BS, false, KS>(t, nt, pos0, L, qop, cscore, j, st, kr, raw_bf16, qlo);
    else if (pos0 < L)
      tile_step<CODE, D, BS, true, KS>(t, nt, pos0, L, qop, cscore, j, st, kr, raw_bf16, qlo);
  }
}

template <bool BF16, int D>
__device__ __forceinline__ void load_query(const uint16_t* qp, float* qf) {
#pragma unroll
  for (int u = 0; u < D / 32; ++u) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(qp + 8 * u);
    unpack2<BF16>(w.x, qf[8 * u + 0], qf[8 * u + 1]);
    unpack2<BF16>(w.y, qf[8 * u + 2], qf[8 * u + 3]);
    unpack2<BF16>(w.z, qf[8 * u + 4], qf[8 * u + 5]);
    unpack2<BF16>(w.w, qf[8 * u + 6], qf[8 * u + 7]);
  }
}

// ---------------------------------------------------------------------------
// 16-bit passthrough (KVQ_CODE_NONE16): rows hold the source values and
// enter both MFMAs in their own format, as the staged rows above do. Keys:
// lane (r, j) holds elements [j d/4, (j+1) d/4) of token r. Values: lane
// (r, j) loads elements [r d/16, (r+1) d/16) of tokens 4j..4j+3, and the
// operand of PV MFMA c is element c of those four tokens -- the same output
// mapping as the 8-bit codes. bf16 rows take two MFMAs per step (the hi and
// lo halves of the query or of the weights).
// ---------------------------------------------------------------------------
template <int D, int BS>
struct TileRaw {
  static constexpr int NT = BS / 16;
  static constexpr int NCH = D / 32;   // 16-byte key vectors per lane per tile
  static constexpr int VW = D / 32;    // 32-bit value words per token per lane
  u32x4 k[NT][NCH];
  uint32_t v[NT][4][VW];               // [tile][token i][word]
};

// NT: value loads are non-temporal, as for load_tile8.
template <int D, int BS, bool NT = false>
__device__ __forceinline__ void load_tile_raw(TileRaw<D, BS>& t, const DecodeArgs& a,
                                              int64_t bh, int lane) {
  const int r = lane & 15, j = lane >> 4;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k_codes) + bh * BS * D;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.v_codes) + bh * BS * D;
#pragma unroll
  for (int nt = 0; nt < TileRaw<D, BS>::NT; ++nt) {
    const uint16_t* kr = kb + (nt * 16 + r) * D + j * (D / 4);
#pragma unroll
    for (int c = 0; c < TileRaw<D, BS>::NCH; ++c)
      t.k[nt][c] = *reinterpret_cast<const u32x4*>(kr + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t* vr = vb + (nt * 16 + 4 * j + i) * D + r * (D / 16);
      if constexpr (D == 128) {
        const u32x4 w = load_codes<NT>(reinterpret_cast<const u32x4*>(vr));
        t.v[nt][i][0] = w.x; t.v[nt][i][1] = w.y; t.v[nt][i][2] = w.z; t.v[nt][i][3] = w.w;
      } else {
        const u32x2 w = load_codes<NT>(reinterpret_cast<const u32x2*>(vr));
        t.v[nt][i][0] = w.x; t.v[nt][i][1] = w.y;
      }
    }
  }
}

// Element c (0 or 1 of word w) of four tokens' value words, as the four
// 16-bit elements of a PV operand (fp16 or bf16 alike).
__device__ __forceinline__ u32x2 raw_vop(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                         bool hi) {
  const uint32_t sel = hi ? 0x07060302u : 0x05040100u;
  return (u32x2){__builtin_amdgcn_perm(w1, w0, sel), __builtin_amdgcn_perm(w3, w2, sel)};
}

template <int D, int BS, bool TAIL>
__device__ __forceinline__ void tile_step_raw(const TileRaw<D, BS>& t, int nt, int pos0, int L,
                                              const half8v* qop, const half8v* qlo, float cscore,
                                              int j, SoftmaxState<D>& st, bool bf16, int Lv = -1,
                                              int lo = 0, int sk = 0) {
  constexpr int NCH = D / 32;
  constexpr int NPV = D / 16;
  const int Ld = Lv < 0 ? L : Lv;   // as in tile_step
  float4v S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < NCH; ++c) S = raw_scores(t.k[nt][c], qop[c], bf16 ? qlo[c] : qop[c], S, bf16);
  bool ok[4];   // as in tile_step
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int tk = pos0 + 4 * j + e;
    ok[e] = !TAIL || (tk < L && (tk >= lo || tk < sk));
  }
  float s[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) s[e] = (TAIL && !ok[e]) ? -INFINITY : S[e] * cscore;
  const float mt = colmax4(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
  const float mn = fmaxf(st.m, mt);
  const float msafe = mn == -INFINITY ? 0.0f : mn;
  if (__any(mn > st.m)) {
    const float alpha = __builtin_amdgcn_exp2f(st.m - msafe);
    st.l *= alpha;
#pragma unroll
    for (int c = 0; c < NPV; ++c) st.acc[c] *= alpha;
  }
  st.m = mn;
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = (TAIL && !ok[e]) ? 0.0f : __builtin_amdgcn_exp2f(s[e] - msafe);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
  // weights: fp16 for fp16 rows, the bf16 pair hi + lo for bf16 rows
  half4v pop;
  short4v phi, plo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (bf16) {
      const __bf16 h = (__bf16)p[e];
      phi[e] = __builtin_bit_cast(short, h);
      plo[e] = __builtin_bit_cast(short, (__bf16)(p[e] - (float)h));
    } else {
      pop[e] = (half_t)p[e];
    }
  }
#pragma unroll
  for (int c = 0; c < NPV; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = t.v[nt][i][c / 2];
      if (TAIL && pos0 + 4 * j + i >= Ld) w[i] = 0u;   // rows past the data may hold NaN
    }
    const u32x2 vw = raw_vop(w[0], w[1], w[2], w[3], c & 1);
    if (bf16) {
      const short4v vop = __builtin_bit_cast(short4v, vw);
      st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, phi, st.acc[c], 0, 0, 0);
      st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, plo, st.acc[c], 0, 0, 0);
    } else {
      st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4v, vw), pop,
                                                        st.acc[c], 0, 0, 0);
    }
  }
}

// Tile-type dispatch for the block streaming below.
template <int D, int BS, bool KCH, bool NT = false>
__device__ __forceinline__ void load_tile(Tile8<D, BS>& t, const DecodeArgs& a, int64_t bh,
                                          int lane) {
  load_tile8<D, BS, KCH, NT>(t, a, bh, lane);
}
template <int D, int BS, bool KCH, bool NT = false>
__device__ __forceinline__ void load_tile(TileRaw<D, BS>& t, const DecodeArgs& a, int64_t bh,
                                          int lane) {
  load_tile_raw<D, BS, NT>(t, a, bh, lane);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// waves per decode / multi-query workgroup
constexpr int kNW = kDecodeWaves;
// Query heads (one wave each) per workgroup of the cross-split merges: up
// to kReduceHeads when the merges number kReduceGroupWaves or more (one-wave
// workgroups by the ten thousand cost dispatch time), else one, which
// spreads a small merge over more CUs.
constexpr int kReduceHeads = 4;
constexpr int64_t kReduceGroupWaves = 4096;
inline int reduce_heads_per_group(int64_t waves) {
  return waves >= kReduceGroupWaves ? kReduceHeads : 1;
}

}  // namespace
}  // namespace kvq
