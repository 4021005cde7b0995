// kvq_int4_tiles.h -- the 4-bit tile machinery shared by decode
// (kvq_decode.hip) and multi-query attention (kvq_prefill.hip): the tile's
// buffer loads, nibble-to-fp16 conversion, row-broadcast scales, and the
// single-tile and two-tile MFMA steps with online softmax. Device code for
// gfx950, internal to the library.
#pragma once

#include <type_traits>

#include "kvq_attn_tiles.h"

namespace kvq {
namespace {

// ---------------------------------------------------------------------------
// 4-bit codes. Row layout (see the header): element 32 i + 2 r + t of a row
// sits in byte n r + i (n = d/32 slices), nibble t. Lane (r, j) feeds the
// score MFMA for token r with key bytes [4 n j, 4 n j + 4 n), i.e. pairs
// r' = 4j .. 4j+3 of every slice: chunk c of the contraction is slice c, so
// that per-slice (group) scales apply to separate accumulators. For P.V, MFMA
// m = 2 i + t covers output rows d = 32 i + 2 r + t and lane (r, j) needs byte
// n r + i of its four tokens.
// ---------------------------------------------------------------------------
template <int D, int MODE>
struct Tile4 {
  static constexpr int NS = D / 32;
  static constexpr int SG = MODE == KVQ_SCALE_GROUP_ASYM ? NS : 1;
  uint32_t k[NS];      // key bytes of token r for pairs 4j..4j+3
  uint32_t v[4];       // value bytes n r .. n r + n - 1 of tokens 4j + e
  // The 4 SG scales of tokens 4j..4j+3 ([token][group]) are spread over the
  // 16 lanes of row j: lane r holds entry r mod 4 SG, read by the others
  // through a row broadcast.
  float sk;            // key scale
  float sv;            // value scale
  uint32_t zk;         // key zero points of token r, byte c = group c
  uint32_t zv[NS];     // value zero points of tokens 4j..4j+3 ([token][group] bytes)
};

// x, known to be equal in every lane, held in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Byte offsets of a lane's loads within a tile's rows, fixed for the wave:
// each load is a wave-uniform base (scalar registers) plus one of these, so
// the loop spends no vector instructions on addresses.
struct Lane4 {
  uint32_t k;   // key bytes [j n, (j + 1) n) of token r, n = d / 8
  uint32_t v;   // value bytes of token 4j (+ e rows for token 4j + e) at r d / 32
  uint32_t s;   // scale entry r mod 4 SG of tokens 4j..4j+3
  uint32_t zk;  // key zero points of token r
  uint32_t zv;  // value zero points of tokens 4j..4j+3
};
template <int D, int MODE>
__device__ __forceinline__ Lane4 lane4_offsets(int lane) {
  constexpr int NS = D / 32;
  constexpr int RB = D / 2;  // bytes per row
  constexpr int SG = Tile4<D, MODE>::SG;
  const int r = lane & 15, j = lane >> 4;
  Lane4 o;
  o.k = (uint32_t)(r * RB + j * (RB / 4));
  o.v = (uint32_t)(4 * j * RB + r * (RB / 16));
  o.s = (uint32_t)(4 * (4 * j * SG + (r & (4 * SG - 1))));
  o.zk = (uint32_t)(r * NS);
  o.zv = (uint32_t)(4 * j * NS);
  return o;
}

// Buffer resource over `base`: raw (untyped) loads at 32-bit byte offsets;
// the record count only bounds the offsets, which stay within a tile.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

template <int D, int BS, int MODE>
__device__ __forceinline__ void load_tile4(Tile4<D, MODE>& t, const DecodeArgs& a, int64_t bh,
                                           int nt, const Lane4& o) {
  constexpr int NS = D / 32;
  constexpr int RB = D / 2;  // bytes per row
  constexpr int SG = Tile4<D, MODE>::SG;
  // first token of the tile: wave-uniform, kept in scalar registers so that
  // each plane's buffer resource is scalar and every load is a buffer load
  // at the lane's fixed 32-bit offset
  const int64_t row0 = uniform64(bh * BS + nt * 16);
  const __amdgpu_buffer_rsrc_t kr = tile_rsrc(a.k_codes + row0 * RB);
  const __amdgpu_buffer_rsrc_t vr = tile_rsrc(a.v_codes + row0 * RB);
  if constexpr (NS == 4) {
    const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, o.k, 0, 0));
    t.k[0] = w.x; t.k[1] = w.y; t.k[2] = w.z; t.k[3] = w.w;
  } else {
    const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(kr, o.k, 0, 0));
    t.k[0] = w.x; t.k[1] = w.y;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (NS == 4)
      t.v[e] = __builtin_amdgcn_raw_buffer_load_b32(vr, o.v + e * RB, 0, 0);
    else
      t.v[e] = __builtin_amdgcn_raw_buffer_load_b16(vr, o.v + e * RB, 0, 0);
  }
  t.sk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(tile_rsrc(a.k_scale + row0 * SG), o.s, 0, 0));
  t.sv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(tile_rsrc(a.v_scale + row0 * SG), o.s, 0, 0));
  if constexpr (MODE == KVQ_SCALE_GROUP_ASYM) {
    const __amdgpu_buffer_rsrc_t zkr = tile_rsrc(a.k_zero + row0 * NS);
    const __amdgpu_buffer_rsrc_t zvr = tile_rsrc(a.v_zero + row0 * NS);
    if constexpr (NS == 4) {
      t.zk = __builtin_amdgcn_raw_buffer_load_b32(zkr, o.zk, 0, 0);
      const u32x4 z = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(zvr, o.zv, 0, 0));
      t.zv[0] = z.x; t.zv[1] = z.y; t.zv[2] = z.z; t.zv[3] = z.w;
    } else {
      t.zk = __builtin_amdgcn_raw_buffer_load_b16(zkr, o.zk, 0, 0);
      const u32x2 z = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(zvr, o.zv, 0, 0));
      t.zv[0] = z.x; t.zv[1] = z.y;
    }
  } else {
    t.zk = 0;
#pragma unroll
    for (int u = 0; u < NS; ++u) t.zv[u] = 0;
  }
}

// Lane F of the caller's row of 16 lanes, for every lane of the row (DPP
// row_newbcast). The compiler folds the move into a following multiply.
template <int F>
__device__ __forceinline__ float row_bcast(float x) {
  static_assert(F >= 0 && F < 16, "a lane within the row");
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + F, 0xF, 0xF, true));
}

// Group combination of the 4-bit asymmetric scores: for each token e of the
// lane, v_e = sum over groups c of S_c[e] times the key scale of (token e,
// group c), which lane NS e + c of the row holds, as one multiply and NS - 1
// multiply-accumulates with a row-broadcast operand (the compiler folds a DPP
// move into a multiply but not into v_fmac). The block reads the score MFMA
// results and a DPP source, hazards the compiler does not track through
// inline assembly, so it opens with 24 wait states: more than an XDL result
// read needs after a 16-pass MFMA and more than a DPP read after a VALU write.
#define KVQ_ROWB(F) " row_newbcast:" #F " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
__device__ __forceinline__ void combine_groups(const float4v* S, float sk, float* v,
                                               std::integral_constant<int, 4>) {
  asm("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
      "v_mul_f32_dpp %0, %4, %5" KVQ_ROWB(0)
      "v_mul_f32_dpp %1, %4, %6" KVQ_ROWB(4)
      "v_mul_f32_dpp %2, %4, %7" KVQ_ROWB(8)
      "v_mul_f32_dpp %3, %4, %8" KVQ_ROWB(12)
      "v_fmac_f32_dpp %0, %4, %9" KVQ_ROWB(1)
      "v_fmac_f32_dpp %1, %4, %10" KVQ_ROWB(5)
      "v_fmac_f32_dpp %2, %4, %11" KVQ_ROWB(9)
      "v_fmac_f32_dpp %3, %4, %12" KVQ_ROWB(13)
      "v_fmac_f32_dpp %0, %4, %13" KVQ_ROWB(2)
      "v_fmac_f32_dpp %1, %4, %14" KVQ_ROWB(6)
      "v_fmac_f32_dpp %2, %4, %15" KVQ_ROWB(10)
      "v_fmac_f32_dpp %3, %4, %16" KVQ_ROWB(14)
      "v_fmac_f32_dpp %0, %4, %17" KVQ_ROWB(3)
      "v_fmac_f32_dpp %1, %4, %18" KVQ_ROWB(7)
      "v_fmac_f32_dpp %2, %4, %19" KVQ_ROWB(11)
      "v_fmac_f32_dpp %3, %4, %20" KVQ_ROWB(15)
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(sk), "v"(S[0][0]), "v"(S[0][1]), "v"(S[0][2]), "v"(S[0][3]),
        "v"(S[1][0]), "v"(S[1][1]), "v"(S[1][2]), "v"(S[1][3]),
        "v"(S[2][0]), "v"(S[2][1]), "v"(S[2][2]), "v"(S[2][3]),
        "v"(S[3][0]), "v"(S[3][1]), "v"(S[3][2]), "v"(S[3][3]));
}
__device__ __forceinline__ void combine_groups(const float4v* S, float sk, float* v,
                                               std::integral_constant<int, 2>) {
  asm("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
      "v_mul_f32_dpp %0, %4, %5" KVQ_ROWB(0)
      "v_mul_f32_dpp %1, %4, %6" KVQ_ROWB(2)
      "v_mul_f32_dpp %2, %4, %7" KVQ_ROWB(4)
      "v_mul_f32_dpp %3, %4, %8" KVQ_ROWB(6)
      "v_fmac_f32_dpp %0, %4, %9" KVQ_ROWB(1)
      "v_fmac_f32_dpp %1, %4, %10" KVQ_ROWB(3)
      "v_fmac_f32_dpp %2, %4, %11" KVQ_ROWB(5)
      "v_fmac_f32_dpp %3, %4, %12" KVQ_ROWB(7)
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(sk), "v"(S[0][0]), "v"(S[0][1]), "v"(S[0][2]), "v"(S[0][3]),
        "v"(S[1][0]), "v"(S[1][1]), "v"(S[1][2]), "v"(S[1][3]));
}
#undef KVQ_ROWB

// f(std::integral_constant<int, I>) for I = B .. E - 1, in order.
template <int B, int E, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Byte c of each of four words w0..w3 as one word [w0.bc, w1.bc, w2.bc, w3.bc]
// for c = 0..3 (a 4x4 byte transpose).
__device__ __forceinline__ void transpose4x4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                             uint32_t* g) {
  const uint32_t a0 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
  const uint32_t a1 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
  const uint32_t c0 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
  const uint32_t c1 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
  g[0] = __builtin_amdgcn_perm(c0, a0, 0x05040100u);
  g[1] = __builtin_amdgcn_perm(c0, a0, 0x07060302u);
  g[2] = __builtin_amdgcn_perm(c1, a1, 0x05040100u);
  g[3] = __builtin_amdgcn_perm(c1, a1, 0x07060302u);
}

// Nibble pairs of bytes 0 and 2 (shift 0 / 4) or 1 and 3 (shift 8 / 12) as
// two fp16 values 1024 + nibble.
// Nibbles SHIFT/4 and SHIFT/4 + 4 of g as the fp16 pair 1024 + q:
// ((g >> SHIFT) & m) | o with m = 0x000F000F and o = 0x64006400 held in
// registers by the caller, so that the and-or is one instruction (a VOP3
// encoding takes no two literal constants on gfx9).
template <int SHIFT>
__device__ __forceinline__ uint32_t nib2u(uint32_t g, uint32_t m, uint32_t o) {
  return ((g >> SHIFT) & m) | o;
}
template <int SHIFT>
__device__ __forceinline__ half2v nib2(uint32_t g, uint32_t m, uint32_t o) {
  return __builtin_bit_cast(half2v, nib2u<SHIFT>(g, m, o));
}

// Register-resident constants of the 4-bit conversions.
struct Nib4Consts {
  uint32_t m;    // 0x000F000F
  uint32_t o;    // 0x64006400
  uint32_t m64;  // 0x64646464, the fp16 exponent byte of 1024 + x for v_perm
  uint32_t e4;   // 0xE4E4E4E4, the same for -(1024 + x)
  uint32_t nb;   // 0xE408E408, the fp16 pair -(1024 + 8)
};
__device__ __forceinline__ Nib4Consts nib4_consts() {
  Nib4Consts k{0x000F000Fu, 0x64006400u, 0x64646464u, 0xE4E4E4E4u, 0xE408E408u};
  asm volatile("" : "+v"(k.m), "+v"(k.o), "+v"(k.m64), "+v"(k.e4), "+v"(k.nb));
  return k;
}

// Per-token scores of one tile before the column scale, for NC column sets
// (qop[cc], v[cc]) that share the key conversion: the score MFMAs (chunk c =
// slice c; one accumulator per 32-element group for asymmetric codes) and,
// for token 4j + e, the sum over groups c of S[c][e] times the key scale of
// (token e, group c), held by lane SG e + c of the row.
template <int D, int MODE, int NC>
__device__ __forceinline__ void tile4_scores(const Tile4<D, MODE>& t, const half8v (*qop)[D / 32],
                                             const Nib4Consts& kc, float (*v)[4]) {
  constexpr int NS = D / 32;
  constexpr bool ASYM = MODE == KVQ_SCALE_GROUP_ASYM;
  uint32_t g[4];
  if constexpr (NS == 4) {
    transpose4x4(t.k[0], t.k[1], t.k[2], t.k[3], g);
  } else {
    g[0] = __builtin_amdgcn_perm(t.k[1], t.k[0], 0x06040200u);
    g[1] = __builtin_amdgcn_perm(t.k[1], t.k[0], 0x07050301u);
  }
  float4v S[NC][ASYM ? NS : 1];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
#pragma unroll
    for (int c = 0; c < (ASYM ? NS : 1); ++c) S[cc][c] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    uint32_t gc = g[c];
    half2v bias;
    if constexpr (ASYM) {  // fp16 pair 1024 + z, z = byte c of zk
      const uint32_t sel = (uint32_t)c | (4u << 8) | ((uint32_t)c << 16) | (4u << 24);
      bias = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kc.m64, t.zk, sel));
    } else {
      gc ^= 0x88888888u;  // two's-complement nibble q -> q + 8
      bias = __builtin_bit_cast(half2v, 0x64086408u);
    }
    const half2v h0 = nib2<0>(gc, kc.m, kc.o) - bias, h1 = nib2<4>(gc, kc.m, kc.o) - bias;
    const half2v h2 = nib2<8>(gc, kc.m, kc.o) - bias, h3 = nib2<12>(gc, kc.m, kc.o) - bias;
    half8v ka;
    ka[0] = h0[0]; ka[1] = h0[1]; ka[2] = h1[0]; ka[3] = h1[1];
    ka[4] = h2[0]; ka[5] = h2[1]; ka[6] = h3[0]; ka[7] = h3[1];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      S[cc][ASYM ? c : 0] =
          __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qop[cc][c], S[cc][ASYM ? c : 0], 0, 0, 0);
  }
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    if constexpr (ASYM) {
      combine_groups(S[cc], t.sk, v[cc], std::integral_constant<int, NS>{});
    } else {
      static_for<0, 4>([&](auto E) {
        constexpr int e = decltype(E)::value;
        v[cc][e] = row_bcast<e>(t.sk) * S[cc][0][e];
      });
    }
  }
}

// Value bytes of a tile regrouped for the PV operands: G[i] (and the zero
// points Z[i]) hold byte i of the four tokens 4j..4j+3.
template <int D, int MODE>
__device__ __forceinline__ void tile4_vbytes(const Tile4<D, MODE>& t, uint32_t* G, uint32_t* Z) {
  constexpr int NS = D / 32;
  constexpr bool ASYM = MODE == KVQ_SCALE_GROUP_ASYM;
  if constexpr (NS == 4) {
    transpose4x4(t.v[0], t.v[1], t.v[2], t.v[3], G);
    if constexpr (ASYM) transpose4x4(t.zv[0], t.zv[1], t.zv[2], t.zv[3], Z);
  } else {
    const uint32_t v01 = t.v[0] | (t.v[1] << 16), v23 = t.v[2] | (t.v[3] << 16);
    G[0] = __builtin_amdgcn_perm(v23, v01, 0x06040200u);
    G[1] = __builtin_amdgcn_perm(v23, v01, 0x07050301u);
    if constexpr (ASYM) {
      Z[0] = __builtin_amdgcn_perm(t.zv[1], t.zv[0], 0x06040200u);
      Z[1] = __builtin_amdgcn_perm(t.zv[1], t.zv[0], 0x07050301u);
    }
  }
}

// PV operand words of group i of one tile, tokens in the order 0, 2, 1, 3:
// x (low nibbles) and y (high nibbles) are the raw codes 1024 + n, c the
// pairs -(1024 + z) (zero point, or 8 for the symmetric offset). A second
// product with c on the same accumulator removes the offset: both are exact
// in fp16 and the two terms cancel in the fp32 accumulator within the step,
// which replaces four fp16 subtractions per group by one more MFMA per
// output tile.
struct VWords4 {
  uint32_t x[2], y[2], c[2];
};
template <bool ASYM>
__device__ __forceinline__ VWords4 vgroup_words(uint32_t Gi, uint32_t Zi, const Nib4Consts& kc) {
  VWords4 w;
  if constexpr (ASYM) {
    w.c[0] = __builtin_amdgcn_perm(kc.e4, Zi, 0x04020400u);
    w.c[1] = __builtin_amdgcn_perm(kc.e4, Zi, 0x04030401u);
  } else {
    Gi ^= 0x88888888u;
    w.c[0] = w.c[1] = kc.nb;
  }
  w.x[0] = nib2u<0>(Gi, kc.m, kc.o);
  w.x[1] = nib2u<8>(Gi, kc.m, kc.o);
  w.y[0] = nib2u<4>(Gi, kc.m, kc.o);
  w.y[1] = nib2u<12>(Gi, kc.m, kc.o);
  return w;
}

// Online-softmax update for N scores per lane (already in log2 units, -inf
// where masked): returns the max to subtract and rescales the state when a
// column's max grows.
template <int D, int N>
__device__ __forceinline__ float softmax_update(const float* s, SoftmaxState<D>& st) {
  float m = s[0];
#pragma unroll
  for (int e = 1; e < N; ++e) m = fmaxf(m, s[e]);
  const float mn = fmaxf(st.m, colmax4(m));
  const float msafe = mn == -INFINITY ? 0.0f : mn;
  if (__any(mn > st.m)) {
    const float alpha = __builtin_amdgcn_exp2f(st.m - msafe);
    st.l *= alpha;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) st.acc[c] *= alpha;
  }
  st.m = mn;
  return msafe;
}

// One 16-token tile for NC column sets (cc: qop[cc], cscore[cc], st[cc],
// limits L[cc], lo[cc]) sharing the code conversions. TAIL: token t of the
// tile counts for this lane's column of set cc only if t < L[cc] and (t >=
// lo[cc] or t < sk) -- the causal limit, and the window start and sink count
// of a windowed column (lo = sk = 0 without a window).
template <int D, int MODE, int NC, bool TAIL>
__device__ __forceinline__ void tile4_step(const Tile4<D, MODE>& t, int pos0, const int* L,
                                           const half8v (*qop)[D / 32], const float* cscore,
                                           int j, SoftmaxState<D>* st, const Nib4Consts& kc,
                                           const int* lo, int sk) {
  constexpr int NS = D / 32;
  constexpr bool ASYM = MODE == KVQ_SCALE_GROUP_ASYM;
  constexpr int SG = Tile4<D, MODE>::SG;
  float v[NC][4];
  tile4_scores<D, MODE, NC>(t, qop, kc, v);
  // Masks that differ between the lanes of a row (per-column limits) must
  // not guard a row-broadcast read: the compiler would move the read under
  // the mask, and a lane whose source lane is masked off reads 0. The empty
  // barriers keep every broadcast ahead of the selects, under the full wave.
  if constexpr (TAIL)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      asm volatile("" : "+v"(v[cc][0]), "+v"(v[cc][1]), "+v"(v[cc][2]), "+v"(v[cc][3]));
  bool ok[NC][4];
  float p[NC][4];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    float s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tk = pos0 + 4 * j + e;
      ok[cc][e] = !TAIL || (tk < L[cc] && (tk >= lo[cc] || tk < sk));
      s[e] = ok[cc][e] ? v[cc][e] * cscore[cc] : -INFINITY;
    }
    const float msafe = softmax_update<D, 4>(s, st[cc]);
#pragma unroll
    for (int e = 0; e < 4; ++e) p[cc][e] = ok[cc][e] ? __builtin_amdgcn_exp2f(s[e] - msafe) : 0.0f;
    st[cc].l += (p[cc][0] + p[cc][1]) + (p[cc][2] + p[cc][3]);
  }
  uint32_t G[4], Z[4] = {0u, 0u, 0u, 0u};
  tile4_vbytes(t, G, Z);
  static_for<0, NS>([&](auto I) {
    constexpr int i = decltype(I)::value;
    float sb[4];
    static_for<0, 4>([&](auto E) {
      constexpr int e = decltype(E)::value;
      sb[e] = row_bcast<SG * e + (ASYM ? i : 0)>(t.sv);
    });
    if constexpr (TAIL) asm volatile("" : "+v"(sb[0]), "+v"(sb[1]), "+v"(sb[2]), "+v"(sb[3]));
    const VWords4 w = vgroup_words<ASYM>(G[i], Z[i], kc);
    const half4v va0 = __builtin_bit_cast(half4v, (u32x2){w.x[0], w.x[1]});
    const half4v va1 = __builtin_bit_cast(half4v, (u32x2){w.y[0], w.y[1]});
    const half4v corr = __builtin_bit_cast(half4v, (u32x2){w.c[0], w.c[1]});
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[e] = ok[cc][e] ? sb[e] * p[cc][e] : 0.0f;
      half4v pop;
      pop[0] = (half_t)pv[0]; pop[1] = (half_t)pv[2]; pop[2] = (half_t)pv[1]; pop[3] = (half_t)pv[3];
      float4v* acc = st[cc].acc;
      acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16f16(va0, pop, acc[2 * i], 0, 0, 0);
      acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(va1, pop, acc[2 * i + 1], 0, 0, 0);
      acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16f16(corr, pop, acc[2 * i], 0, 0, 0);
      acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(corr, pop, acc[2 * i + 1], 0, 0, 0);
    }
  });
}
// One column set (decode).
template <int D, int MODE, bool TAIL>
__device__ __forceinline__ void tile4_step(const Tile4<D, MODE>& t, int pos0, int L,
                                           const half8v* qop, float cscore, int j,
                                           SoftmaxState<D>& st, const Nib4Consts& kc,
                                           int lo = 0, int sk = 0) {
  tile4_step<D, MODE, 1, TAIL>(t, pos0, &L, reinterpret_cast<const half8v(*)[D / 32]>(qop),
                               &cscore, j, &st, kc, &lo, sk);
}

// Two consecutive whole tiles (32 tokens) in one step, for NC column sets
// sharing the code conversions: one softmax update per set for both tiles,
// and the PV products on 16x16x32 MFMAs whose contraction runs over the 32
// tokens (k = 8j + 4T + e' for tile T, token 4j + e' in the order 0, 2, 1, 3,
// the same in the value and probability operands).
template <int D, int MODE, int NC>
__device__ __forceinline__ void tile4_pair_step(const Tile4<D, MODE>& t0, const Tile4<D, MODE>& t1,
                                                const half8v (*qop)[D / 32], const float* cscore,
                                                SoftmaxState<D>* st, const Nib4Consts& kc) {
  constexpr int NS = D / 32;
  constexpr bool ASYM = MODE == KVQ_SCALE_GROUP_ASYM;
  constexpr int SG = Tile4<D, MODE>::SG;
  float v0[NC][4], v1[NC][4];
  tile4_scores<D, MODE, NC>(t0, qop, kc, v0);
  tile4_scores<D, MODE, NC>(t1, qop, kc, v1);
  float p[NC][8];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    float s[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[e] = v0[cc][e] * cscore[cc];
      s[4 + e] = v1[cc][e] * cscore[cc];
    }
    const float msafe = softmax_update<D, 8>(s, st[cc]);
#pragma unroll
    for (int e = 0; e < 8; ++e) p[cc][e] = __builtin_amdgcn_exp2f(s[e] - msafe);
    st[cc].l += ((p[cc][0] + p[cc][1]) + (p[cc][2] + p[cc][3])) +
                ((p[cc][4] + p[cc][5]) + (p[cc][6] + p[cc][7]));
  }
  uint32_t G0[4], Z0[4] = {0u, 0u, 0u, 0u}, G1[4], Z1[4] = {0u, 0u, 0u, 0u};
  tile4_vbytes(t0, G0, Z0);
  tile4_vbytes(t1, G1, Z1);
  static_for<0, NS>([&](auto I) {
    constexpr int i = decltype(I)::value;
    const VWords4 w0 = vgroup_words<ASYM>(G0[i], Z0[i], kc);
    const VWords4 w1 = vgroup_words<ASYM>(G1[i], Z1[i], kc);
    const half8v va0 = __builtin_bit_cast(half8v, (u32x4){w0.x[0], w0.x[1], w1.x[0], w1.x[1]});
    const half8v va1 = __builtin_bit_cast(half8v, (u32x4){w0.y[0], w0.y[1], w1.y[0], w1.y[1]});
    const half8v corr = __builtin_bit_cast(half8v, (u32x4){w0.c[0], w0.c[1], w1.c[0], w1.c[1]});
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      // the row broadcast folds into each multiply (v_mul_f32_dpp)
      float pv[8];
      static_for<0, 4>([&](auto E) {
        constexpr int e = decltype(E)::value;
        pv[e] = row_bcast<SG * e + (ASYM ? i : 0)>(t0.sv) * p[cc][e];
        pv[4 + e] = row_bcast<SG * e + (ASYM ? i : 0)>(t1.sv) * p[cc][4 + e];
      });
      half8v pop;
      pop[0] = (half_t)pv[0]; pop[1] = (half_t)pv[2]; pop[2] = (half_t)pv[1]; pop[3] = (half_t)pv[3];
      pop[4] = (half_t)pv[4]; pop[5] = (half_t)pv[6]; pop[6] = (half_t)pv[5]; pop[7] = (half_t)pv[7];
      float4v* acc = st[cc].acc;
      acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va0, pop, acc[2 * i], 0, 0, 0);
      acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va1, pop, acc[2 * i + 1], 0, 0, 0);
      acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(corr, pop, acc[2 * i], 0, 0, 0);
      acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(corr, pop, acc[2 * i + 1], 0, 0, 0);
    }
  });
}
// One column set (decode).
template <int D, int MODE>
__device__ __forceinline__ void tile4_pair_step(const Tile4<D, MODE>& t0, const Tile4<D, MODE>& t1,
                                                const half8v* qop, float cscore,
                                                SoftmaxState<D>& st, const Nib4Consts& kc) {
  tile4_pair_step<D, MODE, 1>(t0, t1, reinterpret_cast<const half8v(*)[D / 32]>(qop), &cscore,
                              &st, kc);
}

// Query operand for 4-bit keys: chunk c holds elements 32 c + 8 j + perm8[p]
// at position p, matching the nibble order nib2<0,4,8,12> produces.
template <int D>
__device__ __forceinline__ void query_int4(const DecodeArgs& a, const uint16_t* qrow, int j,
                                           bool hcol, half8v* qop, float& cscore) {
  constexpr int NS = D / 32;
  float qf[NS][8];
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * j);
    if (a.q_bf16) {
      unpack2<true>(w.x, qf[c][0], qf[c][1]); unpack2<true>(w.y, qf[c][2], qf[c][3]);
      unpack2<true>(w.z, qf[c][4], qf[c][5]); unpack2<true>(w.w, qf[c][6], qf[c][7]);
    } else {
      unpack2<false>(w.x, qf[c][0], qf[c][1]); unpack2<false>(w.y, qf[c][2], qf[c][3]);
      unpack2<false>(w.z, qf[c][4], qf[c][5]); unpack2<false>(w.w, qf[c][6], qf[c][7]);
    }
  }
  float qmax = 0.0f;
#pragma unroll
  for (int c = 0; c < NS; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf(qf[c][e]));
  qmax = colmax4(qmax);
  int qe = qmax > 0.0f ? (int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127 : 0;
  qe = max(qe, -126);
  const float qdown = __uint_as_float((uint32_t)(127 - qe) << 23);
  const float qup = __uint_as_float((uint32_t)(127 + qe) << 23);
  constexpr int perm8[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
  for (int c = 0; c < NS; ++c)
#pragma unroll
    for (int p = 0; p < 8; ++p) qop[c][p] = hcol ? (half_t)(qf[c][perm8[p]] * qdown) : (half_t)0.0f;
  cscore = hcol ? qup * a.sm_log2 : 0.0f;
}

}  // namespace
}  // namespace kvq
