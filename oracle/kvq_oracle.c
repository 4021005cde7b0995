/*
 * kvq_oracle.c -- plain, slow, scalar CPU oracle. TEST INFRASTRUCTURE ONLY:
 * the test suite, the package smoke check and the benchmark's CPU-baseline
 * leg are its only users. Nothing here is shared with the GPU library.
 *
 * Sources ("the pages"):
 *  [P1] "Dynamic KV Cache Quantization for Fast LLM Inference" (theskillset.io)
 *  [P2] "KV Cache Optimization" glossary (esaholic.com)
 *  [P3] "KV Cache Optimization: Strategies for Faster LLM Inference"
 *       (swarnava.dev)
 * Each function names the passage it follows. Where the pages leave a step
 * open, the reading taken is stated at the function.
 */
#include "kvq_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats, written from their definitions.                          */
/* ------------------------------------------------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  return (float)(sign ? -v : v);
}

/* bfloat16 is the upper half of an IEEE binary32. */
float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float src_to_f32(const void* base, int64_t idx, int dtype) {
  const uint16_t* p = (const uint16_t*)base;
  return dtype == ORC_BF16 ? orc_bf16_to_f32(p[idx]) : orc_f16_to_f32(p[idx]);
}

/* OCP 8-bit floating point, E4M3 variant: 1 sign, 4 exponent (bias 7), 3
 * mantissa bits; exponent field 0 holds subnormals m * 2^-9; S.1111.111 is
 * NaN and there are no infinities, so the largest finite value is
 * 1.75 * 2^8 = 448. (The pages name FP8 KV caches but do not define the
 * format; this is the published format definition.) */
float orc_e4m3_value(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 0xF;
  int m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return (float)(sign ? -v : v);
}

/* Values of the 127 non-negative finite codes, filled once from
 * orc_e4m3_value. */
static double e4m3_table[127];
static pthread_once_t e4m3_once = PTHREAD_ONCE_INIT;
static void e4m3_fill(void) {
  for (int c = 0; c < 127; ++c) e4m3_table[c] = orc_e4m3_value((uint8_t)c);
}

/* Nearest E4M3 value to y, ties to the even code (the code's last bit is the
 * mantissa's last bit), magnitudes above 448 saturate to 448, the sign is kept
 * (so -0 and negatives that round to zero give 0x80). Search over the 127
 * non-negative finite codes, whose values increase with the code. */
uint8_t orc_e4m3_encode(float y) {
  pthread_once(&e4m3_once, e4m3_fill);
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs((double)y);
  if (a >= 448.0) return sign | 0x7E;
  int lo = 0, hi = 126; /* largest k with value(k) <= a */
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (e4m3_table[mid] <= a)
      lo = mid;
    else
      hi = mid - 1;
  }
  int k = lo;
  double below = e4m3_table[k];
  double above = e4m3_table[k + 1];
  double twice = 2.0 * a, mid_sum = below + above; /* both exact in double */
  int pick;
  if (twice < mid_sum)
    pick = k;
  else if (twice > mid_sum)
    pick = k + 1;
  else
    pick = (k % 2 == 0) ? k : k + 1;
  return sign | (uint8_t)pick;
}

/* ------------------------------------------------------------------------ */
/* Row codecs.                                                              */
/* ------------------------------------------------------------------------ */

/* Symmetric absmax quantization of one vector [P1, "Understanding Dynamic
 * Quantization Techniques for KV Caches"]: scale = max|x| / (2^(bits-1) - 1),
 * code = round(x / scale). qmax = 127 for INT8, 7 for INT4. An all-zero
 * vector gives codes 0 and scale 1 (the toy quantizer's early return).
 * Readings: fp32 arithmetic, true division, round half to even (the rounding
 * of torch.round used by the toy quantizer), codes clamped to [-qmax, qmax]. */
void orc_quant_sym(const float* x, int n, int qmax, int8_t* q, float* s) {
  float a = 0.0f;
  for (int i = 0; i < n; ++i) {
    float ax = fabsf(x[i]);
    if (ax > a) a = ax;
  }
  if (a == 0.0f) {
    for (int i = 0; i < n; ++i) q[i] = 0;
    *s = 1.0f;
    return;
  }
  float sc = a / (float)qmax;
  for (int i = 0; i < n; ++i) {
    float r = rintf(x[i] / sc);
    if (r > (float)qmax) r = (float)qmax;
    if (r < (float)-qmax) r = (float)-qmax;
    q[i] = (int8_t)r;
  }
  *s = sc;
}

/* FP8 E4M3 codes with a dynamic per-vector scale. The pages name an FP8 KV
 * cache [P1 "Practical Implementation Challenges", P2 "Technical
 * Architecture", P3 "How vLLM Implements KV Cache Optimization"] but give no
 * scaling rule; the reading taken is the absmax rule of [P1] with the
 * format's largest finite value: scale = max|x| / 448, code = E4M3(x/scale). */
void orc_quant_fp8(const float* x, int n, uint8_t* q, float* s) {
  float a = 0.0f;
  for (int i = 0; i < n; ++i) {
    float ax = fabsf(x[i]);
    if (ax > a) a = ax;
  }
  if (a == 0.0f) {
    for (int i = 0; i < n; ++i) q[i] = orc_e4m3_encode(x[i] / 1.0f);
    *s = 1.0f;
    return;
  }
  float sc = a / 448.0f;
  for (int i = 0; i < n; ++i) q[i] = orc_e4m3_encode(x[i] / sc);
  *s = sc;
}

/* Asymmetric 4-bit quantization of one group: a scale and an integer zero
 * point from the group's range [P1, "Understanding Dynamic Quantization
 * Techniques": the scaling factor and zero point come from the current
 * tensor's range; the toy quantizer returns an integer zero point]. The pages
 * stop there; the reading taken is textbook affine quantization onto [0, 15]
 * with the range widened to contain 0: mn = min(0, min x), mx = max(0, max x),
 * s = (mx - mn) / 15, z = clamp(rne(-mn / s), 0, 15),
 * q = clamp(rne(x / s) + z, 0, 15). A group with mx == mn gets q = 0, s = 1,
 * z = 0. q holds one code per element (unpacked). */
void orc_quant_asym4(const float* x, int n, uint8_t* q, float* s, uint8_t* z) {
  float mn = 0.0f, mx = 0.0f;
  for (int i = 0; i < n; ++i) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  if (mx == mn) {
    for (int i = 0; i < n; ++i) q[i] = 0;
    *s = 1.0f;
    *z = 0;
    return;
  }
  float sc = (mx - mn) / 15.0f;
  float zf = rintf(-mn / sc);
  if (zf < 0.0f) zf = 0.0f;
  if (zf > 15.0f) zf = 15.0f;
  int zi = (int)zf;
  for (int i = 0; i < n; ++i) {
    int qi = (int)rintf(x[i] / sc) + zi;
    if (qi < 0) qi = 0;
    if (qi > 15) qi = 15;
    q[i] = (uint8_t)qi;
  }
  *s = sc;
  *z = (uint8_t)zi;
}

/* Static scales [P1, opening section and "Understanding Dynamic Quantization
 * Techniques for KV Caches": static quantization applies a fixed scaling
 * factor (and zero point) determined in advance, where dynamic quantization
 * derives them from each new vector]. The code rules are those above with
 * the caller's scale s (> 0, finite) and zero point z in place of the ones
 * taken from the vector's range; since the range no longer bounds x / s,
 * the codes saturate: [-qmax, qmax] for the symmetric integers, +-448 for
 * E4M3 (the encoder saturates), [0, 15] for the asymmetric nibbles. The
 * clamps are applied to rne(x / s) before any integer conversion. */
void orc_quant_sym_static(const float* x, int n, int qmax, float s, int8_t* q) {
  for (int i = 0; i < n; ++i) {
    float r = rintf(x[i] / s);
    if (r > (float)qmax) r = (float)qmax;
    if (r < (float)-qmax) r = (float)-qmax;
    q[i] = (int8_t)r;
  }
}

void orc_quant_fp8_static(const float* x, int n, float s, uint8_t* q) {
  for (int i = 0; i < n; ++i) q[i] = orc_e4m3_encode(x[i] / s);
}

void orc_quant_asym4_static(const float* x, int n, float s, uint8_t z, uint8_t* q) {
  for (int i = 0; i < n; ++i) {
    float r = rintf(x[i] / s);
    if (r > 15.0f) r = 15.0f;
    if (r < -15.0f) r = -15.0f;
    int qi = (int)r + (int)z;
    if (qi < 0) qi = 0;
    if (qi > 15) qi = 15;
    q[i] = (uint8_t)qi;
  }
}

/* Per-channel keys [P3, "KV Cache Quantization: When and How to Compress":
 * per-channel scales keep more information than a single scale]. One block of
 * bs rows x[t][c] (c < d): channel c gets the symmetric INT8 rule of
 * orc_quant_sym over its bs values. */
void orc_quant_channel_block(const float* x, int bs, int d, int8_t* q,
                             float* s) {
  float* col = (float*)malloc(sizeof(float) * (size_t)bs);
  int8_t* qc = (int8_t*)malloc((size_t)bs);
  for (int c = 0; c < d; ++c) {
    for (int t = 0; t < bs; ++t) col[t] = x[(size_t)t * d + c];
    orc_quant_sym(col, bs, 127, qc, &s[c]);
    for (int t = 0; t < bs; ++t) q[(size_t)t * d + c] = qc[t];
  }
  free(col);
  free(qc);
}

/* Two 4-bit codes per byte. Placement (a layout choice, not from the pages):
 * with n = d / 32, element e = 32 i + 2 r + t (i < n, r < 16, t < 2) goes to
 * byte n r + i, low nibble for t = 0, high nibble for t = 1. */
void orc_int4_pack(const uint8_t* nib, int d, uint8_t* out) {
  int n = d / 32;
  memset(out, 0, (size_t)d / 2);
  for (int e = 0; e < d; ++e) {
    int i = e / 32, r = (e % 32) / 2, t = e % 2;
    int byte = n * r + i;
    out[byte] |= (uint8_t)((nib[e] & 0xF) << (4 * t));
  }
}

void orc_int4_unpack(const uint8_t* in, int d, uint8_t* nib) {
  int n = d / 32;
  for (int e = 0; e < d; ++e) {
    int i = e / 32, r = (e % 32) / 2, t = e % 2;
    nib[e] = (in[n * r + i] >> (4 * t)) & 0xF;
  }
}

/* ------------------------------------------------------------------------ */
/* Layout arithmetic.                                                       */
/* ------------------------------------------------------------------------ */

static int side_code(const orc_layout* L, int side) {
  return side ? L->v_code : L->k_code;
}
static int side_mode(const orc_layout* L, int side) {
  return side ? L->v_mode : L->k_mode;
}

static int check_side(const orc_layout* L, int side) {
  int code = side_code(L, side), mode = side_mode(L, side);
  if (code < 0 || code > 3 || mode < 0 || mode > 2) return ORC_ERR_INVALID;
  if (mode == ORC_TOKEN_SYM) return ORC_OK;
  if (mode == ORC_GROUP_ASYM)
    return (code == ORC_CODE_INT4 && L->group_size == 32) ? ORC_OK
                                                          : ORC_ERR_UNSUPPORTED;
  /* CHANNEL_BLOCK */
  return (side == 0 && code == ORC_CODE_INT8) ? ORC_OK : ORC_ERR_UNSUPPORTED;
}

static int check_layout(const orc_layout* L) {
  if (!L) return ORC_ERR_INVALID;
  if (L->num_kv_heads < 1) return ORC_ERR_INVALID;
  if (L->head_dim != 64 && L->head_dim != 128) return ORC_ERR_INVALID;
  if (L->block_size != 16 && L->block_size != 32) return ORC_ERR_INVALID;
  if (L->src_dtype != ORC_F16 && L->src_dtype != ORC_BF16)
    return ORC_ERR_INVALID;
  int rc = check_side(L, 0);
  if (rc) return rc;
  return check_side(L, 1);
}

static int code_bits(int code) {
  return code == ORC_CODE_NONE16 ? 16 : code == ORC_CODE_INT4 ? 4 : 8;
}

static int64_t row_bytes(const orc_layout* L, int side) {
  return (int64_t)L->head_dim * code_bits(side_code(L, side)) / 8;
}

/* fp32 scale values per (block, head) of one side. */
static int64_t scales_per_bh(const orc_layout* L, int side) {
  int mode = side_mode(L, side);
  if (side_code(L, side) == ORC_CODE_NONE16) return 0;
  if (mode == ORC_TOKEN_SYM) return L->block_size;
  if (mode == ORC_GROUP_ASYM)
    return (int64_t)L->block_size * (L->head_dim / L->group_size);
  return L->head_dim; /* CHANNEL_BLOCK */
}

static int64_t zeros_per_bh(const orc_layout* L, int side) {
  if (side_mode(L, side) != ORC_GROUP_ASYM) return 0;
  return (int64_t)L->block_size * (L->head_dim / L->group_size);
}

int orc_plane_bytes(const orc_layout* L, int64_t nb, int32_t max_seqs,
                    int64_t out[7]) {
  int rc = check_layout(L);
  if (rc) return rc;
  int64_t H = L->num_kv_heads, bs = L->block_size, d = L->head_dim;
  for (int side = 0; side < 2; ++side) {
    out[0 + side] = nb * H * bs * row_bytes(L, side);
    out[2 + side] = nb * H * scales_per_bh(L, side) * 4;
    out[4 + side] = nb * H * zeros_per_bh(L, side);
  }
  out[6] = (L->k_mode == ORC_CHANNEL_BLOCK) ? (int64_t)max_seqs * H * bs * d * 2
                                            : 0;
  return ORC_OK;
}

/* Cache bytes per token [P2, "Technical Architecture": keys and values, over
 * layers, KV heads and head dimension, at the element width; P3, "What Is KV
 * Cache and Why Does It Balloon Memory Usage?": the same product times
 * sequence length and batch]. The glossary's printed formula carries one
 * factor of 2 too many for its own printed results (327.68 / 163.84 / 81.92
 * KB for 80 layers, 8 KV heads, d = 128 at 16 / 8 / 4 bit); the reading taken
 * is the one that reproduces those results: 2 (K and V) x layers x heads x
 * head_dim x bits / 8. Metadata per layer and side when asked for: TOKEN_SYM
 * H * 4, GROUP_ASYM H * (d / gs) * (4 + 1), CHANNEL_BLOCK ceil(H * d * 4 / bs). */
int64_t orc_bytes_per_token(const orc_layout* L, int32_t num_layers,
                            int32_t include_metadata) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (num_layers < 1) return ORC_ERR_INVALID;
  int64_t H = L->num_kv_heads, d = L->head_dim, bs = L->block_size;
  int64_t per_layer = 0;
  for (int side = 0; side < 2; ++side) {
    per_layer += H * d * code_bits(side_code(L, side)) / 8;
    if (!include_metadata || side_code(L, side) == ORC_CODE_NONE16) continue;
    int mode = side_mode(L, side);
    if (mode == ORC_TOKEN_SYM)
      per_layer += H * 4;
    else if (mode == ORC_GROUP_ASYM)
      per_layer += H * (d / L->group_size) * 5;
    else
      per_layer += (H * d * 4 + bs - 1) / bs;
  }
  return per_layer * num_layers;
}

/* ------------------------------------------------------------------------ */
/* Append: quantize each new row and place it through its slot.              */
/* ------------------------------------------------------------------------ */

/* Quantize one (token, head) row of one side and store it at (blk, h, off).
 * [P1, "Understanding Dynamic Quantization Techniques": the scale is computed
 * for each new piece of keys and values as it enters the cache; P1,
 * "Integrating Dynamic Quantization with PagedAttention": every physical block
 * holds quantized keys and values.] */
static void store_row(const orc_layout* L, const orc_cache* C, int side,
                      const float* x, const uint16_t* raw, int64_t blk, int h,
                      int off) {
  int H = L->num_kv_heads, d = L->head_dim, bs = L->block_size;
  int code = side_code(L, side), mode = side_mode(L, side);
  int64_t bh = blk * H + h;
  int64_t rb = row_bytes(L, side);
  uint8_t* codes = (uint8_t*)(side ? C->v_codes : C->k_codes);
  uint8_t* dst = codes + (bh * bs + off) * rb;
  float* scale = side ? C->v_scale : C->k_scale;
  uint8_t* zero = side ? C->v_zero : C->k_zero;
  if (code == ORC_CODE_NONE16) {
    memcpy(dst, raw, (size_t)rb); /* passthrough: the 16-bit value as given */
    return;
  }
  if (mode == ORC_TOKEN_SYM) {
    float s;
    if (code == ORC_CODE_INT8) {
      orc_quant_sym(x, d, 127, (int8_t*)dst, &s);
    } else if (code == ORC_CODE_FP8) {
      orc_quant_fp8(x, d, dst, &s);
    } else { /* INT4, symmetric: the same rule with bits = 4 */
      int8_t q[128];
      uint8_t nib[128];
      orc_quant_sym(x, d, 7, q, &s);
      for (int e = 0; e < d; ++e) nib[e] = (uint8_t)(q[e] & 0xF);
      orc_int4_pack(nib, d, dst);
    }
    scale[bh * bs + off] = s;
    return;
  }
  /* GROUP_ASYM, INT4: groups of group_size consecutive elements along d. */
  int gs = L->group_size, ng = d / gs;
  uint8_t nib[128];
  for (int g = 0; g < ng; ++g) {
    float s;
    uint8_t z;
    orc_quant_asym4(x + g * gs, gs, nib + g * gs, &s, &z);
    scale[(bh * bs + off) * ng + g] = s;
    zero[(bh * bs + off) * ng + g] = z;
  }
  orc_int4_pack(nib, d, dst);
}

/* Keys under CHANNEL_BLOCK: rows of a block wait raw in the stage row of
 * their sequence; when the block's last slot is written, the whole block is
 * quantized per channel from the staged rows. Reading taken (the pages leave
 * partial blocks open): a block is quantized exactly once, from all its rows,
 * so the result does not depend on how appends were chunked. */
static void store_key_channel_block(const orc_layout* L, const orc_cache* C,
                                    const uint16_t* raw, int64_t blk, int h,
                                    int off, int32_t stage_row) {
  int H = L->num_kv_heads, d = L->head_dim, bs = L->block_size;
  uint16_t* stage = (uint16_t*)C->k_stage;
  uint16_t* srow = stage + (((int64_t)stage_row * H + h) * bs + off) * d;
  memcpy(srow, raw, sizeof(uint16_t) * (size_t)d);
  if (off != bs - 1) return;
  float* x = (float*)malloc(sizeof(float) * (size_t)bs * d);
  uint16_t* sblk = stage + ((int64_t)stage_row * H + h) * bs * d;
  for (int64_t i = 0; i < (int64_t)bs * d; ++i)
    x[i] = L->src_dtype == ORC_BF16 ? orc_bf16_to_f32(sblk[i])
                                    : orc_f16_to_f32(sblk[i]);
  int64_t bh = blk * H + h;
  int8_t* dst = (int8_t*)C->k_codes + bh * bs * d;
  orc_quant_channel_block(x, bs, d, dst, C->k_scale + bh * d);
  free(x);
}

/* Append [P1, "Recap of KV Caching": each new token's keys and values are
 * added to the cache; P1, "Integrating Dynamic Quantization with
 * PagedAttention": blocks are placed through a per-sequence logical-to-
 * physical map]. Token t with slot s goes to block s / bs, offset s % bs;
 * slot -1 writes nothing. Tokens are processed in order t = 0, 1, ... */
int orc_append(const orc_layout* L, const orc_cache* C, const void* k,
               const void* v, int64_t k_row_stride, int64_t v_row_stride,
               int64_t num_tokens, const int64_t* slot_mapping,
               const int32_t* stage_rows) {
  int rc = check_layout(L);
  if (rc) return rc;
  int H = L->num_kv_heads, d = L->head_dim, bs = L->block_size;
  float x[128];
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    int64_t blk = slot / bs;
    int off = (int)(slot % bs);
    if (blk >= C->num_blocks) return ORC_ERR_INVALID;
    for (int side = 0; side < 2; ++side) {
      const void* src = side ? v : k;
      int64_t stride = side ? v_row_stride : k_row_stride;
      for (int h = 0; h < H; ++h) {
        int64_t base = t * stride + (int64_t)h * d;
        const uint16_t* raw = (const uint16_t*)src + base;
        for (int e = 0; e < d; ++e) x[e] = src_to_f32(src, base + e, L->src_dtype);
        if (side_mode(L, side) == ORC_CHANNEL_BLOCK) {
          if (!stage_rows) return ORC_ERR_INVALID;
          store_key_channel_block(L, C, raw, blk, h, off, stage_rows[t]);
        } else {
          store_row(L, C, side, x, raw, blk, h, off);
        }
      }
    }
  }
  return ORC_OK;
}

/* Append with static scales: as orc_append, with side X's codes from the
 * caller's per-KV-head parameters -- TOKEN_SYM: scale x_scale[h]; GROUP_ASYM:
 * scale x_scale[h * ng + g] and zero point x_zero[h * ng + g] for group g of
 * ng = d / group_size; CHANNEL_BLOCK keys: scale k_scale[h * d + c] for
 * channel c. The metadata planes receive those values, so that
 * dequantization is unchanged; NONE16 sides are passthrough as in orc_append.
 * Static per-channel keys (P3, "KV Cache Quantization: When and How to
 * Compress", per-channel scales, here fixed in advance) need no wait for the
 * block: each row is coded at once, and the block's scale row is written with
 * its first slot (offset 0; blocks fill from offset 0 upward). The raw row
 * still goes to the sequence's stage row, because decode reads a sequence's
 * partial last block from there in this mode. */
int orc_append_static(const orc_layout* L, const orc_cache* C, const void* k,
                      const void* v, int64_t k_row_stride, int64_t v_row_stride,
                      int64_t num_tokens, const int64_t* slot_mapping,
                      const int32_t* stage_rows, const float* k_scale,
                      const uint8_t* k_zero, const float* v_scale,
                      const uint8_t* v_zero) {
  int rc = check_layout(L);
  if (rc) return rc;
  if ((L->k_mode == ORC_CHANNEL_BLOCK) != (stage_rows != NULL)) return ORC_ERR_INVALID;
  int H = L->num_kv_heads, d = L->head_dim, bs = L->block_size;
  float x[128];
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    int64_t blk = slot / bs;
    int off = (int)(slot % bs);
    if (blk >= C->num_blocks) return ORC_ERR_INVALID;
    for (int side = 0; side < 2; ++side) {
      const void* src = side ? v : k;
      int64_t stride = side ? v_row_stride : k_row_stride;
      const float* sst = side ? v_scale : k_scale;
      const uint8_t* zst = side ? v_zero : k_zero;
      int code = side_code(L, side), mode = side_mode(L, side);
      for (int h = 0; h < H; ++h) {
        int64_t base = t * stride + (int64_t)h * d;
        int64_t bh = blk * H + h;
        int64_t rb = row_bytes(L, side);
        uint8_t* dst = (uint8_t*)(side ? C->v_codes : C->k_codes) + (bh * bs + off) * rb;
        if (code == ORC_CODE_NONE16) {
          memcpy(dst, (const uint16_t*)src + base, (size_t)rb);
          continue;
        }
        for (int e = 0; e < d; ++e) x[e] = src_to_f32(src, base + e, L->src_dtype);
        float* scale = side ? C->v_scale : C->k_scale;
        if (mode == ORC_CHANNEL_BLOCK) {
          uint16_t* srow = (uint16_t*)C->k_stage +
                           (((int64_t)stage_rows[t] * H + h) * bs + off) * d;
          memcpy(srow, (const uint16_t*)src + base, sizeof(uint16_t) * (size_t)d);
          for (int c = 0; c < d; ++c)
            orc_quant_sym_static(x + c, 1, 127, sst[h * d + c], (int8_t*)dst + c);
          if (off == 0)
            memcpy(scale + bh * d, sst + (int64_t)h * d, sizeof(float) * (size_t)d);
        } else if (mode == ORC_TOKEN_SYM) {
          float sh = sst[h];
          if (code == ORC_CODE_INT8) {
            orc_quant_sym_static(x, d, 127, sh, (int8_t*)dst);
          } else if (code == ORC_CODE_FP8) {
            orc_quant_fp8_static(x, d, sh, dst);
          } else {
            int8_t q[128];
            uint8_t nib[128];
            orc_quant_sym_static(x, d, 7, sh, q);
            for (int e = 0; e < d; ++e) nib[e] = (uint8_t)(q[e] & 0xF);
            orc_int4_pack(nib, d, dst);
          }
          scale[bh * bs + off] = sh;
        } else { /* GROUP_ASYM */
          int gs = L->group_size, ng = d / gs;
          uint8_t nib[128];
          uint8_t* zero = side ? C->v_zero : C->k_zero;
          for (int g = 0; g < ng; ++g) {
            float sg = sst[h * ng + g];
            uint8_t zg = zst[h * ng + g];
            orc_quant_asym4_static(x + g * gs, gs, sg, zg, nib + g * gs);
            scale[(bh * bs + off) * ng + g] = sg;
            zero[(bh * bs + off) * ng + g] = zg;
          }
          orc_int4_pack(nib, d, dst);
        }
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Dequantization and decode attention.                                      */
/* ------------------------------------------------------------------------ */

/* Dequantized fp32 row of logical position pos of one sequence, head h
 * [P1, "Understanding Dynamic Quantization Techniques": the dequantized value
 * is the code as a float times the scale]. Asymmetric: (q - z) * s. Keys under
 * CHANNEL_BLOCK: positions of the partial last block (pos >= floor(len/bs)*bs)
 * come raw from stage row stage_row. */
int orc_dequant_token(const orc_layout* L, const orc_cache* C, int side,
                      const int32_t* table_row, int32_t context_len,
                      int32_t stage_row, int32_t pos, int32_t h, float* out) {
  int H = L->num_kv_heads, d = L->head_dim, bs = L->block_size;
  int code = side_code(L, side), mode = side_mode(L, side);
  if (mode == ORC_CHANNEL_BLOCK && pos >= (context_len / bs) * bs) {
    const uint16_t* stage = (const uint16_t*)C->k_stage;
    const uint16_t* srow =
        stage + (((int64_t)stage_row * H + h) * bs + pos % bs) * d;
    for (int e = 0; e < d; ++e) out[e] = src_to_f32(srow, e, L->src_dtype);
    return ORC_OK;
  }
  int64_t blk = table_row[pos / bs];
  if (blk < 0 || blk >= C->num_blocks) return ORC_ERR_INVALID;
  int off = pos % bs;
  int64_t bh = blk * H + h;
  int64_t rb = row_bytes(L, side);
  const uint8_t* codes = (const uint8_t*)(side ? C->v_codes : C->k_codes);
  const uint8_t* row = codes + (bh * bs + off) * rb;
  const float* scale = side ? C->v_scale : C->k_scale;
  const uint8_t* zero = side ? C->v_zero : C->k_zero;
  if (code == ORC_CODE_NONE16) {
    for (int e = 0; e < d; ++e) out[e] = src_to_f32(row, e, L->src_dtype);
    return ORC_OK;
  }
  if (mode == ORC_CHANNEL_BLOCK) {
    const float* sc = scale + bh * d;
    for (int e = 0; e < d; ++e) out[e] = (float)((const int8_t*)row)[e] * sc[e];
    return ORC_OK;
  }
  if (mode == ORC_GROUP_ASYM) {
    int ng = d / L->group_size;
    uint8_t nib[128];
    orc_int4_unpack(row, d, nib);
    for (int e = 0; e < d; ++e) {
      int g = e / L->group_size;
      float s = scale[(bh * bs + off) * ng + g];
      int z = zero[(bh * bs + off) * ng + g];
      out[e] = (float)((int)nib[e] - z) * s;
    }
    return ORC_OK;
  }
  float s = scale[bh * bs + off]; /* TOKEN_SYM */
  if (code == ORC_CODE_INT8) {
    for (int e = 0; e < d; ++e) out[e] = (float)((const int8_t*)row)[e] * s;
  } else if (code == ORC_CODE_FP8) {
    for (int e = 0; e < d; ++e) out[e] = orc_e4m3_value(row[e]) * s;
  } else {
    uint8_t nib[128];
    orc_int4_unpack(row, d, nib);
    for (int e = 0; e < d; ++e) {
      int qv = nib[e] >= 8 ? (int)nib[e] - 16 : (int)nib[e]; /* sign-extend */
      out[e] = (float)qv * s;
    }
  }
  return ORC_OK;
}

static double q_elem(const void* q, int32_t q_dtype, int64_t idx) {
  if (q_dtype == ORC_F32) return ((const float*)q)[idx];
  return src_to_f32(q, idx, q_dtype);
}

/* Softmax pieces over positions [t_begin, t_end) of sequence b for query
 * head h, in binary64: m = max s_t, l = sum exp(s_t - m),
 * acc = sum exp(s_t - m) v_t, with s_t = (q . k_t) * sm_scale. Query head h
 * reads KV head h / (Hq / H) (contiguous query groups; the pages imply GQA
 * only by pairing 8 KV heads with 64 heads for one model). */
int orc_decode_range(const orc_layout* L, const orc_cache* C, const void* q,
                     int32_t q_dtype, int32_t num_q_heads, int32_t b,
                     int32_t h, const int32_t* table_row, int32_t context_len,
                     int32_t t_begin, int32_t t_end, double sm_scale,
                     double* m_out, double* l_out, double* acc) {
  int H = L->num_kv_heads, d = L->head_dim;
  int G = num_q_heads / H;
  int g = h / G;
  double qv[128];
  float row[128];
  for (int e = 0; e < d; ++e)
    qv[e] = q_elem(q, q_dtype, ((int64_t)b * num_q_heads + h) * d + e);
  for (int e = 0; e < d; ++e) acc[e] = 0.0;
  *m_out = -INFINITY;
  *l_out = 0.0;
  if (t_end <= t_begin) return ORC_OK;
  double* s = (double*)malloc(sizeof(double) * (size_t)(t_end - t_begin));
  double m = -INFINITY;
  for (int t = t_begin; t < t_end; ++t) {
    int rc = orc_dequant_token(L, C, 0, table_row, context_len, b, t, g, row);
    if (rc) {
      free(s);
      return rc;
    }
    double dot = 0.0;
    for (int e = 0; e < d; ++e) dot += qv[e] * (double)row[e];
    s[t - t_begin] = dot * sm_scale;
    if (s[t - t_begin] > m) m = s[t - t_begin];
  }
  double l = 0.0;
  for (int t = t_begin; t < t_end; ++t) {
    double p = exp(s[t - t_begin] - m);
    l += p;
    int rc = orc_dequant_token(L, C, 1, table_row, context_len, b, t, g, row);
    if (rc) {
      free(s);
      return rc;
    }
    for (int e = 0; e < d; ++e) acc[e] += p * (double)row[e];
  }
  free(s);
  *m_out = m;
  *l_out = l;
  return ORC_OK;
}

typedef struct {
  const orc_layout* L;
  const orc_cache* C;
  const void* q;
  int32_t q_dtype, batch, Hq, max_blocks;
  const int32_t* tables;
  const int32_t* lens;
  double sm;
  double* out;
  int64_t next; /* work counter, guarded by mu */
  int rc;
  pthread_mutex_t mu;
} decode_job;

static void* decode_worker(void* arg) {
  decode_job* J = (decode_job*)arg;
  int d = J->L->head_dim;
  double m, l, acc[128];
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t item = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (item >= (int64_t)J->batch * J->Hq) break;
    int b = (int)(item / J->Hq), h = (int)(item % J->Hq);
    double* o = J->out + item * d;
    int rc = orc_decode_range(J->L, J->C, J->q, J->q_dtype, J->Hq, b, h,
                              J->tables + (int64_t)b * J->max_blocks,
                              J->lens[b], 0, J->lens[b], J->sm, &m, &l, acc);
    if (rc) {
      pthread_mutex_lock(&J->mu);
      J->rc = rc;
      pthread_mutex_unlock(&J->mu);
      continue;
    }
    for (int e = 0; e < d; ++e) o[e] = l > 0.0 ? acc[e] / l : 0.0;
  }
  return NULL;
}

/* Decode attention [P1, "Recap of KV Caching": attention of the current query
 * over the cached keys and values of its sequence, scaled dot-product
 * attention softmax(q K^T / sqrt(d)) V]. out[b][h] = sum_t p_t v_t / sum_t p_t,
 * p_t = exp(s_t - max s), over t < context_lens[b]; 0 tokens give 0. All in
 * binary64 from the binary32 dequantized rows. sm_scale = 0 means 1/sqrt(d).
 * (b, h) items are spread over num_threads threads; each item is computed
 * the same way whatever the thread count. */
int orc_decode(const orc_layout* L, const orc_cache* C, const void* q,
               int32_t q_dtype, int32_t batch, int32_t num_q_heads,
               const int32_t* block_tables, int32_t max_blocks_per_seq,
               const int32_t* context_lens, double sm_scale, double* out,
               int32_t num_threads) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (num_q_heads % L->num_kv_heads) return ORC_ERR_INVALID;
  decode_job J;
  J.L = L;
  J.C = C;
  J.q = q;
  J.q_dtype = q_dtype;
  J.batch = batch;
  J.Hq = num_q_heads;
  J.max_blocks = max_blocks_per_seq;
  J.tables = block_tables;
  J.lens = context_lens;
  J.sm = sm_scale != 0.0 ? sm_scale : 1.0 / sqrt((double)L->head_dim);
  J.out = out;
  J.next = 0;
  J.rc = ORC_OK;
  pthread_mutex_init(&J.mu, NULL);
  if (num_threads < 1) num_threads = 1;
  if (num_threads == 1) {
    decode_worker(&J);
  } else {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)num_threads);
    for (int i = 0; i < num_threads; ++i)
      pthread_create(&th[i], NULL, decode_worker, &J);
    for (int i = 0; i < num_threads; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&J.mu);
  return J.rc;
}

/* Multi-query (prefill) attention [P3, "Why KV Cache Is Essential for
 * Efficient LLM Inference": the prompt's tokens are processed together before
 * decoding; P3, "Implementing KV Cache Optimization: A Practical Checklist",
 * common pitfalls: that phase is compute-bound, unlike decode]. Sequence b
 * has nq = query_start[b+1] - query_start[b] query tokens, the last nq of its
 * context_lens[b] = L cached positions (their keys and values are already
 * appended): query i sits at position p = L - nq + i and attends causally to
 * positions 0..p. Query row r = query_start[b] + i, head h (KV head h / G):
 * out[r][h] = sum_{t<=p} e_t v_t / sum_{t<=p} e_t, e_t = exp(s_t - max s),
 * s_t = (q . k_t) sm, in binary64 from the binary32 dequantized rows. Which
 * positions are read raw from the stage (per-channel keys) is decided by the
 * full length L, as in decode. nq = 1 is decode.
 * Sliding window with attention sinks [P3, "Cache Eviction and Compression
 * Strategies": a sliding window keeps only the most recent tokens; a few
 * first tokens kept as sinks next to the window allow unbounded context]:
 * with window > 0 the query at position p sees only positions t <= p with
 * t >= p + 1 - window (its last `window` positions, itself included) or
 * t < sink. window = 0 is full causal attention. */
typedef struct {
  const orc_layout* L;
  const orc_cache* C;
  const void* q;
  int32_t q_dtype, batch, Hq, max_blocks;
  const int32_t* qstart;
  const int32_t* tables;
  const int32_t* lens;
  int32_t window, sink;
  double sm;
  double* out;
  int64_t next;
  int rc;
  pthread_mutex_t mu;
} prefill_job;

static int prefill_sees(const prefill_job* J, int p, int t) {
  return t <= p && (J->window <= 0 || t >= p + 1 - J->window || t < J->sink);
}

static int prefill_one(const prefill_job* J, int b, int i, int h, double* o) {
  const orc_layout* L = J->L;
  int H = L->num_kv_heads, d = L->head_dim, G = J->Hq / H;
  int len = J->lens[b], nq = J->qstart[b + 1] - J->qstart[b];
  int64_t qrow = J->qstart[b] + i;
  int p = len - nq + i; /* the query's own position */
  const int32_t* table_row = J->tables + (int64_t)b * J->max_blocks;
  double qv[128];
  float row[128];
  for (int e = 0; e < d; ++e) qv[e] = q_elem(J->q, J->q_dtype, (qrow * J->Hq + h) * d + e);
  for (int e = 0; e < d; ++e) o[e] = 0.0;
  if (p < 0) return ORC_OK;
  double* sc = (double*)malloc(sizeof(double) * (size_t)(p + 1));
  double m = -INFINITY;
  for (int t = 0; t <= p; ++t) {
    if (!prefill_sees(J, p, t)) continue;
    int rc = orc_dequant_token(L, J->C, 0, table_row, len, b, t, h / G, row);
    if (rc) {
      free(sc);
      return rc;
    }
    double dot = 0.0;
    for (int e = 0; e < d; ++e) dot += qv[e] * (double)row[e];
    sc[t] = dot * J->sm;
    if (sc[t] > m) m = sc[t];
  }
  double l = 0.0;
  for (int t = 0; t <= p; ++t) {
    if (!prefill_sees(J, p, t)) continue;
    double w = exp(sc[t] - m);
    l += w;
    int rc = orc_dequant_token(L, J->C, 1, table_row, len, b, t, h / G, row);
    if (rc) {
      free(sc);
      return rc;
    }
    for (int e = 0; e < d; ++e) o[e] += w * (double)row[e];
  }
  free(sc);
  for (int e = 0; e < d; ++e) o[e] /= l;
  return ORC_OK;
}

static void* prefill_worker(void* arg) {
  prefill_job* J = (prefill_job*)arg;
  int64_t rows = J->qstart[J->batch];
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t item = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (item >= rows * J->Hq) break;
    int64_t r = item / J->Hq;
    int h = (int)(item % J->Hq);
    int b = 0;
    while (J->qstart[b + 1] <= r) ++b; /* the sequence holding row r */
    int rc = prefill_one(J, b, (int)(r - J->qstart[b]), h, J->out + item * J->L->head_dim);
    if (rc) {
      pthread_mutex_lock(&J->mu);
      J->rc = rc;
      pthread_mutex_unlock(&J->mu);
    }
  }
  return NULL;
}

int orc_prefill(const orc_layout* L, const orc_cache* C, const void* q, int32_t q_dtype,
                int32_t batch, int32_t num_q_heads, const int32_t* query_start,
                const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, int32_t window, int32_t sink,
                double sm_scale, double* out, int32_t num_threads) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (num_q_heads % L->num_kv_heads) return ORC_ERR_INVALID;
  for (int b = 0; b < batch; ++b) {
    int nq = query_start[b + 1] - query_start[b];
    if (nq < 0 || nq > context_lens[b]) return ORC_ERR_INVALID;
  }
  prefill_job J;
  J.L = L;
  J.C = C;
  J.q = q;
  J.q_dtype = q_dtype;
  J.batch = batch;
  J.Hq = num_q_heads;
  J.max_blocks = max_blocks_per_seq;
  J.qstart = query_start;
  J.tables = block_tables;
  J.lens = context_lens;
  J.window = window;
  J.sink = sink;
  J.sm = sm_scale != 0.0 ? sm_scale : 1.0 / sqrt((double)L->head_dim);
  J.out = out;
  J.next = 0;
  J.rc = ORC_OK;
  pthread_mutex_init(&J.mu, NULL);
  if (num_threads < 1) num_threads = 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)num_threads);
  for (int i = 0; i < num_threads; ++i) pthread_create(&th[i], NULL, prefill_worker, &J);
  for (int i = 0; i < num_threads; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  return J.rc;
}

/* ------------------------------------------------------------------------ */
/* Block pool [P3, "How vLLM Implements KV Cache Optimization": small fixed- */
/* size blocks handed to sequences on demand; P1, "Integrating Dynamic       */
/* Quantization with PagedAttention": a logical-to-physical block map per    */
/* sequence]. The pages give no allocation order; the one below is a reading */
/* chosen so that the result is unique.                                      */
/* ------------------------------------------------------------------------ */

int orc_pool_init(int32_t* stack, int32_t* top, const int32_t* order,
                  int64_t n) {
  for (int64_t i = 0; i < n; ++i) stack[i] = order ? order[i] : (int32_t)i;
  *top = (int32_t)n;
  return ORC_OK;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Sequence b needs ceil((L+n)/bs) - ceil(L/bs) new blocks. Needs are served in
 * batch order from the top of the stack: with off_b the blocks taken by
 * earlier sequences, b gets stack positions top-off_b-need_b .. top-off_b-1
 * in increasing position order as its next logical blocks. Slots of the new
 * positions follow in batch order. All or nothing. */
int orc_blocks_reserve(int32_t* stack, int32_t* top, int64_t capacity,
                       int32_t* tables, int32_t max_blocks,
                       const int32_t* lens, const int32_t* new_tokens,
                       int32_t batch, int32_t bs, int64_t* slots,
                       int32_t* lens_out, int32_t* status) {
  (void)capacity;
  int64_t total = 0;
  int fits = 1;
  for (int b = 0; b < batch; ++b) {
    int64_t have = ceil_div(lens[b], bs);
    int64_t want = ceil_div((int64_t)lens[b] + new_tokens[b], bs);
    if (want > max_blocks) fits = 0;
    total += want - have;
  }
  if (!fits || total > *top) {
    *status = ORC_ERR_OUT_OF_BLOCKS;
    return ORC_OK;
  }
  int64_t off = 0, tok = 0;
  for (int b = 0; b < batch; ++b) {
    int64_t have = ceil_div(lens[b], bs);
    int64_t need = ceil_div((int64_t)lens[b] + new_tokens[b], bs) - have;
    int32_t* row = tables + (int64_t)b * max_blocks;
    for (int64_t k = 0; k < need; ++k)
      row[have + k] = stack[*top - off - need + k];
    off += need;
    for (int64_t k = 0; k < new_tokens[b]; ++k) {
      int64_t pos = lens[b] + k;
      slots[tok++] = (int64_t)row[pos / bs] * bs + pos % bs;
    }
  }
  *top -= (int32_t)total;
  if (lens_out)
    for (int b = 0; b < batch; ++b) lens_out[b] = lens[b] + new_tokens[b];
  *status = ORC_OK;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Prefix sharing [P3, "How vLLM Implements KV Cache Optimization": requests */
/* sharing a system prompt keep one copy of its cached prefix; P2 glossary, */
/* "Evolution & History" and "Enterprise Use Cases": common prompt prefixes */
/* reused across requests]. refcount[id] counts the table entries that hold  */
/* block id (0 for a free block). A forked sequence shares its source's       */
/* blocks; a shared block that is only partly filled is copied before a     */
/* sequence appends into it (copy on write); a block returns to the free     */
/* stack when its last reference goes.                                       */
/* ------------------------------------------------------------------------ */

/* Fork k (in order): row dst[k] takes row src[k]'s length and its first
 * ceil(len / bs) table entries, each block's count growing by one.
 * Preconditions: destination rows are empty, distinct and not sources. */
int orc_blocks_fork(int32_t* refcount, int32_t* tables, int32_t max_blocks,
                    int32_t* lens, const int32_t* src, const int32_t* dst,
                    int32_t num_forks, int32_t bs) {
  for (int k = 0; k < num_forks; ++k) {
    int64_t nb = ceil_div(lens[src[k]], bs);
    for (int64_t i = 0; i < nb; ++i) {
      int32_t id = tables[(int64_t)src[k] * max_blocks + i];
      tables[(int64_t)dst[k] * max_blocks + i] = id;
      refcount[id] += 1;
    }
    lens[dst[k]] = lens[src[k]];
  }
  return ORC_OK;
}

/* Reservation with counts. Sequence b copies its last block first when it
 * appends (n > 0) into a partly filled block (L % bs != 0) whose count, at
 * the start of the call, exceeds one: need_b = (1 if it copies) +
 * ceil((L+n)/bs) - ceil(L/bs). Needs are served as in orc_blocks_reserve
 * (all or nothing, batch order, increasing stack position); a copying
 * sequence's first block replaces its last table entry and the pair (old,
 * new) is reported (in batch order) for the caller to copy the block's
 * contents. Every block taken gets count 1. After the allocation the copied
 * blocks lose one reference each, in batch order, and a block whose count
 * reaches zero is pushed back onto the stack. */
int orc_blocks_reserve_shared(int32_t* stack, int32_t* top, int64_t capacity,
                              int32_t* refcount, int32_t* tables, int32_t max_blocks,
                              const int32_t* lens, const int32_t* new_tokens,
                              int32_t batch, int32_t bs, int64_t* slots,
                              int32_t* lens_out, int32_t* cow_src, int32_t* cow_dst,
                              int32_t* cow_count, int32_t* status) {
  (void)capacity;
  int64_t total = 0;
  int fits = 1;
  int* cow = (int*)malloc(sizeof(int) * (size_t)(batch > 0 ? batch : 1));
  for (int b = 0; b < batch; ++b) {
    int64_t have = ceil_div(lens[b], bs);
    int64_t want = ceil_div((int64_t)lens[b] + new_tokens[b], bs);
    if (want > max_blocks) fits = 0;
    cow[b] = new_tokens[b] > 0 && lens[b] % bs != 0 &&
             refcount[tables[(int64_t)b * max_blocks + lens[b] / bs]] > 1;
    total += want - have + cow[b];
  }
  if (!fits || total > *top) {
    free(cow);
    *status = ORC_ERR_OUT_OF_BLOCKS;
    return ORC_OK;
  }
  int64_t off = 0, tok = 0;
  int ncow = 0;
  for (int b = 0; b < batch; ++b) {
    int64_t have = ceil_div(lens[b], bs);
    int64_t grow = ceil_div((int64_t)lens[b] + new_tokens[b], bs) - have;
    int64_t need = grow + cow[b];
    int32_t* row = tables + (int64_t)b * max_blocks;
    int64_t first = *top - off - need; /* the sequence's lowest stack position */
    if (cow[b]) {
      int32_t fresh = stack[first];
      cow_src[ncow] = row[lens[b] / bs];
      cow_dst[ncow] = fresh;
      ++ncow;
      row[lens[b] / bs] = fresh;
      refcount[fresh] = 1;
    }
    for (int64_t k = 0; k < grow; ++k) {
      row[have + k] = stack[first + cow[b] + k];
      refcount[row[have + k]] = 1;
    }
    off += need;
    for (int64_t k = 0; k < new_tokens[b]; ++k) {
      int64_t pos = lens[b] + k;
      slots[tok++] = (int64_t)row[pos / bs] * bs + pos % bs;
    }
  }
  *top -= (int32_t)total;
  for (int c = 0; c < ncow; ++c) {
    refcount[cow_src[c]] -= 1;
    if (refcount[cow_src[c]] == 0) stack[(*top)++] = cow_src[c];
  }
  *cow_count = ncow;
  if (lens_out)
    for (int b = 0; b < batch; ++b) lens_out[b] = lens[b] + new_tokens[b];
  free(cow);
  *status = ORC_OK;
  return ORC_OK;
}

/* Release with counts: the masked rows' blocks lose one reference each, in
 * batch order and, within a row, in logical order; a block whose count
 * reaches zero is pushed onto the stack at that moment. */
int orc_blocks_release_shared(int32_t* stack, int32_t* top, int64_t capacity,
                              int32_t* refcount, const int32_t* tables,
                              int32_t max_blocks, const int32_t* lens,
                              const int32_t* mask, int32_t batch, int32_t bs,
                              int32_t* lens_out, int32_t* status) {
  (void)capacity;
  for (int b = 0; b < batch; ++b) {
    if (!mask[b]) continue;
    int64_t nb = ceil_div(lens[b], bs);
    for (int64_t i = 0; i < nb; ++i) {
      int32_t id = tables[(int64_t)b * max_blocks + i];
      refcount[id] -= 1;
      if (refcount[id] == 0) stack[(*top)++] = id;
    }
  }
  if (lens_out)
    for (int b = 0; b < batch; ++b)
      if (mask[b]) lens_out[b] = 0;
  *status = ORC_OK;
  return ORC_OK;
}

/* Copy every plane of block src[k] to block dst[k] (one layer): codes,
 * scales and zero points; per-channel key scales per block. */
int orc_copy_blocks(const orc_layout* L, const orc_cache* C, const int32_t* src,
                    const int32_t* dst, int32_t n) {
  int rc = check_layout(L);
  if (rc) return rc;
  int64_t H = L->num_kv_heads, bs = L->block_size, d = L->head_dim;
  for (int k = 0; k < n; ++k) {
    for (int side = 0; side < 2; ++side) {
      int64_t rb = row_bytes(L, side);
      uint8_t* codes = (uint8_t*)(side ? C->v_codes : C->k_codes);
      memcpy(codes + (int64_t)dst[k] * H * bs * rb, codes + (int64_t)src[k] * H * bs * rb,
             (size_t)(H * bs * rb));
      int code = side_code(L, side), mode = side_mode(L, side);
      if (code == ORC_CODE_NONE16) continue;
      float* scale = side ? C->v_scale : C->k_scale;
      int64_t per = mode == ORC_CHANNEL_BLOCK ? H * d
                    : mode == ORC_GROUP_ASYM ? H * bs * (d / L->group_size)
                                             : H * bs;
      memcpy(scale + dst[k] * per, scale + src[k] * per, sizeof(float) * (size_t)per);
      if (mode == ORC_GROUP_ASYM) {
        uint8_t* zero = side ? C->v_zero : C->k_zero;
        memcpy(zero + dst[k] * per, zero + src[k] * per, (size_t)per);
      }
    }
  }
  return ORC_OK;
}

/* Block recycling under a sliding window [P3, "Cache Eviction and Compression
 * Strategies": with a window of the last N tokens, older tokens are dropped;
 * with sinks, the first tokens stay]. Queries from position L = lens[b] on
 * see positions t >= L + 1 - window and t < sink only, so block i of
 * sequence b is no longer needed when it holds no sink position
 * (i >= ceil(sink / bs)) and ends before the window ((i + 1) bs <=
 * L + 1 - window). Such blocks still in the table are pushed onto the
 * stack (batch order, logical order) and their entries set to -1. All or
 * nothing when the pushes would overflow the stack. */
int orc_blocks_trim(int32_t* stack, int32_t* top, int64_t capacity, int32_t* tables,
                    int32_t max_blocks, const int32_t* lens, int32_t window, int32_t sink,
                    int32_t batch, int32_t bs, int32_t* status) {
  int64_t total = 0;
  if (window > 0) {
    for (int b = 0; b < batch; ++b) {
      int64_t lo = ceil_div(sink, bs), hi = ((int64_t)lens[b] + 1 - window) / bs;
      if (lens[b] + 1 - window < 0) hi = 0;
      for (int64_t i = lo; i < hi && i < max_blocks; ++i)
        total += tables[(int64_t)b * max_blocks + i] >= 0;
    }
  }
  if (*top + total > capacity) {
    *status = ORC_ERR_OUT_OF_BLOCKS;
    return ORC_OK;
  }
  if (window > 0) {
    for (int b = 0; b < batch; ++b) {
      int64_t lo = ceil_div(sink, bs), hi = ((int64_t)lens[b] + 1 - window) / bs;
      if (lens[b] + 1 - window < 0) hi = 0;
      for (int64_t i = lo; i < hi && i < max_blocks; ++i) {
        int32_t* e = &tables[(int64_t)b * max_blocks + i];
        if (*e < 0) continue;
        stack[(*top)++] = *e;
        *e = -1;
      }
    }
  }
  *status = ORC_OK;
  return ORC_OK;
}

/* Offload of quantized blocks [P3, "KV Cache Offloading: Moving Data Between
 * GPU and CPU": inactive cache is moved to CPU memory and brought back when
 * needed, limited by the link's bandwidth; "quantize first": quantized blocks
 * cross the link in 2-4x fewer bytes]. A packed block is the block's slice
 * of every plane of one layer, in the order k_codes, v_codes, k_scale,
 * v_scale, k_zero, v_zero (planes the layout does not have take no bytes);
 * block k of a pack starts at k * orc_block_pack_bytes. */
static int64_t plane_block_bytes(const orc_layout* L, int plane) {
  int64_t H = L->num_kv_heads, bs = L->block_size, d = L->head_dim;
  int side = plane & 1;
  int code = side_code(L, side), mode = side_mode(L, side);
  if (plane < 2) return H * bs * row_bytes(L, side);
  if (code == ORC_CODE_NONE16) return 0;
  int64_t per = mode == ORC_CHANNEL_BLOCK ? H * d
                : mode == ORC_GROUP_ASYM ? H * bs * (d / L->group_size)
                                         : H * bs;
  if (plane < 4) return per * 4;
  return mode == ORC_GROUP_ASYM ? per : 0;
}

int64_t orc_block_pack_bytes(const orc_layout* L) {
  if (check_layout(L)) return ORC_ERR_INVALID;
  int64_t total = 0;
  for (int p = 0; p < 6; ++p) total += plane_block_bytes(L, p);
  return total;
}

static uint8_t* plane_base(const orc_cache* C, int plane) {
  void* b[6] = {C->k_codes, C->v_codes, C->k_scale, C->v_scale, C->k_zero, C->v_zero};
  return (uint8_t*)b[plane];
}

int orc_pack_blocks(const orc_layout* L, const orc_cache* C, const int32_t* ids, int32_t n,
                    uint8_t* dst) {
  int rc = check_layout(L);
  if (rc) return rc;
  int64_t pack = orc_block_pack_bytes(L);
  for (int k = 0; k < n; ++k) {
    if (ids[k] < 0 || ids[k] >= C->num_blocks) return ORC_ERR_INVALID;
    uint8_t* out = dst + (int64_t)k * pack;
    for (int p = 0; p < 6; ++p) {
      int64_t per = plane_block_bytes(L, p);
      if (!per) continue;
      memcpy(out, plane_base(C, p) + (int64_t)ids[k] * per, (size_t)per);
      out += per;
    }
  }
  return ORC_OK;
}

int orc_unpack_blocks(const orc_layout* L, const orc_cache* C, const uint8_t* src,
                      const int32_t* ids, int32_t n) {
  int rc = check_layout(L);
  if (rc) return rc;
  int64_t pack = orc_block_pack_bytes(L);
  for (int k = 0; k < n; ++k) {
    if (ids[k] < 0 || ids[k] >= C->num_blocks) return ORC_ERR_INVALID;
    const uint8_t* in = src + (int64_t)k * pack;
    for (int p = 0; p < 6; ++p) {
      int64_t per = plane_block_bytes(L, p);
      if (!per) continue;
      memcpy(plane_base(C, p) + (int64_t)ids[k] * per, in, (size_t)per);
      in += per;
    }
  }
  return ORC_OK;
}

/* Released sequences push their blocks back in batch order, each in logical
 * order. All or nothing when the pushes would overflow the stack. */
int orc_blocks_release(int32_t* stack, int32_t* top, int64_t capacity,
                       const int32_t* tables, int32_t max_blocks,
                       const int32_t* lens, const int32_t* mask, int32_t batch,
                       int32_t bs, int32_t* lens_out, int32_t* status) {
  int64_t total = 0;
  for (int b = 0; b < batch; ++b)
    if (mask[b]) total += ceil_div(lens[b], bs);
  if (*top + total > capacity) {
    *status = ORC_ERR_OUT_OF_BLOCKS;
    return ORC_OK;
  }
  int64_t pos = *top;
  for (int b = 0; b < batch; ++b) {
    if (!mask[b]) continue;
    int64_t nblk = ceil_div(lens[b], bs);
    for (int64_t k = 0; k < nblk; ++k)
      stack[pos++] = tables[(int64_t)b * max_blocks + k];
  }
  *top = (int32_t)pos;
  if (lens_out)
    for (int b = 0; b < batch; ++b)
      if (mask[b]) lens_out[b] = 0;
  *status = ORC_OK;
  return ORC_OK;
}
