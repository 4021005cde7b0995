// kvq_decode.hip -- split-K paged decode attention over quantized blocks with
// in-register dequantization (gfx950).
//
// What is computed ("KV Cache Optimization" glossary, "Technical
// Architecture", stage 4: the attention kernel dequantizes KV blocks on the
// fly while decoding; "Dynamic KV Cache Quantization for Fast LLM Inference",
// section "Recap of KV Caching": the current query attends over its
// sequence's cached keys and values): for each sequence b and query head h,
// out = sum_t p_t v_t / sum_t p_t with p_t = exp(s_t - max s) and
// s_t = (q . k_t) * sm_scale, over the first context_lens[b] tokens, keys and
// values dequantized from their codes and scales. Online softmax across blocks
// and a log-sum-exp merge across splits follow the Flash-Attention style named
// in "KV Cache Optimization: Strategies for Faster LLM Inference", section
// "Implementing KV Cache Optimization: A Practical Checklist".
//
// Design. Decode is HBM-bound (the same page, "Common pitfalls": decode is
// memory-bound), so the kernel streams each code byte once:
//  * One workgroup of four waves per work item (sequence b, KV head g, split
//    j of split_blocks cache blocks); each wave streams a consecutive quarter
//    of the split and the four softmax states merge through LDS, so the
//    global partials stay few. The G query heads that share KV head g are the
//    16 columns of the MFMA tiles (zero-padded when G < 16).
//  * Scores: S[16 tokens x 16 heads] = K_tile . Q^T with
//    v_mfma_f32_16x16x32_f16. Lane (r, j) = (lane % 16, lane / 16) feeds
//    token r of the tile with elements [j d/4, (j+1) d/4) of its key row,
//    loaded as 16-byte vectors; Q uses the same element assignment.
//  * INT8, E4M3 and INT4 codes are all exactly representable in fp16, so
//    codes are converted in registers (E4M3 by the hardware converter, INT8
//    by the 0x64 exponent trick) and scales are applied after the products:
//    the key scale multiplies the score, the value scale multiplies the
//    probability before it is rounded to fp16.
//  * The accumulator layout of S (lane holds tokens 4j..4j+3 of head r) is
//    exactly the B operand of O^T[d x heads] += V^T[d x 16] . P^T[16 x heads]
//    (v_mfma_f32_16x16x16_f16), so probabilities never leave registers. Lane
//    (r, j) feeds value bytes [r d/16, (r+1) d/16) of tokens 4j..4j+3 and
//    ends up owning outputs [j d/4, (j+1) d/4) of head r.
//  * The query is pre-scaled per head by a power of two into [1, 2) before
//    its fp16 conversion (exact for bf16 values within 2^14 of the head's
//    largest element); the factor returns in the score scale.
//  * A ring of three register buffers keeps two cache blocks in flight while
//    the wave computes on a third; block ids come from one vector load per 64
//    blocks of the split and are read with v_readlane.
//  * Partials (m, l, acc) per split go to the workspace; decode_reduce merges
//    them with the log-sum-exp rule.
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
};

// ---- split planning ---------------------------------------------------------
// Every workgroup of the split kernel and every wave of the reduce derive the
// same plan from context_lens alone, so neither a planning launch nor a host
// synchronization is needed:
//   n_b  = ceil(min(len_b, max_len) / BS)          blocks of sequence b
//   S    = split_blocks, or kDecodeWaves * clamp(ceil(H sum_b n_b / 2^12),
//          ceil(32 / BS), 64)                        blocks per split
//   ns_b = ceil(n_b / S)                            splits of sequence b
// Items (b, j), j < ns_b, are numbered sequence-major. The partial of item
// (b, j) for query head h is row Hq off_b + h ns_b + j of the workspace, with
// off_b = sum_{b' < b} ns_b', so one head's splits are adjacent. The host
// bounds sum_b ns_b from batch and max_len alone (the grid and workspace
// size). Short sequences thus get few splits and the total work is cut into
// about 4096 wave shares whatever the length mix.
struct PlanArgs {
  const int32_t* lens;
  int32_t batch, max_len, bs, H, split_blocks;
};

__device__ __forceinline__ PlanArgs plan_args(const int32_t* lens, int batch, int max_len,
                                              int bs, int H, int split_blocks) {
  PlanArgs p;
  p.lens = lens;
  p.batch = batch;
  p.max_len = max_len;
  p.bs = bs;
  p.H = H;
  p.split_blocks = split_blocks;
  return p;
}

// Cut length of sequence idx (0 past the batch).
__device__ __forceinline__ int plan_len(const PlanArgs& p, int idx) {
  return idx < p.batch ? min(max(p.lens[idx], 0), p.max_len) : 0;
}

// Cut lengths of sequences c0 + 64 u + lane, u < 4, with the four loads
// issued back to back (clamped indices; the empty asm keeps the compiler
// from moving each load into its own branch and wait).
__device__ __forceinline__ void plan_len4(const PlanArgs& p, int c0, int lane, int* len) {
  int v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = p.lens[min(c0 + u * kWave + lane, p.batch - 1)];
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
#pragma unroll
  for (int u = 0; u < 4; ++u)
    len[u] = c0 + u * kWave + lane < p.batch ? min(max(v[u], 0), p.max_len) : 0;
}

// Inclusive prefix sum over the wave with DPP moves (no LDS round trips):
// shifts 1, 2, 4, 8 within each row of 16 lanes, then the last lane of row 0
// and row 2 into rows 1 and 3, then lane 31 into rows 2 and 3. Lanes with no
// source read 0 (the `old` operand).
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
  (void)lane;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ int wave_sum(int x, int lane) {
  return __builtin_amdgcn_readlane(wave_incl_scan(x, lane), kWave - 1);
}

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

// Lengths of sequences c0 + 64 u + lane, u < 4. The first 256 are loaded
// once (len0) and reused by both passes below.
__device__ __forceinline__ void plan_chunk(const PlanArgs& p, int c0, int lane, const int* len0,
                                           int* len) {
  if (c0 == 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) len[u] = len0[u];
  } else {
    plan_len4(p, c0, lane, len);
  }
}

__device__ __forceinline__ int plan_splits_of(const PlanArgs& p, int len, int S) {
  return ((len + p.bs - 1) / p.bs + S - 1) / S;
}

// Blocks per split: the caller's, or planned from the total block count.
// Max over the wave of non-negative ints (DPP, as wave_incl_scan).
template <bool MAX>
__device__ __forceinline__ int wave_reduce_i(int x) {
  const int idle = MAX ? 0 : INT32_MAX;
#define KVQ_DPP_STEP(ctrl, rmask)                                                         \
  {                                                                                        \
    const int y = __builtin_amdgcn_update_dpp(idle, x, ctrl, rmask, 0xF, false);          \
    x = MAX ? max(x, y) : min(x, y);                                                       \
  }
  KVQ_DPP_STEP(0x111, 0xF);
  KVQ_DPP_STEP(0x112, 0xF);
  KVQ_DPP_STEP(0x114, 0xF);
  KVQ_DPP_STEP(0x118, 0xF);
  KVQ_DPP_STEP(0x142, 0xA);
  KVQ_DPP_STEP(0x143, 0xC);
#undef KVQ_DPP_STEP
  return __builtin_amdgcn_readlane(x, kWave - 1);
}

// Blocks per split: the caller's, or planned from the block counts. A batch
// whose non-empty sequences have nearly equal block counts (max <= 9/8 min)
// is cut into one round of shares (2^kDecodeUniformWavesLog2 waves: two
// workgroups per CU, up to kDecodeMaxWaveBlocks blocks each), since equal
// items need no balancing and fewer, longer shares pay the start-up chain
// less often; any other batch into twice as many shorter shares (at most 64
// blocks), which the dispatcher balances.
__device__ __forceinline__ int plan_split_blocks(const PlanArgs& p, int lane, const int* len0) {
  if (p.split_blocks > 0) return p.split_blocks;
  // block counts fit in int32: the host bounds batch * ceil(max_len / bs)
  int tot32 = 0, nmax = 0, nmin = INT32_MAX;
  for (int c0 = 0; c0 < p.batch; c0 += 4 * kWave) {
    int len[4];
    plan_chunk(p, c0, lane, len0, len);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = (len[u] + p.bs - 1) / p.bs;
      tot32 += n;
      nmax = max(nmax, n);
      if (n > 0) nmin = min(nmin, n);
    }
  }
  const int64_t tot = wave_sum(tot32, lane);
  nmax = wave_reduce_i<true>(nmax);
  nmin = wave_reduce_i<false>(nmin);
  const bool uniform = (int64_t)nmax * 8 <= (int64_t)nmin * 9;
  const int lg = uniform ? kDecodeUniformWavesLog2 : kDecodeTargetWavesLog2;
  const int cap = uniform ? kDecodeMaxWaveBlocks : 64;
  int64_t w = (tot * p.H + (int64_t(1) << lg) - 1) >> lg;
  const int wmin = (kDecodeMinWaveTokens + p.bs - 1) / p.bs;
  w = w < wmin ? wmin : w > cap ? cap : w;
  return kDecodeWaves * (int)w;
}

struct PlanItem {
  int b;    // sequence
  int len;  // its cut length
  int j;    // split within the sequence
  int ns;   // splits of the sequence
  int off;  // splits of all earlier sequences
  int S;    // blocks per split
};

// Item `item` of the plan; false past the last item.
__device__ __forceinline__ bool plan_find_item(const PlanArgs& p, int item, int lane,
                                               PlanItem& out) {
  int len0[4];
  plan_len4(p, 0, lane, len0);
  const int S = plan_split_blocks(p, lane, len0);
  out.S = S;
  int off = 0;
  for (int c0 = 0; c0 < p.batch; c0 += 4 * kWave) {
    int len[4];
    plan_chunk(p, c0, lane, len0, len);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ns = plan_splits_of(p, len[u], S);
      const int incl = wave_incl_scan(ns, lane);
      const int tot = __builtin_amdgcn_readlane(incl, kWave - 1);
      if (item < off + tot) {
        const int f = __builtin_ctzll(__ballot(off + incl > item));
        out.b = c0 + u * kWave + f;
        out.len = __builtin_amdgcn_readlane(len[u], f);
        out.ns = __builtin_amdgcn_readlane(ns, f);
        out.off = off + __builtin_amdgcn_readlane(incl, f) - out.ns;
        out.j = item - out.off;
        return out.b < p.batch;   // always, for consistent lengths
      }
      off += tot;
    }
  }
  return false;
}

// Splits of sequence b and of all sequences before it.
__device__ __forceinline__ void plan_sequence(const PlanArgs& p, int b, int lane, int& off,
                                              int& ns) {
  int len0[4];
  plan_len4(p, 0, lane, len0);
  const int S = plan_split_blocks(p, lane, len0);
  int acc = 0;
  for (int c0 = 0; c0 < b; c0 += 4 * kWave) {
    int len[4];
    plan_chunk(p, c0, lane, len0, len);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc += c0 + u * kWave + lane < b ? plan_splits_of(p, len[u], S) : 0;
  }
  off = wave_sum(acc, lane);
  ns = plan_splits_of(p, plan_len(p, b), S);
}

// Block ids of blocks [i0, ilast] of one sequence, 64 at a time: lane k of
// `cur` holds the id of block base + k and lane k of `nxt` that of block
// base + 64 + k (indices past ilast read ilast). A wave asks only for blocks
// in [base, base + 128) and calls advance() once it has passed base + 64, so
// each 64-id load is issued 64 blocks before its first use.
struct IdWindow {
  const int32_t* row;
  int base, ilast;
  int32_t cur, nxt;
  __device__ __forceinline__ void init(const int32_t* trow, int i0, int il, int lane) {
    row = trow;
    base = i0;
    ilast = il;
    cur = row[min(i0 + lane, il)];
    nxt = row[min(i0 + kWave + lane, il)];
  }
  __device__ __forceinline__ int32_t id(int i) const {
    const int k = min(i, ilast) - base;
    return __builtin_amdgcn_readlane(k < kWave ? cur : nxt, k & (kWave - 1));
  }
  __device__ __forceinline__ void advance(int lane) {
    base += kWave;
    cur = nxt;
    nxt = row[min(base + kWave + lane, ilast)];
  }
};

// Per-lane data of one cache block (BS tokens) for 8-bit codes.
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

// KCH: keys carry one scale per channel for the whole block
// (CHANNEL_BLOCK_SYM), loaded as D/64 consecutive floats per lane.
template <int D, int BS, bool KCH>
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
        u32x2 w = *reinterpret_cast<const u32x2*>(vr);
        t.v[nt][i][0] = w.x;
        t.v[nt][i][1] = w.y;
      } else {
        t.v[nt][i][0] = *reinterpret_cast<const uint32_t*>(vr);
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
// the gfx950 lane-swap instructions instead of LDS permutes.
__device__ __forceinline__ float colmax4(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
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

// Eight raw 16-bit key values to fp16 operands: bf16 values are exact in
// fp16 within its range (the same bound as for value scales).
__device__ __forceinline__ half8v raw8_to_h8(const u32x4& w, bool bf16) {
  if (!bf16) return __builtin_bit_cast(half8v, w);
  half8v o;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    o[2 * u] = (half_t)bf16_lo(w[u]);
    o[2 * u + 1] = (half_t)bf16_hi(w[u]);
  }
  return o;
}

// Where the keys of a tile come from.
enum KeySource {
  kKeyTokenScale = 0,  // codes; the score takes the token's key scale
  kKeyChannel = 1,     // codes; per-channel scales are already in the query
  kKeyRaw = 2,         // raw staged rows, kraw[c] = elements of chunk c
};

// One 16-token tile: scores, online softmax, PV. TAIL handles the tile that
// ends past the sequence length: scores of tokens at or past L (this lane's
// column limit) are masked, and value codes of tokens at or past Lv (the rows
// that hold data; Lv < 0 means L) are zeroed, since they may hold NaN bytes.
// In decode both limits are the length; causal multi-query columns differ in
// L while sharing the value operand, so only rows past the data are zeroed.
template <int CODE, int D, int BS, bool TAIL, int KSRC = kKeyTokenScale>
__device__ __forceinline__ void tile_step(const Tile8<D, BS>& t, int nt, int pos0, int L,
                                          const half8v* qop, float cscore, int j,
                                          SoftmaxState<D>& st, const u32x4* kraw = nullptr,
                                          bool raw_bf16 = false, const half8v* qlo = nullptr,
                                          int Lv = -1) {
  constexpr int NCH = D / 32;
  constexpr int NPV = D / 16;
  const int Ld = Lv < 0 ? L : Lv;
  float4v S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    half8v kop;
    if constexpr (KSRC == kKeyRaw) {
      kop = raw8_to_h8(kraw[c], raw_bf16);
    } else {
      const u32x4& kw = t.k[nt][c / 2];
      const uint32_t lo = (c & 1) ? kw.z : kw.x;
      const uint32_t hi = (c & 1) ? kw.w : kw.y;
      kop = codes8_to_h8<CODE>(lo, hi);
    }
    S = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[c], S, 0, 0, 0);
    if constexpr (KSRC == kKeyChannel)  // low half of the split query
      S = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qlo[c], S, 0, 0, 0);
  }
  bool ok[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ok[e] = !TAIL || pos0 + 4 * j + e < L;
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
      const float qp = qs[8 * c + e] * (e < 4 ? s0[e] : s1[e - 4]);
      const half_t hi = (half_t)qp;
      qop[c][e] = hi;
      qlo[c][e] = (half_t)(qp - (float)hi);
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
                                                bool raw_bf16 = false) {
  constexpr int KS = KRAW ? kKeyRaw : kKeyTokenScale;
#pragma unroll
  for (int nt = 0; nt < BS / 16; ++nt) {
    const int pos0 = i * BS + nt * 16;
    const u32x4* kr = KRAW ? kraw[nt] : nullptr;
    if (pos0 + 16 <= L)
      tile_step<CODE, D, BS, false, KS>(t, nt, pos0, L, qop, cscore, j, st, kr, raw_bf16);
    else if (pos0 < L)
      tile_step<CODE, D, BS, true, KS>(t, nt, pos0, L, qop, cscore, j, st, kr, raw_bf16);
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
// 16-bit passthrough (KVQ_CODE_NONE16): rows hold the source values. Keys
// enter the score MFMA as fp16 like the staged rows above (lane (r, j):
// elements [j d/4, (j+1) d/4) of token r). Values: lane (r, j) loads
// elements [r d/16, (r+1) d/16) of tokens 4j..4j+3, and the operand of PV
// MFMA c is element c of those four tokens -- the same output mapping as
// the 8-bit codes. bf16 values convert to fp16 exactly within fp16's range.
// ---------------------------------------------------------------------------
template <int D, int BS>
struct TileRaw {
  static constexpr int NT = BS / 16;
  static constexpr int NCH = D / 32;   // 16-byte key vectors per lane per tile
  static constexpr int VW = D / 32;    // 32-bit value words per token per lane
  u32x4 k[NT][NCH];
  uint32_t v[NT][4][VW];               // [tile][token i][word]
};

template <int D, int BS>
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
        const u32x4 w = *reinterpret_cast<const u32x4*>(vr);
        t.v[nt][i][0] = w.x; t.v[nt][i][1] = w.y; t.v[nt][i][2] = w.z; t.v[nt][i][3] = w.w;
      } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(vr);
        t.v[nt][i][0] = w.x; t.v[nt][i][1] = w.y;
      }
    }
  }
}

// Element c (0 or 1 of word w) of four tokens' value words as fp16.
__device__ __forceinline__ half4v raw_vop(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                          bool hi, bool bf16) {
  half4v o;
  if (bf16) {
    o[0] = (half_t)(hi ? bf16_hi(w0) : bf16_lo(w0));
    o[1] = (half_t)(hi ? bf16_hi(w1) : bf16_lo(w1));
    o[2] = (half_t)(hi ? bf16_hi(w2) : bf16_lo(w2));
    o[3] = (half_t)(hi ? bf16_hi(w3) : bf16_lo(w3));
  } else {
    const uint32_t sel = hi ? 0x07060302u : 0x05040100u;
    const uint32_t x = __builtin_amdgcn_perm(w1, w0, sel), y = __builtin_amdgcn_perm(w3, w2, sel);
    o = __builtin_bit_cast(half4v, (u32x2){x, y});
  }
  return o;
}

template <int D, int BS, bool TAIL>
__device__ __forceinline__ void tile_step_raw(const TileRaw<D, BS>& t, int nt, int pos0, int L,
                                              const half8v* qop, float cscore, int j,
                                              SoftmaxState<D>& st, bool bf16, int Lv = -1) {
  constexpr int NCH = D / 32;
  constexpr int NPV = D / 16;
  const int Ld = Lv < 0 ? L : Lv;   // as in tile_step
  float4v S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    S = __builtin_amdgcn_mfma_f32_16x16x32_f16(raw8_to_h8(t.k[nt][c], bf16), qop[c], S, 0, 0, 0);
  bool ok[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ok[e] = !TAIL || pos0 + 4 * j + e < L;
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
  half4v pop;
#pragma unroll
  for (int e = 0; e < 4; ++e) pop[e] = (half_t)p[e];
#pragma unroll
  for (int c = 0; c < NPV; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = t.v[nt][i][c / 2];
      if (TAIL && pos0 + 4 * j + i >= Ld) w[i] = 0u;   // rows past the data may hold NaN
    }
    st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(raw_vop(w[0], w[1], w[2], w[3], c & 1, bf16),
                                                      pop, st.acc[c], 0, 0, 0);
  }
}

// Tile-type dispatch for the block streaming below.
template <int D, int BS, bool KCH>
__device__ __forceinline__ void load_tile(Tile8<D, BS>& t, const DecodeArgs& a, int64_t bh,
                                          int lane) {
  load_tile8<D, BS, KCH>(t, a, bh, lane);
}
template <int D, int BS, bool KCH>
__device__ __forceinline__ void load_tile(TileRaw<D, BS>& t, const DecodeArgs& a, int64_t bh,
                                          int lane) {
  load_tile_raw<D, BS>(t, a, bh, lane);
}

// One wave's share of a split: blocks [i0, i1) of sequence b, KV head g.
// Leaves the running softmax state in st. KCH: per-channel key scales
// (CHANNEL_BLOCK_SYM), the partial last block's keys read raw from stage
// row b; `lds` is the wave's own scratch of at least D floats.
template <int CODE, int D, int BS, bool KCH = false>
__device__ __forceinline__ void wave_blocks(const DecodeArgs& a, int b, int g, int L, int nblk,
                                            int i0, int i1, int lane, SoftmaxState<D>& st,
                                            float* lds) {
  constexpr int NCH = D / 32;   // k-chunks of the score MFMA
  constexpr int NBUF = BS == 16 ? 3 : 2;  // blocks in the register ring
  const int r = lane & 15, j = lane >> 4;
  const int ilast = i1 - 1;

  // ---- query: heads g*G + r, elements [j d/4, (j+1) d/4) ----------------
  const bool hcol = r < a.G;
  const int h = g * a.G + (hcol ? r : 0);
  float qf[D / 4];
  {
    const uint16_t* qp = a.q + ((int64_t)b * a.Hq + h) * D + j * (D / 4);
    if (a.q_bf16)
      load_query<true, D>(qp, qf);
    else
      load_query<false, D>(qp, qf);
  }
  float qmax = 0.0f;
#pragma unroll
  for (int e = 0; e < D / 4; ++e) qmax = fmaxf(qmax, fabsf(qf[e]));
  qmax = colmax4(qmax);
  int qe = qmax > 0.0f ? (int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127 : 0;
  qe = max(qe, -126);
  const float qdown = __uint_as_float((uint32_t)(127 - qe) << 23);  // 2^-qe
  const float qup = __uint_as_float((uint32_t)(127 + qe) << 23);    // 2^qe
  // qs: the scaled query in fp32; qop: its fp16 operand (with per-channel
  // keys it is only needed for the raw partial block, so it is made there)
#pragma unroll
  for (int e = 0; e < D / 4; ++e) qf[e] = hcol ? qf[e] * qdown : 0.0f;
  const float* qs = qf;
  half8v qop[NCH];
  if constexpr (!KCH) {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[c][e] = (half_t)qs[8 * c + e];
  }
  const float cscore = hcol ? qup * a.sm_log2 : 0.0f;

  // Block ids arrive 64 at a time with one vector load and reach the scalar
  // unit through v_readlane. Ids outside the pool (a broken precondition)
  // are clamped to block 0 so that no load leaves the cache planes.
  IdWindow ids;
  ids.init(a.block_tables + (int64_t)b * a.max_blocks, i0, ilast, lane);
  // Prefetches past the share's last block (the ring's final refills, never
  // computed on) read physical block 0, which every wave shares, so they hit
  // in cache instead of fetching a block from HBM again.
  auto bh_of = [&](int i) -> int64_t {
    const int32_t id = ids.id(i);
    const bool ok = i <= ilast && id >= 0 && id < a.num_blocks;
    return (int64_t)(ok ? id : 0) * a.H + g;
  };
  constexpr bool RAW = CODE == KVQ_CODE_NONE16;
  using TileT = typename std::conditional<RAW, TileRaw<D, BS>, Tile8<D, BS>>::type;
  const bool raw_bf16 = a.stage_bf16 != 0;
  auto block = [&](const TileT& t, int i) {
    if constexpr (RAW) {
#pragma unroll
      for (int nt = 0; nt < BS / 16; ++nt)
        tile_step_raw<D, BS, false>(t, nt, i * BS + nt * 16, L, qop, cscore, j, st, raw_bf16);
    } else if constexpr (KCH) {
      half8v qb[NCH], ql[NCH];
      channel_query<D, BS>(t, lds, qs, lane, qb, ql);
      full_block_step<CODE, D, BS, kKeyChannel>(t, i, L, qb, cscore, j, st, ql);
    } else {
      full_block_step<CODE, D, BS>(t, i, L, qop, cscore, j, st);
    }
  };
  // blocks [i0, ifull) are complete; a partial last block is handled apart
  const bool partial = i1 == nblk && (L % BS) != 0;
  const int ifull = partial ? i1 - 1 : i1;
  TileT buf[NBUF];
#pragma unroll
  for (int u = 0; u < NBUF; ++u) load_tile<D, BS, KCH>(buf[u], a, bh_of(i0 + u), lane);

  // Steady state: every slot computes one block and refills its buffer with
  // the block NBUF ahead (clamped to the split's last block, so the load
  // sequence never branches and the wait counts stay exact).
  int i = i0;
  for (; i + NBUF <= ifull; i += NBUF) {
    if (i - ids.base >= kWave) ids.advance(lane);
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      block(buf[u], i + u);
      load_tile<D, BS, KCH>(buf[u], a, bh_of(i + u + NBUF), lane);
    }
  }
  // Remainder: fewer than NBUF complete blocks, already in buf[0 ..], then
  // the partial block, if any, which sits in the next buffer. Per-channel
  // keys of the partial block are the staged rows of sequence b (rows past
  // the length are masked).
  u32x4 kraw[BS / 16][NCH];
  if constexpr (KCH) {
    if (partial) {
#pragma unroll
      for (int nt = 0; nt < BS / 16; ++nt) {
        const uint16_t* sp =
            a.k_stage + (((int64_t)b * a.H + g) * BS + nt * 16 + r) * D + j * (D / 4);
#pragma unroll
        for (int c = 0; c < NCH; ++c) kraw[nt][c] = *reinterpret_cast<const u32x4*>(sp + 8 * c);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NBUF; ++u) {
    if (i + u < ifull) {
      block(buf[u], i + u);
    } else if (i + u == ifull && partial) {
      if constexpr (RAW) {
#pragma unroll
        for (int nt = 0; nt < BS / 16; ++nt) {
          const int pos0 = (i + u) * BS + nt * 16;
          if (pos0 + 16 <= L)
            tile_step_raw<D, BS, false>(buf[u], nt, pos0, L, qop, cscore, j, st, raw_bf16);
          else if (pos0 < L)
            tile_step_raw<D, BS, true>(buf[u], nt, pos0, L, qop, cscore, j, st, raw_bf16);
        }
      } else if constexpr (KCH) {
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) qop[c][e] = (half_t)qs[8 * c + e];
        last_block_step<CODE, D, BS, true>(buf[u], i + u, L, qop, cscore, j, st, kraw,
                                           a.stage_bf16 != 0);
      } else {
        last_block_step<CODE, D, BS>(buf[u], i + u, L, qop, cscore, j, st);
      }
    }
  }
}

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
  float sk[4 * SG];    // key scales of tokens 4j + e, index 4 group + e
  float sv[4 * SG];    // value scales, same order
  uint32_t zk;         // key zero points of token r, byte c = group c
  uint32_t zv[NS];     // value zero points of tokens 4j..4j+3 ([token][group] bytes)
};

template <int D, int BS, int MODE>
__device__ __forceinline__ void load_tile4(Tile4<D, MODE>& t, const DecodeArgs& a, int64_t bh,
                                           int nt, int lane) {
  constexpr int NS = D / 32;
  constexpr int RB = D / 2;  // bytes per row
  const int r = lane & 15, j = lane >> 4;
  const int64_t row0 = bh * BS + nt * 16;   // first token of the tile
  const uint8_t* kr = a.k_codes + (row0 + r) * RB + j * (RB / 4);
  if constexpr (NS == 4) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(kr);
    t.k[0] = w.x; t.k[1] = w.y; t.k[2] = w.z; t.k[3] = w.w;
  } else {
    const u32x2 w = *reinterpret_cast<const u32x2*>(kr);
    t.k[0] = w.x; t.k[1] = w.y;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint8_t* vr = a.v_codes + (row0 + 4 * j + e) * RB + r * (RB / 16);
    if constexpr (NS == 4)
      t.v[e] = *reinterpret_cast<const uint32_t*>(vr);
    else
      t.v[e] = *reinterpret_cast<const uint16_t*>(vr);
  }
  if constexpr (MODE == KVQ_SCALE_GROUP_ASYM) {
    // the planes hold [token][group]; the tile keeps [group][token]
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const float4v ks = *reinterpret_cast<const float4v*>(a.k_scale + (row0 + 4 * j) * NS + 4 * u);
      const float4v vs = *reinterpret_cast<const float4v*>(a.v_scale + (row0 + 4 * j) * NS + 4 * u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 4 * u + e, tok = f / NS, grp = f % NS;
        t.sk[4 * grp + tok] = ks[e];
        t.sv[4 * grp + tok] = vs[e];
      }
    }
    if constexpr (NS == 4) {
      t.zk = *reinterpret_cast<const uint32_t*>(a.k_zero + (row0 + r) * NS);
      const u32x4 z = *reinterpret_cast<const u32x4*>(a.v_zero + (row0 + 4 * j) * NS);
      t.zv[0] = z.x; t.zv[1] = z.y; t.zv[2] = z.z; t.zv[3] = z.w;
    } else {
      t.zk = *reinterpret_cast<const uint16_t*>(a.k_zero + (row0 + r) * NS);
      const u32x2 z = *reinterpret_cast<const u32x2*>(a.v_zero + (row0 + 4 * j) * NS);
      t.zv[0] = z.x; t.zv[1] = z.y;
    }
  } else {
    const float4v ks = *reinterpret_cast<const float4v*>(a.k_scale + row0 + 4 * j);
    const float4v vs = *reinterpret_cast<const float4v*>(a.v_scale + row0 + 4 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t.sk[e] = ks[e];
      t.sv[e] = vs[e];
    }
    t.zk = 0;
#pragma unroll
    for (int u = 0; u < NS; ++u) t.zv[u] = 0;
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
__device__ __forceinline__ half2v nib2(uint32_t g, uint32_t m, uint32_t o) {
  return __builtin_bit_cast(half2v, ((g >> SHIFT) & m) | o);
}

// Register-resident constants of the 4-bit conversions.
struct Nib4Consts {
  uint32_t m;    // 0x000F000F
  uint32_t o;    // 0x64006400
  uint32_t m64;  // 0x64646464, the fp16 exponent byte for v_perm
};
__device__ __forceinline__ Nib4Consts nib4_consts() {
  Nib4Consts k{0x000F000Fu, 0x64006400u, 0x64646464u};
  asm volatile("" : "+v"(k.m), "+v"(k.o), "+v"(k.m64));
  return k;
}

template <int D, int MODE, bool TAIL>
__device__ __forceinline__ void tile4_step(const Tile4<D, MODE>& t, int pos0, int L,
                                           const half8v* qop, float cscore, int j,
                                           SoftmaxState<D>& st, const Nib4Consts& kc) {
  constexpr bool tail = TAIL;
  constexpr int NS = D / 32;
  constexpr bool ASYM = MODE == KVQ_SCALE_GROUP_ASYM;
  // ---- key operands, chunk c = slice c -----------------------------------
  uint32_t g[4];
  if constexpr (NS == 4) {
    transpose4x4(t.k[0], t.k[1], t.k[2], t.k[3], g);
  } else {
    g[0] = __builtin_amdgcn_perm(t.k[1], t.k[0], 0x06040200u);
    g[1] = __builtin_amdgcn_perm(t.k[1], t.k[0], 0x07050301u);
  }
  float4v S[ASYM ? NS : 1];
#pragma unroll
  for (int c = 0; c < (ASYM ? NS : 1); ++c) S[c] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
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
    S[ASYM ? c : 0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qop[c], S[ASYM ? c : 0], 0, 0, 0);
  }
  bool ok[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ok[e] = !tail || pos0 + 4 * j + e < L;
  float s[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = 0.0f;
    if constexpr (ASYM) {
#pragma unroll
      for (int c = 0; c < NS; ++c) v = __builtin_fmaf(S[c][e], t.sk[4 * c + e], v);
    } else {
      v = S[0][e] * t.sk[e];
    }
    s[e] = ok[e] ? v * cscore : -INFINITY;
  }
  const float mt = colmax4(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
  const float mn = fmaxf(st.m, mt);
  const float msafe = mn == -INFINITY ? 0.0f : mn;
  if (__any(mn > st.m)) {
    const float alpha = __builtin_amdgcn_exp2f(st.m - msafe);
    st.l *= alpha;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) st.acc[c] *= alpha;
  }
  st.m = mn;
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = ok[e] ? __builtin_amdgcn_exp2f(s[e] - msafe) : 0.0f;
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
  // ---- value operands: byte i of the four tokens, tokens in order 0,2,1,3
  uint32_t G[4], Z[4];
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
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = ok[e] ? p[e] * t.sv[ASYM ? 4 * i + e : e] : 0.0f;
    half4v pop;
    pop[0] = (half_t)pv[0]; pop[1] = (half_t)pv[2]; pop[2] = (half_t)pv[1]; pop[3] = (half_t)pv[3];
    uint32_t Gi = G[i];
    half2v b02, b13;
    if constexpr (ASYM) {  // fp16 pairs 1024 + z: bytes 0, 2 and bytes 1, 3 of Z[i]
      b02 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kc.m64, Z[i], 0x04020400u));
      b13 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kc.m64, Z[i], 0x04030401u));
    } else {
      Gi ^= 0x88888888u;
      b02 = b13 = __builtin_bit_cast(half2v, 0x64086408u);
    }
    const half2v x02 = nib2<0>(Gi, kc.m, kc.o) - b02, x13 = nib2<8>(Gi, kc.m, kc.o) - b13;
    const half2v y02 = nib2<4>(Gi, kc.m, kc.o) - b02, y13 = nib2<12>(Gi, kc.m, kc.o) - b13;
    half4v va0, va1;
    va0[0] = x02[0]; va0[1] = x02[1]; va0[2] = x13[0]; va0[3] = x13[1];
    va1[0] = y02[0]; va1[1] = y02[1]; va1[2] = y13[0]; va1[3] = y13[1];
    st.acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16f16(va0, pop, st.acc[2 * i], 0, 0, 0);
    st.acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(va1, pop, st.acc[2 * i + 1], 0, 0, 0);
  }
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

// One wave's share of a split for 4-bit codes, in 16-token tiles with a ring
// of NBUF tiles in registers.
template <int D, int BS, int MODE>
__device__ __forceinline__ void wave_blocks_int4(const DecodeArgs& a, int b, int g, int L,
                                                 int nblk, int i0, int i1, int lane,
                                                 SoftmaxState<D>& st) {
  constexpr int TPB = BS / 16;  // tiles per block
  constexpr int NBUF = MODE == KVQ_SCALE_GROUP_ASYM ? 2 : 3;
  const int r = lane & 15, j = lane >> 4;
  const int ilast = i1 - 1;
  const bool hcol = r < a.G;
  const int h = g * a.G + (hcol ? r : 0);
  half8v qop[D / 32];
  float cscore;
  query_int4<D>(a, a.q + ((int64_t)b * a.Hq + h) * D, j, hcol, qop, cscore);
  const Nib4Consts kc = nib4_consts();
  (void)nblk;

  IdWindow ids;
  ids.init(a.block_tables + (int64_t)b * a.max_blocks, i0, ilast, lane);
  const int t0 = i0 * TPB;
  const int t1 = min(i1 * TPB, (L + 15) / 16);   // tiles holding tokens < L
  const int tfull = min(t1, L / 16);               // tiles wholly below L
  const int tlast = t1 - 1;
  auto load = [&](Tile4<D, MODE>& t, int tile) {
    // refills past the last tile read tile 0 of the shared block 0
    const bool past = tile > tlast;
    const int ti = past ? 0 : tile;
    const int32_t id = ids.id(past ? ids.base : ti / TPB);
    const bool ok = !past && id >= 0 && id < a.num_blocks;
    const int64_t bh = (int64_t)(ok ? id : 0) * a.H + g;
    load_tile4<D, BS, MODE>(t, a, bh, ti % TPB, lane);
  };
  Tile4<D, MODE> buf[NBUF];
#pragma unroll
  for (int u = 0; u < NBUF; ++u) load(buf[u], t0 + u);
  int tt = t0;
  for (; tt + NBUF <= tfull; tt += NBUF) {
    if (tt / TPB - ids.base >= kWave) ids.advance(lane);
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      tile4_step<D, MODE, false>(buf[u], (tt + u) * 16, L, qop, cscore, j, st, kc);
      load(buf[u], tt + u + NBUF);
    }
  }
#pragma unroll
  for (int u = 0; u < NBUF; ++u) {
    if (tt + u < tfull)
      tile4_step<D, MODE, false>(buf[u], (tt + u) * 16, L, qop, cscore, j, st, kc);
    else if (tt + u < t1)
      tile4_step<D, MODE, true>(buf[u], (tt + u) * 16, L, qop, cscore, j, st, kc);
  }
}

// Workgroup -> (item, KV head). The KV head varies fastest, so the H
// workgroups of one item read the same blocks (whose heads are adjacent in
// memory) at about the same time. Consecutive workgroups go to the 8 XCDs in
// turn, and each XCD has its own L2; with H dividing 16 the order within
// each run of 16 workgroups also puts heads 2m and 2m + 1 of an item on the
// same XCD (workgroups q and q + 8), so that a 128-byte line holding both
// heads' 64-byte scale tiles (block 16) is fetched by one L2, not two.
__device__ __forceinline__ void workgroup_item(int H, int w, int& item, int& g) {
  if ((H & 1) == 0 && 16 % H == 0) {
    const int per = H >> 1;                  // head pairs per item
    const int x = w & 7, slot = (w >> 3) & 1;
    item = (w >> 4) * (8 / per) + x / per;
    g = 2 * (x % per) + slot;
  } else {
    item = w / H;
    g = w % H;
  }
}

// One item of the plan per workgroup and KV head: the split's S blocks are
// cut into kNW consecutive shares of at most 64 blocks, one per wave; the
// waves merge their softmax states through LDS and wave 0 writes the split's
// partial.
constexpr int kNW = kDecodeWaves;

template <int CODE, int MODE, int D, int BS>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_kernel(DecodeArgs a) {
  constexpr int NPV = D / 16;   // output MFMAs (16 d-rows each)
  constexpr int NV = D / 4;     // accumulator values per lane
  __shared__ float red[kNW][NV + 2][kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, j = lane >> 4;
  int wg_item, g;
  workgroup_item(a.H, blockIdx.x, wg_item, g);
  // every wave derives the same plan, so the early exit is workgroup-uniform
  const PlanArgs pa = plan_args(a.context_lens, a.batch, a.max_len, BS, a.H, a.split_blocks);
  PlanItem it;
  if (!plan_find_item(pa, wg_item, lane, it)) return;
  const int S = it.S;
  const int b = it.b, L = it.len;
  const int nblk = (L + BS - 1) / BS;
  const int s0 = it.j * S;
  const int s1 = min(s0 + S, nblk);
  // the item's blocks split evenly over the waves (a short last split or a
  // short sequence keeps every wave busy)
  const int share = (s1 - s0 + kNW - 1) / kNW;
  const int i0 = s0 + wave * share;
  const int i1 = min(i0 + share, s1);

  SoftmaxState<D> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int c = 0; c < NPV; ++c) st.acc[c] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
  if (i0 < i1) {
    if constexpr (CODE == KVQ_CODE_INT4)
      wave_blocks_int4<D, BS, MODE>(a, b, g, L, nblk, i0, i1, lane, st);
    else
      wave_blocks<CODE, D, BS, MODE == KVQ_SCALE_CHANNEL_BLOCK_SYM>(a, b, g, L, nblk, i0, i1,
                                                                     lane, st, &red[wave][0][0]);
  }

  // ---- merge the waves' states, then write the split's partial ----------
  const float lsum = colsum4(st.l);
#pragma unroll
  for (int c = 0; c < NPV; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][4 * c + e][lane] = st.acc[c][e];
  red[wave][NV][lane] = st.m;
  red[wave][NV + 1][lane] = lsum;
  __syncthreads();
  if (wave != 0) return;
  float M = red[0][NV][lane];
#pragma unroll
  for (int w = 1; w < kNW; ++w) M = fmaxf(M, red[w][NV][lane]);
  float acc[NV], l = 0.0f;
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = 0.0f;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    const float mw = red[w][NV][lane];
    const float sc = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
    l += sc * red[w][NV + 1][lane];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] += sc * red[w][v][lane];
  }
  if (r >= a.G) return;
  const int h = g * a.G + r;
  const int64_t item = (int64_t)a.Hq * it.off + (int64_t)h * it.ns + it.j;
  if (j == 0) {
    float2 ml = {M, l};
    *reinterpret_cast<float2*>(a.ws_ml + item * 2) = ml;
  }
  if constexpr (CODE == KVQ_CODE_INT4) {
    // acc[4 m + e], m = 2 i + t, holds output element 32 i + 8 j + 2 e + t
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      float* dst = a.ws_acc + item * D + 32 * i + 8 * j;
      const float* A0 = acc + 8 * i;      // t = 0
      const float* A1 = acc + 8 * i + 4;  // t = 1
      float4v lo = {A0[0], A1[0], A0[1], A1[1]};
      float4v hi = {A0[2], A1[2], A0[3], A1[3]};
      *reinterpret_cast<float4v*>(dst) = lo;
      *reinterpret_cast<float4v*>(dst + 4) = hi;
    }
  } else {
    // acc[4 c + e] holds output element (d/16) (4 j + e) + c of head r
    float* dst = a.ws_acc + item * D + j * (D / 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (NPV == 8) {
        float4v lo = {acc[0 + e], acc[4 + e], acc[8 + e], acc[12 + e]};
        float4v hi = {acc[16 + e], acc[20 + e], acc[24 + e], acc[28 + e]};
        *reinterpret_cast<float4v*>(dst + 8 * e) = lo;
        *reinterpret_cast<float4v*>(dst + 8 * e + 4) = hi;
      } else {
        float4v v4 = {acc[0 + e], acc[4 + e], acc[8 + e], acc[12 + e]};
        *reinterpret_cast<float4v*>(dst + 4 * e) = v4;
      }
    }
  }
}

// Cross-split merge: M = max m_j, out = sum_j 2^(m_j - M) acc_j /
// sum_j 2^(m_j - M) l_j; a sequence with no tokens gets 0.
struct ReduceArgs {
  const float* ws_acc;
  const float* ws_ml;
  const int32_t* context_lens;
  void* out;
  int32_t out_dtype;
  int32_t Hq;
  int32_t H;
  int32_t BS;
  int32_t batch;
  int32_t max_len;
  int32_t split_blocks;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// One wave per (sequence, query head). Lane s holds split s's (m, l); the
// partial accumulators of up to 32 splits are loaded in the same batch, so a
// sequence with up to 32 splits is merged after a single memory round trip.
template <int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(ReduceArgs a) {
  constexpr int EPL = D / 64;  // output elements per lane
  constexpr int KB = 32;       // splits per batch of loads
  typedef float floatE __attribute__((ext_vector_type(EPL)));
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const PlanArgs pa = plan_args(a.context_lens, a.batch, a.max_len, a.BS, a.H, a.split_blocks);
  int off, ns;
  plan_sequence(pa, b, lane, off, ns);
  const int64_t base = (int64_t)a.Hq * off + (int64_t)h * ns;
  floatE o;
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.0f;
  float M = -INFINITY, den = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += KB) {
    const int cnt = min(KB, ns - s0);
    float2 ml = {-INFINITY, 0.0f};
    if (lane < cnt) ml = *reinterpret_cast<const float2*>(a.ws_ml + (base + s0 + lane) * 2);
    floatE v[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (u < cnt)
        v[u] = *reinterpret_cast<const floatE*>(a.ws_acc + (base + s0 + u) * D + EPL * lane);
    // running merge across batches: M is the max over all splits seen so far
    const float mb = wave_reduce_f<true>(ml.x);
    const float Mn = fmaxf(M, mb);
    const float rescale = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
    o *= rescale;
    den *= rescale;
    M = Mn;
    const float w = ml.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml.x - M);
    den += w * ml.y;
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (u < cnt) {
        const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
        o += wu * v[u];
      }
  }
  den = wave_reduce_f<false>(den);
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  o *= inv;
  const int64_t ob = ((int64_t)b * a.Hq + h) * D + EPL * lane;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    if (a.out_dtype == KVQ_F32)
      static_cast<float*>(a.out)[ob + e] = o[e];
    else if (a.out_dtype == KVQ_F16)
      static_cast<half_t*>(a.out)[ob + e] = (half_t)o[e];
    else
      static_cast<uint16_t*>(a.out)[ob + e] = f32_to_bf16_rne(o[e]);
  }
}

template <int CODE, int MODE, int D, int BS>
hipError_t launch_split(const DecodeArgs& a, int items, hipStream_t stream) {
  // whole runs of 16 workgroups (see workgroup_item); the extra ones find no item
  dim3 grid((items * a.H + 15) / 16 * 16);
  decode_split_kernel<CODE, MODE, D, BS><<<grid, 64 * kNW, 0, stream>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Multi-query (prefill) attention over the same cache ("KV Cache
// Optimization: Strategies for Faster LLM Inference", sections "Why KV Cache
// Is Essential for Efficient LLM Inference" -- the prompt is processed as a
// whole before decoding -- and "Implementing KV Cache Optimization: A
// Practical Checklist" -- that phase is compute-bound). Sequence b's queries
// are its last nq positions; query i (position L - nq + i) sees positions
// 0 .. L - nq + i.
//
// The 16 MFMA columns of a wave are 16 consecutive (query, head) pairs
// c = i G + r of one KV head g, a column tile: the G heads of a query are
// adjacent, a tile spans 16 / G queries (or a query G / 16 tiles). A wave
// takes one unit (sequence b, split j of S blocks, KV head g, column tile
// ct), streams the split's blocks with a double buffer and runs the decode's
// tile steps with its own causal limit per lane (column); every block it
// loads serves 16 columns, and the units of one (b, j, g) are adjacent in
// the grid so that their repeated block reads meet in L2. Each unit writes a
// partial (m, l, acc) per column; prefill_reduce merges the splits.
// ---------------------------------------------------------------------------
struct PrefillArgs {
  DecodeArgs a;
  const int32_t* qstart;
  int32_t J;    // splits per sequence in the grid
  int32_t S;    // blocks per split
  int32_t CT;   // column tiles per (sequence, KV head)
};

template <int CODE, int MODE, int D, int BS>
__global__ __launch_bounds__(256) void prefill_split_kernel(PrefillArgs pa) {
  constexpr int NCH = D / 32;
  constexpr int NPV = D / 16;
  constexpr bool KCH = MODE == KVQ_SCALE_CHANNEL_BLOCK_SYM;
  constexpr bool RAW = CODE == KVQ_CODE_NONE16;
  using TileT = typename std::conditional<RAW, TileRaw<D, BS>, Tile8<D, BS>>::type;
  __shared__ float lds[4][D];
  const DecodeArgs& a = pa.a;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, jj = lane >> 4;
  int64_t u = (int64_t)blockIdx.x * 4 + wave;
  const int ct = (int)(u % pa.CT);
  u /= pa.CT;
  const int g = (int)(u % a.H);
  u /= a.H;
  const int j = (int)(u % pa.J);
  const int b = (int)(u / pa.J);
  if (b >= a.batch) return;
  const int L = min(a.context_lens[b], a.max_len);
  const int q0 = pa.qstart[b];
  const int nq = min(pa.qstart[b + 1] - q0, L);
  const int ncol = nq * a.G;
  const int cbase = ct * 16;
  const int nblk = (L + BS - 1) / BS;
  const int s0 = j * pa.S;
  if (cbase >= ncol || s0 >= nblk) return;  // no such column tile or split

  // ---- columns: lane (r, jj) serves column c = cbase + r -------------------
  const int c = cbase + r;
  const bool valid = c < ncol;
  const int qi = valid ? c / a.G : 0;
  const int hq = g * a.G + (valid ? c % a.G : 0);
  const int Lr = valid ? L - nq + qi + 1 : 0;                 // this column's limit
  const int Lmin = L - nq + cbase / a.G + 1;                  // over the tile's columns
  const int Lmax = L - nq + (min(ncol, cbase + 16) - 1) / a.G + 1;
  const int i0 = s0;
  const int i1 = min(min(s0 + pa.S, nblk), (Lmax + BS - 1) / BS);

  float qf[D / 4];
  {
    const uint16_t* qp = a.q + ((int64_t)(q0 + qi) * a.Hq + hq) * D + jj * (D / 4);
    if (a.q_bf16)
      load_query<true, D>(qp, qf);
    else
      load_query<false, D>(qp, qf);
  }
  float qmax = 0.0f;
#pragma unroll
  for (int e = 0; e < D / 4; ++e) qmax = fmaxf(qmax, fabsf(qf[e]));
  qmax = colmax4(qmax);
  int qe = qmax > 0.0f ? (int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127 : 0;
  qe = max(qe, -126);
  const float qdown = __uint_as_float((uint32_t)(127 - qe) << 23);
  const float qup = __uint_as_float((uint32_t)(127 + qe) << 23);
#pragma unroll
  for (int e = 0; e < D / 4; ++e) qf[e] = valid ? qf[e] * qdown : 0.0f;
  half8v qop[NCH];
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) qop[cc][e] = (half_t)qf[8 * cc + e];
  const float cscore = valid ? qup * a.sm_log2 : 0.0f;
  const bool raw_bf16 = a.stage_bf16 != 0;

  SoftmaxState<D> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int cc = 0; cc < NPV; ++cc) st.acc[cc] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  // per-channel keys: a partly filled last block is read raw from stage row b
  const bool staged = KCH && (L % BS) != 0;
  u32x4 kraw[BS / 16][NCH];
  if constexpr (KCH) {
    if (staged && i1 == nblk) {
#pragma unroll
      for (int nt = 0; nt < BS / 16; ++nt) {
        const uint16_t* sp =
            a.k_stage + (((int64_t)b * a.H + g) * BS + nt * 16 + r) * D + jj * (D / 4);
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) kraw[nt][cc] = *reinterpret_cast<const u32x4*>(sp + 8 * cc);
      }
    }
  }
  const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks;
  // loads past the split read physical block 0 (shared, cached); ids outside
  // the pool (a broken precondition) are read as block 0 too
  auto bh_of = [&](int i) -> int64_t {
    const int32_t id = i < i1 ? trow[i] : 0;
    return (int64_t)(id >= 0 && id < a.num_blocks ? id : 0) * a.H + g;
  };
  auto block = [&](const TileT& t, int i) {
    const bool rawk = KCH && staged && i == nblk - 1;
    if (!rawk && (i + 1) * BS <= Lmin) {  // every column sees the whole block
      if constexpr (RAW) {
#pragma unroll
        for (int nt = 0; nt < BS / 16; ++nt)
          tile_step_raw<D, BS, false>(t, nt, i * BS + nt * 16, L, qop, cscore, jj, st, raw_bf16);
      } else if constexpr (KCH) {
        half8v qb[NCH], ql[NCH];
        channel_query<D, BS>(t, lds[wave], qf, lane, qb, ql);
        full_block_step<CODE, D, BS, kKeyChannel>(t, i, L, qb, cscore, jj, st, ql);
      } else {
        full_block_step<CODE, D, BS>(t, i, L, qop, cscore, jj, st);
      }
      return;
    }
    half8v qb[NCH], ql[NCH];
    if constexpr (KCH && !RAW) {
      if (!rawk) channel_query<D, BS>(t, lds[wave], qf, lane, qb, ql);
    }
#pragma unroll
    for (int nt = 0; nt < BS / 16; ++nt) {
      const int pos0 = i * BS + nt * 16;
      if (pos0 >= Lmax) continue;
      const bool masked = pos0 + 16 > Lmin;
      if constexpr (RAW) {
        if (masked)
          tile_step_raw<D, BS, true>(t, nt, pos0, Lr, qop, cscore, jj, st, raw_bf16, L);
        else
          tile_step_raw<D, BS, false>(t, nt, pos0, Lr, qop, cscore, jj, st, raw_bf16, L);
      } else if constexpr (KCH) {
        if (rawk) {
          if (masked)
            tile_step<CODE, D, BS, true, kKeyRaw>(t, nt, pos0, Lr, qop, cscore, jj, st,
                                                  kraw[nt], raw_bf16, nullptr, L);
          else
            tile_step<CODE, D, BS, false, kKeyRaw>(t, nt, pos0, Lr, qop, cscore, jj, st,
                                                   kraw[nt], raw_bf16, nullptr, L);
        } else if (masked) {
          tile_step<CODE, D, BS, true, kKeyChannel>(t, nt, pos0, Lr, qb, cscore, jj, st,
                                                    nullptr, false, ql, L);
        } else {
          tile_step<CODE, D, BS, false, kKeyChannel>(t, nt, pos0, Lr, qb, cscore, jj, st,
                                                     nullptr, false, ql, L);
        }
      } else {
        if (masked)
          tile_step<CODE, D, BS, true>(t, nt, pos0, Lr, qop, cscore, jj, st, nullptr, false,
                                       nullptr, L);
        else
          tile_step<CODE, D, BS, false>(t, nt, pos0, Lr, qop, cscore, jj, st, nullptr, false,
                                        nullptr, L);
      }
    }
  };
  // double buffer: block i + 1 loads while block i computes
  TileT t0, t1;
  if (i0 < i1) load_tile<D, BS, KCH>(t0, a, bh_of(i0), lane);
  for (int i = i0; i < i1; i += 2) {
    load_tile<D, BS, KCH>(t1, a, bh_of(i + 1), lane);
    block(t0, i);
    if (i + 1 >= i1) break;
    load_tile<D, BS, KCH>(t0, a, bh_of(i + 2), lane);
    block(t1, i + 1);
  }

  // ---- this unit's partial, one per valid column ---------------------------
  const float lsum = colsum4(st.l);
  if (!valid) return;
  const int64_t pidx = (((int64_t)b * pa.J + j) * a.H + g) * (pa.CT * 16) + c;
  if (jj == 0) *reinterpret_cast<float2*>(a.ws_ml + pidx * 2) = make_float2(st.m, lsum);
  // st.acc[cc][e] holds output element (d/16) (4 jj + e) + cc of column c
  float* dst = a.ws_acc + pidx * D + jj * (D / 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (NPV == 8) {
      float4v lo = {st.acc[0][e], st.acc[1][e], st.acc[2][e], st.acc[3][e]};
      float4v hi = {st.acc[4][e], st.acc[5][e], st.acc[6][e], st.acc[7][e]};
      *reinterpret_cast<float4v*>(dst + 8 * e) = lo;
      *reinterpret_cast<float4v*>(dst + 8 * e + 4) = hi;
    } else {
      float4v v4 = {st.acc[0][e], st.acc[1][e], st.acc[2][e], st.acc[3][e]};
      *reinterpret_cast<float4v*>(dst + 4 * e) = v4;
    }
  }
}

// Cross-split merge for multi-query attention, as decode_reduce: one wave
// per (query head, query i, sequence b); split j's partial of column
// c = i G + h % G sits at ((b J + j) H + g) CT16 + c.
struct PrefillReduceArgs {
  const float* ws_acc;
  const float* ws_ml;
  const int32_t* context_lens;
  const int32_t* qstart;
  void* out;
  int32_t out_dtype;
  int32_t Hq, H, G, BS, max_len, J, S, CT;
};

template <int D>
__global__ __launch_bounds__(64) void prefill_reduce_kernel(PrefillReduceArgs a) {
  constexpr int EPL = D / 64;
  constexpr int KB = 32;
  typedef float floatE __attribute__((ext_vector_type(EPL)));
  const int h = blockIdx.x, i = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int L = min(a.context_lens[b], a.max_len);
  const int q0 = a.qstart[b];
  const int nq = min(a.qstart[b + 1] - q0, L);
  if (i >= nq) return;
  const int ns = ((L + a.BS - 1) / a.BS + a.S - 1) / a.S;
  const int64_t cols = (int64_t)a.CT * 16;
  const int64_t base = ((int64_t)b * a.J * a.H + h / a.G) * cols + (int64_t)i * a.G + h % a.G;
  const int64_t stride = (int64_t)a.H * cols;
  floatE o;
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.0f;
  float M = -INFINITY, den = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += KB) {
    const int cnt = min(KB, ns - s0);
    float2 ml = {-INFINITY, 0.0f};
    if (lane < cnt) ml = *reinterpret_cast<const float2*>(a.ws_ml + (base + (s0 + lane) * stride) * 2);
    floatE v[KB];
#pragma unroll
    for (int uu = 0; uu < KB; ++uu)
      if (uu < cnt)
        v[uu] = *reinterpret_cast<const floatE*>(a.ws_acc + (base + (s0 + uu) * stride) * D + EPL * lane);
    const float mb = wave_reduce_f<true>(ml.x);
    const float Mn = fmaxf(M, mb);
    const float rescale = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
    o *= rescale;
    den *= rescale;
    M = Mn;
    const float w = ml.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml.x - M);
    den += w * ml.y;
#pragma unroll
    for (int uu = 0; uu < KB; ++uu)
      if (uu < cnt) {
        const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), uu));
        o += wu * v[uu];
      }
  }
  den = wave_reduce_f<false>(den);
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  o *= inv;
  const int64_t ob = ((int64_t)(q0 + i) * a.Hq + h) * D + EPL * lane;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    if (a.out_dtype == KVQ_F32)
      static_cast<float*>(a.out)[ob + e] = o[e];
    else if (a.out_dtype == KVQ_F16)
      static_cast<half_t*>(a.out)[ob + e] = (half_t)o[e];
    else
      static_cast<uint16_t*>(a.out)[ob + e] = f32_to_bf16_rne(o[e]);
  }
}

template <int CODE, int MODE>
hipError_t launch_prefill_shape(const PrefillArgs& pa, int d, int bs, int64_t units,
                                hipStream_t stream) {
  const dim3 grid((unsigned)((units + 3) / 4));
  if (d == 128) {
    if (bs == 16)
      prefill_split_kernel<CODE, MODE, 128, 16><<<grid, 256, 0, stream>>>(pa);
    else
      prefill_split_kernel<CODE, MODE, 128, 32><<<grid, 256, 0, stream>>>(pa);
  } else {
    if (bs == 16)
      prefill_split_kernel<CODE, MODE, 64, 16><<<grid, 256, 0, stream>>>(pa);
    else
      prefill_split_kernel<CODE, MODE, 64, 32><<<grid, 256, 0, stream>>>(pa);
  }
  return hipGetLastError();
}

template <int CODE, int MODE>
hipError_t launch_split_shape(const DecodeArgs& a, int d, int bs, int items, hipStream_t stream) {
  if (d == 128)
    return bs == 16 ? launch_split<CODE, MODE, 128, 16>(a, items, stream)
                    : launch_split<CODE, MODE, 128, 32>(a, items, stream);
  return bs == 16 ? launch_split<CODE, MODE, 64, 16>(a, items, stream)
                  : launch_split<CODE, MODE, 64, 32>(a, items, stream);
}

}  // namespace

bool prefill_supported(int32_t k_code, int32_t v_code, int32_t k_mode, int32_t v_mode) {
  if (k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM)
    return k_code == KVQ_CODE_INT8 && v_code == KVQ_CODE_INT8 && v_mode == KVQ_SCALE_TOKEN_SYM;
  if (k_code != v_code || k_mode != v_mode) return false;
  if (k_code == KVQ_CODE_NONE16) return true;
  return k_mode == KVQ_SCALE_TOKEN_SYM &&
         (k_code == KVQ_CODE_INT8 || k_code == KVQ_CODE_FP8_E4M3);
}

hipError_t launch_prefill(const PrefillPlan& pp, hipStream_t stream) {
  const DecodePlan& p = pp.d;
  PrefillArgs pa;
  DecodeArgs& a = pa.a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k_codes = static_cast<const uint8_t*>(p.k_codes);
  a.v_codes = static_cast<const uint8_t*>(p.v_codes);
  a.k_scale = p.k_scale;
  a.v_scale = p.v_scale;
  a.k_zero = p.k_zero;
  a.v_zero = p.v_zero;
  a.k_stage = static_cast<const uint16_t*>(p.k_stage);
  a.block_tables = p.block_tables;
  a.context_lens = p.context_lens;
  a.ws_acc = p.ws_acc;
  a.ws_ml = p.ws_ml;
  a.num_blocks = p.num_blocks;
  a.q_bf16 = p.q_bf16;
  a.stage_bf16 = p.src_bf16;
  a.Hq = p.num_q_heads;
  a.H = p.num_kv_heads;
  a.G = p.num_q_heads / p.num_kv_heads;
  a.max_blocks = p.max_blocks_per_seq;
  a.batch = p.batch;
  a.max_len = p.max_context_len;
  a.split_blocks = pp.split_blocks;
  a.sm_log2 = p.sm_scale * kLog2e;
  pa.qstart = pp.query_start;
  pa.J = pp.splits;
  pa.S = pp.split_blocks;
  pa.CT = pp.col_tiles;
  const int64_t units = (int64_t)p.batch * pp.splits * p.num_kv_heads * pp.col_tiles;
  const int d = p.head_dim, bs = p.block_size;
  hipError_t e;
  if (p.k_code == KVQ_CODE_NONE16)
    e = launch_prefill_shape<KVQ_CODE_NONE16, KVQ_SCALE_TOKEN_SYM>(pa, d, bs, units, stream);
  else if (p.k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM)
    e = launch_prefill_shape<KVQ_CODE_INT8, KVQ_SCALE_CHANNEL_BLOCK_SYM>(pa, d, bs, units, stream);
  else if (p.k_code == KVQ_CODE_FP8_E4M3)
    e = launch_prefill_shape<KVQ_CODE_FP8_E4M3, KVQ_SCALE_TOKEN_SYM>(pa, d, bs, units, stream);
  else
    e = launch_prefill_shape<KVQ_CODE_INT8, KVQ_SCALE_TOKEN_SYM>(pa, d, bs, units, stream);
  if (e != hipSuccess) return e;
  PrefillReduceArgs ra;
  ra.ws_acc = p.ws_acc;
  ra.ws_ml = p.ws_ml;
  ra.context_lens = p.context_lens;
  ra.qstart = pp.query_start;
  ra.out = p.out;
  ra.out_dtype = p.out_dtype;
  ra.Hq = p.num_q_heads;
  ra.H = p.num_kv_heads;
  ra.G = p.num_q_heads / p.num_kv_heads;
  ra.BS = p.block_size;
  ra.max_len = p.max_context_len;
  ra.J = pp.splits;
  ra.S = pp.split_blocks;
  ra.CT = pp.col_tiles;
  const dim3 grid(p.num_q_heads, pp.max_query_len, p.batch);
  if (d == 128)
    prefill_reduce_kernel<128><<<grid, 64, 0, stream>>>(ra);
  else
    prefill_reduce_kernel<64><<<grid, 64, 0, stream>>>(ra);
  return hipGetLastError();
}

bool decode_supported(int32_t k_code, int32_t v_code, int32_t k_mode,
                      int32_t v_mode) {
  if (k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM)
    return k_code == KVQ_CODE_INT8 && v_code == KVQ_CODE_INT8 && v_mode == KVQ_SCALE_TOKEN_SYM;
  if (k_code != v_code || k_mode != v_mode) return false;
  if (k_code == KVQ_CODE_NONE16) return true;
  if (k_mode == KVQ_SCALE_TOKEN_SYM)
    return k_code == KVQ_CODE_INT8 || k_code == KVQ_CODE_FP8_E4M3 || k_code == KVQ_CODE_INT4;
  return k_mode == KVQ_SCALE_GROUP_ASYM && k_code == KVQ_CODE_INT4;
}

hipError_t launch_decode(const DecodePlan& p, hipStream_t stream) {
  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k_codes = static_cast<const uint8_t*>(p.k_codes);
  a.v_codes = static_cast<const uint8_t*>(p.v_codes);
  a.k_scale = p.k_scale;
  a.v_scale = p.v_scale;
  a.block_tables = p.block_tables;
  a.context_lens = p.context_lens;
  a.ws_acc = p.ws_acc;
  a.ws_ml = p.ws_ml;
  a.num_blocks = p.num_blocks;
  a.q_bf16 = p.q_bf16;
  a.Hq = p.num_q_heads;
  a.H = p.num_kv_heads;
  a.G = p.num_q_heads / p.num_kv_heads;
  a.max_blocks = p.max_blocks_per_seq;
  a.batch = p.batch;
  a.max_len = p.max_context_len;
  a.split_blocks = p.split_blocks;
  a.sm_log2 = p.sm_scale * kLog2e;
  a.k_zero = p.k_zero;
  a.v_zero = p.v_zero;
  a.k_stage = static_cast<const uint16_t*>(p.k_stage);
  a.stage_bf16 = p.src_bf16;
  hipError_t e;
  const int d = p.head_dim, bs = p.block_size;
  if (p.k_code == KVQ_CODE_NONE16)
    e = launch_split_shape<KVQ_CODE_NONE16, KVQ_SCALE_TOKEN_SYM>(a, d, bs, p.item_bound, stream);
  else if (p.k_code == KVQ_CODE_FP8_E4M3)
    e = launch_split_shape<KVQ_CODE_FP8_E4M3, KVQ_SCALE_TOKEN_SYM>(a, d, bs, p.item_bound, stream);
  else if (p.k_code == KVQ_CODE_INT8 && p.k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM)
    e = launch_split_shape<KVQ_CODE_INT8, KVQ_SCALE_CHANNEL_BLOCK_SYM>(a, d, bs, p.item_bound,
                                                                      stream);
  else if (p.k_code == KVQ_CODE_INT8)
    e = launch_split_shape<KVQ_CODE_INT8, KVQ_SCALE_TOKEN_SYM>(a, d, bs, p.item_bound, stream);
  else if (p.k_mode == KVQ_SCALE_GROUP_ASYM)
    e = launch_split_shape<KVQ_CODE_INT4, KVQ_SCALE_GROUP_ASYM>(a, d, bs, p.item_bound, stream);
  else
    e = launch_split_shape<KVQ_CODE_INT4, KVQ_SCALE_TOKEN_SYM>(a, d, bs, p.item_bound, stream);
  if (e != hipSuccess) return e;
  ReduceArgs ra;
  ra.ws_acc = p.ws_acc;
  ra.ws_ml = p.ws_ml;
  ra.context_lens = p.context_lens;
  ra.out = p.out;
  ra.out_dtype = p.out_dtype;
  ra.Hq = p.num_q_heads;
  ra.H = p.num_kv_heads;
  ra.BS = p.block_size;
  ra.batch = p.batch;
  ra.max_len = p.max_context_len;
  ra.split_blocks = p.split_blocks;
  dim3 grid(p.num_q_heads, p.batch);
  if (p.head_dim == 128)
    decode_reduce_kernel<128><<<grid, 64, 0, stream>>>(ra);
  else
    decode_reduce_kernel<64><<<grid, 64, 0, stream>>>(ra);
  return hipGetLastError();
}

}  // namespace kvq
