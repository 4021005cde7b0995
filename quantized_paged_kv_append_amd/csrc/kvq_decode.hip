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
#include "kvq_attn_tiles.h"

namespace kvq {
namespace {

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

// Per-token scores of one tile before the column scale: the score MFMAs
// (chunk c = slice c; one accumulator per 32-element group for asymmetric
// codes) and, for token 4j + e, the sum over groups c of S[c][e] times the
// key scale of (token e, group c), held by lane SG e + c of the row.
template <int D, int MODE>
__device__ __forceinline__ void tile4_scores(const Tile4<D, MODE>& t, const half8v* qop,
                                             const Nib4Consts& kc, float* v) {
  constexpr int NS = D / 32;
  constexpr bool ASYM = MODE == KVQ_SCALE_GROUP_ASYM;
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
  if constexpr (ASYM) {
    combine_groups(S, t.sk, v, std::integral_constant<int, NS>{});
  } else {
    static_for<0, 4>([&](auto E) {
      constexpr int e = decltype(E)::value;
      v[e] = row_bcast<e>(t.sk) * S[0][e];
    });
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

template <int D, int MODE, bool TAIL>
__device__ __forceinline__ void tile4_step(const Tile4<D, MODE>& t, int pos0, int L,
                                           const half8v* qop, float cscore, int j,
                                           SoftmaxState<D>& st, const Nib4Consts& kc) {
  constexpr int NS = D / 32;
  constexpr bool ASYM = MODE == KVQ_SCALE_GROUP_ASYM;
  constexpr int SG = Tile4<D, MODE>::SG;
  float v[4], s[4];
  tile4_scores(t, qop, kc, v);
  bool ok[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ok[e] = !TAIL || pos0 + 4 * j + e < L;
#pragma unroll
  for (int e = 0; e < 4; ++e) s[e] = ok[e] ? v[e] * cscore : -INFINITY;
  const float msafe = softmax_update<D, 4>(s, st);
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = ok[e] ? __builtin_amdgcn_exp2f(s[e] - msafe) : 0.0f;
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
  uint32_t G[4], Z[4] = {0u, 0u, 0u, 0u};
  tile4_vbytes(t, G, Z);
  static_for<0, NS>([&](auto I) {
    constexpr int i = decltype(I)::value;
    float pv[4];
    static_for<0, 4>([&](auto E) {
      constexpr int e = decltype(E)::value;
      pv[e] = ok[e] ? row_bcast<SG * e + (ASYM ? i : 0)>(t.sv) * p[e] : 0.0f;
    });
    half4v pop;
    pop[0] = (half_t)pv[0]; pop[1] = (half_t)pv[2]; pop[2] = (half_t)pv[1]; pop[3] = (half_t)pv[3];
    const VWords4 w = vgroup_words<ASYM>(G[i], Z[i], kc);
    const half4v va0 = __builtin_bit_cast(half4v, (u32x2){w.x[0], w.x[1]});
    const half4v va1 = __builtin_bit_cast(half4v, (u32x2){w.y[0], w.y[1]});
    const half4v corr = __builtin_bit_cast(half4v, (u32x2){w.c[0], w.c[1]});
    st.acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16f16(va0, pop, st.acc[2 * i], 0, 0, 0);
    st.acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(va1, pop, st.acc[2 * i + 1], 0, 0, 0);
    st.acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16f16(corr, pop, st.acc[2 * i], 0, 0, 0);
    st.acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(corr, pop, st.acc[2 * i + 1], 0, 0, 0);
  });
}

// Two consecutive whole tiles (32 tokens) in one step: one softmax update
// for both, and the PV products on 16x16x32 MFMAs whose contraction runs over
// the 32 tokens (k = 8j + 4T + e' for tile T, token 4j + e' in the order
// 0, 2, 1, 3, the same in the value and probability operands).
template <int D, int MODE>
__device__ __forceinline__ void tile4_pair_step(const Tile4<D, MODE>& t0, const Tile4<D, MODE>& t1,
                                                const half8v* qop, float cscore,
                                                SoftmaxState<D>& st, const Nib4Consts& kc) {
  constexpr int NS = D / 32;
  constexpr bool ASYM = MODE == KVQ_SCALE_GROUP_ASYM;
  constexpr int SG = Tile4<D, MODE>::SG;
  float v[8], s[8];
  tile4_scores(t0, qop, kc, v);
  tile4_scores(t1, qop, kc, v + 4);
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = v[e] * cscore;
  const float msafe = softmax_update<D, 8>(s, st);
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(s[e] - msafe);
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  uint32_t G0[4], Z0[4] = {0u, 0u, 0u, 0u}, G1[4], Z1[4] = {0u, 0u, 0u, 0u};
  tile4_vbytes(t0, G0, Z0);
  tile4_vbytes(t1, G1, Z1);
  static_for<0, NS>([&](auto I) {
    constexpr int i = decltype(I)::value;
    float pv[8];
    static_for<0, 4>([&](auto E) {
      constexpr int e = decltype(E)::value;
      pv[e] = row_bcast<SG * e + (ASYM ? i : 0)>(t0.sv) * p[e];
      pv[4 + e] = row_bcast<SG * e + (ASYM ? i : 0)>(t1.sv) * p[4 + e];
    });
    half8v pop;
    pop[0] = (half_t)pv[0]; pop[1] = (half_t)pv[2]; pop[2] = (half_t)pv[1]; pop[3] = (half_t)pv[3];
    pop[4] = (half_t)pv[4]; pop[5] = (half_t)pv[6]; pop[6] = (half_t)pv[5]; pop[7] = (half_t)pv[7];
    const VWords4 w0 = vgroup_words<ASYM>(G0[i], Z0[i], kc);
    const VWords4 w1 = vgroup_words<ASYM>(G1[i], Z1[i], kc);
    const half8v va0 = __builtin_bit_cast(half8v, (u32x4){w0.x[0], w0.x[1], w1.x[0], w1.x[1]});
    const half8v va1 = __builtin_bit_cast(half8v, (u32x4){w0.y[0], w0.y[1], w1.y[0], w1.y[1]});
    const half8v corr = __builtin_bit_cast(half8v, (u32x4){w0.c[0], w0.c[1], w1.c[0], w1.c[1]});
    st.acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va0, pop, st.acc[2 * i], 0, 0, 0);
    st.acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va1, pop, st.acc[2 * i + 1], 0, 0, 0);
    st.acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(corr, pop, st.acc[2 * i], 0, 0, 0);
    st.acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(corr, pop, st.acc[2 * i + 1], 0, 0, 0);
  });
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

// One wave's share of a split for 4-bit codes, in pairs of 16-token tiles
// from a ring of NBUF tiles in registers; the last tiles go one at a time.
template <int D, int BS, int MODE>
__device__ __forceinline__ void wave_blocks_int4(const DecodeArgs& a, int b, int g, int L,
                                                 int nblk, int i0, int i1, int lane,
                                                 SoftmaxState<D>& st) {
  constexpr int TPB = BS / 16;  // tiles per block
  constexpr int NBUF = 4;  // tiles in the register ring: two pairs
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
  const Lane4 lo4 = lane4_offsets<D, MODE>(lane);
  auto load = [&](Tile4<D, MODE>& t, int tile) {
    // refills past the last tile read tile 0 of the shared block 0
    const bool past = tile > tlast;
    const int ti = past ? 0 : tile;
    const int32_t id = ids.id(past ? ids.base : ti / TPB);
    const bool ok = !past && id >= 0 && id < a.num_blocks;
    const int64_t bh = (int64_t)(ok ? id : 0) * a.H + g;
    load_tile4<D, BS, MODE>(t, a, bh, ti % TPB, lo4);
  };
  Tile4<D, MODE> buf[NBUF];
#pragma unroll
  for (int u = 0; u < NBUF; ++u) load(buf[u], t0 + u);
  int tt = t0;
  for (; tt + NBUF <= tfull; tt += NBUF) {
    if (tt / TPB - ids.base >= kWave) ids.advance(lane);
    tile4_pair_step<D, MODE>(buf[0], buf[1], qop, cscore, st, kc);
    load(buf[0], tt + NBUF);
    load(buf[1], tt + NBUF + 1);
    tile4_pair_step<D, MODE>(buf[2], buf[3], qop, cscore, st, kc);
    load(buf[2], tt + NBUF + 2);
    load(buf[3], tt + NBUF + 3);
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

template <int CODE, int MODE>
hipError_t launch_split_shape(const DecodeArgs& a, int d, int bs, int items, hipStream_t stream) {
  if (d == 128)
    return bs == 16 ? launch_split<CODE, MODE, 128, 16>(a, items, stream)
                    : launch_split<CODE, MODE, 128, 32>(a, items, stream);
  return bs == 16 ? launch_split<CODE, MODE, 64, 16>(a, items, stream)
                  : launch_split<CODE, MODE, 64, 32>(a, items, stream);
}

}  // namespace

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
