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
//  * 8-bit codes with per-token scales take two 16-token tiles per softmax
//    update, with PV on v_mfma_f32_16x16x32_f16 over both tiles' tokens.
//  * A ring of register buffers (four 16-token blocks as two pairs, or three
//    / two blocks) keeps the next blocks in flight while the wave computes;
//    block ids come from one vector load per 64 blocks of the split and are
//    read with v_readlane.
//  * Partials (m, l, acc) per split go to the workspace; decode_reduce merges
//    them with the log-sum-exp rule.
#include <atomic>
#include <mutex>

#include "kvq_attn_tiles.h"
#include "kvq_encode.h"
#include "kvq_int4_tiles.h"

// Partials of kvq_decode_attention_noalloc: a fixed array in device memory
// (one copy per GPU, held until the process ends), so that callers that cannot
// allocate still get a workspace. Host code never names it in a launch: its
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[KVQ_DECODE_SCRATCH_BYTES];

namespace kvq {
namespace {

// ---- split planning ---------------------------------------------------------
// Every workgroup of the split kernel and every wave of the reduce derive the
// same plan from context_lens alone, so neither a planning launch nor a host
// synchronization is needed:
//   n_b  = ceil(min(len_b, max_len) / BS)          blocks of sequence b
//   S    = split_blocks, or kDecodeWaves * clamp(ceil(H sum_b n_b / 2^lg),
//          ceil(32 / BS), cap)                       blocks per split
//          (lg, cap = 11, 256 for nearly equal lengths; otherwise 12, 32 for
//          INT4, 12, 64 for per-channel keys, 11, 64 for other layouts)
//   ns_b = ceil(n_b / S)                            splits of sequence b
// Items (b, j), j < ns_b, are numbered sequence-major. The partial of item
// (b, j) for query head h is row Hq off_b + h ns_b + j of the workspace, with
// off_b = sum_{b' < b} ns_b', so one head's splits are adjacent. The host
// bounds sum_b ns_b from batch and max_len alone (the grid and workspace
// size). Short sequences thus get few splits and the total work is cut into
// about 2^lg wave shares whatever the length mix.
struct PlanArgs {
  const int32_t* lens;
  int32_t batch, max_len, bs, H, split_blocks;
  int32_t skew_cap;  // per-wave share cap for batches of unequal lengths
  int32_t skew_lg;   // their wave target, log2
};

__device__ __forceinline__ PlanArgs plan_args(const int32_t* lens, int batch, int max_len,
                                              int bs, int H, int split_blocks, int skew_cap,
                                              int skew_lg) {
  PlanArgs p;
  p.lens = lens;
  p.batch = batch;
  p.max_len = max_len;
  p.bs = bs;
  p.H = H;
  p.split_blocks = split_blocks;
  p.skew_cap = skew_cap;
  p.skew_lg = skew_lg;
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
// less often; any other batch into 2^decode_skew_lg shares of at most
// decode_skew_cap blocks (twice as many, shorter ones for INT4 and
// per-channel keys), which the dispatcher balances.
__device__ __forceinline__ int plan_split_blocks(const PlanArgs& p, int lane, const int* len0,
                                                 bool& uniform) {
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
  uniform = (int64_t)nmax * 8 <= (int64_t)nmin * 9;
  if (p.split_blocks > 0) return p.split_blocks;
  const int lg = uniform ? kDecodeUniformWavesLog2 : p.skew_lg;
  const int cap = uniform ? kDecodeMaxWaveBlocks : p.skew_cap;
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

// Splits of sequence b (ns) and of all sequences before it (off), for S
// blocks per split; len0 holds the first 256 lengths (plan_len4).
__device__ __forceinline__ void plan_sequence_of(const PlanArgs& p, int b, int lane,
                                                 const int* len0, int S, int& off, int& ns) {
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

// Sequences (of the batch) whose last split is partial with at least r of
// its S blocks (r >= 1).
__device__ __forceinline__ int plan_partials_from(const PlanArgs& p, const int* len0, int S,
                                                  int r, int lane) {
  int cnt = 0;
#pragma unroll 1
  for (int c0 = 0; c0 < p.batch; c0 += 4 * kWave) {
    int len[4];
    plan_chunk(p, c0, lane, len0, len);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      cnt += __builtin_popcountll(__ballot(((len[u] + p.bs - 1) / p.bs) % S >= r));
  }
  return cnt;
}

// What every item lookup of one launch shares: the first 256 lengths, the
// blocks per split and whether the batch has nearly equal lengths.
struct PlanCtx {
  int len0[4];
  int S;
  bool uniform;
};

__device__ __forceinline__ PlanCtx plan_ctx(const PlanArgs& p, int lane) {
  PlanCtx c;
  plan_len4(p, 0, lane, c.len0);
  c.S = plan_split_blocks(p, lane, c.len0, c.uniform);
  return c;
}

// Workgroups the plan occupies: its items times the KV heads, in whole runs
// of 16 (see workgroup_item).
__device__ __forceinline__ int plan_workgroups(const PlanArgs& p, const PlanCtx& c, int lane) {
  int total = 0;
  for (int c0 = 0; c0 < p.batch; c0 += 4 * kWave) {
    int len[4];
    plan_chunk(p, c0, lane, c.len0, len);
    int t4 = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) t4 += plan_splits_of(p, len[u], c.S);
    total += wave_sum(t4, lane);
  }
  return (total * p.H + 15) / 16 * 16;
}

// Item `item` of the plan; false past the last item. The partial row of
// item (b, j) is fixed by (b, j) alone (see plan_sequence); only which
// workgroup computes it depends on the order here. A batch of nearly equal
// lengths is taken sequence-major. Any other batch is taken longest first,
// so that its short splits, not long ones, close the launch: first every
// full split (S blocks) in sequence order, then the sequences' partial last
// splits by size, largest first, in sequence order among equal sizes.
__device__ __forceinline__ bool plan_find_item(const PlanArgs& p, const PlanCtx& ctx, int item,
                                               int lane, PlanItem& out) {
  const int* len0 = ctx.len0;
  const bool uniform = ctx.uniform;
  const int S = ctx.S;
  out.S = S;
  if (uniform) {
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
  // counts of full splits and of all splits: the grid is sized for the
  // longest possible contexts, so most workgroups of a skewed batch find no
  // item and leave here
  int full = 0, total = 0;
  for (int c0 = 0; c0 < p.batch; c0 += 4 * kWave) {
    int len[4];
    plan_chunk(p, c0, lane, len0, len);
    int f4 = 0, t4 = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = (len[u] + p.bs - 1) / p.bs;
      f4 += n / S;
      t4 += (n + S - 1) / S;
    }
    full += wave_sum(f4, lane);
    total += wave_sum(t4, lane);
  }
  if (item >= total) return false;
  int b = -1, j = 0;
  if (item < full) {   // the item-th full split, sequence order
    int off = 0;
#pragma unroll 1
    for (int c0 = 0; c0 < p.batch && b < 0; c0 += 4 * kWave) {
      int len[4];
      plan_chunk(p, c0, lane, len0, len);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int F = (len[u] + p.bs - 1) / p.bs / S;
        const int incl = wave_incl_scan(F, lane);
        const int tot = __builtin_amdgcn_readlane(incl, kWave - 1);
        if (b < 0 && item < off + tot) {
          const int f = __builtin_ctzll(__ballot(off + incl > item));
          b = c0 + u * kWave + f;
          j = item - (off + __builtin_amdgcn_readlane(incl, f) - __builtin_amdgcn_readlane(F, f));
        }
        off += tot;
      }
    }
  } else {             // a partial last split: its size r, then its rank there
    const int w = item - full;
    // the largest r with more than w partial splits of at least r blocks
    int lo = 1, hi = S - 1;
#pragma unroll 1
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (plan_partials_from(p, len0, S, mid, lane) > w)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int r = lo;
    int k = w - (r + 1 < S ? plan_partials_from(p, len0, S, r + 1, lane) : 0);
#pragma unroll 1
    for (int c0 = 0; c0 < p.batch && b < 0; c0 += 4 * kWave) {
      int len[4];
      plan_chunk(p, c0, lane, len0, len);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int n = (len[u] + p.bs - 1) / p.bs;
        const uint64_t m = __ballot(n % S == r);
        const int pc = __builtin_popcountll(m);
        if (b < 0 && k < pc) {
          // the lane holding the k-th set bit of m
          const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
          const int f = __builtin_ctzll(__ballot(((m >> lane) & 1) && rank == k));
          b = c0 + u * kWave + f;
          j = __builtin_amdgcn_readlane(n / S, f);   // the last split
        }
        if (b < 0) k -= pc;
      }
    }
  }
  if (b < 0 || b >= p.batch) return false;
  out.b = b;
  plan_sequence_of(p, b, lane, len0, S, out.off, out.ns);
  out.len = plan_len(p, b);
  out.j = j;
  return true;
}

// Splits of sequence b and of all sequences before it.
__device__ __forceinline__ void plan_sequence(const PlanArgs& p, int b, int lane, int& off,
                                              int& ns) {
  int len0[4];
  plan_len4(p, 0, lane, len0);
  bool uniform;
  const int S = plan_split_blocks(p, lane, len0, uniform);
  plan_sequence_of(p, b, lane, len0, S, off, ns);
}

// Block ids of blocks [i0, ilast] of one sequence, 64 at a time: lane k of
// `cur` holds the id of block base + k and lane k of `nxt` that of block
// base + 64 + k (indices past ilast read ilast). A wave asks only for blocks
// in [base, base + 128) and calls advance() once it has passed base + 64.
// Each new window is waited for where it is loaded: vector loads retire in
// order, and a window still in flight where id() reads it (the read of
// `nxt` sits on every path) would make every ring turn wait for all of its
// block loads, where this way only the turns that advance, one per 64
// blocks, do.
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
    asm volatile("" ::"v"(cur), "v"(nxt));  // wait for both windows here
  }
  __device__ __forceinline__ int32_t id(int i) const {
    const int k = min(i, ilast) - base;
    return __builtin_amdgcn_readlane(k < kWave ? cur : nxt, k & (kWave - 1));
  }
  __device__ __forceinline__ void advance(int lane) {
    base += kWave;
    cur = nxt;
    nxt = row[min(base + kWave + lane, ilast)];
    asm volatile("" ::"v"(nxt));  // wait for the new window here
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
  constexpr bool RAW = CODE == KVQ_CODE_NONE16;
  // Per-token 8-bit codes step two 16-token tiles at a time; 16-token
  // blocks then ride a ring of two pairs.
  constexpr bool PAIR = !RAW && !KCH;
  constexpr int NBUF = BS == 16 ? (PAIR ? 4 : 3) : 2;  // blocks in the register ring
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
  // qs: the scaled query in fp32; qop: its fp16 operand, or for bf16 raw
  // rows the bf16 pair qop + qlo (with per-channel keys it is only needed
  // for the raw partial block, so it is made there)
#pragma unroll
  for (int e = 0; e < D / 4; ++e) qf[e] = hcol ? qf[e] * qdown : 0.0f;
  const float* qs = qf;
  const bool raw_bf16 = a.stage_bf16 != 0;
  half8v qop[NCH], qlo[NCH];
  auto make_qop = [&](bool pair) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (pair) {
        bf16_split8(qs + 8 * c, qop[c], qlo[c]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qop[c][e] = (half_t)qs[8 * c + e];
      }
    }
  };
  if constexpr (!KCH) make_qop(RAW && raw_bf16);
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
  using TileT = typename std::conditional<RAW, TileRaw<D, BS>, Tile8<D, BS>>::type;
  auto block = [&](const TileT& t, int i) {
    if constexpr (RAW) {
#pragma unroll
      for (int nt = 0; nt < BS / 16; ++nt)
        tile_step_raw<D, BS, false>(t, nt, i * BS + nt * 16, L, qop, qlo, cscore, j, st,
                                    raw_bf16);
    } else if constexpr (KCH) {
      half8v qb[NCH], ql[NCH];
      channel_query<D, BS>(t, lds, qs, lane, qb, ql);
      full_block_step<CODE, D, BS, kKeyChannel>(t, i, L, qb, cscore, j, st, ql);
    } else if constexpr (PAIR && BS >= 32) {
#pragma unroll
      for (int nt = 0; nt < BS / 16; nt += 2) tile_pair_step<CODE, D, BS>(t, nt, t, nt + 1, qop, cscore, st);
    } else {
      full_block_step<CODE, D, BS>(t, i, L, qop, cscore, j, st);
    }
  };
  // blocks [i0, ifull) are complete; a partial last block is handled apart
  const bool partial = i1 == nblk && (L % BS) != 0;
  const int ifull = partial ? i1 - 1 : i1;
  TileT buf[NBUF];
#pragma unroll
  for (int u = 0; u < NBUF; ++u) load_tile<D, BS, KCH, true>(buf[u], a, bh_of(i0 + u), lane);

  // Steady state: every slot computes one block and refills its buffer with
  // the block NBUF ahead (clamped to the split's last block, so the load
  // sequence never branches and the wait counts stay exact).
  int i = i0;
  for (; i + NBUF <= ifull; i += NBUF) {
    if (i - ids.base >= kWave) ids.advance(lane);
    if constexpr (PAIR && BS == 16) {
#pragma unroll
      for (int u = 0; u < NBUF; u += 2) {
        tile_pair_step<CODE, D, BS>(buf[u], 0, buf[u + 1], 0, qop, cscore, st);
        load_tile<D, BS, KCH, true>(buf[u], a, bh_of(i + u + NBUF), lane);
        load_tile<D, BS, KCH, true>(buf[u + 1], a, bh_of(i + u + 1 + NBUF), lane);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        block(buf[u], i + u);
        load_tile<D, BS, KCH, true>(buf[u], a, bh_of(i + u + NBUF), lane);
      }
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
  bool paired = false;  // the first two remaining 16-token blocks as one pair
  if constexpr (PAIR && BS == 16) {
    if (i + 1 < ifull) {
      tile_pair_step<CODE, D, BS>(buf[0], 0, buf[1], 0, qop, cscore, st);
      paired = true;
    }
  }
#pragma unroll
  for (int u = 0; u < NBUF; ++u) {
    if (u < 2 && paired) continue;
    if (i + u < ifull) {
      block(buf[u], i + u);
    } else if (i + u == ifull && partial) {
      if constexpr (RAW) {
#pragma unroll
        for (int nt = 0; nt < BS / 16; ++nt) {
          const int pos0 = (i + u) * BS + nt * 16;
          if (pos0 + 16 <= L)
            tile_step_raw<D, BS, false>(buf[u], nt, pos0, L, qop, qlo, cscore, j, st, raw_bf16);
          else if (pos0 < L)
            tile_step_raw<D, BS, true>(buf[u], nt, pos0, L, qop, qlo, cscore, j, st, raw_bf16);
        }
      } else if constexpr (KCH) {
        make_qop(raw_bf16);
        last_block_step<CODE, D, BS, true>(buf[u], i + u, L, qop, cscore, j, st, kraw, raw_bf16,
                                           qlo);
      } else {
        last_block_step<CODE, D, BS>(buf[u], i + u, L, qop, cscore, j, st);
      }
    }
  }
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

// Wave 0: merge the kNW wave states in red and write the split's partial.
template <int CODE, int D>
__device__ __forceinline__ void split_write(const DecodeArgs& a, const PlanItem& it, int g,
                                            int lane, float (*red)[D / 4 + 2][kWave]) {
  constexpr int NPV = D / 16;
  constexpr int NV = D / 4;
  const int r = lane & 15, j = lane >> 4;
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

// The step's new token of sequence b, KV head g, coded into the cache at
// position L - 1 before the wave that owns the sequence's last block reads
// it: quad 0 codes the key row and quad 1 the value row with the append's
// own coder, so the bytes equal those kvq_append writes. The wave's stores
// complete before its loads are issued; the block's other readers do not
// exist in this launch (each block belongs to one wave's share).
template <int CODE, int D, int BS>
__device__ __forceinline__ void append_new_token(const DecodeArgs& a, int b, int g, int L,
                                                 int lane) {
  constexpr int NV = D / 32;   // 16-byte pieces per lane of a row
  // a length past max_context_len (a broken precondition) was cut to L: the
  // row would land on a cached token, so the sequence takes none
  if (a.context_lens[b] != L) return;
  const int pos = L - 1;
  const int32_t id = a.block_tables[(int64_t)b * a.max_blocks + pos / BS];
  const int quad = lane >> 2, k = lane & 3;
  const bool isv = quad == 1;
  const bool live = quad < 2 && id >= 0 && id < a.num_blocks;
  const int64_t rowi = ((int64_t)(live ? id : 0) * a.H + g) * BS + pos % BS;
  const uint16_t* src = (isv ? a.new_v + (int64_t)b * a.new_v_stride
                             : a.new_k + (int64_t)b * a.new_k_stride) + g * D + 8 * k;
  u32x4 w[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u)
    w[u] = live ? *reinterpret_cast<const u32x4*>(src + 32 * u) : (u32x4){0u, 0u, 0u, 0u};
  if constexpr (CODE == KVQ_CODE_NONE16) {
    uint8_t* dst = (isv ? a.v_codes_w : a.k_codes_w) + rowi * (2 * D);
    if (live) {
#pragma unroll
      for (int u = 0; u < NV; ++u)
        *reinterpret_cast<u32x4*>(dst + 2 * (32 * u + 8 * k)) = w[u];
    }
  } else {
    uint8_t* dst = (isv ? a.v_codes_w : a.k_codes_w) + rowi * D;
    float* sc = (isv ? a.v_scale_w : a.k_scale_w) + rowi;
    if (a.new_bf16)
      code_row8<CODE, D, true, false>(w, k, 0.0f, dst, sc, live);
    else
      code_row8<CODE, D, false, false>(w, k, 0.0f, dst, sc, live);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// One item of the plan: the split's S blocks are cut into kNW consecutive
// shares, one per wave; the waves merge their softmax states through LDS and
// wave 0 writes the split's partial. Every wave calls this (it holds
// workgroup barriers); with ROUNDS the waves wait for wave 0 at the end, so
// that a next item may reuse red.
template <int CODE, int MODE, int D, int BS, bool ROUNDS>
__device__ __forceinline__ void split_item(const DecodeArgs& a, const PlanItem& it, int g,
                                           int lane, int wave,
                                           float (*red)[D / 4 + 2][kWave]) {
  constexpr int NPV = D / 16;   // output MFMAs (16 d-rows each)
  constexpr int NV = D / 4;     // accumulator values per lane
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
  if constexpr (!ROUNDS && MODE == KVQ_SCALE_TOKEN_SYM && CODE != KVQ_CODE_INT4) {
    if (a.new_k != nullptr && i0 < i1 && i1 == nblk) append_new_token<CODE, D, BS>(a, b, g, L, lane);
  }
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
  if (wave == 0) split_write<CODE, D>(a, it, g, lane, red);
  // the next item's waves write red only after wave 0 has read it
  if constexpr (ROUNDS) __syncthreads();
}

// Workgroup w takes the plan's (item, KV head) pair w. ROUNDS (a grid of
// kDecodeMaxGrid workgroups, for plans the host can only bound above that,
// i.e. large skewed batches whose bound assumes every context at its
// longest): the workgroups take the pairs x = 0, 1, ... in rounds of the grid
// size G, round 0 pair w and later rounds pair x0 + w or x0 + G - 1 - w (odd
// rounds), so that the extra pairs go first to the workgroups dispatched
// last, which hold the shortest items; without it such a batch would launch
// thousands of workgroups that find no item. Only scalars cross the rounds
// (each derives the plan again from the cached lengths): the rounds cost
// registers, so plans within the bound take the single-pair kernel.
template <int CODE, int MODE, int D, int BS, bool ROUNDS>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_kernel(DecodeArgs a) {
  constexpr int NV = D / 4;
  __shared__ float red[kNW][NV + 2][kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  // every wave derives the same plan, so every branch below is
  // workgroup-uniform
  const PlanArgs pa = plan_args(a.context_lens, a.batch, a.max_len, BS, a.H, a.split_blocks,
                                decode_skew_cap(CODE, MODE), decode_skew_lg(CODE, MODE));
  if constexpr (!ROUNDS) {
    int wg_item, g;
    workgroup_item(a.H, blockIdx.x, wg_item, g);
    const PlanCtx ctx = plan_ctx(pa, lane);
    PlanItem it;
    if (!plan_find_item(pa, ctx, wg_item, lane, it)) return;
    split_item<CODE, MODE, D, BS, false>(a, it, g, lane, wave, red);
  } else {
    const int G = (int)gridDim.x, w = (int)blockIdx.x;
    int need = 0;
    for (int x0 = 0, odd = 0; x0 == 0 || x0 < need; x0 += G, odd ^= 1) {
      const PlanCtx ctx = plan_ctx(pa, lane);
      need = __builtin_amdgcn_readfirstlane(plan_workgroups(pa, ctx, lane));
      const int x = x0 + (odd ? G - 1 - w : w);
      if (x >= need) continue;
      int wg_item, g;
      workgroup_item(a.H, x, wg_item, g);
      PlanItem it;
      if (!plan_find_item(pa, ctx, wg_item, lane, it)) continue;
      split_item<CODE, MODE, D, BS, true>(a, it, g, lane, wave, red);
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
  int32_t skew_cap;  // the split kernel's plan: decode_skew_cap / _lg of the layout
  int32_t skew_lg;
};


// One wave per (sequence, query head), one or kReduceHeads heads per
// workgroup.
// Lane s holds split s's (m, l); the partial accumulators of up to 32
// splits are loaded in the same batch, so a sequence with up to 32 splits is
// merged after a single memory round trip.
template <int D>
__global__ __launch_bounds__(64 * kReduceHeads) void decode_reduce_kernel(ReduceArgs a) {
  constexpr int EPL = D / 64;  // output elements per lane
  constexpr int KB = 32;       // splits per batch of loads
  typedef float floatE __attribute__((ext_vector_type(EPL)));
  const int lane = threadIdx.x & (kWave - 1);
  const int h = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave, b = blockIdx.y;
  if (h >= a.Hq) return;
  const PlanArgs pa = plan_args(a.context_lens, a.batch, a.max_len, a.BS, a.H, a.split_blocks,
                                a.skew_cap, a.skew_lg);
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
  // whole runs of 16 workgroups (see workgroup_item); the extra ones find no
  // item. Beyond kDecodeMaxGrid workgroups, the grid is capped and takes
  // rounds, except when the launch also appends the step's tokens: that code
  // lives in the single-pass kernel only (it would cost the rounds kernel
  // registers), whose surplus workgroups exit at once.
  const int64_t pairs = ((int64_t)items * a.H + 15) / 16 * 16;
  if (pairs <= kDecodeMaxGrid || a.new_k != nullptr)
    decode_split_kernel<CODE, MODE, D, BS, false><<<dim3((unsigned)pairs), 64 * kNW, 0, stream>>>(a);
  else
    decode_split_kernel<CODE, MODE, D, BS, true><<<dim3(kDecodeMaxGrid), 64 * kNW, 0, stream>>>(a);
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

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t decode_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      // with `dev` current: each GPU holds its own copy at its own address
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
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
  if (p.new_k != nullptr) {
    a.new_k = static_cast<const uint16_t*>(p.new_k);
    a.new_v = static_cast<const uint16_t*>(p.new_v);
    a.new_k_stride = p.new_k_stride;
    a.new_v_stride = p.new_v_stride;
    a.k_codes_w = static_cast<uint8_t*>(const_cast<void*>(p.k_codes));
    a.v_codes_w = static_cast<uint8_t*>(const_cast<void*>(p.v_codes));
    a.k_scale_w = const_cast<float*>(p.k_scale);
    a.v_scale_w = const_cast<float*>(p.v_scale);
    a.new_bf16 = p.src_bf16;
  }
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
  ra.skew_cap = decode_skew_cap(p.k_code, p.k_mode);
  ra.skew_lg = decode_skew_lg(p.k_code, p.k_mode);
  const int hpg = reduce_heads_per_group((int64_t)p.num_q_heads * p.batch);
  dim3 grid((p.num_q_heads + hpg - 1) / hpg, p.batch);
  if (p.head_dim == 128)
    decode_reduce_kernel<128><<<grid, kWave * hpg, 0, stream>>>(ra);
  else
    decode_reduce_kernel<64><<<grid, kWave * hpg, 0, stream>>>(ra);
  return hipGetLastError();
}

}  // namespace kvq
