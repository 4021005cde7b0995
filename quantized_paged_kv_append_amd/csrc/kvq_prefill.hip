// kvq_prefill.hip -- multi-query (prefill) attention over the quantized
// paged cache (gfx950): several causal queries per sequence at once.
#include "kvq_attn_tiles.h"
#include "kvq_int4_tiles.h"

namespace kvq {
namespace {

// ---------------------------------------------------------------------------
// Multi-query (prefill) attention over the same cache ("KV Cache
// Optimization: Strategies for Faster LLM Inference", sections "Why KV Cache
// Is Essential for Efficient LLM Inference" -- the prompt is processed as a
// whole before decoding -- and "Implementing KV Cache Optimization: A
// Practical Checklist" -- that phase is compute-bound). Sequence b's queries
// are its last nq positions; query i (position L - nq + i) sees positions
// 0 .. L - nq + i.
//
// The 16 MFMA columns of a tile are 16 consecutive (query, head) pairs
// c = i G + r of one KV head g: the G heads of a query are adjacent, a tile
// spans 16 / G queries (or a query G / 16 tiles). A wave serves one or two
// tiles (each block it loads and converts then serves 16 or 32 columns), with
// a causal limit (and window start) per lane and tile. A workgroup takes one
// unit (sequence b, split j of S blocks, KV head g, group of up to four
// waves' tiles); waves on the same tiles stream consecutive shares of the
// split through the decode's register ring and tile steps and merge their
// softmax states through LDS. The waves of a workgroup read the same blocks,
// which meet in L1. Each unit writes a partial (m, l, acc) per column;
// prefill_reduce merges the splits.
// ---------------------------------------------------------------------------
struct PrefillArgs {
  DecodeArgs a;
  const int32_t* qstart;
  int32_t J;    // splits per sequence (rows of partials in the workspace)
  int32_t S;    // blocks per split
  int32_t CT;   // column tiles per (sequence, KV head)
  int32_t max_q;  // bound on every sequence's query count (sizes CT and the grid)
  int32_t TW;   // column tiles per workgroup: 1, 2 or 4 (4 / TW waves per tile)
  int32_t window;   // > 0: each query sees its last `window` positions ...
  int32_t sink;     // ... and the first `sink` positions
  int32_t bs_log2;  // log2 of the block size (the LDS-staged kernel)
  int32_t Jg;       // splits per sequence enumerated by the grid (J rounded up to
                    // odd; splits j >= J start past every sequence and exit)
};

// NC: 16-column tiles per wave. With NC = 2 a block's codes are loaded and
// converted once for 32 columns (per-channel keys keep NC = 1: their
// per-block query folding needs the fp32 query of every column).
// A wave's share of a split over 4-bit codes for its NC column tiles: the
// visible blocks as positions [x0, x1) in the sink blocks A = [s0, s0 + nA)
// then the window's blocks from bstart. Blocks seen whole by every column
// stream through a four-tile register ring in pairs of tiles; the others
// (sink blocks, the window's first blocks, the context's last one or two)
// go tile by tile with this lane's column masks (limit Lr, window start lo,
// sink count).
template <int D, int BS, int MODE, int NC>
__device__ __forceinline__ void prefill_blocks_int4(const PrefillArgs& pa, int b, int g, int L,
                                                    int s0, int x0, int x1, int nA, int bstart,
                                                    int Lmin, int Lmax, int lo_min, int lo_max,
                                                    const int* Lr, const int* lo,
                                                    const half8v (*qop)[D / 32],
                                                    const float* cscore, int lane,
                                                    SoftmaxState<D>* st) {
  constexpr int TPB = BS / 16;  // tiles per block
  constexpr int NBUF = 4;       // tiles in the ring: two pairs
  const DecodeArgs& a = pa.a;
  const int jj = lane >> 4;
  const int W = pa.window, SK = pa.window > 0 ? pa.sink : 0;
  const Nib4Consts kc = nib4_consts();
  const Lane4 lo4 = lane4_offsets<D, MODE>(lane);
  const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks;
  // ids outside the pool (a broken precondition, or a block dropped from a
  // window) are read as block 0, which every wave shares
  auto bh_of = [&](int i) -> int64_t {
    const int32_t id = trow[i];
    return (int64_t)(id >= 0 && id < a.num_blocks ? id : 0) * a.H + g;
  };
  const int b0 = bstart + max(x0, nA) - nA, b1 = bstart + x1 - nA;
  const int iseen = Lmin / BS;
  const int wf0 = W > 0 ? (max(lo_max, 0) + BS - 1) / BS : 0;
  const int ra = min(max(wf0, b0), max(b1, b0));
  const int rb = min(max(iseen, ra), max(b1, ra));
  auto edge_run = [&](int e0, int e1) {
    for (int i = e0; i < e1; ++i) {
      const int64_t bh = bh_of(i);
#pragma unroll
      for (int nt = 0; nt < TPB; ++nt) {
        const int pos0 = i * BS + nt * 16;
        // no column sees the tile: past every limit, or between the sinks
        // and every window
        if (pos0 >= Lmax || (W > 0 && pos0 >= SK && pos0 + 16 <= lo_min)) continue;
        const bool masked = pos0 + 16 > Lmin || (W > 0 && pos0 < lo_max && pos0 + 16 > SK);
        Tile4<D, MODE> t;
        load_tile4<D, BS, MODE>(t, a, bh, nt, lo4);
        if (masked)
          tile4_step<D, MODE, NC, true>(t, pos0, Lr, qop, cscore, jj, st, kc, lo, SK);
        else
          tile4_step<D, MODE, NC, false>(t, pos0, Lr, qop, cscore, jj, st, kc, lo, SK);
      }
    }
  };
  edge_run(s0 + x0, s0 + min(x1, nA));   // sink blocks
  edge_run(b0, ra);
  if (ra < rb) {
    // tiles [T0, T1) of the whole blocks; refills past T1 read tile 0 of
    // block 0, which every wave shares
    const int T0 = ra * TPB, T1 = rb * TPB;
    auto load = [&](Tile4<D, MODE>& t, int tile) {
      const bool past = tile >= T1;
      load_tile4<D, BS, MODE>(t, a, past ? (int64_t)g : bh_of(tile / TPB), past ? 0 : tile % TPB,
                              lo4);
    };
    Tile4<D, MODE> buf[NBUF];
#pragma unroll
    for (int u = 0; u < NBUF; ++u) load(buf[u], T0 + u);
    int tt = T0;
    for (; tt + NBUF <= T1; tt += NBUF) {
      tile4_pair_step<D, MODE, NC>(buf[0], buf[1], qop, cscore, st, kc);
      load(buf[0], tt + NBUF);
      load(buf[1], tt + NBUF + 1);
      tile4_pair_step<D, MODE, NC>(buf[2], buf[3], qop, cscore, st, kc);
      load(buf[2], tt + NBUF + 2);
      load(buf[3], tt + NBUF + 3);
    }
#pragma unroll
    for (int u = 0; u < NBUF; ++u)
      if (tt + u < T1)
        tile4_step<D, MODE, NC, false>(buf[u], (tt + u) * 16, Lr, qop, cscore, jj, st, kc, lo, SK);
  }
  edge_run(rb, b1);
}

template <int CODE, int MODE, int D, int BS, int NC>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_split_kernel(PrefillArgs pa) {
  constexpr int NCH = D / 32;
  constexpr int NPV = D / 16;
  constexpr int NV = D / 4;
  constexpr int NBUF = BS == 16 ? 3 : 2;  // blocks in the register ring
  constexpr bool KCH = MODE == KVQ_SCALE_CHANNEL_BLOCK_SYM;
  constexpr bool RAW = CODE == KVQ_CODE_NONE16;
  constexpr bool I4 = CODE == KVQ_CODE_INT4;
  static_assert(!KCH || NC == 1, "per-channel keys take one column tile per wave");
  using TileT = typename std::conditional<RAW, TileRaw<D, BS>, Tile8<D, BS>>::type;
  __shared__ float red[kNW][NV + 2][kWave];
  const DecodeArgs& a = pa.a;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, jj = lane >> 4;
  // unit (b, j, g, tile group); wave w serves column tiles NC (tg TW + w % TW)
  // .. + NC - 1 and the (w / TW)-th of the 4 / TW shares of the split's blocks
  const int cts = (pa.CT + NC - 1) / NC;
  const int ctg = (cts + pa.TW - 1) / pa.TW;
  int64_t u = blockIdx.x;
  const int tg = (int)(u % ctg);
  u /= ctg;
  const int g = (int)(u % a.H);
  u /= a.H;
  const int j = (int)(u % pa.Jg);
  const int b = (int)(u / pa.Jg);
  if (b >= a.batch) return;
  const int L = min(a.context_lens[b], a.max_len);
  const int q0 = pa.qstart[b];
  // queries past max_q would index past the CT * 16 columns of a partial row
  const int nq = min(min(pa.qstart[b + 1] - q0, L), pa.max_q);
  const int ncol = nq * a.G;
  const int nblk = (L + BS - 1) / BS;
  const int s0 = j * pa.S;
  // workgroup-uniform exits: no split here, or no column in the tile group
  if (s0 >= nblk || tg * pa.TW * NC * 16 >= ncol) return;
  const int nshare = kNW / pa.TW;
  const int cbase = (tg * pa.TW + wave % pa.TW) * NC * 16;
  const bool active = cbase < ncol;   // tiles past the columns only join the merge

  // ---- columns: lane (r, jj) serves columns cbase + 16 c + r, c < NC -------
  int col[NC], Lr[NC], lo_r[NC];
  bool valid[NC];
  float cscore[NC];
  const int W = pa.window, SK = pa.window > 0 ? pa.sink : 0;
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    col[cc] = cbase + 16 * cc + r;
    valid[cc] = col[cc] < ncol;
    Lr[cc] = valid[cc] ? L - nq + col[cc] / a.G + 1 : 0;   // the column's limit
    lo_r[cc] = W > 0 ? Lr[cc] - W : 0;                       // its window start
  }
  // bounds over the wave's columns
  const int Lmin = L - nq + cbase / a.G + 1;
  const int Lmax = active ? L - nq + (min(ncol, cbase + 16 * NC) - 1) / a.G + 1 : 0;
  const int lo_min = W > 0 ? Lmin - W : 0;
  const int lo_max = W > 0 ? Lmax - W : 0;
  // the visible blocks of the split (none past what any of the columns
  // sees): the sink blocks A = [s0, a_end) and the window's blocks
  // B = [bstart, s1), with nothing between them read
  const int s1 = min(min(s0 + pa.S, nblk), (Lmax + BS - 1) / BS);
  const int nsb = (SK + BS - 1) / BS;
  const int wb0 = max(lo_min, 0) / BS;   // first block any window reaches
  const bool gap = wb0 > nsb;
  const int a_end = gap ? max(s0, min(s1, nsb)) : s0;
  const int bstart = gap ? max(a_end, max(s0, wb0)) : s0;
  const int nA = a_end - s0, nV = nA + max(s1 - bstart, 0);
  // the wave's share of the visible blocks, as positions x in A then B
  const int share = (nV + nshare - 1) / nshare;
  const int x0 = (wave / pa.TW) * share, x1 = min(x0 + share, nV);

  // ---- queries, each column pre-scaled by a power of two (as in decode) ---
  float qf[D / 4];      // the last column's fp32 query (per-channel keys: NC = 1)
  half8v qop[NC][NCH];  // fp16 operands (made later with per-channel keys), or
  half8v qlo[NC][NCH];  // for bf16 raw rows the bf16 pairs qop + qlo
  const bool raw_bf16 = a.stage_bf16 != 0;
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    const int qi = valid[cc] ? col[cc] / a.G : 0;
    const int hq = g * a.G + (valid[cc] ? col[cc] % a.G : 0);
    if constexpr (I4) {   // the 4-bit operand order, made from the whole row
      query_int4<D>(a, a.q + ((int64_t)(q0 + qi) * a.Hq + hq) * D, jj, valid[cc], qop[cc],
                    cscore[cc]);
      continue;
    }
    const uint16_t* qp = a.q + ((int64_t)(q0 + qi) * a.Hq + hq) * D + jj * (D / 4);
    if (a.q_bf16)
      load_query<true, D>(qp, qf);
    else
      load_query<false, D>(qp, qf);
    float qmax = 0.0f;
#pragma unroll
    for (int e = 0; e < D / 4; ++e) qmax = fmaxf(qmax, fabsf(qf[e]));
    qmax = colmax4(qmax);
    int qe = qmax > 0.0f ? (int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127 : 0;
    qe = max(qe, -126);
    const float qdown = __uint_as_float((uint32_t)(127 - qe) << 23);
    const float qup = __uint_as_float((uint32_t)(127 + qe) << 23);
#pragma unroll
    for (int e = 0; e < D / 4; ++e) qf[e] = valid[cc] ? qf[e] * qdown : 0.0f;
    if constexpr (!KCH) {
#pragma unroll
      for (int k8 = 0; k8 < NCH; ++k8) {
        if (RAW && raw_bf16) {
          bf16_split8(qf + 8 * k8, qop[cc][k8], qlo[cc][k8]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) qop[cc][k8][e] = (half_t)qf[8 * k8 + e];
        }
      }
    }
    cscore[cc] = valid[cc] ? qup * a.sm_log2 : 0.0f;
  }

  SoftmaxState<D> st[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    st[cc].m = -INFINITY;
    st[cc].l = 0.0f;
#pragma unroll
    for (int k = 0; k < NPV; ++k) st[cc].acc[k] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
  }

  if constexpr (I4) {
    if (x0 < x1) prefill_blocks_int4<D, BS, MODE, NC>(pa, b, g, L, s0, x0, x1, nA, bstart, Lmin,
                                                      Lmax, lo_min, lo_max, Lr, lo_r, qop, cscore,
                                                      lane, st);
  } else if (x0 < x1) {
    // per-channel keys: a partly filled last block is read raw from stage row b
    const bool staged = KCH && (L % BS) != 0;
    // the wave's LDS slice for the per-channel query (the merge area, unused
    // until the waves have finished streaming)
    float* xs = &red[wave][0][0];
    const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks;
    // ids outside the pool (a broken precondition, or a block dropped from a
    // window) are read as block 0, which every wave shares
    auto bh_of = [&](int i) -> int64_t {
      const int32_t id = trow[i];
      return (int64_t)(id >= 0 && id < a.num_blocks ? id : 0) * a.H + g;
    };
    // the share's blocks of B: [b0, b1); of those, [ra, rb) are seen whole by
    // every column (and hold codes) and stream through the register ring;
    // the rest -- sink blocks, the first blocks of the window, the last one
    // or two of the context, a staged one -- take per-column masks
    const int b0 = bstart + max(x0, nA) - nA, b1 = bstart + x1 - nA;
    const int iseen = (KCH && staged) ? min(Lmin / BS, nblk - 1) : Lmin / BS;
    const int wf0 = W > 0 ? (max(lo_max, 0) + BS - 1) / BS : 0;
    const int ra = min(max(wf0, b0), max(b1, b0));
    const int rb = min(max(iseen, ra), max(b1, ra));
    auto full_block = [&](const TileT& t, int i) {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        if constexpr (RAW) {
#pragma unroll
          for (int nt = 0; nt < BS / 16; ++nt)
            tile_step_raw<D, BS, false>(t, nt, i * BS + nt * 16, L, qop[cc], qlo[cc],
                                        cscore[cc], jj, st[cc], raw_bf16);
        } else if constexpr (KCH) {
          half8v qb[NCH], ql[NCH];
          channel_query<D, BS>(t, xs, qf, lane, qb, ql);
          full_block_step<CODE, D, BS, kKeyChannel>(t, i, L, qb, cscore[cc], jj, st[cc], ql);
        } else {
          full_block_step<CODE, D, BS>(t, i, L, qop[cc], cscore[cc], jj, st[cc]);
        }
      }
    };
    auto edge_block = [&](const TileT& t, int i) {
      const bool rawk = KCH && staged && i == nblk - 1;
      half8v qb[NCH], ql[NCH];
      u32x4 kraw[BS / 16][NCH];   // the staged rows, loaded here only
      if constexpr (KCH && !RAW) {
        if (!rawk) {
          channel_query<D, BS>(t, xs, qf, lane, qb, ql);
        } else {
#pragma unroll
          for (int nt = 0; nt < BS / 16; ++nt) {
            const uint16_t* sp =
                a.k_stage + (((int64_t)b * a.H + g) * BS + nt * 16 + r) * D + jj * (D / 4);
#pragma unroll
            for (int k8 = 0; k8 < NCH; ++k8)
              kraw[nt][k8] = *reinterpret_cast<const u32x4*>(sp + 8 * k8);
          }
#pragma unroll
          for (int k8 = 0; k8 < NCH; ++k8) {
            if (raw_bf16) {
              bf16_split8(qf + 8 * k8, qb[k8], ql[k8]);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) qb[k8][e] = (half_t)qf[8 * k8 + e];
            }
          }
        }
      }
#pragma unroll
      for (int nt = 0; nt < BS / 16; ++nt) {
        const int pos0 = i * BS + nt * 16;
        // no column sees the tile: past every limit, or between the sinks
        // and every window
        if (pos0 >= Lmax || (W > 0 && pos0 >= SK && pos0 + 16 <= lo_min)) continue;
        const bool masked =
            pos0 + 16 > Lmin || (W > 0 && pos0 < lo_max && pos0 + 16 > SK);
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          if constexpr (RAW) {
            if (masked)
              tile_step_raw<D, BS, true>(t, nt, pos0, Lr[cc], qop[cc], qlo[cc], cscore[cc], jj,
                                         st[cc], raw_bf16, L, lo_r[cc], SK);
            else
              tile_step_raw<D, BS, false>(t, nt, pos0, Lr[cc], qop[cc], qlo[cc], cscore[cc], jj,
                                          st[cc], raw_bf16, L);
          } else if constexpr (KCH) {
            if (rawk) {   // qb holds the plain fp16 query here, or qb + ql the bf16 pair
              if (masked)
                tile_step<CODE, D, BS, true, kKeyRaw>(t, nt, pos0, Lr[cc], qb, cscore[cc], jj,
                                                      st[cc], kraw[nt], raw_bf16, ql, L,
                                                      lo_r[cc], SK);
              else
                tile_step<CODE, D, BS, false, kKeyRaw>(t, nt, pos0, Lr[cc], qb, cscore[cc], jj,
                                                       st[cc], kraw[nt], raw_bf16, ql, L);
            } else if (masked) {
              tile_step<CODE, D, BS, true, kKeyChannel>(t, nt, pos0, Lr[cc], qb, cscore[cc], jj,
                                                        st[cc], nullptr, false, ql, L, lo_r[cc],
                                                        SK);
            } else {
              tile_step<CODE, D, BS, false, kKeyChannel>(t, nt, pos0, Lr[cc], qb, cscore[cc],
                                                         jj, st[cc], nullptr, false, ql, L);
            }
          } else {
            if (masked)
              tile_step<CODE, D, BS, true>(t, nt, pos0, Lr[cc], qop[cc], cscore[cc], jj, st[cc],
                                           nullptr, false, nullptr, L, lo_r[cc], SK);
            else
              tile_step<CODE, D, BS, false>(t, nt, pos0, Lr[cc], qop[cc], cscore[cc], jj,
                                            st[cc], nullptr, false, nullptr, L);
          }
        }
      }
    };
    auto edge_run = [&](int e0, int e1) {
      for (int i = e0; i < e1; ++i) {
        TileT t;
        load_tile<D, BS, KCH>(t, a, bh_of(i), lane);
        edge_block(t, i);
      }
    };
    edge_run(s0 + x0, s0 + min(x1, nA));   // sink blocks
    edge_run(b0, ra);
    // register ring over the whole blocks: every slot computes one block and
    // refills its buffer with the block NBUF ahead (past rb: block 0)
    if (ra < rb) {
      auto bh_full = [&](int i) -> int64_t { return i < rb ? bh_of(i) : (int64_t)g; };
      TileT buf[NBUF];
#pragma unroll
      for (int v = 0; v < NBUF; ++v) load_tile<D, BS, KCH>(buf[v], a, bh_full(ra + v), lane);
      for (int i = ra; i < rb; i += NBUF) {
#pragma unroll
        for (int v = 0; v < NBUF; ++v) {
          if (i + v < rb) full_block(buf[v], i + v);
          load_tile<D, BS, KCH>(buf[v], a, bh_full(i + v + NBUF), lane);
        }
      }
    }
    edge_run(rb, b1);
  }

  // ---- merge the waves' states, then write one partial per column ---------
  // one column tile at a time through the same LDS area
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    const float lsum = colsum4(st[cc].l);
    __syncthreads();   // every wave is done with the LDS area
#pragma unroll
    for (int k = 0; k < NPV; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][4 * k + e][lane] = st[cc].acc[k][e];
    red[wave][NV][lane] = st[cc].m;
    red[wave][NV + 1][lane] = lsum;
    __syncthreads();
    // waves w < TW merge the shares of their columns: waves w, w + TW, ...
    if (wave < pa.TW && valid[cc]) {
      float M = -INFINITY;
      for (int w = wave; w < kNW; w += pa.TW) M = fmaxf(M, red[w][NV][lane]);
      float acc[NV], l = 0.0f;
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] = 0.0f;
      for (int w = wave; w < kNW; w += pa.TW) {
        const float mw = red[w][NV][lane];
        const float sc = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        l += sc * red[w][NV + 1][lane];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] += sc * red[w][v][lane];
      }
      const int64_t pidx = (((int64_t)b * pa.J + j) * a.H + g) * (pa.CT * 16) + col[cc];
      if (jj == 0) *reinterpret_cast<float2*>(a.ws_ml + pidx * 2) = make_float2(M, l);
      if constexpr (I4) {
        // acc[4 m + e], m = 2 i + t, holds output element 32 i + 8 jj + 2 e + t
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
          float* dst = a.ws_acc + pidx * D + 32 * i + 8 * jj;
          const float* A0 = acc + 8 * i;      // t = 0
          const float* A1 = acc + 8 * i + 4;  // t = 1
          *reinterpret_cast<float4v*>(dst) = (float4v){A0[0], A1[0], A0[1], A1[1]};
          *reinterpret_cast<float4v*>(dst + 4) = (float4v){A0[2], A1[2], A0[3], A1[3]};
        }
        continue;
      }
      // acc[4 k + e] holds output element (d/16) (4 jj + e) + k of the column
      float* dst = a.ws_acc + pidx * D + jj * (D / 4);
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
}

// ---------------------------------------------------------------------------
// Multi-query attention with the cache converted once per workgroup (8-bit
// codes with per-token scales, no window). A workgroup takes one unit
// (sequence b, split j, KV head g, column group) and streams the split in
// chunks of 16 tokens per wave (64 with four waves, 32 with two): its
// threads load each chunk's key and value codes once, 16 bytes per load,
// convert them to fp16 (exact for INT8 and E4M3 codes) and store them with
// the per-token scales in one of two LDS buffers; the waves then take their
// MFMA operands from LDS, so a block is fetched and converted once for all
// the columns of the workgroup, not once per wave. Wave w serves NCW column
// tiles (16 (query, head) columns each, numbered as in prefill_split_kernel)
// and the (w / TW)-th of NW / TW interleaved shares of a chunk's 16-token
// tiles. The next two chunks are in flight in registers while a chunk is
// computed. Rows past the split's last visible position carry scale 0 and
// every lane's mask excludes them (its column's causal limit).
// LDS key and value rows hold D fp16 values and 8 halves of padding: the 16
// lanes of a 16-byte key read then start on 16 different 4-bank groups, and
// the 16 rows of a transposing value read (below) on 16 different ones.
// ---------------------------------------------------------------------------
// ds_read_b64_tr_b16 (gfx950): each lane gives the LDS address of 4 fp16
// values; in each group of 16 lanes, lane i receives as its value k the
// (i % 4)-th value of those that lane 4 k + i / 4 points at.
__device__ __forceinline__ half4v lds_read_tr16(const half_t* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      half4v, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(p)));
}

constexpr int kMqMaxSplit = 512;  // blocks per split at most (the ids staged in LDS)
static_assert(kMqMaxSplit >= kPrefillMaxSplitBlocks, "a split's ids fit in LDS");

template <int D, int CH, int NW>
struct MqLds {
  static constexpr int KSTR = D + 8;                      // halves per key row
  static constexpr int VSTR = D + 8;                      // halves per value row
  static constexpr int PLANE = CH * KSTR * 2;             // bytes: the keys of a chunk
  static constexpr int VPLANE = CH * VSTR * 2;            // bytes: its values
  static constexpr int SCALES = PLANE + VPLANE;           // then key and value scales
  static constexpr int BUF = SCALES + 2 * CH * 4;
  static constexpr int BYTES = 2 * BUF;                   // double buffer
  static constexpr int IDS = BYTES;                       // then the split's block ids
  static constexpr int TOTAL = IDS + kMqMaxSplit * 4;
  static constexpr int RED = NW * (D / 4 + 2) * kWave * 4;   // the waves' merge area
  static_assert(RED <= BYTES, "the merge reuses the chunk buffers");
};

// One online-softmax step of each of a wave's NCW column tiles over its NT
// tiles of a chunk, in two parts: mq_scores (scaled scores and column
// maxima) and mq_weights (rescale, then weights). S[cc][k] are the raw scores of tile k (token 4 jj + e of
// the tile in element e), sk / sv the key / value scales of those tokens,
// cscore[cc] > 0 the column's score factor, so the largest scaled score is
// cscore times the largest S sk (the column maxima of both tiles in one
// lane exchange when NCW = 2). The reference st.m moves only when a score exceeds it, and
// then to that score plus kMqHeadroom (log2 units): weights stay below
// 2^-kMqHeadroom and the smaller increases that follow cost no rescale of
// the accumulators (with 16 columns to a tile one of them reaches a new
// maximum in almost every chunk). The merges need a common reference for l
// and acc, not the maximum itself. Writes the PV operands pop[cc][k] =
// fp16(p sv). MASKED: token t counts for the lane's column only if t < lim[cc].
// st.m starts at the finite kMqNone, below every real reference, so that no
// step needs a guard for an infinite one: a masked score (-inf) gives
// exp2(-inf) = 0 against it, and the first visible score replaces it.
constexpr float kMqHeadroom = 2.0f;
constexpr float kMqNone = -3.0e38f;

template <int NCW, int NT, bool MASKED>
__device__ __forceinline__ void mq_scores(const float4v (&S)[NCW][NT], const float4v* sk,
                                          const int* lim, const int* pos0, int jj,
                                          float (&u)[NCW][NT][4], float (&mt)[NCW]) {
  float mx[NCW];
#pragma unroll
  for (int cc = 0; cc < NCW; ++cc) {
    mx[cc] = -INFINITY;
#pragma unroll
    for (int k = 0; k < NT; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u[cc][k][e] = S[cc][k][e] * sk[k][e];
        if (MASKED && pos0[k] + 4 * jj + e >= lim[cc]) u[cc][k][e] = -INFINITY;
        mx[cc] = fmaxf(mx[cc], u[cc][k][e]);
      }
  }
  if constexpr (NCW == 2)
    colmax4x2(mx[0], mx[1], mt[0], mt[1]);
  else
    mt[0] = colmax4(mx[0]);
}

template <int D, int NCW, int NT>
__device__ __forceinline__ void mq_weights(const float (&u)[NCW][NT][4], const float (&mt)[NCW],
                                           const float4v* sv, const float* cscore,
                                           SoftmaxState<D>* st, half4v (&pop)[NCW][NT]) {
  constexpr int NPV = D / 16;
  // the rescales first (branches), then the weights of every column tile
  // in one basic block
#pragma unroll
  for (int cc = 0; cc < NCW; ++cc) {
    SoftmaxState<D>& s = st[cc];
    const float m = mt[cc] * cscore[cc];
    if (__any(m > s.m)) {
      const float mn = m > s.m ? m + kMqHeadroom : s.m;
      const float alpha = __builtin_amdgcn_exp2f(s.m - mn);   // 1 where s.m stays
      s.l *= alpha;
#pragma unroll
      for (int c = 0; c < NPV; ++c) s.acc[c] *= alpha;
      s.m = mn;
    }
  }
#pragma unroll
  for (int cc = 0; cc < NCW; ++cc) {
    SoftmaxState<D>& s = st[cc];
    float lsum;
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)   // masked: exp2(-inf) = 0
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(u[cc][k][e], cscore[cc], -s.m));
      const float ps = (p[0] + p[1]) + (p[2] + p[3]);
      lsum = k == 0 ? ps : lsum + ps;
#pragma unroll
      for (int e = 0; e < 4; ++e) pop[cc][k][e] = (half_t)(p[e] * sv[k][e]);
    }
    s.l += lsum;
  }
}

// Multi-query kernel over LDS chunks. NW waves per workgroup and CH = 16 NW
// tokens per chunk (one 16-token tile per wave). TW: column-tile groups per
// workgroup (and tiles per wave per chunk: wave w takes tiles w / TW + k
// (NW / TW), k < TW, one softmax step per two of them); NCW: column tiles
// per wave.
template <int CODE, int D, int NCW, int TW, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void mq_split_kernel(PrefillArgs pa) {
  constexpr int NCH = D / 32;
  constexpr int NPV = D / 16;
  constexpr int NV = D / 4;
  constexpr int CH = 16 * NW;
  constexpr int NTC = CH / 16;        // 16-token tiles per chunk
  constexpr int NSH = NTC / TW;       // waves sharing a column tile group (tile stride)
  constexpr int SG = TW < 2 ? TW : 2; // tiles per softmax step
  constexpr int PPT = D / 64;         // 16-byte code pieces per thread per plane and chunk
  using Lds = MqLds<D, CH, NW>;
  constexpr int KSTR = Lds::KSTR;
  constexpr int VSTR = Lds::VSTR;
  constexpr int DL = D == 128 ? 7 : 6;  // log2 D
  constexpr int NPF = 2;              // chunks in flight in registers
  static_assert(NTC == NW && CH * D / 16 == PPT * 64 * NW, "chunk shape");
  __shared__ __align__(16) unsigned char smem[Lds::TOTAL];
  const DecodeArgs& a = pa.a;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int r = lane & 15, jj = lane >> 4;
  const int bsl = pa.bs_log2, BS = 1 << bsl;   // block size 16 or 32

  // ---- unit: workgroup x runs on XCD x % 8; the column groups of one
  // (b, j, g) are consecutive there, so they share that XCD's L2 ----------
  const int cts = (pa.CT + NCW - 1) / NCW;
  const int CG = (cts + TW - 1) / TW;
  const int64_t x = blockIdx.x;
  const int64_t k8 = x >> 3;
  const int cg = (int)(k8 % CG);
  int64_t item = (k8 / CG) * 8 + (x & 7);
  const int g = (int)(item % a.H);
  item /= a.H;
  const int j = (int)(item % pa.Jg);
  const int b = (int)(item / pa.Jg);
  if (b >= a.batch) return;
  const int L = min(a.context_lens[b], a.max_len);
  const int q0 = pa.qstart[b];
  const int nq = min(min(pa.qstart[b + 1] - q0, L), pa.max_q);
  const int ncol = nq * a.G;
  const int nblk = (L + BS - 1) >> bsl;
  const int s0 = j * pa.S;
  const int cw0 = cg * TW * NCW * 16;   // the workgroup's first column
  if (s0 >= nblk || cw0 >= ncol) return;   // workgroup-uniform
  const int sh = wave / TW;
  const int cbase = cw0 + (wave % TW) * NCW * 16;   // the wave's first column
  const bool active = cbase < ncol;
  // tokens [t0, t1) of the split that some column of the workgroup sees
  const int Lmax = L - nq + (min(ncol, cw0 + TW * NCW * 16) - 1) / a.G + 1;
  const int s1 = min(min(s0 + pa.S, nblk), (Lmax + BS - 1) >> bsl);
  const int t0 = s0 << bsl, t1 = max(min(s1 << bsl, Lmax), t0);
  // the wave's least limit (its first column's)
  const int lim_lo = min(L - nq + cbase / a.G + 1, t1);

  // ---- columns: lane (r, jj) serves columns cbase + 16 cc + r ---------------
  int col[NCW], lim[NCW];
  bool valid[NCW];
  float cscore[NCW];
  half8v qop[NCW][NCH];
#pragma unroll
  for (int cc = 0; cc < NCW; ++cc) {
    col[cc] = cbase + 16 * cc + r;
    valid[cc] = col[cc] < ncol;
    lim[cc] = valid[cc] ? min(L - nq + col[cc] / a.G + 1, t1) : 0;
    const int qi = valid[cc] ? col[cc] / a.G : 0;
    const int hq = g * a.G + (valid[cc] ? col[cc] % a.G : 0);
    const uint16_t* qp = a.q + ((int64_t)(q0 + qi) * a.Hq + hq) * D + jj * (D / 4);
    float qf[D / 4];
    if (a.q_bf16)
      load_query<true, D>(qp, qf);
    else
      load_query<false, D>(qp, qf);
    float qmax = 0.0f;
#pragma unroll
    for (int e = 0; e < D / 4; ++e) qmax = fmaxf(qmax, fabsf(qf[e]));
    qmax = colmax4(qmax);
    int qe = qmax > 0.0f ? (int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127 : 0;
    qe = max(qe, -126);
    const float qdown = __uint_as_float((uint32_t)(127 - qe) << 23);
    const float qup = __uint_as_float((uint32_t)(127 + qe) << 23);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[cc][c][e] = (half_t)(valid[cc] ? qf[8 * c + e] * qdown : 0.0f);
    // positive in every lane (mq_softmax takes the maximum through it);
    // columns past the last have zero queries and are never written
    cscore[cc] = valid[cc] ? qup * a.sm_log2 : 1.0f;
  }
  SoftmaxState<D> st[NCW];
#pragma unroll
  for (int cc = 0; cc < NCW; ++cc) {
    st[cc].m = kMqNone;
    st[cc].l = 0.0f;
#pragma unroll
    for (int k = 0; k < NPV; ++k) st[cc].acc[k] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
  }

  // ---- the split's block ids go to LDS first: a chunk's code loads then
  // wait on no other vector load (those complete in order, so waiting on an
  // id just loaded would also wait on the chunks already in flight). Ids
  // outside the pool (a broken precondition) are read as block 0. --------
  int32_t* ids = reinterpret_cast<int32_t*>(smem + Lds::IDS);
  {
    const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks;
    for (int i = tid; i < s1 - s0; i += kWave * NW) {
      const int32_t id = trow[s0 + i];
      ids[i] = id >= 0 && id < a.num_blocks ? id : 0;
    }
    __syncthreads();
  }
  // ---- chunk loads: piece p of thread tid is code bytes [d0, d0 + 16) of
  // token T of the chunk; threads tid and tid + 128 (tid < 128) also load
  // the key (tid % 128 < 64) or value scale of token tid % 64. Positions
  // past t1 read the codes of the split's last visible token (cached), a
  // finite copy, and are stored with scale 0: every column's mask excludes
  // them, so their weights are exactly 0. A wave's pieces p cover 8 (d 128)
  // or 16 (d 64) consecutive positions of one block -- also when clamped to
  // t1 - 1 -- so their block id and row base are wave-uniform. The store
  // has no branch, so it can share a basic block with MFMAs. -------------
  struct Regs {
    u32x4 k[PPT], v[PPT];
    float s;
  };
  auto load_chunk = [&](Regs& R, int c) {
    const int tc = t0 + c * CH;
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int q = tid + kWave * NW * p;
      const int T = q / (D / 16), d0 = (q % (D / 16)) * 16;
      const int tok = min(tc + T, t1 - 1);
      const int blk = __builtin_amdgcn_readfirstlane(tok >> bsl);
      const int id = __builtin_amdgcn_readfirstlane(ids[blk - s0]);
      const int64_t base = ((int64_t)id * a.H + g) << (bsl + DL);
      const uint32_t off = ((uint32_t)(tok & (BS - 1)) << DL) + d0;
      R.k[p] = *reinterpret_cast<const u32x4*>(a.k_codes + base + off);
      R.v[p] = load_codes<true>(reinterpret_cast<const u32x4*>(a.v_codes + base + off));
    }
    const int tok = min(tc + (tid & (CH - 1)), t1 - 1);
    const int64_t row = ((int64_t)ids[(tok >> bsl) - s0] * a.H + g) * BS + (tok & (BS - 1));
    R.s = ((tid & CH) ? a.v_scale : a.k_scale)[row];
  };
  auto store_chunk = [&](const Regs& R, int c, unsigned char* buf) {
    const int tc = t0 + c * CH;
    half_t* K = reinterpret_cast<half_t*>(buf);
    half_t* V = reinterpret_cast<half_t*>(buf + Lds::PLANE);
    float* SC = reinterpret_cast<float*>(buf + Lds::SCALES);   // [2][CH]
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int q = tid + kWave * NW * p;
      const int T = q / (D / 16), d0 = (q % (D / 16)) * 16;
      const half8v k0 = codes8_to_h8<CODE>(R.k[p].x, R.k[p].y);
      const half8v k1 = codes8_to_h8<CODE>(R.k[p].z, R.k[p].w);
      const half8v v0 = codes8_to_h8<CODE>(R.v[p].x, R.v[p].y);
      const half8v v1 = codes8_to_h8<CODE>(R.v[p].z, R.v[p].w);
      *reinterpret_cast<half8v*>(K + T * KSTR + d0) = k0;
      *reinterpret_cast<half8v*>(K + T * KSTR + d0 + 8) = k1;
      *reinterpret_cast<half8v*>(V + T * VSTR + d0) = v0;
      *reinterpret_cast<half8v*>(V + T * VSTR + d0 + 8) = v1;
    }
    // threads tid and tid + 128 write the same scale to the same place
    SC[tid & (2 * CH - 1)] = tc + (tid & (CH - 1)) < t1 ? R.s : 0.0f;
  };
  // a wave's TW tiles of chunk c, in groups of SG: qk_group computes the
  // group's raw scores, finish_group takes one softmax step per column tile
  // and then the PV MFMAs
  auto qk_group = [&](const unsigned char* buf, int k0, float4v (&S)[NCW][SG]) {
    const half_t* K = reinterpret_cast<const half_t*>(buf);
#pragma unroll
    for (int k = 0; k < SG; ++k) {
      const int nt = sh + (k0 + k) * NSH;
      half8v kop[NCH];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
        kop[ch] = *reinterpret_cast<const half8v*>(K + (nt * 16 + r) * KSTR + jj * (D / 4) + 8 * ch);
#pragma unroll
      for (int cc = 0; cc < NCW; ++cc) {
        float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[ch], qop[cc][ch], acc, 0, 0, 0);
        S[cc][k] = acc;
      }
    }
  };
  auto group_scales = [&](int c, const unsigned char* buf, int k0, int (&pos0)[SG],
                          float4v (&sk)[SG], float4v (&sv)[SG]) {
    const float* SK = reinterpret_cast<const float*>(buf + Lds::SCALES);
    const float* SV = SK + CH;
#pragma unroll
    for (int k = 0; k < SG; ++k) {
      const int nt = sh + (k0 + k) * NSH;
      pos0[k] = t0 + c * CH + nt * 16;
      sk[k] = *reinterpret_cast<const float4v*>(SK + nt * 16 + 4 * jj);
      sv[k] = *reinterpret_cast<const float4v*>(SV + nt * 16 + 4 * jj);
    }
  };
  // PV MFMA e: output elements 16 e + 4 jj + i of every column (row 4 jj
  // + i of the MFMA's output is element 16 e + 4 jj + i). Its value
  // operand, the values of elements 16 e .. 16 e + 15 over the group's
  // tokens, comes from one transposing LDS read per tile: in each 16-lane
  // group, lane i receives as its value k the (i % 4)-th of the 4 values
  // that lane 4 k + i / 4 points at. Lane (r, jj) points at elements 16 e
  // + 4 (r % 4) .. + 3 of token 4 jj + r / 4, and so receives element 16 e
  // + r of tokens 4 jj .. 4 jj + 3 -- the tokens whose weights it holds.
  // One tile: 16 tokens (16x16x16). Two tiles: 32 tokens (16x16x32),
  // contraction index 8 jj + i taking token 4 jj + i of the first tile for
  // i < 4 and token 4 jj + i - 4 of the second for i >= 4.
  auto pv_group = [&](const unsigned char* buf, int k0, const half4v (&pop)[NCW][SG]) {
    const half_t* V = reinterpret_cast<const half_t*>(buf + Lds::PLANE);
    const int vo = (4 * jj + (r >> 2)) * VSTR + 4 * (r & 3);
#pragma unroll
    for (int e = 0; e < NPV; ++e) {
      const half4v v0 = lds_read_tr16(V + (sh + k0 * NSH) * 16 * VSTR + vo + 16 * e);
      if constexpr (SG == 2) {
        const half4v v1 = lds_read_tr16(V + (sh + (k0 + 1) * NSH) * 16 * VSTR + vo + 16 * e);
        const half8v va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int cc = 0; cc < NCW; ++cc) {
          const half8v pb = __builtin_shufflevector(pop[cc][0], pop[cc][1], 0, 1, 2, 3, 4, 5, 6, 7);
          st[cc].acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, st[cc].acc[e], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < NCW; ++cc)
          st[cc].acc[e] =
              __builtin_amdgcn_mfma_f32_16x16x16f16(v0, pop[cc][0], st[cc].acc[e], 0, 0, 0);
      }
    }
  };
  // the rest of chunk c for a wave whose first group's scores are S0: per
  // group, the weights and PV MFMAs, then the next group's scores (between
  // one group's rescale branches and the next's, one basic block). MASKED:
  // the chunk holds a position at or past the wave's least column limit.
  auto compute_rest = [&](auto masked, int c, const unsigned char* buf,
                          const float4v (&S0)[NCW][SG]) {
    constexpr bool MASKED = decltype(masked)::value;
    int pos0[SG];
    float4v sk[SG], sv[SG];
    float u[NCW][SG][4], mt[NCW];
    group_scales(c, buf, 0, pos0, sk, sv);
    mq_scores<NCW, SG, MASKED>(S0, sk, lim, pos0, jj, u, mt);
#pragma unroll
    for (int k0 = 0; k0 < TW; k0 += SG) {
      half4v pop[NCW][SG];
      mq_weights<D, NCW, SG>(u, mt, sv, cscore, st, pop);
      pv_group(buf, k0, pop);
      if (k0 + SG < TW) {
        float4v S[NCW][SG];
        qk_group(buf, k0 + SG, S);
        group_scales(c, buf, k0 + SG, pos0, sk, sv);
        mq_scores<NCW, SG, MASKED>(S, sk, lim, pos0, jj, u, mt);
      }
    }
  };

  // ---- the chunk loop. Step c: one barrier (chunk c is in LDS, and every
  // wave has finished chunk c - 1, whose buffer chunk c + 1 takes next);
  // the scores of the wave's first tile group of chunk c; chunk c + 1
  // converted from registers into the other buffer; chunk c + 1 + NPF
  // loads started into the registers that freed; then the rest of chunk c.
  // The scores and the conversion sit in one basic block, so the
  // conversion's vector instructions issue while the score MFMAs run. The
  // score MFMAs run in every wave, also where none of its columns or tiles
  // counts (the results are then unused). Every step issues the same loads
  // (chunks past the last one read its rows again, clamped; stored past the
  // end they are zeros and never computed), so that the wait before a
  // conversion covers that chunk's loads only, not the ones behind it.
  const int nch = (t1 - t0 + CH - 1) / CH;
  if (nch > 0) {
    // register set (c + 1) % 2 holds chunk c + 1 at step c
    static_assert(NPF == 2, "two register sets alternate with the two buffers");
    Regs R[NPF];
    load_chunk(R[0], 0);
    load_chunk(R[1], 1);
    store_chunk(R[0], 0, smem);
    load_chunk(R[0], 2);
    auto step = [&](Regs& Rn, int c, const unsigned char* buf, unsigned char* nbuf) {
      __syncthreads();
      float4v S[NCW][SG];
      qk_group(buf, 0, S);
      store_chunk(Rn, c + 1, nbuf);
      load_chunk(Rn, c + 1 + NPF);
      const int tc = t0 + c * CH;
      if (active && tc + sh * 16 < t1) {   // some tile of the wave has a visible position
        if (tc + (sh + (TW - 1) * NSH) * 16 + 16 > lim_lo)
          compute_rest(std::true_type{}, c, buf, S);
        else
          compute_rest(std::false_type{}, c, buf, S);
      }
    };
    unsigned char* const b0 = smem;
    unsigned char* const b1 = smem + Lds::BUF;
    int c0 = 0;
    for (; c0 + 2 <= nch; c0 += 2) {
      step(R[1], c0, b0, b1);
      step(R[0], c0 + 1, b1, b0);
    }
    if (c0 < nch) step(R[1], c0, b0, b1);   // at most one chunk left
  }

  // ---- merge the waves' states, then write one partial per column ---------
  float (*red)[NV + 2][kWave] = reinterpret_cast<float (*)[NV + 2][kWave]>(smem);
#pragma unroll
  for (int cc = 0; cc < NCW; ++cc) {
    const float lsum = colsum4(st[cc].l);
    __syncthreads();   // every wave is done with the LDS area
#pragma unroll
    for (int k = 0; k < NPV; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][4 * k + e][lane] = st[cc].acc[k][e];
    red[wave][NV][lane] = st[cc].m == kMqNone ? -INFINITY : st[cc].m;   // no visible score
    red[wave][NV + 1][lane] = lsum;
    __syncthreads();
    // waves w < TW merge the shares of their columns: waves w, w + TW, ...
    if (wave < TW && valid[cc]) {
      float M = -INFINITY;
#pragma unroll
      for (int w = wave; w < NW; w += TW) M = fmaxf(M, red[w][NV][lane]);
      float acc[NV], l = 0.0f;
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] = 0.0f;
#pragma unroll
      for (int w = wave; w < NW; w += TW) {
        const float mw = red[w][NV][lane];
        const float sc = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        l += sc * red[w][NV + 1][lane];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] += sc * red[w][v][lane];
      }
      const int64_t pidx = (((int64_t)b * pa.J + j) * a.H + g) * (pa.CT * 16) + col[cc];
      if (jj == 0) *reinterpret_cast<float2*>(a.ws_ml + pidx * 2) = make_float2(M, l);
      // acc[4 k + e] holds output element 16 k + 4 jj + e of the column
      float* dst = a.ws_acc + pidx * D + 4 * jj;
#pragma unroll
      for (int k = 0; k < NPV; ++k)
        *reinterpret_cast<float4v*>(dst + 16 * k) =
            (float4v){acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]};
    }
  }
}

// Cross-split merge for multi-query attention, as decode_reduce: one wave
// per (query head, query i, sequence b), one or kReduceHeads heads per
// workgroup;
// split j's partial of column
// c = i G + h % G sits at ((b J + j) H + g) CT16 + c.
struct PrefillReduceArgs {
  const float* ws_acc;
  const float* ws_ml;
  const int32_t* context_lens;
  const int32_t* qstart;
  void* out;
  int32_t out_dtype;
  int32_t Hq, H, G, BS, max_len, J, S, CT;
  int32_t max_q;  // as in PrefillArgs
};

template <int D>
__global__ __launch_bounds__(64 * kReduceHeads) void prefill_reduce_kernel(PrefillReduceArgs a) {
  constexpr int EPL = D / 64;
  // splits per batch of loads: 16 holds the kernel at 80 VGPRs (six waves
  // per SIMD; with 32, each load's 64-bit address among them, 144 and three),
  // at one more round trip per 16 splits past the first 16
  constexpr int KB = 16;
  typedef float floatE __attribute__((ext_vector_type(EPL)));
  const int lane = threadIdx.x & (kWave - 1);
  const int h = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave, i = blockIdx.y,
            b = blockIdx.z;
  if (h >= a.Hq) return;
  const int L = min(a.context_lens[b], a.max_len);
  const int q0 = a.qstart[b];
  const int nq = min(min(a.qstart[b + 1] - q0, L), a.max_q);
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
    // a partial with m = -inf is empty (no position of the split seen): its
    // accumulator is not read
    const uint64_t full = __ballot(ml.x != -INFINITY);   // lanes past cnt hold -inf
    floatE v[KB];
#pragma unroll
    for (int uu = 0; uu < KB; ++uu)
      if ((full >> uu) & 1)
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
      if ((full >> uu) & 1) {
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

template <int CODE, int MODE, int NC>
hipError_t launch_prefill_nc(const PrefillArgs& pa, int d, int bs, int64_t units,
                             hipStream_t stream) {
  const dim3 grid((unsigned)units);   // one workgroup per unit
  if (d == 128) {
    if (bs == 16)
      prefill_split_kernel<CODE, MODE, 128, 16, NC><<<grid, 64 * kNW, 0, stream>>>(pa);
    else
      prefill_split_kernel<CODE, MODE, 128, 32, NC><<<grid, 64 * kNW, 0, stream>>>(pa);
  } else {
    if (bs == 16)
      prefill_split_kernel<CODE, MODE, 64, 16, NC><<<grid, 64 * kNW, 0, stream>>>(pa);
    else
      prefill_split_kernel<CODE, MODE, 64, 32, NC><<<grid, 64 * kNW, 0, stream>>>(pa);
  }
  return hipGetLastError();
}

// Two column tiles per wave whenever there are two and the second set of
// accumulators fits in registers next to the ring without spilling (d 64;
// d 128 with 16-token blocks of 8-bit codes; 4-bit codes, whose conversion
// the two tiles then share); per-channel keys: one.
template <int CODE, int MODE>
hipError_t launch_prefill_shape(PrefillArgs pa, int d, int bs, int64_t units_per_tg,
                                hipStream_t stream) {
  const bool fits = d == 64 || (bs == 16 && CODE != KVQ_CODE_NONE16) || CODE == KVQ_CODE_INT4;
  const int nc = (MODE != KVQ_SCALE_CHANNEL_BLOCK_SYM && pa.CT >= 2 && fits) ? 2 : 1;
  const int cts = (pa.CT + nc - 1) / nc;
  // the column tiles of a split share a workgroup (one wave or pair of waves
  // each), so that their reads of the same blocks meet in L1
  pa.TW = cts >= 4 ? 4 : (cts >= 2 ? 2 : 1);
  const int64_t units = units_per_tg * ((cts + pa.TW - 1) / pa.TW);
  if constexpr (MODE == KVQ_SCALE_CHANNEL_BLOCK_SYM) {
    return launch_prefill_nc<CODE, MODE, 1>(pa, d, bs, units, stream);
  } else {
    if (nc == 2) return launch_prefill_nc<CODE, MODE, 2>(pa, d, bs, units, stream);
    return launch_prefill_nc<CODE, MODE, 1>(pa, d, bs, units, stream);
  }
}

// The LDS-staged kernel: two column tiles per wave where there are two, and
// 1, 2 or 4 waves' column tiles per workgroup (the other waves of a column
// tile group share its token tiles). Grid: 8 x (column groups) x
// ceil(units / 8), so that the column groups of a unit meet on one XCD.
template <int CODE, int NCW, int TW, int NW>
hipError_t launch_mq_shape(const PrefillArgs& pa, int d, hipStream_t stream) {
  static_assert(TW <= NW, "a column-tile group has at least one wave");
  const int64_t cts = (pa.CT + NCW - 1) / NCW;
  const int64_t cgs = (cts + TW - 1) / TW;
  const int64_t items = (int64_t)pa.a.batch * pa.Jg * pa.a.H;
  const dim3 grid((unsigned)(8 * cgs * ((items + 7) / 8)));
  if (d == 128)
    mq_split_kernel<CODE, 128, NCW, TW, NW><<<grid, 64 * NW, 0, stream>>>(pa);
  else
    mq_split_kernel<CODE, 64, NCW, TW, NW><<<grid, 64 * NW, 0, stream>>>(pa);
  return hipGetLastError();
}

// Two column-tile groups per workgroup run as two waves over 32-token
// chunks (about 37 KB of LDS, so four workgroups share a CU and each
// barrier waits for two waves, not four): 70B shape, 8 queries per
// sequence, 16 layers at steady clocks, 265 -> 253 us. One group keeps four
// waves (8B layer: two waves 185 us against 182).

// Jg: the k-th workgroup of an XCD goes to its CUs in turn, so with the
// split index cycling through the item order and J dividing 32, each CU
// would keep one split index: with uneven lengths some CUs would take every
// full first split and others the mostly empty last ones (8B layer, 8
// queries: 4 splits 248 us, 5 splits 197 us). An odd split count in the
// enumeration cycles every CU through all of them.
template <int CODE>
hipError_t launch_mq(PrefillArgs pa, int d, int bs, hipStream_t stream) {
  pa.bs_log2 = bs == 32 ? 5 : 4;
  if (pa.CT < 2) return launch_mq_shape<CODE, 1, 1, 4>(pa, d, stream);
  const int cts = (pa.CT + 1) / 2;
  if (cts >= 4) return launch_mq_shape<CODE, 2, 4, 4>(pa, d, stream);
  if (cts >= 2) return launch_mq_shape<CODE, 2, 2, 2>(pa, d, stream);
  return launch_mq_shape<CODE, 2, 1, 4>(pa, d, stream);
}

}  // namespace

bool prefill_supported(int32_t k_code, int32_t v_code, int32_t k_mode, int32_t v_mode) {
  if (k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM)
    return k_code == KVQ_CODE_INT8 && v_code == KVQ_CODE_INT8 && v_mode == KVQ_SCALE_TOKEN_SYM;
  if (k_code != v_code || k_mode != v_mode) return false;
  if (k_code == KVQ_CODE_NONE16) return true;
  if (k_code == KVQ_CODE_INT4)
    return k_mode == KVQ_SCALE_TOKEN_SYM || k_mode == KVQ_SCALE_GROUP_ASYM;
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
  pa.max_q = pp.max_query_len;
  pa.window = pp.window;
  pa.sink = pp.sink;
  pa.TW = 1;   // set per launch shape
  pa.Jg = pp.splits | 1;   // odd, as for the LDS-staged kernel (see launch_mq)
  const int64_t units = (int64_t)p.batch * pa.Jg * p.num_kv_heads;
  const int d = p.head_dim, bs = p.block_size;
  hipError_t e;
  const bool tok8 = p.k_mode == KVQ_SCALE_TOKEN_SYM &&
                    (p.k_code == KVQ_CODE_INT8 || p.k_code == KVQ_CODE_FP8_E4M3);
  if (tok8 && pp.window == 0 && p.k_code == KVQ_CODE_FP8_E4M3)
    e = launch_mq<KVQ_CODE_FP8_E4M3>(pa, d, bs, stream);
  else if (tok8 && pp.window == 0)
    e = launch_mq<KVQ_CODE_INT8>(pa, d, bs, stream);
  else if (p.k_code == KVQ_CODE_NONE16)
    e = launch_prefill_shape<KVQ_CODE_NONE16, KVQ_SCALE_TOKEN_SYM>(pa, d, bs, units, stream);
  else if (p.k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM)
    e = launch_prefill_shape<KVQ_CODE_INT8, KVQ_SCALE_CHANNEL_BLOCK_SYM>(pa, d, bs, units, stream);
  else if (p.k_code == KVQ_CODE_FP8_E4M3)
    e = launch_prefill_shape<KVQ_CODE_FP8_E4M3, KVQ_SCALE_TOKEN_SYM>(pa, d, bs, units, stream);
  else if (p.k_code == KVQ_CODE_INT4 && p.k_mode == KVQ_SCALE_GROUP_ASYM)
    e = launch_prefill_shape<KVQ_CODE_INT4, KVQ_SCALE_GROUP_ASYM>(pa, d, bs, units, stream);
  else if (p.k_code == KVQ_CODE_INT4)
    e = launch_prefill_shape<KVQ_CODE_INT4, KVQ_SCALE_TOKEN_SYM>(pa, d, bs, units, stream);
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
  ra.max_q = pp.max_query_len;
  const int hpg =
      reduce_heads_per_group((int64_t)p.num_q_heads * pp.max_query_len * p.batch);
  const dim3 grid((p.num_q_heads + hpg - 1) / hpg, pp.max_query_len, p.batch);
  if (d == 128)
    prefill_reduce_kernel<128><<<grid, kWave * hpg, 0, stream>>>(ra);
  else
    prefill_reduce_kernel<64><<<grid, kWave * hpg, 0, stream>>>(ra);
  return hipGetLastError();
}

}  // namespace kvq
