// kvq_prefill.hip -- multi-query (prefill) attention over the quantized
// paged cache (gfx950): several causal queries per sequence at once.
#include "kvq_attn_tiles.h"

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
// The 16 MFMA columns of a wave are 16 consecutive (query, head) pairs
// c = i G + r of one KV head g, a column tile: the G heads of a query are
// adjacent, a tile spans 16 / G queries (or a query G / 16 tiles). A
// workgroup takes one unit (sequence b, split j of S blocks, KV head g,
// column tile ct); its four waves stream consecutive quarters of the split
// through the decode's register ring and tile steps, with a causal limit
// per lane (column), and merge their softmax states through LDS. Every block
// a wave loads serves 16 columns; the units of one (b, j, g) are adjacent in
// the grid, so their repeated block reads meet in L2. Each unit writes a
// partial (m, l, acc) per column; prefill_reduce merges the splits.
// ---------------------------------------------------------------------------
struct PrefillArgs {
  DecodeArgs a;
  const int32_t* qstart;
  int32_t J;    // splits per sequence in the grid
  int32_t S;    // blocks per split
  int32_t CT;   // column tiles per (sequence, KV head)
  int32_t TW;   // column tiles per workgroup: 1, 2 or 4 (4 / TW waves per tile)
  int32_t window;   // > 0: each query sees its last `window` positions ...
  int32_t sink;     // ... and the first `sink` positions
};

template <int CODE, int MODE, int D, int BS>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_split_kernel(PrefillArgs pa) {
  constexpr int NCH = D / 32;
  constexpr int NPV = D / 16;
  constexpr int NV = D / 4;
  constexpr int NBUF = BS == 16 ? 3 : 2;  // blocks in the register ring
  constexpr bool KCH = MODE == KVQ_SCALE_CHANNEL_BLOCK_SYM;
  constexpr bool RAW = CODE == KVQ_CODE_NONE16;
  using TileT = typename std::conditional<RAW, TileRaw<D, BS>, Tile8<D, BS>>::type;
  __shared__ float red[kNW][NV + 2][kWave];
  const DecodeArgs& a = pa.a;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, jj = lane >> 4;
  // unit (b, j, g, tile group); wave w serves column tile tg TW + w % TW and
  // the (w / TW)-th of the 4 / TW shares of the split's blocks
  const int ctg = (pa.CT + pa.TW - 1) / pa.TW;
  int64_t u = blockIdx.x;
  const int tg = (int)(u % ctg);
  u /= ctg;
  const int g = (int)(u % a.H);
  u /= a.H;
  const int j = (int)(u % pa.J);
  const int b = (int)(u / pa.J);
  if (b >= a.batch) return;
  const int L = min(a.context_lens[b], a.max_len);
  const int q0 = pa.qstart[b];
  const int nq = min(pa.qstart[b + 1] - q0, L);
  const int ncol = nq * a.G;
  const int nblk = (L + BS - 1) / BS;
  const int s0 = j * pa.S;
  // workgroup-uniform exits: no split here, or no column in the tile group
  if (s0 >= nblk || tg * pa.TW * 16 >= ncol) return;
  const int nshare = kNW / pa.TW;
  const int ct = tg * pa.TW + wave % pa.TW;
  const int cbase = ct * 16;
  const bool active = cbase < ncol;   // a tile past the columns only joins the merge

  // ---- columns: lane (r, jj) serves column c = cbase + r -------------------
  const int c = cbase + r;
  const bool valid = c < ncol;
  const int qi = valid ? c / a.G : 0;
  const int hq = g * a.G + (valid ? c % a.G : 0);
  const int Lr = valid ? L - nq + qi + 1 : 0;                 // this column's limit
  const int Lmin = L - nq + cbase / a.G + 1;                  // over the tile's columns
  const int Lmax = active ? L - nq + (min(ncol, cbase + 16) - 1) / a.G + 1 : 0;
  // sliding window with sinks: the lane's column sees t >= lo_r (and t < SK);
  // lo_min / lo_max bound the window starts over the tile's columns
  const int W = pa.window, SK = pa.window > 0 ? pa.sink : 0;
  const int lo_r = W > 0 ? Lr - W : 0;
  const int lo_min = W > 0 ? Lmin - W : 0;
  const int lo_max = W > 0 ? Lmax - W : 0;
  // the tile's visible blocks of the split (none past what any of its columns
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
  // fp16 query operand; with per-channel keys it is made where it is needed
  // (the staged block), to keep registers for the ring
  half8v qop[NCH];
  if constexpr (!KCH) {
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[cc][e] = (half_t)qf[8 * cc + e];
  }
  const float cscore = valid ? qup * a.sm_log2 : 0.0f;
  const bool raw_bf16 = a.stage_bf16 != 0;

  SoftmaxState<D> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int cc = 0; cc < NPV; ++cc) st.acc[cc] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  if (x0 < x1) {
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
      if constexpr (RAW) {
#pragma unroll
        for (int nt = 0; nt < BS / 16; ++nt)
          tile_step_raw<D, BS, false>(t, nt, i * BS + nt * 16, L, qop, cscore, jj, st, raw_bf16);
      } else if constexpr (KCH) {
        half8v qb[NCH], ql[NCH];
        channel_query<D, BS>(t, xs, qf, lane, qb, ql);
        full_block_step<CODE, D, BS, kKeyChannel>(t, i, L, qb, cscore, jj, st, ql);
      } else {
        full_block_step<CODE, D, BS>(t, i, L, qop, cscore, jj, st);
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
            for (int cc = 0; cc < NCH; ++cc)
              kraw[nt][cc] = *reinterpret_cast<const u32x4*>(sp + 8 * cc);
          }
#pragma unroll
          for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
            for (int e = 0; e < 8; ++e) qb[cc][e] = (half_t)qf[8 * cc + e];
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
        if constexpr (RAW) {
          if (masked)
            tile_step_raw<D, BS, true>(t, nt, pos0, Lr, qop, cscore, jj, st, raw_bf16, L,
                                       lo_r, SK);
          else
            tile_step_raw<D, BS, false>(t, nt, pos0, Lr, qop, cscore, jj, st, raw_bf16, L);
        } else if constexpr (KCH) {
          if (rawk) {   // qb holds the plain fp16 query here
            if (masked)
              tile_step<CODE, D, BS, true, kKeyRaw>(t, nt, pos0, Lr, qb, cscore, jj, st,
                                                    kraw[nt], raw_bf16, nullptr, L, lo_r, SK);
            else
              tile_step<CODE, D, BS, false, kKeyRaw>(t, nt, pos0, Lr, qb, cscore, jj, st,
                                                     kraw[nt], raw_bf16, nullptr, L);
          } else if (masked) {
            tile_step<CODE, D, BS, true, kKeyChannel>(t, nt, pos0, Lr, qb, cscore, jj, st,
                                                      nullptr, false, ql, L, lo_r, SK);
          } else {
            tile_step<CODE, D, BS, false, kKeyChannel>(t, nt, pos0, Lr, qb, cscore, jj, st,
                                                       nullptr, false, ql, L);
          }
        } else {
          if (masked)
            tile_step<CODE, D, BS, true>(t, nt, pos0, Lr, qop, cscore, jj, st, nullptr, false,
                                         nullptr, L, lo_r, SK);
          else
            tile_step<CODE, D, BS, false>(t, nt, pos0, Lr, qop, cscore, jj, st, nullptr, false,
                                          nullptr, L);
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
  const float lsum = colsum4(st.l);
  __syncthreads();   // every wave is done with its LDS slice
#pragma unroll
  for (int cc = 0; cc < NPV; ++cc)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][4 * cc + e][lane] = st.acc[cc][e];
  red[wave][NV][lane] = st.m;
  red[wave][NV + 1][lane] = lsum;
  __syncthreads();
  // waves w < TW merge the shares of their tile: waves w, w + TW, ...
  if (wave >= pa.TW || !valid) return;
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
  const int64_t pidx = (((int64_t)b * pa.J + j) * a.H + g) * (pa.CT * 16) + c;
  if (jj == 0) *reinterpret_cast<float2*>(a.ws_ml + pidx * 2) = make_float2(M, l);
  // acc[4 cc + e] holds output element (d/16) (4 jj + e) + cc of column c
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
  const dim3 grid((unsigned)units);   // one workgroup per unit
  if (d == 128) {
    if (bs == 16)
      prefill_split_kernel<CODE, MODE, 128, 16><<<grid, 64 * kNW, 0, stream>>>(pa);
    else
      prefill_split_kernel<CODE, MODE, 128, 32><<<grid, 64 * kNW, 0, stream>>>(pa);
  } else {
    if (bs == 16)
      prefill_split_kernel<CODE, MODE, 64, 16><<<grid, 64 * kNW, 0, stream>>>(pa);
    else
      prefill_split_kernel<CODE, MODE, 64, 32><<<grid, 64 * kNW, 0, stream>>>(pa);
  }
  return hipGetLastError();
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
  pa.window = pp.window;
  pa.sink = pp.sink;
  // the column tiles of a split share a workgroup (one tile per wave or
  // pair of waves), so that their reads of the same blocks meet in L1
  pa.TW = pp.col_tiles >= 4 ? 4 : (pp.col_tiles >= 2 ? 2 : 1);
  const int64_t units = (int64_t)p.batch * pp.splits * p.num_kv_heads *
                        ((pp.col_tiles + pa.TW - 1) / pa.TW);
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

}  // namespace kvq
