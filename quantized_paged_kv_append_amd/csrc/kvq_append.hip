// kvq_append.hip -- quantize-on-append into paged blocks (gfx950).
//
// What is computed ("Dynamic KV Cache Quantization for Fast LLM Inference",
// section "Understanding Dynamic Quantization Techniques for KV Caches"): for
// every new (token, head) vector a scale from its own range, computed when it
// enters the cache, then codes round(x / scale); section "Integrating Dynamic
// Quantization with PagedAttention": each physical block stores the quantized
// keys and values, placed through the sequence's block map (here the slot
// mapping). The per-channel key mode follows "KV Cache Optimization:
// Strategies for Faster LLM Inference", section "KV Cache Quantization: When
// and How to Compress".
//
// Design (HBM-bound single streaming pass): a row of d 16-bit elements is
// handled by d/8 lanes, each with one 16-byte load (or, for 4-bit codes, the
// loads that feed whole output bytes of the slice-interleaved nibble layout);
// the row's absmax (or per-group min/max) is a lane-group shuffle reduction;
// the scale is one correctly rounded fp32 division per row; codes use the
// reciprocal with a near-tie check that falls back to the exact quotient, so
// stored bytes equal rne(x / s) exactly. Codes leave as one 8-byte (INT8/FP8)
// or 4-byte (INT4) store per lane.
//
// Static scales (same pages, "Understanding Dynamic Quantization Techniques
// for KV Caches", the static alternative): the STATIC kernels take the scale
// (and zero point) of each head, or head and group, from the caller instead
// of the row's range, skip the range reduction, and saturate the codes at the
// code range, since the range no longer bounds x / s; the metadata planes
// receive the given values.
#include "kvq_device.h"
#include "kvq_encode.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

struct SideArgs {
  const uint16_t* src;
  int64_t row_stride;
  uint8_t* codes;
  float* scale;
  uint8_t* zero;
  const float* st_scale;   // static parameters (STATIC kernels only)
  const uint8_t* st_zero;
};

struct RowArgs {
  SideArgs side[2];
  const int64_t* slots;
  const int32_t* stage_rows;  // static per-channel keys only
  uint16_t* stage;
  int64_t num_tokens;
  int64_t num_blocks;
  int32_t H;
  int32_t bs;
  int32_t max_seqs;
  int32_t side0;     // first side handled; blockIdx.y adds to it
  uint32_t h_mul;    // t = r / H as ((mulhi(r, h_mul) + r) >> h_shift), r < 2^31
  uint32_t h_shift;
  uint32_t bs_shift; // log2(bs)
};

__device__ __forceinline__ uint32_t div_h(uint32_t r, const RowArgs& a) {
  return (__umulhi(r, a.h_mul) + r) >> a.h_shift;
}

// Byte codes (INT8 / FP8 / 16-bit passthrough). A wave covers 16 consecutive
// tokens of one KV head (rows r = ((tg H + h) 16 + i), token 16 tg + i), so a
// block's scales leave as one contiguous store when its slots are
// consecutive. Four lanes share a row of d elements: lane k holds elements
// 32 u + 8 k + e (u < d/32, e < 8); each 16-byte load instruction reads a
// contiguous 64-byte piece of every row.
template <int CODE, int D, bool BF16, bool STATIC>
__global__ __launch_bounds__(256) void append_bytes_kernel(RowArgs a) {
  constexpr int NV = D / 32;        // 16-byte vectors per lane
  constexpr int RPW = kWave / 4;    // rows per wave (= tokens of one group)
  const SideArgs S = a.side[a.side0 + blockIdx.y];
  const int lane = threadIdx.x & (kWave - 1);
  const int k = lane & 3;
  const uint32_t groups = ((uint32_t)a.num_tokens + 15u) / 16u;
  const uint32_t items = groups * (uint32_t)a.H;   // (token group, head) pairs
  const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const uint32_t nwaves = gridDim.x * blockDim.x / kWave;
  // The inputs of one (token group, head) item: the lane row's slot and its
  // 16-byte pieces. For E4M3 and 16-bit codes each wave loads its next item
  // before it codes the current one, so two items' loads are in flight while
  // it computes (measured: +9% on E4M3); INT8 keeps one item at a time, whose
  // lower register use holds eight waves per SIMD instead of six (the
  // prefetch cost it 4%).
  struct Rows {
    int64_t slot;
    u32x4 w[NV];
  };
  auto fetch = [&](uint32_t it, Rows& R) {
    const uint32_t tg = div_h(it, a);
    const uint32_t h = it - tg * (uint32_t)a.H;
    const uint32_t t = tg * RPW + (uint32_t)(lane >> 2);
    const bool in = it < items && t < (uint32_t)a.num_tokens;
    R.slot = in ? a.slots[t] : -1;
    const uint16_t* src = S.src + (int64_t)(in ? t : 0) * S.row_stride + h * D + 8 * k;
#pragma unroll
    for (int u = 0; u < NV; ++u)
      R.w[u] = in ? *reinterpret_cast<const u32x4*>(src + 32 * u) : (u32x4){0u, 0u, 0u, 0u};
  };
  auto code = [&](uint32_t it, const Rows& R) {
    const uint32_t tg = div_h(it, a);
    const uint32_t h = it - tg * (uint32_t)a.H;
    const int64_t slot = R.slot;
    const int64_t blk = slot >> a.bs_shift;
    const bool live = slot >= 0 && blk < a.num_blocks;
    const int64_t rowi = (blk * a.H + h) * a.bs + (slot & (a.bs - 1));
    const u32x4* w = R.w;
    if constexpr (CODE == KVQ_CODE_NONE16) {
      if (live) {
#pragma unroll
        for (int u = 0; u < NV; ++u)
          *reinterpret_cast<u32x4*>(S.codes + rowi * (2 * D) + 2 * (32 * u + 8 * k)) = w[u];
      }
      return;
    }
    code_row8<CODE, D, BF16, STATIC>(w, k, STATIC ? S.st_scale[h] : 0.0f, S.codes + rowi * D,
                                     S.scale + rowi, live);
  };
  if constexpr (CODE == KVQ_CODE_INT8) {
    for (uint32_t it = wave; it < items; it += nwaves) {
      Rows cur;
      fetch(it, cur);
      code(it, cur);
    }
  } else {
    if (wave >= items) return;
    Rows cur, nxt;
    fetch(wave, cur);
    for (uint32_t it = wave; it < items; it += nwaves) {
      fetch(it + nwaves, nxt);
      code(it, cur);
      cur = nxt;
    }
  }
}

// min over the four lanes of a quad (DPP quad permutations, no LDS)
__device__ __forceinline__ float quad_min(float v) {
  v = fminf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true)));
  v = fminf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true)));
  return v;
}

// the value of lane `src` of each quad, in every lane of that quad
template <int SRC>
__device__ __forceinline__ float quad_bcast(float v) {
  constexpr int ctrl = SRC | (SRC << 2) | (SRC << 4) | (SRC << 6);
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, true));
}

// 4-bit codes. Nibble layout: with n = D/32 slices (= 32-element groups),
// element 32 i + 2 r + t sits in byte n r + i (nibble t). A wave covers 16
// consecutive tokens of one head, four lanes per row; lane k of a row loads
// elements [32 i + 8 k, 32 i + 8 k + 8) of every slice i (16-byte loads) and
// so owns pairs r in [4 k, 4 k + 4), i.e. the n * 4 contiguous output bytes
// starting at byte 4 n k.
// MODE TOKEN_SYM: symmetric codes in [-7, 7] stored as q & 0xF.
// MODE GROUP_ASYM: unsigned codes with a zero point per slice; lane k of a
// quad computes slice k's scale and zero point (k < n) and the quad shares
// them by DPP broadcasts.
template <int MODE, int D, bool BF16, bool STATIC>
__global__ __launch_bounds__(256) void append_int4_kernel(RowArgs a) {
  constexpr int NS = D / 32;       // slices per row, one 16-byte load each
  constexpr int RPW = kWave / 4;   // rows per wave (tokens of one group)
  const SideArgs S = a.side[a.side0 + blockIdx.y];
  const int lane = threadIdx.x & (kWave - 1);
  const int k = lane & 3;
  const uint32_t groups = ((uint32_t)a.num_tokens + 15u) / 16u;
  const uint32_t items = groups * (uint32_t)a.H;   // (token group, head) pairs
  const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const uint32_t nwaves = gridDim.x * blockDim.x / kWave;
  for (uint32_t it = wave; it < items; it += nwaves) {
    const uint32_t tg = div_h(it, a);
    const uint32_t h = it - tg * (uint32_t)a.H;
    const uint32_t t = tg * RPW + (uint32_t)(lane >> 2);
    const bool in = t < (uint32_t)a.num_tokens;
    const int64_t slot = in ? a.slots[t] : -1;
    const int64_t blk = slot >> a.bs_shift;
    const bool live = slot >= 0 && blk < a.num_blocks;
    const int64_t rowi = (blk * a.H + h) * a.bs + (slot & (a.bs - 1));
    const uint16_t* src = S.src + (int64_t)(in ? t : 0) * S.row_stride + h * D + 8 * k;
    float x[NS][8];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const u32x4 w = in ? *reinterpret_cast<const u32x4*>(src + 32 * i) : (u32x4){0u, 0u, 0u, 0u};
      unpack2<BF16>(w.x, x[i][0], x[i][1]);
      unpack2<BF16>(w.y, x[i][2], x[i][3]);
      unpack2<BF16>(w.z, x[i][4], x[i][5]);
      unpack2<BF16>(w.w, x[i][6], x[i][7]);
    }
    int q[NS][8];
    if constexpr (MODE == KVQ_SCALE_TOKEN_SYM) {
      float s;
      if constexpr (STATIC) {
        s = S.st_scale[h];
      } else {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < NS; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
        amax = quad_max(amax);
        s = amax == 0.0f ? 1.0f : div_rn(amax, 7.0f);
      }
      const float inv = __builtin_amdgcn_rcpf(s);   // within 1 ulp of 1/s
      const bool unsafe = recip_unsafe(s);
      // an element near a rounding boundary (rare) takes the exact quotient
      // on its own, so a wave redoes only the elements some lane needs
#pragma unroll
      for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = x[i][e] * inv;
          float qq = rne(y);
          if (unsafe || near_half(y, qq)) qq = rne(div_rn(x[i][e], s));
          q[i][e] = (int)fminf(fmaxf(qq, -7.0f), 7.0f);
        }
      if (live && k == 0) S.scale[rowi] = s;
    } else {
      float sg[NS];
      int zg[NS];
      if constexpr (STATIC) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          sg[i] = S.st_scale[h * NS + i];
          zg[i] = S.st_zero[h * NS + i];
        }
      } else {
      // per-slice range, widened to contain 0
      float mn[NS], mx[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        mn[i] = 0.0f;
        mx[i] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          mn[i] = fminf(mn[i], x[i][e]);
          mx[i] = fmaxf(mx[i], x[i][e]);
        }
        mn[i] = quad_min(mn[i]);
        mx[i] = quad_max(mx[i]);
      }
      // lane k computes slice k's scalars (k < NS), the quad shares them
      float mno = mn[0], mxo = mx[0];
#pragma unroll
      for (int i = 1; i < NS; ++i)
        if (k == i) {
          mno = mn[i];
          mxo = mx[i];
        }
      float so = 1.0f, zf = 0.0f;
      if (mxo != mno) {
        so = div_rn(mxo - mno, 15.0f);
        zf = fminf(fmaxf(rne(div_rn(-mno, so)), 0.0f), 15.0f);
      }
      sg[0] = quad_bcast<0>(so);
      zg[0] = (int)quad_bcast<0>(zf);
      sg[1] = quad_bcast<1>(so);
      zg[1] = (int)quad_bcast<1>(zf);
      if constexpr (NS == 4) {
        sg[2] = quad_bcast<2>(so);
        zg[2] = (int)quad_bcast<2>(zf);
        sg[3] = quad_bcast<3>(so);
        zg[3] = (int)quad_bcast<3>(zf);
      }
      }
      // A dynamic range bounds |x / s| by 15; static scales do not, so the
      // rounded quotient is clipped to +-15 before the integer conversion.
      // an element near a rounding boundary (rare) takes the exact quotient
      // on its own, so a wave redoes only the elements some lane needs
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const bool unsafe = recip_unsafe(sg[i]);
        const float inv = __builtin_amdgcn_rcpf(sg[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = x[i][e] * inv;
          float qq = rne(y);
          if (unsafe || near_half(y, qq)) qq = rne(div_rn(x[i][e], sg[i]));
          if constexpr (STATIC) qq = fminf(fmaxf(qq, -15.0f), 15.0f);
          q[i][e] = min(max((int)qq + zg[i], 0), 15);
        }
      }
      if (live && k == 0) {
        float* sp = S.scale + rowi * NS;
        uint8_t* zp = S.zero + rowi * NS;
        if constexpr (NS == 4) {
          *reinterpret_cast<float4v*>(sp) = (float4v){sg[0], sg[1], sg[2], sg[3]};
          *reinterpret_cast<uint32_t*>(zp) = (uint32_t)zg[0] | ((uint32_t)zg[1] << 8) |
                                             ((uint32_t)zg[2] << 16) | ((uint32_t)zg[3] << 24);
        } else {
          *reinterpret_cast<float2*>(sp) = make_float2(sg[0], sg[1]);
          *reinterpret_cast<uint16_t*>(zp) = (uint16_t)(zg[0] | (zg[1] << 8));
        }
      }
    }
    // output byte NS r' + i (r' = r - 4 k) holds elements 2 r', 2 r' + 1 of
    // this lane's run of slice i
    uint32_t out[NS];
#pragma unroll
    for (int wd = 0; wd < NS; ++wd) {
      uint32_t v = 0;
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const int byte = 4 * wd + b4, rr = byte / NS, i = byte % NS;
        v |= ((uint32_t)(q[i][2 * rr] & 0xF) | ((uint32_t)(q[i][2 * rr + 1] & 0xF) << 4)) << (8 * b4);
      }
      out[wd] = v;
    }
    if (live) {
      uint8_t* dst = S.codes + rowi * (D / 2) + 4 * NS * k;
      if constexpr (NS == 4)
        *reinterpret_cast<u32x4*>(dst) = (u32x4){out[0], out[1], out[2], out[3]};
      else
        *reinterpret_cast<u32x2*>(dst) = (u32x2){out[0], out[1]};
    }
  }
}

// ---- per-channel-per-block keys -----------------------------------------
// Phase 1: every token whose slot is the last of its block completes that
// block: the block's rows come from this call (the run of preceding tokens
// with consecutive slots and the same stage row) and, for earlier offsets,
// from the stage row. One wave per (token, head) item (items whose token
// completes no block end after reading its slot); lane l owns channels
// 2l, 2l+1 (D = 128) or channel l (D = 64) over all bs rows.
struct ChanArgs {
  const uint16_t* src;
  int64_t row_stride;
  const int64_t* slots;
  const int32_t* stage_rows;
  uint16_t* stage;  // [max_seqs][H][bs][D]
  int8_t* codes;
  float* scale;
  int64_t num_tokens;
  int64_t num_blocks;
  int32_t H;
  int32_t max_seqs;
};

// Quantize the block completed by token t (its slot, the block's last, is
// `slot`; its stage row `srow`) for head h: the whole wave, lane l owning
// channels CPL l .. CPL l + CPL - 1 over all BS rows.
template <int D, int BS, bool BF16>
__device__ __forceinline__ void chan_block(const ChanArgs& a, int64_t t, int h, int64_t slot,
                                           int32_t srow, int lane) {
  constexpr int CPL = D / kWave;  // channels per lane (1 or 2)
  const int64_t blk = slot / BS;
  // rows of this block provided by this call: t - k for k < n_new, the
  // run of preceding tokens with consecutive slots and the same stage row;
  // lane l checks token t - 1 - l, all lanes at once
  bool match = false;
  if (lane < BS - 1 && t - 1 - lane >= 0) {
    const int64_t tp = t - 1 - lane;
    match = a.slots[tp] == slot - 1 - lane && a.stage_rows[tp] == srow;
  }
  // at most BS - 1 < 64 bits are set, so the complement is never 0
  const int n_new = 1 + __builtin_ctzll(~(uint64_t)__ballot(match));
  float x[BS][CPL];
  float amax[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) amax[c] = 0.0f;
#pragma unroll
  for (int o = 0; o < BS; ++o) {
    const int k = BS - 1 - o;  // token t - k holds offset o when k < n_new
    const uint16_t* p;
    if (k < n_new)
      p = a.src + (t - k) * a.row_stride + (int64_t)h * D;
    else
      p = a.stage + (((int64_t)srow * a.H + h) * BS + o) * D;
    if constexpr (CPL == 2) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(p + 2 * lane);
      unpack2<BF16>(w, x[o][0], x[o][1]);
    } else {
      uint16_t w = p[lane];
      x[o][0] = BF16 ? bf16_lo(w) : f16_lo(w);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) amax[c] = fmaxf(amax[c], fabsf(x[o][c]));
  }
  float s[CPL], inv[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    s[c] = amax[c] == 0.0f ? 1.0f : div_rn(amax[c], 127.0f);
    inv[c] = div_rn(1.0f, s[c]);
  }
  int8_t* cb = a.codes + ((blk * a.H + h) * BS) * D;
#pragma unroll
  for (int o = 0; o < BS; ++o) {
    int q[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float y = x[o][c] * inv[c];
      float r = rne(y);
      if (near_half(y, r) || recip_unsafe(s[c])) r = rne(div_rn(x[o][c], s[c]));
      q[c] = (int)fminf(fmaxf(r, -127.0f), 127.0f);
    }
    if constexpr (CPL == 2) {
      *reinterpret_cast<uint16_t*>(cb + o * D + 2 * lane) =
          (uint16_t)((q[0] & 0xFF) | ((q[1] & 0xFF) << 8));
    } else {
      cb[o * D + lane] = (int8_t)q[0];
    }
  }
  float* sp = a.scale + (blk * a.H + h) * D;
  if constexpr (CPL == 2) {
    float2 sv = {s[0], s[1]};
    *reinterpret_cast<float2*>(sp + 2 * lane) = sv;
  } else {
    sp[lane] = s[0];
  }
}

// The slot and stage row of token t, when they complete a block (else
// slot = -1).
template <int BS>
__device__ __forceinline__ void chan_completing(const ChanArgs& a, int64_t t, int64_t& slot,
                                                int32_t& srow) {
  slot = a.slots[t];
  srow = a.stage_rows[t];
  if (slot < 0 || slot % BS != BS - 1 || slot / BS >= a.num_blocks || srow < 0 ||
      srow >= a.max_seqs)
    slot = -1;
}

// Small appends (a decode step's few tokens per sequence): one wave per
// (token, head) item, so that the items that complete no block (all but about
// one in BS) cost a single slot load each, side by side.
template <int D, int BS, bool BF16>
__global__ __launch_bounds__(256) void chan_complete_kernel(ChanArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  const int64_t items = a.num_tokens * a.H;
  for (int64_t it = wave; it < items; it += nwaves) {
    const int64_t t = it / a.H;
    const int h = (int)(it % a.H);
    int64_t slot;
    int32_t srow;
    chan_completing<BS>(a, t, slot, srow);
    if (slot >= 0) chan_block<D, BS, BF16>(a, t, h, slot, srow, lane);
  }
}

// Bulk appends (prompts): one wave per (64-token chunk, head): lane l reads
// token 64 c + l's slot and stage row, and the wave quantizes the blocks the
// chunk's tokens complete, one after another, instead of paying a dependent
// slot load per (token, head).
template <int D, int BS, bool BF16>
__global__ __launch_bounds__(256) void chan_complete_chunked_kernel(ChanArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  const int64_t items = (a.num_tokens + kWave - 1) / kWave * a.H;
  for (int64_t it = wave; it < items; it += nwaves) {
    const int64_t t0 = it / a.H * kWave;
    const int h = (int)(it % a.H);
    int64_t slot = -1;
    int32_t srow = -1;
    if (t0 + lane < a.num_tokens) chan_completing<BS>(a, t0 + lane, slot, srow);
    for (uint64_t m = __ballot(slot >= 0); m; m &= m - 1) {
      const int i = __builtin_ctzll(m);
      const int64_t st = ((int64_t)__builtin_amdgcn_readlane((int)(slot >> 32), i) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((int)slot, i);
      chan_block<D, BS, BF16>(a, t0 + i, h, st, __builtin_amdgcn_readlane(srow, i), lane);
    }
  }
}

// Static per-channel keys: channel c of head h has the caller's scale
// s[h d + c], so a row is coded as soon as it arrives (no wait for its block).
// Lane layout as in append_bytes_kernel (16 tokens of one head per wave, four
// lanes per row); each lane also reads the scales of its 8 D/32 channels, and
// writes them as the block's scale row when its token holds offset 0. Rows of
// a block that this call does not complete still go, raw, to the stage row,
// where decode reads a partial last block (at most one such row per stage
// position per call, so no two writes race).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void append_chan_static_kernel(RowArgs a) {
  constexpr int NV = D / 32;
  constexpr int RPW = kWave / 4;
  const SideArgs S = a.side[0];
  const int lane = threadIdx.x & (kWave - 1);
  const int k = lane & 3;
  const uint32_t groups = ((uint32_t)a.num_tokens + 15u) / 16u;
  const uint32_t items = groups * (uint32_t)a.H;
  const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const uint32_t nwaves = gridDim.x * blockDim.x / kWave;
  for (uint32_t it = wave; it < items; it += nwaves) {
    const uint32_t tg = div_h(it, a);
    const uint32_t h = it - tg * (uint32_t)a.H;
    const uint32_t t = tg * RPW + (uint32_t)(lane >> 2);
    const bool in = t < (uint32_t)a.num_tokens;
    const int64_t slot = in ? a.slots[t] : -1;
    const int32_t srow = in ? a.stage_rows[t] : -1;
    const int64_t blk = slot >> a.bs_shift;
    const int off = (int)(slot & (a.bs - 1));
    const bool live = slot >= 0 && blk < a.num_blocks && srow >= 0 && srow < a.max_seqs;
    const int64_t rowi = (blk * a.H + h) * a.bs + off;
    const uint16_t* src = S.src + (int64_t)(in ? t : 0) * S.row_stride + h * D + 8 * k;
    const float* sp = S.st_scale + h * D + 8 * k;
    u32x4 w[NV];
    float4v sv[NV][2];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      w[u] = in ? *reinterpret_cast<const u32x4*>(src + 32 * u) : (u32x4){0u, 0u, 0u, 0u};
      sv[u][0] = *reinterpret_cast<const float4v*>(sp + 32 * u);
      sv[u][1] = *reinterpret_cast<const float4v*>(sp + 32 * u + 4);
    }
    uint32_t o[NV][2];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      float x[8];
      unpack2<BF16>(w[u].x, x[0], x[1]);
      unpack2<BF16>(w[u].y, x[2], x[3]);
      unpack2<BF16>(w[u].z, x[4], x[5]);
      unpack2<BF16>(w[u].w, x[6], x[7]);
      int c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float sc = sv[u][e >> 2][e & 3];
        const float y = x[e] * __builtin_amdgcn_rcpf(sc);
        float q = rne(y);
        if (near_half(y, q) || recip_unsafe(sc)) q = rne(div_rn(x[e], sc));  // rare
        c[e] = (int)fminf(fmaxf(q, -127.0f), 127.0f);
      }
      o[u][0] = pack_bytes(c[0], c[1], c[2], c[3]);
      o[u][1] = pack_bytes(c[4], c[5], c[6], c[7]);
    }
    if (live) {
      // completed in this call iff the token holding the block's last offset
      // follows in the same run
      const int64_t tl = (int64_t)t + (a.bs - 1 - off);
      const bool completes = tl < a.num_tokens && a.slots[tl] == slot + (a.bs - 1 - off) &&
                             a.stage_rows[tl] == srow;
      uint16_t* st = a.stage + (((int64_t)srow * a.H + h) * a.bs + off) * D + 8 * k;
      int8_t* cd = reinterpret_cast<int8_t*>(S.codes) + rowi * D + 8 * k;
      float* sd = S.scale + (blk * a.H + h) * D + 8 * k;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        *reinterpret_cast<u32x2*>(cd + 32 * u) = (u32x2){o[u][0], o[u][1]};
        if (!completes) *reinterpret_cast<u32x4*>(st + 32 * u) = w[u];
        if (off == 0) {
          *reinterpret_cast<float4v*>(sd + 32 * u) = sv[u][0];
          *reinterpret_cast<float4v*>(sd + 32 * u + 4) = sv[u][1];
        }
      }
    }
  }
}

// Phase 2: rows whose block is not completed within this call go, raw, to
// their stage row. Runs after phase 1 (same stream), which may still read
// stage rows of a block that this call completes. One row per D/8 lanes.
template <int D, int BS>
__global__ __launch_bounds__(256) void chan_stage_kernel(ChanArgs a) {
  constexpr int RL = D / 8;
  constexpr int RPW = kWave / RL;
  const int lane = threadIdx.x & (kWave - 1);
  const int j = lane % RL;
  const int64_t rows = a.num_tokens * a.H;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  for (int64_t base = wave * RPW; base < rows; base += nwaves * RPW) {
    const int64_t r = base + lane / RL;
    if (r >= rows) continue;
    const int64_t t = r / a.H;
    const int h = (int)(r % a.H);
    const int64_t slot = a.slots[t];
    if (slot < 0) continue;
    const int32_t srow = a.stage_rows[t];
    if (srow < 0 || srow >= a.max_seqs || slot / BS >= a.num_blocks) continue;
    const int off = (int)(slot % BS);
    // completed in this call iff the token holding the block's last offset
    // follows in the same run
    const int64_t tl = t + (BS - 1 - off);
    const bool completes = tl < a.num_tokens && a.slots[tl] == slot + (BS - 1 - off) &&
                           a.stage_rows[tl] == srow;
    if (completes) continue;
    const u32x4 w = *reinterpret_cast<const u32x4*>(a.src + t * a.row_stride + (int64_t)h * D + 8 * j);
    *reinterpret_cast<u32x4*>(a.stage + (((int64_t)srow * a.H + h) * BS + off) * D + 8 * j) = w;
  }
}

// Phase 2 for bulk appends: lane l of a wave holds the metadata of row
// 64 c + l (row = token H + head), and the wave copies the rows that need the
// stage, four at a time (16 lanes of 16 bytes per row at D = 128, eight per
// row at D = 64).
template <int D, int BS>
__global__ __launch_bounds__(256) void chan_stage_chunked_kernel(ChanArgs a) {
  constexpr int RL = D / 8;          // lanes per row
  constexpr int RPW = kWave / RL;    // rows per copy step
  const int lane = threadIdx.x & (kWave - 1);
  const int j = lane % RL;
  const int64_t rows = a.num_tokens * a.H;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  for (int64_t base = wave * kWave; base < rows; base += nwaves * kWave) {
    const int64_t r = base + lane;
    bool need = false;
    int64_t dst = 0;
    if (r < rows) {
      const int64_t t = r / a.H;
      const int h = (int)(r % a.H);
      const int64_t slot = a.slots[t];
      const int32_t srow = a.stage_rows[t];
      if (slot >= 0 && srow >= 0 && srow < a.max_seqs && slot / BS < a.num_blocks) {
        const int off = (int)(slot % BS);
        const int64_t tl = t + (BS - 1 - off);
        const bool completes = tl < a.num_tokens && a.slots[tl] == slot + (BS - 1 - off) &&
                               a.stage_rows[tl] == srow;
        need = !completes;
        dst = (((int64_t)srow * a.H + h) * BS + off) * D;
      }
    }
    // the rows that need the stage, RPW at a time: lane group q copies the
    // row of the q-th lowest remaining set bit (the picks are wave-uniform)
    uint64_t rem = __ballot(need);
    const int q = lane / RL;
    while (rem) {
      int src = -1;
#pragma unroll
      for (int z = 0; z < RPW; ++z) {
        const int b = rem ? __builtin_ctzll(rem) : -1;
        rem &= rem - 1;   // rem = 0 stays 0
        if (z == q) src = b;
      }
      const int64_t dd = __shfl(dst, src < 0 ? 0 : src);
      if (src >= 0) {
        const int64_t rr = base + src;
        const int64_t t = rr / a.H;
        const int h = (int)(rr % a.H);
        const u32x4 w =
            *reinterpret_cast<const u32x4*>(a.src + t * a.row_stride + (int64_t)h * D + 8 * j);
        *reinterpret_cast<u32x4*>(a.stage + dd + 8 * j) = w;
      }
    }
  }
}

// (token, head) items above which a per-channel key append takes the chunked
// kernels: two items per wave of the largest grid (256 CUs x 16 workgroups of
// four waves).
constexpr int64_t kChanBulkItems = 2 * 256 * 16 * 4;

int grid_for(int64_t waves_needed, int cu_count) {
  int64_t blocks = (waves_needed + 3) / 4;
  int64_t cap = (int64_t)cu_count * 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

template <int D, bool BF16, bool STATIC>
void launch_rows_t(dim3 grid, const RowArgs& ra, int code, int mode, hipStream_t stream) {
  if (code == KVQ_CODE_INT8)
    append_bytes_kernel<KVQ_CODE_INT8, D, BF16, STATIC><<<grid, 256, 0, stream>>>(ra);
  else if (code == KVQ_CODE_FP8_E4M3)
    append_bytes_kernel<KVQ_CODE_FP8_E4M3, D, BF16, STATIC><<<grid, 256, 0, stream>>>(ra);
  else if (code == KVQ_CODE_NONE16)
    append_bytes_kernel<KVQ_CODE_NONE16, D, BF16, false><<<grid, 256, 0, stream>>>(ra);
  else if (mode == KVQ_SCALE_TOKEN_SYM)
    append_int4_kernel<KVQ_SCALE_TOKEN_SYM, D, BF16, STATIC><<<grid, 256, 0, stream>>>(ra);
  else
    append_int4_kernel<KVQ_SCALE_GROUP_ASYM, D, BF16, STATIC><<<grid, 256, 0, stream>>>(ra);
}

template <int D, bool BF16>
hipError_t launch_rows(const AppendPlan& p, const RowArgs& ra, int code, int mode,
                       int nsides, hipStream_t stream) {
  // every row kernel: one wave per (16-token group, head)
  const int64_t waves = (p.num_tokens + 15) / 16 * p.num_kv_heads;
  dim3 grid(grid_for(waves, p.cu_count), nsides);
  if (p.is_static)
    launch_rows_t<D, BF16, true>(grid, ra, code, mode, stream);
  else
    launch_rows_t<D, BF16, false>(grid, ra, code, mode, stream);
  return hipGetLastError();
}

template <int D, int BS, bool BF16>
hipError_t launch_chan(const AppendPlan& p, hipStream_t stream) {
  ChanArgs c;
  c.src = static_cast<const uint16_t*>(p.side[0].src);
  c.row_stride = p.side[0].row_stride;
  c.slots = p.slots;
  c.stage_rows = p.stage_rows;
  c.stage = static_cast<uint16_t*>(p.k_stage);
  c.codes = static_cast<int8_t*>(p.side[0].codes);
  c.scale = p.side[0].scale;
  c.num_tokens = p.num_tokens;
  c.num_blocks = p.num_blocks;
  c.H = p.num_kv_heads;
  c.max_seqs = p.max_seqs;
  const int64_t items = p.num_tokens * p.num_kv_heads;
  // Up to a few items per wave of the full grid (a decode step's append),
  // one wave per (token, head) item; beyond, the chunked kernels, whose
  // waves read 64 tokens' slots at once
  const bool bulk = items > kChanBulkItems;
  hipError_t e;
  if (bulk) {
    const int64_t chunk_items = (p.num_tokens + kWave - 1) / kWave * p.num_kv_heads;
    chan_complete_chunked_kernel<D, BS, BF16>
        <<<grid_for(chunk_items, p.cu_count), 256, 0, stream>>>(c);
  } else {
    chan_complete_kernel<D, BS, BF16><<<grid_for(items, p.cu_count), 256, 0, stream>>>(c);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (bulk) {
    chan_stage_chunked_kernel<D, BS>
        <<<grid_for((items + kWave - 1) / kWave, p.cu_count), 256, 0, stream>>>(c);
  } else {
    const int64_t waves = (items + (kWave / (D / 8)) - 1) / (kWave / (D / 8));
    chan_stage_kernel<D, BS><<<grid_for(waves, p.cu_count), 256, 0, stream>>>(c);
  }
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_append_d(const AppendPlan& p, hipStream_t stream) {
  RowArgs ra;
  for (int s = 0; s < 2; ++s) {
    ra.side[s].src = static_cast<const uint16_t*>(p.side[s].src);
    ra.side[s].row_stride = p.side[s].row_stride;
    ra.side[s].codes = static_cast<uint8_t*>(p.side[s].codes);
    ra.side[s].scale = p.side[s].scale;
    ra.side[s].zero = p.side[s].zero;
    ra.side[s].st_scale = p.side[s].st_scale;
    ra.side[s].st_zero = p.side[s].st_zero;
  }
  ra.slots = p.slots;
  ra.stage_rows = p.stage_rows;
  ra.stage = static_cast<uint16_t*>(p.k_stage);
  ra.max_seqs = p.max_seqs;
  ra.num_tokens = p.num_tokens;
  ra.num_blocks = p.num_blocks;
  ra.H = p.num_kv_heads;
  ra.bs = p.block_size;
  {
    const uint32_t d = (uint32_t)p.num_kv_heads;
    uint32_t l = 0;
    while ((1u << l) < d) ++l;  // ceil(log2 d)
    ra.h_shift = l;
    ra.h_mul = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
    ra.bs_shift = p.block_size == 16 ? 4 : 5;
  }
  hipError_t e;
  const bool chan = p.mode[0] == KVQ_SCALE_CHANNEL_BLOCK_SYM;
  if (!chan && p.code[0] == p.code[1] && p.mode[0] == p.mode[1]) {
    ra.side0 = 0;
    return launch_rows<D, BF16>(p, ra, p.code[0], p.mode[0], 2, stream);
  }
  if (!chan) {
    ra.side0 = 0;
    e = launch_rows<D, BF16>(p, ra, p.code[0], p.mode[0], 1, stream);
    if (e != hipSuccess) return e;
  } else if (p.is_static) {
    ra.side0 = 0;
    const int64_t waves = (p.num_tokens + 15) / 16 * p.num_kv_heads;
    append_chan_static_kernel<D, BF16><<<grid_for(waves, p.cu_count), 256, 0, stream>>>(ra);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    e = p.block_size == 16 ? launch_chan<D, 16, BF16>(p, stream)
                           : launch_chan<D, 32, BF16>(p, stream);
    if (e != hipSuccess) return e;
  }
  ra.side0 = 1;
  return launch_rows<D, BF16>(p, ra, p.code[1], p.mode[1], 1, stream);
}

}  // namespace

hipError_t launch_append(const AppendPlan& p, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  if (p.head_dim == 128)
    return p.src_bf16 ? launch_append_d<128, true>(p, stream) : launch_append_d<128, false>(p, stream);
  return p.src_bf16 ? launch_append_d<64, true>(p, stream) : launch_append_d<64, false>(p, stream);
}

}  // namespace kvq
