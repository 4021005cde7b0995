// kvq_api.cpp -- the library's C ABI: argument checks, sizes, split planning
// and dispatch to the HIP launchers. Every check runs on the host before any
// launch; the library allocates nothing and keeps no state.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include <hip/hip_runtime.h>

#include "kvq.h"
#include "kvq_internal.h"
#include "kvq_sharing.h"

namespace {

// Largest caller-given split (cache blocks shared by a workgroup's waves).
constexpr int64_t kMaxSplitBlocks = 256;
// Tokens per append launch: keeps row indices within int32 inside kernels.
constexpr int64_t kAppendChunk = int64_t(1) << 22;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int code_bits(int32_t code) {
  return code == KVQ_CODE_NONE16 ? 16 : code == KVQ_CODE_INT4 ? 4 : 8;
}

kvq_status check_side(const kvq_layout* L, int side) {
  const int32_t code = side ? L->v_code : L->k_code;
  const int32_t mode = side ? L->v_mode : L->k_mode;
  if (code < KVQ_CODE_NONE16 || code > KVQ_CODE_INT4) return KVQ_ERR_INVALID_ARGUMENT;
  if (mode < KVQ_SCALE_TOKEN_SYM || mode > KVQ_SCALE_CHANNEL_BLOCK_SYM)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (mode == KVQ_SCALE_TOKEN_SYM) return KVQ_OK;
  if (mode == KVQ_SCALE_GROUP_ASYM)
    return (code == KVQ_CODE_INT4 && L->group_size == 32) ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
  return (side == 0 && code == KVQ_CODE_INT8) ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
}

int64_t scales_per_bh(const kvq_layout* L, int side) {
  const int32_t code = side ? L->v_code : L->k_code;
  const int32_t mode = side ? L->v_mode : L->k_mode;
  if (code == KVQ_CODE_NONE16) return 0;
  if (mode == KVQ_SCALE_TOKEN_SYM) return L->block_size;
  if (mode == KVQ_SCALE_GROUP_ASYM) return (int64_t)L->block_size * (L->head_dim / L->group_size);
  return L->head_dim;
}

int64_t zeros_per_bh(const kvq_layout* L, int side) {
  const int32_t mode = side ? L->v_mode : L->k_mode;
  return mode == KVQ_SCALE_GROUP_ASYM ? (int64_t)L->block_size * (L->head_dim / L->group_size)
                                      : 0;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Upper bound on the (sequence, split) items the device plan can produce for
// any lengths within [0, max_context_len]: sum_b ceil(n_b / S) with n_b
// <= nmax = ceil(max_context_len / bs) blocks. For an explicit S it is
// batch * ceil(nmax / S). For a planned S = 4w, w = clamp(ceil(H N / 2^12),
// wmin, 64) with N = sum_b n_b: each non-empty sequence adds at most one
// split beyond n_b / S, so the sum is at most batch + N / S, and N / S is
// at most 2^12 / (4 H) while w is below 64 and batch nmax / 256 once it is
// 64. Also at most batch * ceil(nmax / (4 wmin)). The plan for nearly equal
// lengths, w = clamp(ceil(H N / 2^11), wmin, 128), gives fewer items than
// either term.
int64_t decode_item_bound(const kvq_layout* L, int64_t batch, int64_t max_context_len,
                          int64_t split_blocks) {
  const int64_t bs = L->block_size;
  const int64_t nmax = ceil_div(max_context_len, bs);
  if (batch == 0 || nmax == 0) return 1;
  if (split_blocks > 0) return batch * ceil_div(nmax, split_blocks);
  const int64_t W = kvq::kDecodeWaves;
  const int64_t wmin = ceil_div(kvq::kDecodeMinWaveTokens, bs);
  const int64_t a = batch * ceil_div(nmax, W * wmin);
  const int64_t c = batch + std::max(ceil_div(int64_t(1) << kvq::kDecodeTargetWavesLog2,
                                              W * L->num_kv_heads),
                                     ceil_div(batch * nmax, W * kvq::kDecodeSkewWaveBlocks));
  return std::min(a, c);
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace

extern "C" {

const char* kvq_status_string(kvq_status status) {
  switch (status) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_INVALID_ARGUMENT: return "KVQ_ERR_INVALID_ARGUMENT";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED";
    case KVQ_ERR_WORKSPACE_TOO_SMALL: return "KVQ_ERR_WORKSPACE_TOO_SMALL";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP";
    case KVQ_ERR_OUT_OF_BLOCKS: return "KVQ_ERR_OUT_OF_BLOCKS";
    default: return "KVQ_UNKNOWN_STATUS";
  }
}

kvq_status kvq_layout_check(const kvq_layout* L) {
  if (!L) return KVQ_ERR_INVALID_ARGUMENT;
  if (L->reserved != 0 || L->num_kv_heads < 1 || L->num_kv_heads > 4096)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (L->head_dim != 64 && L->head_dim != 128) return KVQ_ERR_INVALID_ARGUMENT;
  if (L->block_size != 16 && L->block_size != 32) return KVQ_ERR_INVALID_ARGUMENT;
  if (L->src_dtype != KVQ_F16 && L->src_dtype != KVQ_BF16) return KVQ_ERR_INVALID_ARGUMENT;
  kvq_status s = check_side(L, 0);
  if (s != KVQ_OK) return s;
  return check_side(L, 1);
}

int64_t kvq_bytes_per_token(const kvq_layout* L, int32_t num_layers, int32_t include_metadata) {
  kvq_status s = kvq_layout_check(L);
  if (s != KVQ_OK) return s;
  if (num_layers < 1) return KVQ_ERR_INVALID_ARGUMENT;
  const int64_t H = L->num_kv_heads, d = L->head_dim, bs = L->block_size;
  int64_t per_layer = 0;
  for (int side = 0; side < 2; ++side) {
    const int32_t code = side ? L->v_code : L->k_code;
    const int32_t mode = side ? L->v_mode : L->k_mode;
    per_layer += H * d * code_bits(code) / 8;
    if (!include_metadata || code == KVQ_CODE_NONE16) continue;
    if (mode == KVQ_SCALE_TOKEN_SYM)
      per_layer += H * 4;
    else if (mode == KVQ_SCALE_GROUP_ASYM)
      per_layer += H * (d / L->group_size) * 5;
    else
      per_layer += (H * d * 4 + bs - 1) / bs;
  }
  return per_layer * num_layers;
}

kvq_status kvq_cache_plane_bytes(const kvq_layout* L, int64_t num_blocks, int32_t max_seqs,
                                 int64_t out_bytes[7]) {
  kvq_status s = kvq_layout_check(L);
  if (s != KVQ_OK) return s;
  if (!out_bytes || num_blocks < 0 || max_seqs < 0) return KVQ_ERR_INVALID_ARGUMENT;
  const int64_t H = L->num_kv_heads, bs = L->block_size, d = L->head_dim;
  for (int side = 0; side < 2; ++side) {
    const int32_t code = side ? L->v_code : L->k_code;
    out_bytes[0 + side] = num_blocks * H * bs * d * code_bits(code) / 8;
    out_bytes[2 + side] = num_blocks * H * scales_per_bh(L, side) * 4;
    out_bytes[4 + side] = num_blocks * H * zeros_per_bh(L, side);
  }
  out_bytes[6] = L->k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM ? (int64_t)max_seqs * H * bs * d * 2 : 0;
  return KVQ_OK;
}

static kvq_status check_cache(const kvq_layout* L, const kvq_cache* C) {
  if (!C || C->reserved != 0 || C->num_blocks < 1 || C->max_seqs < 0)
    return KVQ_ERR_INVALID_ARGUMENT;
  for (int side = 0; side < 2; ++side) {
    const void* codes = side ? C->v_codes : C->k_codes;
    const float* scale = side ? C->v_scale : C->k_scale;
    const uint8_t* zero = side ? C->v_zero : C->k_zero;
    if (!codes || !aligned16(codes)) return KVQ_ERR_INVALID_ARGUMENT;
    if ((scales_per_bh(L, side) > 0) != (scale != nullptr)) return KVQ_ERR_INVALID_ARGUMENT;
    if (scale && !aligned16(scale)) return KVQ_ERR_INVALID_ARGUMENT;
    if ((zeros_per_bh(L, side) > 0) != (zero != nullptr)) return KVQ_ERR_INVALID_ARGUMENT;
    if (zero && !aligned16(zero)) return KVQ_ERR_INVALID_ARGUMENT;
  }
  const bool chan = L->k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM;
  if (chan != (C->k_stage != nullptr)) return KVQ_ERR_INVALID_ARGUMENT;
  if (chan && (C->max_seqs < 1 || !aligned16(C->k_stage))) return KVQ_ERR_INVALID_ARGUMENT;
  return KVQ_OK;
}

namespace {

// Both append entry points: st[side] / sz[side] are the static parameters
// (null on the dynamic path).
kvq_status append_common(const kvq_layout* L, const kvq_cache* C, const void* k, const void* v,
                         int64_t k_row_stride, int64_t v_row_stride, int64_t num_tokens,
                         const int64_t* slot_mapping, const int32_t* stage_rows,
                         const float* const st[2], const uint8_t* const sz[2], bool is_static,
                         void* stream) {
  kvq_status s = kvq_layout_check(L);
  if (s != KVQ_OK) return s;
  s = check_cache(L, C);
  if (s != KVQ_OK) return s;
  if (num_tokens < 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return KVQ_OK;
  const int64_t row = (int64_t)L->num_kv_heads * L->head_dim;
  if (!k || !v || !slot_mapping || !aligned16(k) || !aligned16(v)) return KVQ_ERR_INVALID_ARGUMENT;
  // per-channel keys are appended in one launch pair; row indices stay int32
  if (L->k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM && num_tokens * L->num_kv_heads >= (int64_t(1) << 31))
    return KVQ_ERR_UNSUPPORTED;
  if (k_row_stride < row || v_row_stride < row) return KVQ_ERR_INVALID_ARGUMENT;
  if ((k_row_stride * 2) % 16 || (v_row_stride * 2) % 16) return KVQ_ERR_INVALID_ARGUMENT;
  const bool chan = L->k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM;
  if (chan != (stage_rows != nullptr)) return KVQ_ERR_INVALID_ARGUMENT;
  kvq::AppendPlan p;
  p.side[0] = {k, k_row_stride, C->k_codes, C->k_scale, C->k_zero, st[0], sz[0]};
  p.side[1] = {v, v_row_stride, C->v_codes, C->v_scale, C->v_zero, st[1], sz[1]};
  p.is_static = is_static;
  p.k_stage = C->k_stage;
  p.num_blocks = C->num_blocks;
  p.num_kv_heads = L->num_kv_heads;
  p.head_dim = L->head_dim;
  p.block_size = L->block_size;
  p.src_bf16 = L->src_dtype == KVQ_BF16;
  p.code[0] = L->k_code;
  p.code[1] = L->v_code;
  p.mode[0] = L->k_mode;
  p.mode[1] = L->v_mode;
  p.max_seqs = C->max_seqs;
  p.cu_count = 256;
  // Chunks keep kernel row indices small. A per-channel key append is not
  // chunked: a chunk boundary inside one sequence's run would split the rows
  // of a completing block between launches.
  const int64_t max_chunk = std::min<int64_t>(kAppendChunk, (int64_t(1) << 31) / L->num_kv_heads - 1);
  const int64_t chunk = chan ? num_tokens : max_chunk;
  for (int64_t t0 = 0; t0 < num_tokens; t0 += chunk) {
    const int64_t n = num_tokens - t0 < chunk ? num_tokens - t0 : chunk;
    p.side[0].src = static_cast<const uint16_t*>(k) + t0 * k_row_stride;
    p.side[1].src = static_cast<const uint16_t*>(v) + t0 * v_row_stride;
    p.slots = slot_mapping + t0;
    p.stage_rows = stage_rows ? stage_rows + t0 : nullptr;
    p.num_tokens = n;
    hipError_t e = kvq::launch_append(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return KVQ_ERR_HIP;
  }
  return KVQ_OK;
}

}  // namespace

kvq_status kvq_append(const kvq_layout* L, const kvq_cache* C, const void* k, const void* v,
                      int64_t k_row_stride, int64_t v_row_stride, int64_t num_tokens,
                      const int64_t* slot_mapping, const int32_t* stage_rows, void* stream) {
  const float* const st[2] = {nullptr, nullptr};
  const uint8_t* const sz[2] = {nullptr, nullptr};
  return append_common(L, C, k, v, k_row_stride, v_row_stride, num_tokens, slot_mapping,
                       stage_rows, st, sz, false, stream);
}

kvq_status kvq_append_static(const kvq_layout* L, const kvq_cache* C, const void* k,
                             const void* v, int64_t k_row_stride, int64_t v_row_stride,
                             int64_t num_tokens, const int64_t* slot_mapping,
                             const int32_t* stage_rows, const float* k_scales,
                             const uint8_t* k_zeros, const float* v_scales,
                             const uint8_t* v_zeros, void* stream) {
  kvq_status s = kvq_layout_check(L);
  if (s != KVQ_OK) return s;
  const float* const st[2] = {k_scales, v_scales};
  const uint8_t* const sz[2] = {k_zeros, v_zeros};
  const int32_t code[2] = {L->k_code, L->v_code}, mode[2] = {L->k_mode, L->v_mode};
  for (int i = 0; i < 2; ++i) {
    // a passthrough side takes no parameters; a quantized one its scales,
    // and zero points exactly when it is asymmetric
    const bool quant = code[i] != KVQ_CODE_NONE16;
    const bool asym = quant && mode[i] == KVQ_SCALE_GROUP_ASYM;
    if ((st[i] != nullptr) != quant || (sz[i] != nullptr) != asym)
      return KVQ_ERR_INVALID_ARGUMENT;
    // per-channel scales are read as 16-byte vectors
    const uintptr_t align = mode[i] == KVQ_SCALE_CHANNEL_BLOCK_SYM ? 16 : 4;
    if (st[i] && reinterpret_cast<uintptr_t>(st[i]) % align) return KVQ_ERR_INVALID_ARGUMENT;
  }
  return append_common(L, C, k, v, k_row_stride, v_row_stride, num_tokens, slot_mapping,
                       stage_rows, st, sz, true, stream);
}

int64_t kvq_decode_workspace_bytes(const kvq_layout* L, int32_t batch, int32_t num_q_heads,
                                   int32_t max_context_len, int32_t split_blocks) {
  kvq_status s = kvq_layout_check(L);
  if (s != KVQ_OK) return s;
  if (batch < 0 || num_q_heads < 1 || max_context_len < 0 || split_blocks < 0 ||
      split_blocks > kMaxSplitBlocks)
    return KVQ_ERR_INVALID_ARGUMENT;
  const int64_t items = decode_item_bound(L, batch, max_context_len, split_blocks) * num_q_heads;
  return round_up(items * L->head_dim * 4, 256) + round_up(items * 2 * 4, 256);
}

namespace {

// Host checks shared by both decode entry points (every check before any
// launch); on success *need is the workspace the call needs.
kvq_status decode_check(const kvq_layout* L, const kvq_cache* C, const void* q, int32_t q_dtype,
                        int32_t batch, int32_t num_q_heads, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t max_context_len, float sm_scale, int32_t split_blocks,
                        void* out, int32_t out_dtype, int64_t* need) {
  *need = 0;
  kvq_status s = kvq_layout_check(L);
  if (s != KVQ_OK) return s;
  s = check_cache(L, C);
  if (s != KVQ_OK) return s;
  if (batch < 0 || num_q_heads < 1 || num_q_heads % L->num_kv_heads) return KVQ_ERR_INVALID_ARGUMENT;
  if (num_q_heads / L->num_kv_heads > 16) return KVQ_ERR_UNSUPPORTED;
  if (q_dtype != KVQ_F16 && q_dtype != KVQ_BF16) return KVQ_ERR_INVALID_ARGUMENT;
  if (out_dtype != KVQ_F32 && out_dtype != KVQ_F16 && out_dtype != KVQ_BF16)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (max_context_len < 0 || split_blocks < 0 || split_blocks > kMaxSplitBlocks ||
      max_blocks_per_seq < 1)
    return KVQ_ERR_INVALID_ARGUMENT;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * L->block_size)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (!(sm_scale >= 0.0f) || isinf(sm_scale)) return KVQ_ERR_INVALID_ARGUMENT;
  if (!kvq::decode_supported(L->k_code, L->v_code, L->k_mode, L->v_mode)) return KVQ_ERR_UNSUPPORTED;
  // per-channel keys: row b of the batch reads stage row b
  if (L->k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM && batch > C->max_seqs)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (batch == 0) return KVQ_OK;
  if (!q || !out || !block_tables || !context_lens) return KVQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(out)) return KVQ_ERR_INVALID_ARGUMENT;
  // the device planner counts blocks in int32
  if ((int64_t)batch * ceil_div(max_context_len, L->block_size) > INT32_MAX)
    return KVQ_ERR_UNSUPPORTED;
  const int64_t bound = decode_item_bound(L, batch, max_context_len, split_blocks);
  if (bound * L->num_kv_heads > INT32_MAX - 16) return KVQ_ERR_UNSUPPORTED;  // 1-D grid
  *need = kvq_decode_workspace_bytes(L, batch, num_q_heads, max_context_len, split_blocks);
  return KVQ_OK;
}

// Enqueue the split and reduce kernels; the arguments passed decode_check.
kvq_status decode_launch(const kvq_layout* L, const kvq_cache* C, const void* q, int32_t q_dtype,
                         int32_t batch, int32_t num_q_heads, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t max_context_len, float sm_scale, int32_t split_blocks,
                         void* out, int32_t out_dtype, void* workspace, void* stream,
                         const void* new_k = nullptr, const void* new_v = nullptr,
                         int64_t new_k_stride = 0, int64_t new_v_stride = 0) {
  const int64_t bound = decode_item_bound(L, batch, max_context_len, split_blocks);
  const int64_t items = bound * num_q_heads;
  kvq::DecodePlan p;
  p.q = q;
  p.q_bf16 = q_dtype == KVQ_BF16;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = L->num_kv_heads;
  p.head_dim = L->head_dim;
  p.block_size = L->block_size;
  p.k_code = L->k_code;
  p.v_code = L->v_code;
  p.k_mode = L->k_mode;
  p.v_mode = L->v_mode;
  p.src_bf16 = L->src_dtype == KVQ_BF16;
  p.k_codes = C->k_codes;
  p.v_codes = C->v_codes;
  p.k_scale = C->k_scale;
  p.v_scale = C->v_scale;
  p.k_zero = C->k_zero;
  p.v_zero = C->v_zero;
  p.k_stage = C->k_stage;
  p.num_blocks = C->num_blocks;
  p.block_tables = block_tables;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.context_lens = context_lens;
  p.max_context_len = max_context_len;
  p.split_blocks = split_blocks;
  p.item_bound = (int32_t)bound;
  p.sm_scale = sm_scale > 0.0f ? sm_scale : (float)(1.0 / sqrt((double)L->head_dim));
  p.out = out;
  p.out_dtype = out_dtype;
  p.ws_acc = static_cast<float*>(workspace);
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                     round_up(items * L->head_dim * 4, 256));
  p.new_k = new_k;
  p.new_v = new_v;
  p.new_k_stride = new_k_stride;
  p.new_v_stride = new_v_stride;
  return hip_status(kvq::launch_decode(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

kvq_status kvq_decode_attention(const kvq_layout* L, const kvq_cache* C, const void* q,
                                int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t max_context_len,
                                float sm_scale, int32_t split_blocks, void* out,
                                int32_t out_dtype, void* workspace, int64_t workspace_bytes,
                                void* stream) {
  int64_t need = 0;
  kvq_status s = decode_check(L, C, q, q_dtype, batch, num_q_heads, block_tables,
                              max_blocks_per_seq, context_lens, max_context_len, sm_scale,
                              split_blocks, out, out_dtype, &need);
  if (s != KVQ_OK || batch == 0) return s;
  if (!workspace || !aligned16(workspace)) return KVQ_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  return decode_launch(L, C, q, q_dtype, batch, num_q_heads, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, sm_scale, split_blocks, out, out_dtype,
                       workspace, stream);
}

kvq_status kvq_append_decode_attention(const kvq_layout* L, const kvq_cache* C, const void* k,
                                       const void* v, int64_t k_row_stride, int64_t v_row_stride,
                                       const void* q, int32_t q_dtype, int32_t batch,
                                       int32_t num_q_heads, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                                       int32_t max_context_len, float sm_scale,
                                       int32_t split_blocks, void* out, int32_t out_dtype,
                                       void* workspace, int64_t workspace_bytes, void* stream) {
  int64_t need = 0;
  kvq_status s = decode_check(L, C, q, q_dtype, batch, num_q_heads, block_tables,
                              max_blocks_per_seq, context_lens, max_context_len, sm_scale,
                              split_blocks, out, out_dtype, &need);
  if (s != KVQ_OK) return s;
  // byte codes with per-token scales, or 16-bit rows, on both sides
  const bool bytes = L->k_code == L->v_code && L->k_mode == KVQ_SCALE_TOKEN_SYM &&
                     L->v_mode == KVQ_SCALE_TOKEN_SYM &&
                     (L->k_code == KVQ_CODE_INT8 || L->k_code == KVQ_CODE_FP8_E4M3);
  const bool raw = L->k_code == KVQ_CODE_NONE16 && L->v_code == KVQ_CODE_NONE16;
  if (!bytes && !raw) return KVQ_ERR_UNSUPPORTED;
  if (batch == 0) return KVQ_OK;
  // every context holds at least its new token
  if (max_context_len < 1) return KVQ_ERR_INVALID_ARGUMENT;
  const int64_t row = (int64_t)L->num_kv_heads * L->head_dim;
  if (!k || !v || !aligned16(k) || !aligned16(v)) return KVQ_ERR_INVALID_ARGUMENT;
  if (k_row_stride < row || v_row_stride < row) return KVQ_ERR_INVALID_ARGUMENT;
  if ((k_row_stride * 2) % 16 || (v_row_stride * 2) % 16) return KVQ_ERR_INVALID_ARGUMENT;
  if (!workspace || !aligned16(workspace)) return KVQ_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  return decode_launch(L, C, q, q_dtype, batch, num_q_heads, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, sm_scale, split_blocks, out, out_dtype,
                       workspace, stream, k, v, k_row_stride, v_row_stride);
}

kvq_status kvq_decode_attention_noalloc(const kvq_layout* L, const kvq_cache* C, const void* q,
                                        int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t max_context_len,
                                        float sm_scale, int32_t split_blocks, void* out,
                                        int32_t out_dtype, void* stream) {
  int64_t need = 0;
  kvq_status s = decode_check(L, C, q, q_dtype, batch, num_q_heads, block_tables,
                              max_blocks_per_seq, context_lens, max_context_len, sm_scale,
                              split_blocks, out, out_dtype, &need);
  if (s != KVQ_OK || batch == 0) return s;
  // sizes beyond the library's scratch are refused before the device is touched
  if (need > (int64_t)KVQ_DECODE_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  void* scratch = nullptr;
  if (kvq::decode_scratch(&scratch) != hipSuccess || !scratch) return KVQ_ERR_HIP;
  return decode_launch(L, C, q, q_dtype, batch, num_q_heads, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, sm_scale, split_blocks, out, out_dtype,
                       scratch, stream);
}

namespace {

// Multi-query splits: S blocks per split, J = splits of the longest context,
// CT = 16-column tiles of max_query_len queries times G heads. S is the
// caller's, else:
//  - 8-bit codes with per-token scales (the LDS-staged kernel, whose
//    workgroups each pay a fixed start -- block ids, first loads, queries --
//    and a fixed merge): the launch's block visits, counted at the longest
//    context (sequences x KV heads x groups of up to eight column tiles x
//    blocks), over kPrefillUnits workgroups -- two rounds of two per CU --
//    within [32, kPrefillMaxSplitBlocks] blocks (fewer, longer splits also
//    mean fewer partials written and merged). Batches of 32 sequences or
//    more take twice the workgroups: their lengths usually spread below the
//    longest, so its visits overstate the work, and shorter splits balance
//    the unequal sequences (a heuristic: the lengths stay on the device).
//    S is a multiple of 32 blocks;
//  - other layouts (register-streaming kernel): a sixteenth of the longest
//    context within [32, 64], short enough that a batch of mostly short
//    sequences still fills the GPU.
constexpr int64_t kPrefillUnits = 1024;

struct PrefillShape {
  int64_t S, J, CT, partials;
};

bool prefill_staged(const kvq_layout* L) {
  return L->k_mode == KVQ_SCALE_TOKEN_SYM && L->v_mode == KVQ_SCALE_TOKEN_SYM &&
         L->k_code == L->v_code &&
         (L->k_code == KVQ_CODE_INT8 || L->k_code == KVQ_CODE_FP8_E4M3);
}

PrefillShape prefill_shape(const kvq_layout* L, int64_t batch, int64_t num_q_heads,
                           int64_t max_query_len, int64_t max_context_len, int64_t split_blocks) {
  PrefillShape sh;
  const int64_t maxblk = std::max<int64_t>(1, ceil_div(max_context_len, L->block_size));
  sh.CT = ceil_div(max_query_len * (num_q_heads / L->num_kv_heads), 16);
  if (split_blocks > 0) {
    sh.S = split_blocks;
  } else if (prefill_staged(L)) {
    const int64_t visits = batch * L->num_kv_heads * ceil_div(sh.CT, 8) * maxblk;
    // rounded down to 32 blocks: a split is whole 64-token chunks
    const int64_t units = batch >= 32 ? 2 * kPrefillUnits : kPrefillUnits;
    int64_t S = std::min<int64_t>(kvq::kPrefillMaxSplitBlocks,
                                  std::max<int64_t>(32, ceil_div(visits, units) / 32 * 32));
    // a last split shorter than a quarter of the others is spread over them
    // (whole chunks still, and no split past the LDS bound)
    const int64_t J = ceil_div(maxblk, S);
    if (J > 1 && maxblk - (J - 1) * S < S / 4) {
      const int64_t per_chunk = std::max<int64_t>(1, 64 / L->block_size);
      const int64_t S2 = round_up(ceil_div(maxblk, J - 1), per_chunk);
      if (S2 <= kvq::kPrefillMaxSplitBlocks) S = S2;
    }
    sh.S = S;
  } else {
    sh.S = std::min<int64_t>(64, std::max<int64_t>(32, ceil_div(maxblk, 16)));
  }
  sh.J = ceil_div(maxblk, sh.S);
  sh.partials = batch * sh.J * L->num_kv_heads * sh.CT * 16;
  return sh;
}

}  // namespace

int64_t kvq_prefill_workspace_bytes(const kvq_layout* L, int32_t batch, int32_t num_q_heads,
                                    int32_t max_query_len, int32_t max_context_len,
                                    int32_t split_blocks) {
  kvq_status s = kvq_layout_check(L);
  if (s != KVQ_OK) return s;
  if (batch < 0 || num_q_heads < 1 || num_q_heads % L->num_kv_heads || max_query_len < 0 ||
      max_context_len < max_query_len || split_blocks < 0 || split_blocks > kMaxSplitBlocks)
    return KVQ_ERR_INVALID_ARGUMENT;
  const PrefillShape sh = prefill_shape(L, batch, num_q_heads, max_query_len, max_context_len,
                                        split_blocks);
  return round_up(sh.partials * L->head_dim * 4, 256) + round_up(sh.partials * 2 * 4, 256);
}

kvq_status kvq_prefill_attention(const kvq_layout* L, const kvq_cache* C, const void* q,
                                 int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                                 const int32_t* query_start, int32_t max_query_len,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t max_context_len,
                                 float sm_scale, int32_t window, int32_t sink,
                                 int32_t split_blocks, void* out, int32_t out_dtype,
                                 void* workspace, int64_t workspace_bytes, void* stream) {
  kvq_status s = kvq_layout_check(L);
  if (s != KVQ_OK) return s;
  s = check_cache(L, C);
  if (s != KVQ_OK) return s;
  if (batch < 0 || num_q_heads < 1 || num_q_heads % L->num_kv_heads) return KVQ_ERR_INVALID_ARGUMENT;
  if (window < 0 || sink < 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (q_dtype != KVQ_F16 && q_dtype != KVQ_BF16) return KVQ_ERR_INVALID_ARGUMENT;
  if (out_dtype != KVQ_F32 && out_dtype != KVQ_F16 && out_dtype != KVQ_BF16)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (max_query_len < 0 || max_context_len < max_query_len || split_blocks < 0 ||
      split_blocks > kMaxSplitBlocks || max_blocks_per_seq < 1)
    return KVQ_ERR_INVALID_ARGUMENT;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * L->block_size)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (!(sm_scale >= 0.0f) || isinf(sm_scale)) return KVQ_ERR_INVALID_ARGUMENT;
  if (!kvq::prefill_supported(L->k_code, L->v_code, L->k_mode, L->v_mode))
    return KVQ_ERR_UNSUPPORTED;
  if (L->k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM && batch > C->max_seqs)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (batch == 0 || max_query_len == 0) return KVQ_OK;
  if (!q || !out || !query_start || !block_tables || !context_lens || !workspace)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return KVQ_ERR_INVALID_ARGUMENT;
  const int64_t need = kvq_prefill_workspace_bytes(L, batch, num_q_heads, max_query_len,
                                                   max_context_len, split_blocks);
  if (workspace_bytes < need) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  const PrefillShape sh = prefill_shape(L, batch, num_q_heads, max_query_len, max_context_len,
                                        split_blocks);
  // one workgroup per unit in a 1-D grid; the reduce grid is (heads,
  // queries, sequences)
  if (sh.partials / 16 > (int64_t)INT32_MAX || max_query_len > 65535 || batch > 65535)
    return KVQ_ERR_UNSUPPORTED;
  kvq::PrefillPlan pp;
  kvq::DecodePlan& p = pp.d;
  p.q = q;
  p.q_bf16 = q_dtype == KVQ_BF16;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = L->num_kv_heads;
  p.head_dim = L->head_dim;
  p.block_size = L->block_size;
  p.k_code = L->k_code;
  p.v_code = L->v_code;
  p.k_mode = L->k_mode;
  p.v_mode = L->v_mode;
  p.src_bf16 = L->src_dtype == KVQ_BF16;
  p.k_codes = C->k_codes;
  p.v_codes = C->v_codes;
  p.k_scale = C->k_scale;
  p.v_scale = C->v_scale;
  p.k_zero = C->k_zero;
  p.v_zero = C->v_zero;
  p.k_stage = C->k_stage;
  p.num_blocks = C->num_blocks;
  p.block_tables = block_tables;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.context_lens = context_lens;
  p.max_context_len = max_context_len;
  p.split_blocks = (int32_t)sh.S;
  p.item_bound = 0;
  p.sm_scale = sm_scale > 0.0f ? sm_scale : (float)(1.0 / sqrt((double)L->head_dim));
  p.out = out;
  p.out_dtype = out_dtype;
  p.ws_acc = static_cast<float*>(workspace);
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                     round_up(sh.partials * L->head_dim * 4, 256));
  pp.query_start = query_start;
  pp.max_query_len = max_query_len;
  pp.splits = (int32_t)sh.J;
  pp.split_blocks = (int32_t)sh.S;
  pp.col_tiles = (int32_t)sh.CT;
  pp.window = window;
  pp.sink = window > 0 ? sink : 0;
  return hip_status(kvq::launch_prefill(pp, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_pool_init(int32_t* free_stack, int32_t* free_top, const int32_t* initial_order,
                         int64_t num_blocks, void* stream) {
  if (!free_stack || !free_top || num_blocks < 1 || num_blocks > INT32_MAX)
    return KVQ_ERR_INVALID_ARGUMENT;
  return hip_status(kvq::launch_pool_init(free_stack, free_top, initial_order, num_blocks,
                                          static_cast<hipStream_t>(stream)));
}

kvq_status kvq_blocks_reserve(int32_t* free_stack, int32_t* free_top, int64_t pool_capacity,
                              int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, const int32_t* new_tokens,
                              int32_t batch, int32_t block_size, int64_t* slot_mapping_out,
                              int64_t slot_capacity, int32_t* context_lens_out,
                              int32_t* status_flag, void* stream) {
  if (!free_stack || !free_top || !status_flag || pool_capacity < 1 || pool_capacity > INT32_MAX)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (batch < 0 || max_blocks_per_seq < 1 || block_size < 1 || slot_capacity < 0)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (batch > 0 && (!block_tables || !context_lens || !new_tokens ||
                    (!slot_mapping_out && slot_capacity > 0)))
    return KVQ_ERR_INVALID_ARGUMENT;
  return hip_status(kvq::launch_blocks_reserve(
      free_stack, free_top, pool_capacity, block_tables, max_blocks_per_seq, context_lens,
      new_tokens, batch, block_size, slot_mapping_out, slot_capacity, context_lens_out,
      status_flag, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_blocks_release(int32_t* free_stack, int32_t* free_top, int64_t pool_capacity,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, const int32_t* release_mask,
                              int32_t batch, int32_t block_size, int32_t* context_lens_out,
                              int32_t* status_flag, void* stream) {
  if (!free_stack || !free_top || !status_flag || pool_capacity < 1 || pool_capacity > INT32_MAX)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (batch < 0 || max_blocks_per_seq < 1 || block_size < 1) return KVQ_ERR_INVALID_ARGUMENT;
  if (batch > 0 && (!block_tables || !context_lens || !release_mask)) return KVQ_ERR_INVALID_ARGUMENT;
  return hip_status(kvq::launch_blocks_release(
      free_stack, free_top, pool_capacity, block_tables, max_blocks_per_seq, context_lens,
      release_mask, batch, block_size, context_lens_out, status_flag,
      static_cast<hipStream_t>(stream)));
}

kvq_status kvq_check_block_tables(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t batch,
                                  int32_t block_size, int64_t num_blocks, int64_t* first_bad,
                                  int32_t* status_flag, void* stream) {
  if (!first_bad || !status_flag || batch < 0 || max_blocks_per_seq < 1 || block_size < 1 ||
      num_blocks < 1)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (batch > 0 && (!block_tables || !context_lens)) return KVQ_ERR_INVALID_ARGUMENT;
  return hip_status(kvq::launch_check_tables(block_tables, max_blocks_per_seq, context_lens,
                                             batch, block_size, num_blocks, first_bad,
                                             status_flag, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_check_slots(const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                           int32_t block_size, int64_t* first_bad, int32_t* status_flag,
                           void* stream) {
  if (!first_bad || !status_flag || num_tokens < 0 || num_blocks < 1 || block_size < 1 ||
      num_blocks > INT64_MAX / block_size)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (num_tokens > 0 && !slot_mapping) return KVQ_ERR_INVALID_ARGUMENT;
  return hip_status(kvq::launch_check_slots(slot_mapping, num_tokens, num_blocks, block_size,
                                            first_bad, status_flag,
                                            static_cast<hipStream_t>(stream)));
}

kvq_status kvq_blocks_trim(int32_t* free_stack, int32_t* free_top, int64_t pool_capacity,
                           int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t window, int32_t sink,
                           int32_t batch, int32_t block_size, int32_t* status_flag,
                           void* stream) {
  if (!free_stack || !free_top || !status_flag || pool_capacity < 1 || pool_capacity > INT32_MAX)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (batch < 0 || max_blocks_per_seq < 1 || block_size < 1 || window < 0 || sink < 0)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (batch > 0 && (!block_tables || !context_lens)) return KVQ_ERR_INVALID_ARGUMENT;
  return hip_status(kvq::launch_blocks_trim(free_stack, free_top, pool_capacity, block_tables,
                                            max_blocks_per_seq, context_lens, window, sink,
                                            batch, block_size, status_flag,
                                            static_cast<hipStream_t>(stream)));
}

kvq_status kvq_blocks_fork(int32_t* refcount, int64_t pool_capacity, int32_t* block_tables,
                           int32_t max_blocks_per_seq, int32_t* context_lens, int32_t batch,
                           const int32_t* src_rows, const int32_t* dst_rows, int32_t num_forks,
                           int32_t block_size, void* stream) {
  if (!refcount || pool_capacity < 1 || pool_capacity > INT32_MAX || batch < 0 ||
      max_blocks_per_seq < 1 || block_size < 1 || num_forks < 0)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (num_forks == 0) return KVQ_OK;
  if (!block_tables || !context_lens || !src_rows || !dst_rows) return KVQ_ERR_INVALID_ARGUMENT;
  return hip_status(kvq::launch_blocks_fork(refcount, pool_capacity, block_tables,
                                            max_blocks_per_seq, context_lens, batch, src_rows,
                                            dst_rows, num_forks, block_size,
                                            static_cast<hipStream_t>(stream)));
}

kvq_status kvq_blocks_reserve_shared(int32_t* free_stack, int32_t* free_top,
                                     int64_t pool_capacity, int32_t* refcount,
                                     int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, const int32_t* new_tokens,
                                     int32_t batch, int32_t block_size,
                                     int64_t* slot_mapping_out, int64_t slot_capacity,
                                     int32_t* context_lens_out, int32_t* cow_src,
                                     int32_t* cow_dst, int32_t* cow_count,
                                     int32_t* status_flag, void* stream) {
  if (!free_stack || !free_top || !status_flag || !refcount || !cow_count ||
      pool_capacity < 1 || pool_capacity > INT32_MAX)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (batch < 0 || max_blocks_per_seq < 1 || block_size < 1 || slot_capacity < 0)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (batch > 0 && (!block_tables || !context_lens || !new_tokens ||
                    (!slot_mapping_out && slot_capacity > 0) || !cow_src || !cow_dst))
    return KVQ_ERR_INVALID_ARGUMENT;
  return hip_status(kvq::launch_blocks_reserve_shared(
      free_stack, free_top, pool_capacity, refcount, block_tables, max_blocks_per_seq,
      context_lens, new_tokens, batch, block_size, slot_mapping_out, slot_capacity,
      context_lens_out, cow_src, cow_dst, cow_count, status_flag,
      static_cast<hipStream_t>(stream)));
}

kvq_status kvq_blocks_release_shared(int32_t* free_stack, int32_t* free_top,
                                     int64_t pool_capacity, int32_t* refcount,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, const int32_t* release_mask,
                                     int32_t batch, int32_t block_size,
                                     int32_t* context_lens_out, int32_t* status_flag,
                                     void* stream) {
  if (!free_stack || !free_top || !status_flag || !refcount || pool_capacity < 1 ||
      pool_capacity > INT32_MAX)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (batch < 0 || max_blocks_per_seq < 1 || block_size < 1) return KVQ_ERR_INVALID_ARGUMENT;
  if (batch > 0 && (!block_tables || !context_lens || !release_mask)) return KVQ_ERR_INVALID_ARGUMENT;
  return hip_status(kvq::launch_blocks_release_shared(
      free_stack, free_top, pool_capacity, refcount, block_tables, max_blocks_per_seq,
      context_lens, release_mask, batch, block_size, context_lens_out, status_flag,
      static_cast<hipStream_t>(stream)));
}

kvq_status kvq_copy_blocks(const kvq_layout* L, const kvq_cache* C, const int32_t* src_ids,
                           const int32_t* dst_ids, const int32_t* count, int32_t max_pairs,
                           void* stream) {
  kvq_status s = kvq_layout_check(L);
  if (s != KVQ_OK) return s;
  s = check_cache(L, C);
  if (s != KVQ_OK) return s;
  if (max_pairs < 0 || max_pairs > 65535 * 1024) return KVQ_ERR_INVALID_ARGUMENT;
  if (max_pairs == 0) return KVQ_OK;
  if (!src_ids || !dst_ids || !count) return KVQ_ERR_INVALID_ARGUMENT;
  int64_t planes[7];
  s = kvq_cache_plane_bytes(L, C->num_blocks, C->max_seqs, planes);
  if (s != KVQ_OK) return s;
  uint8_t* const base[6] = {static_cast<uint8_t*>(C->k_codes), static_cast<uint8_t*>(C->v_codes),
                            reinterpret_cast<uint8_t*>(C->k_scale),
                            reinterpret_cast<uint8_t*>(C->v_scale), C->k_zero, C->v_zero};
  int64_t per_block[6];
  for (int i = 0; i < 6; ++i) per_block[i] = planes[i] / C->num_blocks;
  return hip_status(kvq::launch_copy_blocks(base, per_block, src_ids, dst_ids, count, max_pairs,
                                            C->num_blocks, static_cast<hipStream_t>(stream)));
}

namespace {

// The six planes of one layer (k_codes, v_codes, k_scale, v_scale, k_zero,
// v_zero) and their bytes per block.
kvq_status block_planes(const kvq_layout* L, const kvq_cache* C, uint8_t* base[6],
                        int64_t per_block[6]) {
  int64_t planes[7];
  kvq_status s = kvq_cache_plane_bytes(L, C->num_blocks, C->max_seqs, planes);
  if (s != KVQ_OK) return s;
  uint8_t* const b[6] = {static_cast<uint8_t*>(C->k_codes), static_cast<uint8_t*>(C->v_codes),
                         reinterpret_cast<uint8_t*>(C->k_scale),
                         reinterpret_cast<uint8_t*>(C->v_scale), C->k_zero, C->v_zero};
  for (int i = 0; i < 6; ++i) {
    base[i] = b[i];
    per_block[i] = b[i] ? planes[i] / C->num_blocks : 0;
  }
  return KVQ_OK;
}

kvq_status pack_common(const kvq_layout* L, const kvq_cache* C, const int32_t* ids, int32_t n,
                       void* packed, bool pack, void* stream) {
  kvq_status s = kvq_layout_check(L);
  if (s != KVQ_OK) return s;
  s = check_cache(L, C);
  if (s != KVQ_OK) return s;
  if (n < 0 || n > 65535 * 1024) return KVQ_ERR_INVALID_ARGUMENT;
  if (n == 0) return KVQ_OK;
  if (!ids || !packed || !aligned16(packed)) return KVQ_ERR_INVALID_ARGUMENT;
  uint8_t* base[6];
  int64_t per[6];
  s = block_planes(L, C, base, per);
  if (s != KVQ_OK) return s;
  return hip_status(kvq::launch_pack_blocks(base, per, ids, n, static_cast<uint8_t*>(packed),
                                            pack, C->num_blocks,
                                            static_cast<hipStream_t>(stream)));
}

}  // namespace

int64_t kvq_block_pack_bytes(const kvq_layout* L) {
  kvq_status s = kvq_layout_check(L);
  if (s != KVQ_OK) return s;
  int64_t planes[7];
  kvq_cache_plane_bytes(L, 1, 0, planes);
  int64_t total = 0;
  for (int i = 0; i < 6; ++i) total += planes[i];
  return total;
}

kvq_status kvq_pack_blocks(const kvq_layout* L, const kvq_cache* C, const int32_t* ids,
                           int32_t n, void* dst, void* stream) {
  return pack_common(L, C, ids, n, dst, true, stream);
}

kvq_status kvq_unpack_blocks(const kvq_layout* L, const kvq_cache* C, const void* src,
                             const int32_t* ids, int32_t n, void* stream) {
  return pack_common(L, C, ids, n, const_cast<void*>(src), false, stream);
}

}  // extern "C"
