// kvq_internal.h -- host-side interface between the C ABI layer
// (kvq_api.cpp) and the kernel launchers (kvq_*.hip). Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// One side (keys or values) of an append.
struct AppendSide {
  const void* src;     // 16-bit rows, token t head h element e at
                       // src[t * row_stride + h * d + e]
  int64_t row_stride;  // elements
  void* codes;
  float* scale;
  uint8_t* zero;
  const float* st_scale;   // static scales ([H] or [H][d/32]); null: dynamic
  const uint8_t* st_zero;  // static zero points ([H][d/32], GROUP_ASYM)
};

struct AppendPlan {
  AppendSide side[2];  // [0] keys, [1] values
  const int64_t* slots;
  const int32_t* stage_rows;
  void* k_stage;
  int64_t num_tokens;
  int64_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t src_bf16;
  int32_t code[2];
  int32_t mode[2];
  int32_t max_seqs;
  int32_t cu_count;
  int32_t is_static;   // codes from the sides' st_scale / st_zero
};

hipError_t launch_append(const AppendPlan& p, hipStream_t stream);

struct DecodePlan {
  const void* q;
  int32_t q_bf16;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t k_code, v_code, k_mode, v_mode;
  int32_t src_bf16;
  const void* k_codes;
  const void* v_codes;
  const float* k_scale;
  const float* v_scale;
  const uint8_t* k_zero;
  const uint8_t* v_zero;
  const void* k_stage;
  int64_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;
  int32_t max_context_len;
  int32_t split_blocks;  // cache blocks per split, 0 = planned on the device
  int32_t item_bound;    // upper bound on (sequence, split) items: grid size
  float sm_scale;
  void* out;
  int32_t out_dtype;
  float* ws_acc;  // [item_bound][Hq][d]
  float* ws_ml;   // [item_bound][Hq][2]
  // kvq_append_decode_attention: the step's new rows, else nullptr
  const void* new_k = nullptr;
  const void* new_v = nullptr;
  int64_t new_k_stride = 0;
  int64_t new_v_stride = 0;
};

// Split planning constants, shared by the host (grid and workspace bounds)
// and the device (the plan itself). A workgroup of kDecodeWaves waves takes
// one (sequence, KV head, split) item. When the caller leaves split_blocks
// at 0 the per-wave share is ceil(H * total_blocks / 2^lg) blocks, clamped to
// [ceil(kDecodeMinWaveTokens / bs), cap], with lg, cap =
// kDecodeUniformWavesLog2, kDecodeMaxWaveBlocks for a batch of nearly equal
// lengths and kDecodeTargetWavesLog2, kDecodeSkewWaveBlocks otherwise. The
// host's item bound assumes the second pair, which yields more items for any
// lengths.
constexpr int kDecodeWaves = 4;
constexpr int kDecodeMaxWaveBlocks = 256;
constexpr int kDecodeTargetWavesLog2 = 12;
constexpr int kDecodeUniformWavesLog2 = 11;
constexpr int kDecodeMinWaveTokens = 32;
// Per-wave share cap for batches of unequal lengths: 32 blocks, or 64 with
// per-channel keys, whose items cost more to start (each block folds its
// scales into the query); the host bound takes the smaller, which yields
// more items.
// Byte codes and 16-bit rows with per-token scales take longer shares, 64
// blocks, over half as many waves (2^11): their blocks cost less to convert
// than INT4 tiles, and a wave's fixed start (query, id window, first loads)
// then weighs less (the 8B layer, 64 sequences of 1-8K tokens: 118 against
// 124-129 us per launch at 128-block splits); INT4, whose loop is bound by
// its instruction latency, measured slower with longer shares.
constexpr int kDecodeSkewWaveBlocks = 32;
constexpr int kDecodeSkewWaveBlocksBytes = 64;
constexpr int kDecodeSkewWaveBlocksChannel = 64;
constexpr int kDecodeSkewWavesLog2Bytes = 11;
__host__ __device__ constexpr int decode_skew_cap(int32_t k_code, int32_t k_mode) {
  return k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM ? kDecodeSkewWaveBlocksChannel
         : k_code == KVQ_CODE_INT4             ? kDecodeSkewWaveBlocks
                                               : kDecodeSkewWaveBlocksBytes;
}
// the wave target (log2) of a batch of unequal lengths
__host__ __device__ constexpr int decode_skew_lg(int32_t k_code, int32_t k_mode) {
  return k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM || k_code == KVQ_CODE_INT4
             ? kDecodeTargetWavesLog2
             : kDecodeSkewWavesLog2Bytes;
}

// Largest decode split grid: sixteen workgroups of kDecodeWaves waves per
// CU of a 256-CU chip, a multiple of 16; when the host's bound on the (item,
// KV head) pairs is larger, a grid of this size takes the pairs in rounds.
constexpr int kDecodeMaxGrid = 4096;

hipError_t launch_decode(const DecodePlan& p, hipStream_t stream);
// Device address of the current device's decode scratch array
// (KVQ_DECODE_SCRATCH_BYTES, 256-byte aligned), looked up once per device.
hipError_t decode_scratch(void** ptr);
bool decode_supported(int32_t k_code, int32_t v_code, int32_t k_mode,
                      int32_t v_mode);

// Multi-query (prefill) attention: the decode fields (q is [Tq][Hq][d], out
// [Tq][Hq][d], the workspace [batch][splits][H][col_tiles * 16] partials)
// plus the query rows of each sequence.
struct PrefillPlan {
  DecodePlan d;
  const int32_t* query_start;  // [batch + 1]
  int32_t max_query_len;
  int32_t splits;              // J: splits per sequence (upper bound)
  int32_t split_blocks;        // S: cache blocks per split
  int32_t col_tiles;           // CT: 16-column tiles per (sequence, KV head)
  int32_t window;              // > 0: sliding window of the last `window` positions
  int32_t sink;                // sink positions kept next to the window
};

// Longest split the multi-query kernels take (the library's own choice for
// 8-bit per-token caches may exceed the caller's bound on split_blocks).
constexpr int kPrefillMaxSplitBlocks = 512;

hipError_t launch_prefill(const PrefillPlan& p, hipStream_t stream);
bool prefill_supported(int32_t k_code, int32_t v_code, int32_t k_mode, int32_t v_mode);

hipError_t launch_pool_init(int32_t* stack, int32_t* top, const int32_t* order,
                            int64_t n, hipStream_t stream);
hipError_t launch_blocks_reserve(int32_t* stack, int32_t* top, int64_t capacity,
                                 int32_t* tables, int32_t max_blocks,
                                 const int32_t* lens, const int32_t* new_tokens,
                                 int32_t batch, int32_t bs, int64_t* slots,
                                 int64_t slot_capacity, int32_t* lens_out, int32_t* status,
                                 hipStream_t stream);
hipError_t launch_blocks_release(int32_t* stack, int32_t* top,
                                 int64_t capacity, const int32_t* tables,
                                 int32_t max_blocks, const int32_t* lens,
                                 const int32_t* mask, int32_t batch, int32_t bs,
                                 int32_t* lens_out, int32_t* status,
                                 hipStream_t stream);
hipError_t launch_check_tables(const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                               int32_t batch, int32_t bs, int64_t num_blocks, int64_t* first_bad,
                               int32_t* status, hipStream_t stream);
hipError_t launch_check_slots(const int64_t* slots, int64_t n, int64_t num_blocks, int32_t bs,
                              int64_t* first_bad, int32_t* status, hipStream_t stream);

}  // namespace kvq
