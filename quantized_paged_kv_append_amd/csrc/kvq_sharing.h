// kvq_sharing.h -- host-side interface between the C ABI layer (kvq_api.cpp)
// and the pool kernels for prefix sharing, window trimming and block offload
// (kvq_pool.hip).
// Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

hipError_t launch_blocks_fork(int32_t* refcount, int64_t capacity, int32_t* tables,
                              int32_t max_blocks, int32_t* lens, int32_t batch,
                              const int32_t* src, const int32_t* dst, int32_t num_forks,
                              int32_t bs, hipStream_t stream);
hipError_t launch_blocks_reserve_shared(int32_t* stack, int32_t* top, int64_t capacity,
                                        int32_t* refcount, int32_t* tables, int32_t max_blocks,
                                        const int32_t* lens, const int32_t* new_tokens,
                                        int32_t batch, int32_t bs, int64_t* slots,
                                        int64_t slot_capacity, int32_t* lens_out,
                                        int32_t* cow_src, int32_t* cow_dst,
                                        int32_t* cow_count, int32_t* status,
                                        hipStream_t stream);
hipError_t launch_blocks_release_shared(int32_t* stack, int32_t* top, int64_t capacity,
                                        int32_t* refcount, const int32_t* tables,
                                        int32_t max_blocks, const int32_t* lens,
                                        const int32_t* mask, int32_t batch, int32_t bs,
                                        int32_t* lens_out, int32_t* status,
                                        hipStream_t stream);
// base / per_block: the six planes of one layer (k_codes, v_codes, k_scale,
// v_scale, k_zero, v_zero) and their bytes per block; NULL planes are skipped.
hipError_t launch_copy_blocks(uint8_t* const base[6], const int64_t per_block[6],
                              const int32_t* src, const int32_t* dst, const int32_t* count,
                              int32_t max_pairs, int64_t num_blocks, hipStream_t stream);

hipError_t launch_blocks_trim(int32_t* stack, int32_t* top, int64_t capacity, int32_t* tables,
                              int32_t max_blocks, const int32_t* lens, int32_t window,
                              int32_t sink, int32_t batch, int32_t bs, int32_t* status,
                              hipStream_t stream);

// pack (pack = true) or unpack the six planes of blocks ids[0 .. n) to / from
// `packed` (block k at k * sum(per_block), planes in order)
hipError_t launch_pack_blocks(uint8_t* const base[6], const int64_t per_block[6],
                              const int32_t* ids, int32_t n, uint8_t* packed, bool pack,
                              int64_t num_blocks, hipStream_t stream);

}  // namespace kvq
