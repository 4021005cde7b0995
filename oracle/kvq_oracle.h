/*
 * kvq_oracle.h -- plain, slow, scalar CPU oracle for quantized paged KV append
 * and decode attention.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load or call this code. It shares no code,
 * header or constant generator with the GPU library: the enumerations below
 * carry the same numbers as the library's public header because both follow
 * the same written layout, and a test checks that the two agree.
 *
 * Arithmetic: codecs run in IEEE binary32 with true division and rintf
 * (round half to even) under the default rounding mode, built with
 * -ffp-contract=off and without -ffast-math; attention runs in binary64 from
 * the binary32 dequantized values.
 */
#ifndef KVQ_ORACLE_H_
#define KVQ_ORACLE_H_

#include <stdint.h>

#define ORC_OK 0
#define ORC_ERR_INVALID (-1)
#define ORC_ERR_UNSUPPORTED (-2)
#define ORC_ERR_OUT_OF_BLOCKS (-5)

#define ORC_F16 0
#define ORC_BF16 1
#define ORC_F32 2

#define ORC_CODE_NONE16 0
#define ORC_CODE_INT8 1
#define ORC_CODE_FP8 2
#define ORC_CODE_INT4 3

#define ORC_TOKEN_SYM 0
#define ORC_GROUP_ASYM 1
#define ORC_CHANNEL_BLOCK 2

typedef struct {
  int32_t num_kv_heads, head_dim, block_size, group_size;
  int32_t k_code, v_code, k_mode, v_mode, src_dtype, reserved;
} orc_layout;

/* Host copies of one layer's planes, same shapes as the library's cache. */
typedef struct {
  void* k_codes;
  void* v_codes;
  float* k_scale;
  float* v_scale;
  uint8_t* k_zero;
  uint8_t* v_zero;
  void* k_stage;
  int64_t num_blocks;
  int32_t max_seqs, reserved;
} orc_cache;

/* number formats */
float orc_f16_to_f32(uint16_t h);
float orc_bf16_to_f32(uint16_t h);
float orc_e4m3_value(uint8_t c);
uint8_t orc_e4m3_encode(float y);

/* row codecs (x already in fp32) */
void orc_quant_sym(const float* x, int n, int qmax, int8_t* q, float* s);
void orc_quant_fp8(const float* x, int n, uint8_t* q, float* s);
void orc_quant_asym4(const float* x, int n, uint8_t* q, float* s, uint8_t* z);
void orc_quant_channel_block(const float* x, int bs, int d, int8_t* q, float* s);
void orc_quant_sym_static(const float* x, int n, int qmax, float s, int8_t* q);
void orc_quant_fp8_static(const float* x, int n, float s, uint8_t* q);
void orc_quant_asym4_static(const float* x, int n, float s, uint8_t z, uint8_t* q);
void orc_int4_pack(const uint8_t* nib, int d, uint8_t* out);
void orc_int4_unpack(const uint8_t* in, int d, uint8_t* nib);

/* sizes */
int64_t orc_bytes_per_token(const orc_layout* L, int32_t num_layers,
                            int32_t include_metadata);
int orc_plane_bytes(const orc_layout* L, int64_t num_blocks, int32_t max_seqs,
                    int64_t out[7]);

/* the two steps of the hot path */
int orc_append(const orc_layout* L, const orc_cache* C, const void* k,
               const void* v, int64_t k_row_stride, int64_t v_row_stride,
               int64_t num_tokens, const int64_t* slot_mapping,
               const int32_t* stage_rows);
int orc_append_static(const orc_layout* L, const orc_cache* C, const void* k,
                      const void* v, int64_t k_row_stride, int64_t v_row_stride,
                      int64_t num_tokens, const int64_t* slot_mapping,
                      const int32_t* stage_rows, const float* k_scale,
                      const uint8_t* k_zero, const float* v_scale,
                      const uint8_t* v_zero);
int orc_prefill(const orc_layout* L, const orc_cache* C, const void* q, int32_t q_dtype,
                int32_t batch, int32_t num_q_heads, const int32_t* query_start,
                const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, int32_t window, int32_t sink,
                double sm_scale, double* out, int32_t num_threads);
int orc_blocks_trim(int32_t* stack, int32_t* top, int64_t capacity, int32_t* tables,
                    int32_t max_blocks, const int32_t* lens, int32_t window, int32_t sink,
                    int32_t batch, int32_t bs, int32_t* status);
int orc_blocks_fork(int32_t* refcount, int32_t* tables, int32_t max_blocks,
                    int32_t* lens, const int32_t* src, const int32_t* dst,
                    int32_t num_forks, int32_t bs);
int orc_blocks_reserve_shared(int32_t* stack, int32_t* top, int64_t capacity,
                              int32_t* refcount, int32_t* tables, int32_t max_blocks,
                              const int32_t* lens, const int32_t* new_tokens,
                              int32_t batch, int32_t bs, int64_t* slots,
                              int32_t* lens_out, int32_t* cow_src, int32_t* cow_dst,
                              int32_t* cow_count, int32_t* status);
int orc_blocks_release_shared(int32_t* stack, int32_t* top, int64_t capacity,
                              int32_t* refcount, const int32_t* tables,
                              int32_t max_blocks, const int32_t* lens,
                              const int32_t* mask, int32_t batch, int32_t bs,
                              int32_t* lens_out, int32_t* status);
int orc_copy_blocks(const orc_layout* L, const orc_cache* C, const int32_t* src,
                    const int32_t* dst, int32_t n);
int64_t orc_block_pack_bytes(const orc_layout* L);
int orc_pack_blocks(const orc_layout* L, const orc_cache* C, const int32_t* ids, int32_t n,
                    uint8_t* dst);
int orc_unpack_blocks(const orc_layout* L, const orc_cache* C, const uint8_t* src,
                      const int32_t* ids, int32_t n);
int orc_dequant_token(const orc_layout* L, const orc_cache* C, int side,
                      const int32_t* table_row, int32_t context_len,
                      int32_t stage_row, int32_t pos, int32_t head, float* out);
int orc_decode(const orc_layout* L, const orc_cache* C, const void* q,
               int32_t q_dtype, int32_t batch, int32_t num_q_heads,
               const int32_t* block_tables, int32_t max_blocks_per_seq,
               const int32_t* context_lens, double sm_scale, double* out,
               int32_t num_threads);
int orc_decode_range(const orc_layout* L, const orc_cache* C, const void* q,
                     int32_t q_dtype, int32_t num_q_heads, int32_t b,
                     int32_t h, const int32_t* table_row, int32_t context_len,
                     int32_t t_begin, int32_t t_end, double sm_scale,
                     double* m, double* l, double* acc);

/* the block pool */
int orc_pool_init(int32_t* stack, int32_t* top, const int32_t* order,
                  int64_t n);
int orc_blocks_reserve(int32_t* stack, int32_t* top, int64_t capacity,
                       int32_t* tables, int32_t max_blocks,
                       const int32_t* lens, const int32_t* new_tokens,
                       int32_t batch, int32_t bs, int64_t* slots,
                       int32_t* lens_out, int32_t* status);
int orc_blocks_release(int32_t* stack, int32_t* top, int64_t capacity,
                       const int32_t* tables, int32_t max_blocks,
                       const int32_t* lens, const int32_t* mask, int32_t batch,
                       int32_t bs, int32_t* lens_out, int32_t* status);

#endif /* KVQ_ORACLE_H_ */
