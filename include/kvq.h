/*
 * kvq.h -- C ABI of a quantized paged KV-cache library for AMD Instinct MI355X
 * (gfx950, CDNA4).
 *
 * The library covers the decode-time hot path that the three source pages
 * describe:
 *
 *   kvq_append            quantize freshly computed key/value vectors (fp16 or
 *                         bf16) with scales computed at run time from each
 *                         vector's own range, and scatter the codes into
 *                         fixed-size cache blocks through a slot mapping.
 *                         ("Dynamic KV Cache Quantization for Fast LLM
 *                         Inference", sections "Understanding Dynamic
 *                         Quantization Techniques for KV Caches" and
 *                         "Integrating Dynamic Quantization with PagedAttention";
 *                         "KV Cache Optimization" glossary, "Technical
 *                         Architecture", stages 2 and 3.)
 *   kvq_append_static     the same with scales (and zero points) fixed in
 *                         advance by the caller ("Dynamic KV Cache
 *                         Quantization ...", static versus dynamic scales).
 *   kvq_decode_attention  single-query GQA attention softmax(q.K^T*scale).V of
 *                         every sequence of a batch over its cached blocks,
 *                         dequantizing the codes in registers ("KV Cache
 *                         Optimization" glossary, "Technical Architecture",
 *                         stage 4 "fused dequantization attention kernel";
 *                         "Dynamic KV Cache Quantization ...", section "Recap
 *                         of KV Caching", the append-then-attend loop).
 *   kvq_append_decode_attention
 *                         a decode step's append of one token per sequence
 *                         and its attention in one launch (byte codes with
 *                         per-token scales, 16-bit rows).
 *   kvq_prefill_attention several causal queries per sequence at once
 *                         (prompt chunks, checking several new tokens).
 *   kvq_bytes_per_token   the cache-size closed form ("KV Cache Optimization"
 *                         glossary, "Technical Architecture"; "KV Cache
 *                         Optimization: Strategies for Faster LLM Inference",
 *                         section "What Is KV Cache and Why Does It Balloon
 *                         Memory Usage?").
 *   kvq_pool_init / kvq_blocks_reserve / kvq_blocks_release
 *                         a device-side pool of physical blocks that hands
 *                         blocks to sequences on demand and maps logical to
 *                         physical blocks ("KV Cache Optimization: Strategies
 *                         ...", section "How vLLM Implements KV Cache
 *                         Optimization").
 *   kvq_pack_blocks / kvq_unpack_blocks
 *                         quantized blocks packed for offload to host memory
 *                         and back ("KV Cache Optimization: Strategies ...",
 *                         section "KV Cache Offloading ...").
 *   kvq_blocks_trim       blocks a sliding window no longer reaches go back
 *                         to the pool (section "Cache Eviction ...").
 *   kvq_blocks_fork / kvq_blocks_reserve_shared / kvq_blocks_release_shared /
 *   kvq_copy_blocks       prefix sharing: reference-counted blocks, copy on
 *                         write of a shared, partly filled block (same
 *                         section, prefix caching).
 *   kvq_check_block_tables / kvq_check_slots
 *                         debugging aids: report block ids and slots outside
 *                         the pool through a status word.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Ownership: the caller owns every buffer. Pointers named "device" must be
 *    device memory (hipMalloc or a torch CUDA tensor); all others are host
 *    memory. The library never allocates or frees memory and keeps no state
 *    between calls, so every call is re-entrant.
 *  - Streams: `stream` is a hipStream_t passed as an opaque pointer (NULL is
 *    the null stream). Calls only enqueue work on it and return; results are
 *    visible to later work on the same stream.
 *  - Errors: every argument check happens on the host before any launch; a
 *    failing check returns a negative kvq_status and enqueues nothing.
 *    Conditions only the device can see (pool exhaustion) are written to a
 *    caller-provided device status word. Values that the host cannot check
 *    (block ids, slots, lengths inside device arrays) are preconditions:
 *    breaking one gives unspecified results. Decode and multi-query attention
 *    never read outside the cache planes: a block id outside
 *    [0, num_blocks) is read as block 0 (its positions then count with block
 *    0's data), and no error is reported. kvq_check_block_tables and
 *    kvq_check_slots report such values (a debugging aid, run on the device
 *    with no trap).
 *  - Alignment: every device pointer must be 16-byte aligned and every row
 *    stride must keep rows 16-byte aligned.
 *  - Inputs must be finite.
 *
 * Cache layout (one kvq_cache = one transformer layer; block tables are shared
 * by all layers). H = num_kv_heads, d = head_dim, bs = block_size,
 * NB = num_blocks. A token stored in slot s lives in block s / bs at offset
 * s % bs.
 *  codes      [NB][H][bs][row_bytes], row_bytes = d (INT8, FP8_E4M3),
 *             d / 2 (INT4) or 2 d (NONE16, the raw fp16/bf16 value).
 *             INT8 codes are two's complement in [-127, 127]; FP8 codes are
 *             OCP E4M3 (bias 7, max 448, 0x7F / 0xFF never written).
 *             INT4 codes pack two elements per byte, with the 32-element
 *             slice interleave described at KVQ_CODE_INT4.
 *  TOKEN_SYM scale            float [NB][H][bs]
 *  GROUP_ASYM scale / zero    float / uint8 [NB][H][bs][d / group_size]
 *  CHANNEL_BLOCK_SYM scale    float [NB][H][d]            (keys only)
 *  k_stage (CHANNEL_BLOCK_SYM keys only)  src dtype [max_seqs][H][bs][d]:
 *             raw rows of each sequence's not yet complete last block.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
typedef int32_t kvq_status;
#define KVQ_OK 0
#define KVQ_ERR_INVALID_ARGUMENT (-1)    /* bad pointer, size, enum or shape     */
#define KVQ_ERR_UNSUPPORTED (-2)         /* valid request the library lacks       */
#define KVQ_ERR_WORKSPACE_TOO_SMALL (-3) /* decode workspace below required size */
#define KVQ_ERR_HIP (-4)                 /* a HIP launch or runtime call failed   */
#define KVQ_ERR_OUT_OF_BLOCKS (-5)       /* pool cannot serve a reservation       */

/* ---- enumerations (stored as int32 in the structs below) ---------------- */
/* Floating-point types of inputs and outputs. */
#define KVQ_F16 0
#define KVQ_BF16 1
#define KVQ_F32 2

/* Code types of the cache.
 * KVQ_CODE_NONE16: unquantized; the row is stored as given (fp16 or bf16),
 *   no scale. Lets the same decode run on a 16-bit cache.
 * KVQ_CODE_INT8: signed integer codes q = clamp(rne(x / s), -127, 127) with
 *   s = max|x| / 127 ("Dynamic KV Cache Quantization ...", section
 *   "Understanding Dynamic Quantization Techniques", the absmax scale with
 *   2^(bits-1) - 1 in the denominator).
 * KVQ_CODE_FP8_E4M3: the OCP E4M3 byte nearest x / s, ties to even mantissa,
 *   saturating at +-448, with s = max|x| / 448 (FP8 KV cache named on all
 *   three pages; the pages give no scaling rule, so the absmax rule above is
 *   used with the format's largest finite value).
 * KVQ_CODE_INT4: 4-bit codes, symmetric q in [-7, 7] under TOKEN_SYM (the
 *   same absmax rule with bits = 4) or unsigned q in [0, 15] with a zero point
 *   under GROUP_ASYM. Nibble placement inside a row of d elements, with
 *   n = d / 32: element e = 32 i + 2 r + t (i < n, r < 16, t < 2) sits in
 *   byte n r + i, low nibble when t = 0 and high nibble when t = 1. Signed
 *   codes are stored as q & 0xF. */
#define KVQ_CODE_NONE16 0
#define KVQ_CODE_INT8 1
#define KVQ_CODE_FP8_E4M3 2
#define KVQ_CODE_INT4 3

/* Scale granularity ("Dynamic KV Cache Quantization ...", section
 * "Understanding Dynamic Quantization Techniques": per token or per head;
 * "KV Cache Optimization: Strategies ...", section "KV Cache Quantization:
 * When and How to Compress": per channel keeps more information).
 * KVQ_SCALE_TOKEN_SYM: one fp32 scale per (token, head), zero point 0. An
 *   all-zero row gets codes 0 and scale 1.
 * KVQ_SCALE_GROUP_ASYM: per group of group_size consecutive elements of a
 *   (token, head) row: mn = min(0, min x), mx = max(0, max x),
 *   s = (mx - mn) / 15, z = clamp(rne(-mn / s), 0, 15),
 *   q = clamp(rne(x / s) + z, 0, 15); dequantized value (q - z) s. A group
 *   with mx == mn gets codes 0, s = 1, z = 0. INT4 only.
 * KVQ_SCALE_CHANNEL_BLOCK_SYM: keys only, INT8 only. One fp32 scale per
 *   (block, head, channel) from the absmax of that channel over the block's
 *   bs tokens. Rows of a block that is not yet full wait, raw, in k_stage and
 *   are quantized together when an append writes the block's last slot. */
#define KVQ_SCALE_TOKEN_SYM 0
#define KVQ_SCALE_GROUP_ASYM 1
#define KVQ_SCALE_CHANNEL_BLOCK_SYM 2

/* ---- structs (host memory, passed by pointer) ----------------------------
 * kvq_layout: the static description of one layer's cache.
 *   num_kv_heads  H >= 1
 *   head_dim      d in {64, 128}
 *   block_size    bs in {16, 32}
 *   group_size    32 for GROUP_ASYM, ignored (set 0) otherwise
 *   k_code/v_code KVQ_CODE_*; k_mode/v_mode KVQ_SCALE_*
 *   src_dtype     KVQ_F16 or KVQ_BF16: the type of rows given to kvq_append
 *                 and of the NONE16 cache and the k_stage plane
 *   reserved      must be 0 */
typedef struct kvq_layout {
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t group_size;
  int32_t k_code;
  int32_t v_code;
  int32_t k_mode;
  int32_t v_mode;
  int32_t src_dtype;
  int32_t reserved;
} kvq_layout;

/* kvq_cache: device planes of one layer (see the layout comment at the top).
 * Pointers a layout does not use must be NULL. */
typedef struct kvq_cache {
  void* k_codes;
  void* v_codes;
  float* k_scale;
  float* v_scale;
  uint8_t* k_zero;
  uint8_t* v_zero;
  void* k_stage;
  int64_t num_blocks; /* NB, physical blocks in every plane */
  int32_t max_seqs;   /* rows of k_stage (0 when k_stage is unused) */
  int32_t reserved;   /* must be 0 */
} kvq_cache;

/* ---- entry points -------------------------------------------------------- */

/* Human-readable name of a status code (static storage, never NULL). */
const char* kvq_status_string(kvq_status status);

/* Checks a layout without touching the device: KVQ_OK, or
 * KVQ_ERR_INVALID_ARGUMENT for malformed fields, or KVQ_ERR_UNSUPPORTED for a
 * well-formed combination the library does not implement. */
kvq_status kvq_layout_check(const kvq_layout* layout);

/* Cache bytes per token over num_layers layers ("KV Cache Optimization"
 * glossary, "Technical Architecture": keys and values, times layers, KV heads,
 * head dimension and bytes per element; for 80 layers, 8 KV heads and d = 128
 * this is 327 680 B at 16 bit, 163 840 B at 8 bit and 81 920 B at 4 bit).
 * include_metadata = 0 counts codes only: 2 * num_layers * H * d * bits / 8
 * summed over K and V with their own code widths. include_metadata = 1 adds,
 * per layer and side, H * 4 (TOKEN_SYM scale), H * (d / group_size) * 5
 * (GROUP_ASYM scale and zero point) or ceil(H * d * 4 / bs) (CHANNEL_BLOCK
 * scales amortized over a block). Returns the byte count, or a negative
 * kvq_status for a bad layout or num_layers < 1. Host arithmetic only. */
int64_t kvq_bytes_per_token(const kvq_layout* layout, int32_t num_layers,
                            int32_t include_metadata);

/* Size in bytes of every plane of one layer's cache, in the order k_codes,
 * v_codes, k_scale, v_scale, k_zero, v_zero, k_stage (0 for planes the layout
 * does not use). out_bytes is a host array of 7 int64. Host only. */
kvq_status kvq_cache_plane_bytes(const kvq_layout* layout, int64_t num_blocks,
                                 int32_t max_seqs, int64_t out_bytes[7]);

/* Quantize num_tokens new K and V rows and write them to their slots.
 *  k, v          device, src_dtype; token t, head h, element e at
 *                k[t * k_row_stride + h * d + e] (strides in elements; the H*d
 *                elements of one token are contiguous).
 *  slot_mapping  device int64[num_tokens]; slot of token t, or -1 to skip it.
 *  stage_rows    device int32[num_tokens] when either side is
 *                CHANNEL_BLOCK_SYM, else NULL: the k_stage row (the decode
 *                batch row) of token t's sequence.
 * Scales are computed in fp32 with correctly rounded division and codes with
 * round-half-to-even, so the stored bytes are a pure function of the input.
 * Preconditions: slots are distinct and inside the cache; for
 * CHANNEL_BLOCK_SYM keys, the tokens of one sequence appear in the call
 * contiguously and in position order, and each sequence's blocks fill from
 * offset 0 upward across calls. Returns KVQ_OK after enqueueing. */
kvq_status kvq_append(const kvq_layout* layout, const kvq_cache* cache,
                      const void* k, const void* v, int64_t k_row_stride,
                      int64_t v_row_stride, int64_t num_tokens,
                      const int64_t* slot_mapping, const int32_t* stage_rows,
                      void* stream);

/* kvq_append with static scales: the scale (and zero point) of each code is
 * given by the caller, fixed in advance, instead of being computed from each
 * new vector's range ("Dynamic KV Cache Quantization for Fast LLM Inference",
 * opening section and section "Understanding Dynamic Quantization Techniques
 * for KV Caches", the static scheme that dynamic quantization is set against).
 *  k_scales, v_scales  device float: TOKEN_SYM [H], one per KV head;
 *                GROUP_ASYM [H][d / group_size], one per head and group;
 *                CHANNEL_BLOCK_SYM keys [H][d], one per head and channel
 *                (16-byte aligned). Positive and finite. NULL exactly for a
 *                NONE16 side.
 *  k_zeros, v_zeros    device uint8 [H][d / group_size] zero points in
 *                [0, 15] for a GROUP_ASYM side; NULL otherwise.
 * The other arguments are those of kvq_append, stage_rows included. Codes are
 * rne(x / s), or rne(x / s) + z, with x / s in fp32 and correctly rounded,
 * then saturated at the code range: [-127, 127] (INT8), [-7, 7] (INT4
 * symmetric), +-448 (E4M3), [0, 15] (INT4 asymmetric, the quotient clipped to
 * [-15, 15] first). Each token's metadata entries receive the given values,
 * so the cache reads back through kvq_decode_attention unchanged. Per-channel
 * keys are coded at once (the scale is known, so rows need not wait for their
 * block); a block's scale row is written with its offset-0 slot, and the
 * rows of each sequence's not yet complete last block still go, raw, to its
 * stage row, where decode reads them.
 * Scale and zero arrays other than per-channel ones need only their element
 * alignment.
 * Errors: KVQ_ERR_INVALID_ARGUMENT if a pointer is NULL where one is required
 * or given where none is, or for kvq_append's argument errors. */
kvq_status kvq_append_static(const kvq_layout* layout, const kvq_cache* cache,
                             const void* k, const void* v, int64_t k_row_stride,
                             int64_t v_row_stride, int64_t num_tokens,
                             const int64_t* slot_mapping, const int32_t* stage_rows,
                             const float* k_scales, const uint8_t* k_zeros,
                             const float* v_scales, const uint8_t* v_zeros,
                             void* stream);

/* Device workspace bytes kvq_decode_attention needs for these sizes and this
 * split_blocks (1..256, or 0 = the library's own choice), or a negative
 * kvq_status. */
int64_t kvq_decode_workspace_bytes(const kvq_layout* layout, int32_t batch,
                                   int32_t num_q_heads, int32_t max_context_len,
                                   int32_t split_blocks);

/* Single-query decode attention over the paged cache.
 *  q              device [batch][num_q_heads][d] in q_dtype (F16 or BF16).
 *  block_tables   device int32 [batch][max_blocks_per_seq]: physical block of
 *                 each logical block of each sequence.
 *  context_lens   device int32 [batch]: cached tokens each sequence attends
 *                 over, 0 <= len <= max_context_len <= max_blocks_per_seq*bs.
 *  max_context_len host bound on context_lens, sizes the launch.
 *  sm_scale       score scale; 0 means 1/sqrt(d).
 *  split_blocks   cache blocks per split-K chunk, 1..256; 0 lets the library
 *                 choose.
 *  out            device [batch][num_q_heads][d] in out_dtype (F32, F16 or
 *                 BF16), RNE-rounded from fp32.
 *  workspace      device, at least kvq_decode_workspace_bytes(...) bytes.
 * Query head h reads KV head h / (num_q_heads / H). out = sum_t p_t v_t /
 * sum_t p_t with p_t = exp(s_t - max s), s_t = (q . k_t) * sm_scale, over the
 * first context_lens[b] tokens; a sequence with no tokens gets out = 0.
 * Keys and values are dequantized as the scale mode defines; under
 * CHANNEL_BLOCK_SYM the partial last block is read raw from k_stage row b;
 * a NONE16 cache is read as stored.
 * The result depends on physical block ids only through the data they hold.
 * Supported: both sides INT8, E4M3 or INT4 under TOKEN_SYM, both INT4 under
 * GROUP_ASYM, INT8 CHANNEL_BLOCK_SYM keys with INT8 TOKEN_SYM values, and
 * both NONE16; other layouts return KVQ_ERR_UNSUPPORTED.
 * Preconditions: num_q_heads is a multiple of H and num_q_heads / H <= 16;
 * dequantized values v satisfy |v| / 127 < 65504 (fp16 range of the folded
 * value scale). Rows read raw (NONE16, staged rows) enter the matrix
 * instructions in their own 16-bit format, so bf16 rows keep bf16's range;
 * only sums past fp32's range overflow. */
kvq_status kvq_decode_attention(const kvq_layout* layout, const kvq_cache* cache,
                                const void* q, int32_t q_dtype, int32_t batch,
                                int32_t num_q_heads, const int32_t* block_tables,
                                int32_t max_blocks_per_seq,
                                const int32_t* context_lens,
                                int32_t max_context_len, float sm_scale,
                                int32_t split_blocks, void* out,
                                int32_t out_dtype, void* workspace,
                                int64_t workspace_bytes, void* stream);

/* kvq_append followed by kvq_decode_attention in one launch, for a decode
 * step's one new token per sequence ("Dynamic KV Cache Quantization for Fast
 * LLM Inference", section "Integrating Dynamic Quantization with
 * PagedAttention": the new key and value are quantized as they enter their
 * block, and the step's attention reads them from there).
 *  k, v          device, src_dtype; the new row of sequence b, KV head h,
 *                element e at k[b * k_row_stride + h * d + e] (strides in
 *                elements, 16-byte aligned rows as for kvq_append).
 * Row b is coded into position context_lens[b] - 1 of sequence b, the slot
 * block_tables[b][(len - 1) / bs] * bs + (len - 1) % bs that
 * kvq_blocks_reserve handed out for it, with kvq_append's arithmetic (same
 * bytes); the decode then attends over all context_lens[b] tokens, the new
 * one included. The other arguments, the result and the workspace are those
 * of kvq_decode_attention. A sequence with no tokens takes no row, nor does
 * one whose length exceeds max_context_len (a broken precondition: the row
 * would land on a cached token); a table entry outside the pool receives
 * nothing (the decode reads block 0 there).
 * Supported: both sides INT8 or E4M3 under TOKEN_SYM, and both NONE16; other
 * layouts return KVQ_ERR_UNSUPPORTED (use kvq_append, then decode).
 * Errors: those of kvq_decode_attention, and KVQ_ERR_INVALID_ARGUMENT for a
 * missing or misaligned k or v, a row stride below H * d or not a multiple of
 * 8 elements, or max_context_len < 1 with batch > 0. */
kvq_status kvq_append_decode_attention(const kvq_layout* layout, const kvq_cache* cache,
                                       const void* k, const void* v, int64_t k_row_stride,
                                       int64_t v_row_stride, const void* q, int32_t q_dtype,
                                       int32_t batch, int32_t num_q_heads,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len,
                                       float sm_scale, int32_t split_blocks, void* out,
                                       int32_t out_dtype, void* workspace,
                                       int64_t workspace_bytes, void* stream);

/* kvq_decode_attention for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It takes no workspace: the partials go to a fixed array the
 * library holds in each GPU's memory (KVQ_DECODE_SCRATCH_BYTES per GPU, kept
 * until the process ends, its address looked up once per device on the first
 * call). The call allocates nothing: no hipMalloc, no hipFree, no allocating
 * library routine.
 *  Arguments, results and errors are those of kvq_decode_attention, minus
 *  workspace and workspace_bytes. The stream must belong to the current
 *  device. A call whose kvq_decode_workspace_bytes(...) exceeds
 *  KVQ_DECODE_SCRATCH_BYTES returns KVQ_ERR_WORKSPACE_TOO_SMALL before
 *  touching the device; KVQ_ERR_HIP if the array's address cannot be had.
 *  Every call on one GPU shares that GPU's array: calls that may overlap on
 *  one GPU (different streams, or threads) race and must be serialized by
 *  the caller. Nothing in the array needs to start at any value. */
#define KVQ_DECODE_SCRATCH_BYTES 134217728 /* 128 MiB */
kvq_status kvq_decode_attention_noalloc(const kvq_layout* layout, const kvq_cache* cache,
                                        const void* q, int32_t q_dtype, int32_t batch,
                                        int32_t num_q_heads, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq,
                                        const int32_t* context_lens,
                                        int32_t max_context_len, float sm_scale,
                                        int32_t split_blocks, void* out, int32_t out_dtype,
                                        void* stream);

/* Device workspace bytes kvq_prefill_attention needs for these sizes and this
 * split_blocks (1..256, or 0 = the library's own choice), or a negative
 * kvq_status. */
int64_t kvq_prefill_workspace_bytes(const kvq_layout* layout, int32_t batch,
                                    int32_t num_q_heads, int32_t max_query_len,
                                    int32_t max_context_len, int32_t split_blocks);

/* Multi-query (prefill) attention over the paged cache: several query
 * tokens per sequence at once, causally, as when a prompt chunk is processed
 * or several new tokens are checked together ("KV Cache Optimization:
 * Strategies for Faster LLM Inference", sections "Why KV Cache Is Essential
 * for Efficient LLM Inference" and "Implementing KV Cache Optimization: A
 * Practical Checklist", prefill versus decode).
 *  q              device [Tq][num_q_heads][d] in q_dtype (F16 or BF16),
 *                 Tq = query_start[batch].
 *  query_start    device int32 [batch + 1], non-decreasing, query_start[0] =
 *                 0: sequence b's queries are rows query_start[b] ..
 *                 query_start[b + 1] - 1, nq_b of them, and they are its last
 *                 nq_b cached positions (their keys and values already
 *                 appended): query i sits at position context_lens[b] - nq_b
 *                 + i and attends to positions 0 .. that position.
 *  max_query_len  host bound on every nq_b (sizes the launch).
 *  window, sink   sliding-window attention with attention sinks ("KV Cache
 *                 Optimization: Strategies ...", section "Cache Eviction and
 *                 Compression Strategies"): with window > 0 the query at
 *                 position p sees only positions t <= p with
 *                 t >= p + 1 - window or t < sink; window = 0 (sink
 *                 ignored) is full causal attention. Positions no query
 *                 sees are never read, so their table entries may be -1
 *                 (kvq_blocks_trim).
 *  split_blocks   cache blocks per split-K chunk, 1..256; 0 lets the library
 *                 choose.
 *  out            device [Tq][num_q_heads][d] in out_dtype.
 * The other arguments are those of kvq_decode_attention; nq_b = 1 computes
 * the same function as decode. Under CHANNEL_BLOCK_SYM the positions of the
 * partial last block (decided by context_lens[b]) are read raw from k_stage
 * row b. Supported: both sides INT8, E4M3 or INT4 under TOKEN_SYM, both INT4
 * under GROUP_ASYM, INT8 CHANNEL_BLOCK_SYM keys with INT8 TOKEN_SYM values,
 * and both NONE16 (the layouts decode supports); other layouts return
 * KVQ_ERR_UNSUPPORTED. Preconditions: nq_b <= context_lens[b]
 * <= max_context_len; the value-range preconditions of decode. */
kvq_status kvq_prefill_attention(const kvq_layout* layout, const kvq_cache* cache,
                                 const void* q, int32_t q_dtype, int32_t batch,
                                 int32_t num_q_heads, const int32_t* query_start,
                                 int32_t max_query_len, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t max_context_len, float sm_scale, int32_t window,
                                 int32_t sink, int32_t split_blocks, void* out,
                                 int32_t out_dtype, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/* Fill a pool: free_stack[i] = initial_order[i] (or i when initial_order is
 * NULL) for i < num_blocks, and *free_top = num_blocks. free_stack, free_top
 * and initial_order are device memory; initial_order must be a permutation of
 * [0, num_blocks). */
kvq_status kvq_pool_init(int32_t* free_stack, int32_t* free_top,
                         const int32_t* initial_order, int64_t num_blocks,
                         void* stream);

/* Give each sequence b the blocks it needs to grow from context_lens[b] to
 * context_lens[b] + new_tokens[b] tokens ("KV Cache Optimization: Strategies
 * ...", section "How vLLM Implements KV Cache Optimization": blocks are
 * handed out on demand rather than reserved for the worst case).
 *  need_b = ceil((L_b + n_b) / bs) - ceil(L_b / bs); off_b is the exclusive
 *  prefix sum of need in batch order; with top = *free_top, sequence b takes
 *  free_stack[top - off_b - need_b + k], k = 0..need_b-1, as logical blocks
 *  ceil(L_b / bs) + k of block_tables[b]; *free_top drops by sum(need).
 *  slot_mapping_out[o_b + k] (o_b = exclusive prefix sum of new_tokens) gets
 *  the slot of position L_b + k, k < n_b. context_lens_out (may be NULL or
 *  alias context_lens) gets L_b + n_b.
 * All or nothing: if sum(new_tokens) > slot_capacity (the entries of
 * slot_mapping_out), nothing is written except *status_flag =
 * KVQ_ERR_INVALID_ARGUMENT; else if sum(need) > top, or a sequence would
 * exceed max_blocks_per_seq blocks, nothing is written except *status_flag =
 * KVQ_ERR_OUT_OF_BLOCKS; on success *status_flag = KVQ_OK. The token count
 * is checked on the device, so the call reads nothing back to the host.
 * All pointers are device memory; pool_capacity is the length of
 * free_stack. A negative slot_capacity is KVQ_ERR_INVALID_ARGUMENT. */
kvq_status kvq_blocks_reserve(int32_t* free_stack, int32_t* free_top,
                              int64_t pool_capacity, int32_t* block_tables,
                              int32_t max_blocks_per_seq,
                              const int32_t* context_lens,
                              const int32_t* new_tokens, int32_t batch,
                              int32_t block_size, int64_t* slot_mapping_out,
                              int64_t slot_capacity, int32_t* context_lens_out,
                              int32_t* status_flag, void* stream);

/* Return the blocks of every sequence b with release_mask[b] != 0 to the
 * pool: its ceil(context_lens[b] / bs) blocks are pushed in batch order and,
 * within a sequence, in logical order: free_stack[top + roff_b + k] =
 * block_tables[b][k]. context_lens_out (may be NULL or alias context_lens)
 * gets 0 for released rows. If the pushes would exceed pool_capacity, nothing
 * changes and *status_flag = KVQ_ERR_OUT_OF_BLOCKS; else KVQ_OK. All pointers
 * are device memory. */
kvq_status kvq_blocks_release(int32_t* free_stack, int32_t* free_top,
                              int64_t pool_capacity,
                              const int32_t* block_tables,
                              int32_t max_blocks_per_seq,
                              const int32_t* context_lens,
                              const int32_t* release_mask, int32_t batch,
                              int32_t block_size, int32_t* context_lens_out,
                              int32_t* status_flag, void* stream);

/* ---- prefix sharing ("KV Cache Optimization: Strategies ...", section "How
 * vLLM Implements KV Cache Optimization": requests that share a system prompt
 * keep one cached copy of its prefix; "KV Cache Optimization" glossary,
 * "Evolution & History" and "Enterprise Use Cases": common prompt prefixes
 * reused across requests). A pool used with these calls also keeps
 * refcount, a device int32 [pool_capacity]: the number of table entries
 * holding each block, 0 for a free block (all zero after kvq_pool_init; the
 * caller zero-fills it). Use the _shared reserve and release with such a
 * pool; the plain ones do not keep the counts. */

/* Block recycling under a sliding window ("KV Cache Optimization:
 * Strategies ...", section "Cache Eviction and Compression Strategies": only
 * the recent tokens, and the sinks, are kept). Queries from position
 * L = context_lens[b] on see only t >= L + 1 - window and t < sink, so the
 * blocks i of sequence b with ceil(sink / bs) <= i and (i + 1) bs <=
 * L + 1 - window that are still in its table are pushed onto the stack
 * (batch order, logical order) and their entries set to -1. window = 0 trims
 * nothing. For the plain pool (no counts); a trimmed table is for windowed
 * kvq_prefill_attention only (decode reads every block). All or nothing if
 * the pushes would overflow the stack (*status_flag = KVQ_ERR_OUT_OF_BLOCKS).
 * All pointers are device memory. */
kvq_status kvq_blocks_trim(int32_t* free_stack, int32_t* free_top, int64_t pool_capacity,
                           int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t window, int32_t sink,
                           int32_t batch, int32_t block_size, int32_t* status_flag,
                           void* stream);

/* Debugging aids for the block map the attention calls read ("Dynamic KV
 * Cache Quantization for Fast LLM Inference", section "Integrating Dynamic
 * Quantization with PagedAttention": a table maps each sequence's logical
 * blocks to physical ones). Block ids and slots live in device arrays that
 * the host does not read; these calls check them on the device, with no
 * trap, and report through device words.
 *
 * kvq_check_block_tables: every entry block_tables[b][k] with
 * k < ceil(context_lens[b] / bs) must lie in [0, num_blocks), and every
 * context_lens[b] in [0, max_blocks_per_seq * bs]. *first_bad (device int64)
 * gets the smallest flat index b * max_blocks_per_seq + k of an entry that
 * breaks this (a length outside its range counts at k = 0), or -1;
 * *status_flag (device int32) gets KVQ_ERR_INVALID_ARGUMENT or KVQ_OK. One
 * workgroup, so the answer does not depend on timing; intended for debug
 * builds of a serving loop (it reads the whole table). */
kvq_status kvq_check_block_tables(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t batch,
                                  int32_t block_size, int64_t num_blocks, int64_t* first_bad,
                                  int32_t* status_flag, void* stream);

/* kvq_check_slots: every slot_mapping[t], t < num_tokens, must be -1 (skip)
 * or lie in [0, num_blocks * block_size). Reports as kvq_check_block_tables
 * (first_bad = the smallest bad t, or -1). */
kvq_status kvq_check_slots(const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                           int32_t block_size, int64_t* first_bad, int32_t* status_flag,
                           void* stream);

/* Fork k (k < num_forks): row dst_rows[k] takes row src_rows[k]'s length and
 * its first ceil(len / bs) table entries, each block gaining one reference.
 * Destination rows must be empty (length 0), distinct, and not sources of
 * the same call. With CHANNEL_BLOCK_SYM keys the destination's k_stage row
 * must also be given the source's (a plain device copy), since a partly
 * filled last block lives there. All pointers are device memory. */
kvq_status kvq_blocks_fork(int32_t* refcount, int64_t pool_capacity,
                           int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t* context_lens, int32_t batch,
                           const int32_t* src_rows, const int32_t* dst_rows,
                           int32_t num_forks, int32_t block_size, void* stream);

/* kvq_blocks_reserve for a pool with counts, with copy on write: a sequence
 * that appends (n_b > 0) into a partly filled last block (L_b % bs != 0)
 * held by more than one table (count > 1 at the start of the call) first
 * takes one extra block, the lowest of its stack positions, which replaces
 * that table entry; the pair (old, new) goes to cow_src[c], cow_dst[c]
 * (c in batch order, *cow_count pairs; arrays of at least batch entries) and
 * the caller must copy each pair's contents in every layer
 * (kvq_copy_blocks) before appending. need_b counts the extra block; taken
 * blocks get count 1; after the allocation each copied block loses one
 * reference and one left at zero is pushed onto the stack (in the order of
 * its last copy). Otherwise as kvq_blocks_reserve, all or nothing. */
kvq_status kvq_blocks_reserve_shared(int32_t* free_stack, int32_t* free_top,
                                     int64_t pool_capacity, int32_t* refcount,
                                     int32_t* block_tables,
                                     int32_t max_blocks_per_seq,
                                     const int32_t* context_lens,
                                     const int32_t* new_tokens, int32_t batch,
                                     int32_t block_size, int64_t* slot_mapping_out,
                                     int64_t slot_capacity, int32_t* context_lens_out,
                                     int32_t* cow_src, int32_t* cow_dst,
                                     int32_t* cow_count, int32_t* status_flag,
                                     void* stream);

/* kvq_blocks_release for a pool with counts: every table entry of a masked
 * row drops one reference (rows in batch order, entries in logical order)
 * and a block left at zero is pushed onto the stack in the order of its
 * last entry. */
kvq_status kvq_blocks_release_shared(int32_t* free_stack, int32_t* free_top,
                                     int64_t pool_capacity, int32_t* refcount,
                                     const int32_t* block_tables,
                                     int32_t max_blocks_per_seq,
                                     const int32_t* context_lens,
                                     const int32_t* release_mask, int32_t batch,
                                     int32_t block_size, int32_t* context_lens_out,
                                     int32_t* status_flag, void* stream);

/* Copy every plane of block src_ids[k] onto block dst_ids[k] in one layer's
 * cache (codes, scales, zero points; not k_stage), for k < *count (device
 * int32, at most max_pairs): the copy-on-write pairs of
 * kvq_blocks_reserve_shared. Ids outside [0, num_blocks) are skipped. */
kvq_status kvq_copy_blocks(const kvq_layout* layout, const kvq_cache* cache,
                           const int32_t* src_ids, const int32_t* dst_ids,
                           const int32_t* count, int32_t max_pairs, void* stream);

/* ---- block offload ("KV Cache Optimization: Strategies ...", section "KV
 * Cache Offloading: Moving Data Between GPU and CPU": inactive cache moves to
 * CPU memory and back, bounded by the link; quantized blocks cross it in 2-4x
 * fewer bytes than 16-bit ones). A packed block is the block's slice of every
 * plane of one layer, in the order k_codes, v_codes, k_scale, v_scale,
 * k_zero, v_zero (absent planes take no bytes; k_stage is not part of it);
 * block k of a pack starts at k * kvq_block_pack_bytes(layout). The pack
 * lives in device memory, or in host memory the device can address
 * (hipHostMalloc); the caller moves it across the link (hipMemcpyAsync). */

/* Bytes of one packed block of this layout = kvq_bytes_per_token(layout, 1, 1)
 * * block_size (per-channel key scales are per block), or a negative
 * kvq_status. Host only. */
int64_t kvq_block_pack_bytes(const kvq_layout* layout);

/* Pack blocks ids[0 .. n) (device int32) of one layer into dst, 16-byte
 * aligned, n * kvq_block_pack_bytes bytes. Ids outside [0, num_blocks) are
 * skipped (their slot in dst is left as it was). */
kvq_status kvq_pack_blocks(const kvq_layout* layout, const kvq_cache* cache,
                           const int32_t* ids, int32_t n, void* dst, void* stream);

/* The inverse: write packed block k of src into block ids[k] of one layer. */
kvq_status kvq_unpack_blocks(const kvq_layout* layout, const kvq_cache* cache,
                             const void* src, const int32_t* ids, int32_t n,
                             void* stream);

/* ---- measurement aid -------------------------------------------------- */
/* Decode is bound by the memory stream ("KV Cache Optimization: Strategies
 * for Faster LLM Inference", "Implementing KV Cache Optimization: A Practical
 * Checklist": decode is memory-bound), so its rate is judged against what a
 * kernel that only reads can reach on the device. kvq_read_probe reads
 * `bytes` bytes of device memory at buf (16-byte aligned, a multiple of 16)
 * once, with 16-byte non-temporal loads, each workgroup of up to 2048
 * streaming one contiguous chunk, and
 * stores nothing except, in the practically impossible case that the XOR of
 * everything it read equals 0x9E3779B9, that value to sink[0] (device
 * uint32). The launch's duration (events on `stream`) gives the read rate.
 * Errors: KVQ_ERR_INVALID_ARGUMENT for a NULL pointer, misalignment or a size
 * that is not a positive multiple of 16. */
kvq_status kvq_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* KVQ_H_ */
