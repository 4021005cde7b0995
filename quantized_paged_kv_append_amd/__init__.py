"""Quantized paged KV-cache append and fused-dequantization decode attention
for AMD Instinct MI355X (gfx950).

The work happens in libkvq.so (hand-written HIP kernels behind the C ABI of
include/kvq.h); `kvq` is its ctypes binding. Importing this package fails
loudly when the library has not been built.
"""
from .kvq import (  # noqa: F401
    KVQ_DECODE_SCRATCH_BYTES, KvqError, PagedCache, kvq_append, kvq_append_static,
    kvq_blocks_fork, kvq_blocks_release,
    kvq_block_pack_bytes, kvq_blocks_release_shared, kvq_blocks_reserve_shared, kvq_blocks_trim,
    kvq_copy_blocks, kvq_pack_blocks, kvq_unpack_blocks, kvq_blocks_reserve,
    kvq_bytes_per_token, kvq_cache_plane_bytes, kvq_check_block_tables, kvq_check_slots,
    kvq_decode_attention,
    kvq_append_decode_attention,
    kvq_decode_attention_noalloc,
    kvq_decode_workspace_bytes, kvq_layout_check, kvq_pool_init, kvq_prefill_attention,
    kvq_prefill_workspace_bytes, kvq_read_probe,
    kvq_status_string, make_layout)
