"""Thin ctypes binding of libkvq.so (the C ABI in include/kvq.h).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels. torch supplies device memory (tensors) and the current stream.
The functions keep the C names; they take torch tensors and raise KvqError on
a non-zero status.
"""
import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libkvq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: the HIP library has not been built. Build it "
        "with `python -c 'import __graft_entry__ as g; g.build()'` (or "
        "`python quantized_paged_kv_append_amd/_build.py`) from the repository root.")

_lib = C.CDLL(LIB_PATH)

# ---- numbers from include/kvq.h (a test checks that they agree) ------------
KVQ_OK = 0
KVQ_ERR_INVALID_ARGUMENT = -1
KVQ_ERR_UNSUPPORTED = -2
KVQ_ERR_WORKSPACE_TOO_SMALL = -3
KVQ_ERR_HIP = -4
KVQ_ERR_OUT_OF_BLOCKS = -5

KVQ_F16, KVQ_BF16, KVQ_F32 = 0, 1, 2
KVQ_CODE_NONE16, KVQ_CODE_INT8, KVQ_CODE_FP8_E4M3, KVQ_CODE_INT4 = 0, 1, 2, 3
KVQ_SCALE_TOKEN_SYM, KVQ_SCALE_GROUP_ASYM, KVQ_SCALE_CHANNEL_BLOCK_SYM = 0, 1, 2

CODES = {"none16": KVQ_CODE_NONE16, "int8": KVQ_CODE_INT8, "fp8": KVQ_CODE_FP8_E4M3,
         "int4": KVQ_CODE_INT4}
MODES = {"token_sym": KVQ_SCALE_TOKEN_SYM, "group_asym": KVQ_SCALE_GROUP_ASYM,
         "channel_block": KVQ_SCALE_CHANNEL_BLOCK_SYM}
DTYPES = {torch.float16: KVQ_F16, torch.bfloat16: KVQ_BF16, torch.float32: KVQ_F32}


class kvq_layout(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "num_kv_heads", "head_dim", "block_size", "group_size", "k_code",
        "v_code", "k_mode", "v_mode", "src_dtype", "reserved")]


class kvq_cache(C.Structure):
    _fields_ = [("k_codes", C.c_void_p), ("v_codes", C.c_void_p),
                ("k_scale", C.c_void_p), ("v_scale", C.c_void_p),
                ("k_zero", C.c_void_p), ("v_zero", C.c_void_p),
                ("k_stage", C.c_void_p), ("num_blocks", C.c_int64),
                ("max_seqs", C.c_int32), ("reserved", C.c_int32)]


_vp, _i32, _i64, _f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
_LP, _CP = C.POINTER(kvq_layout), C.POINTER(kvq_cache)
_SIGS = {
    "kvq_status_string": (C.c_char_p, [_i32]),
    "kvq_layout_check": (_i32, [_LP]),
    "kvq_bytes_per_token": (_i64, [_LP, _i32, _i32]),
    "kvq_cache_plane_bytes": (_i32, [_LP, _i64, _i32, _vp]),
    "kvq_append": (_i32, [_LP, _CP, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "kvq_append_static": (_i32, [_LP, _CP, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp]),
    "kvq_decode_workspace_bytes": (_i64, [_LP, _i32, _i32, _i32, _i32]),
    "kvq_decode_attention": (_i32, [_LP, _CP, _vp, _i32, _i32, _i32, _vp, _i32, _vp,
                                    _i32, _f32, _i32, _vp, _i32, _vp, _i64, _vp]),
    "kvq_prefill_workspace_bytes": (_i64, [_LP, _i32, _i32, _i32, _i32, _i32]),
    "kvq_prefill_attention": (_i32, [_LP, _CP, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _i32,
                                     _vp, _i32, _f32, _i32, _i32, _i32, _vp, _i32, _vp, _i64,
                                     _vp]),
    "kvq_blocks_trim": (_i32, [_vp, _vp, _i64, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp,
                               _vp]),
    "kvq_pool_init": (_i32, [_vp, _vp, _vp, _i64, _vp]),
    "kvq_blocks_fork": (_i32, [_vp, _i64, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _vp]),
    "kvq_blocks_reserve_shared": (_i32, [_vp, _vp, _i64, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                         _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "kvq_blocks_release_shared": (_i32, [_vp, _vp, _i64, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                         _vp, _vp, _vp]),
    "kvq_copy_blocks": (_i32, [_LP, _CP, _vp, _vp, _vp, _i32, _vp]),
    "kvq_block_pack_bytes": (_i64, [_LP]),
    "kvq_pack_blocks": (_i32, [_LP, _CP, _vp, _i32, _vp, _vp]),
    "kvq_unpack_blocks": (_i32, [_LP, _CP, _vp, _vp, _i32, _vp]),
    "kvq_blocks_reserve": (_i32, [_vp, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _i32,
                                  _vp, _vp, _vp, _vp]),
    "kvq_blocks_release": (_i32, [_vp, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _i32,
                                  _vp, _vp, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class KvqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {kvq_status_string(status)} ({status})")


def _check(fn, status):
    if status != KVQ_OK:
        raise KvqError(fn, status)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def kvq_status_string(status: int) -> str:
    return _lib.kvq_status_string(status).decode()


def make_layout(num_kv_heads, head_dim, block_size, k_code="int8", v_code=None,
                k_mode="token_sym", v_mode=None, group_size=0,
                src_dtype=torch.bfloat16) -> kvq_layout:
    """Build a kvq_layout from names ("int8", "fp8", "int4", "none16";
    "token_sym", "group_asym", "channel_block")."""
    v_code = k_code if v_code is None else v_code
    if v_mode is None:
        v_mode = "token_sym" if k_mode == "channel_block" else k_mode
    return kvq_layout(num_kv_heads, head_dim, block_size, group_size,
                      CODES[k_code], CODES[v_code], MODES[k_mode], MODES[v_mode],
                      DTYPES[src_dtype], 0)


def kvq_layout_check(layout) -> int:
    return _lib.kvq_layout_check(C.byref(layout))


def kvq_bytes_per_token(layout, num_layers: int, include_metadata: int = 0) -> int:
    n = _lib.kvq_bytes_per_token(C.byref(layout), num_layers, include_metadata)
    if n < 0:
        raise KvqError("kvq_bytes_per_token", n)
    return n


def kvq_cache_plane_bytes(layout, num_blocks: int, max_seqs: int = 0):
    out = (C.c_int64 * 7)()
    _check("kvq_cache_plane_bytes",
           _lib.kvq_cache_plane_bytes(C.byref(layout), num_blocks, max_seqs, out))
    return list(out)


class PagedCache:
    """One layer's device planes (torch uint8 tensors), sized by the library."""

    NAMES = ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero", "k_stage")

    def __init__(self, layout, num_blocks, max_seqs=0, device="cuda"):
        self.layout, self.num_blocks, self.max_seqs = layout, num_blocks, max_seqs
        sizes = kvq_cache_plane_bytes(layout, num_blocks, max_seqs)
        self.planes = {n: (torch.empty(s, dtype=torch.uint8, device=device) if s else None)
                       for n, s in zip(self.NAMES, sizes)}
        self.struct = kvq_cache(*(_ptr(self.planes[n]) for n in self.NAMES),
                                num_blocks, max_seqs, 0)


def kvq_append(layout, cache: PagedCache, k, v, slot_mapping, stage_rows=None,
               stream=None):
    """k, v: device [T][H][d] (or [T][H*d], rows may be strided) in the layout's
    source dtype; slot_mapping: device int64 [T]; stage_rows: device int32 [T]
    for per-channel keys."""
    T = k.shape[0]
    _check("kvq_append", _lib.kvq_append(
        C.byref(layout), C.byref(cache.struct), _ptr(k), _ptr(v),
        k.stride(0) if T else 0, v.stride(0) if T else 0, T, _ptr(slot_mapping),
        _ptr(stage_rows), _stream(stream)))


def kvq_append_static(layout, cache: PagedCache, k, v, slot_mapping, k_scales,
                      v_scales, k_zeros=None, v_zeros=None, stage_rows=None, stream=None):
    """kvq_append with caller-given scales: k_scales / v_scales device float32
    [H] (TOKEN_SYM), [H][d/32] (GROUP_ASYM, with uint8 zero points of that
    shape) or [H][d] (per-channel keys, with stage_rows as for kvq_append);
    None for a 16-bit passthrough side."""
    T = k.shape[0]
    _check("kvq_append_static", _lib.kvq_append_static(
        C.byref(layout), C.byref(cache.struct), _ptr(k), _ptr(v),
        k.stride(0) if T else 0, v.stride(0) if T else 0, T, _ptr(slot_mapping),
        _ptr(stage_rows), _ptr(k_scales), _ptr(k_zeros), _ptr(v_scales), _ptr(v_zeros),
        _stream(stream)))


def kvq_decode_workspace_bytes(layout, batch, num_q_heads, max_context_len,
                               split_blocks=0) -> int:
    n = _lib.kvq_decode_workspace_bytes(C.byref(layout), batch, num_q_heads,
                                        max_context_len, split_blocks)
    if n < 0:
        raise KvqError("kvq_decode_workspace_bytes", n)
    return n


def kvq_decode_attention(layout, cache: PagedCache, q, block_tables, context_lens,
                         max_context_len, out, workspace, sm_scale=0.0,
                         split_blocks=0, stream=None):
    """q: device [B][Hq][d] fp16/bf16; block_tables: int32 [B][max_blocks];
    context_lens: int32 [B]; out: device [B][Hq][d] fp32/fp16/bf16;
    workspace: device uint8 tensor of kvq_decode_workspace_bytes(...)."""
    B, Hq, _ = q.shape
    _check("kvq_decode_attention", _lib.kvq_decode_attention(
        C.byref(layout), C.byref(cache.struct), _ptr(q), DTYPES[q.dtype], B, Hq,
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        int(max_context_len), float(sm_scale), int(split_blocks), _ptr(out),
        DTYPES[out.dtype], _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def kvq_prefill_workspace_bytes(layout, batch, num_q_heads, max_query_len, max_context_len,
                                split_blocks=0) -> int:
    n = _lib.kvq_prefill_workspace_bytes(C.byref(layout), batch, num_q_heads, max_query_len,
                                         max_context_len, split_blocks)
    if n < 0:
        raise KvqError("kvq_prefill_workspace_bytes", n)
    return n


def kvq_prefill_attention(layout, cache: PagedCache, q, query_start, max_query_len,
                          block_tables, context_lens, max_context_len, out, workspace,
                          sm_scale=0.0, split_blocks=0, window=0, sink=0, stream=None):
    """q: device [Tq][Hq][d] fp16/bf16; query_start: int32 [B+1] (sequence b's
    queries are its last query_start[b+1]-query_start[b] positions);
    block_tables: int32 [B][max_blocks]; context_lens: int32 [B]; out: device
    [Tq][Hq][d]; workspace: device uint8 tensor of
    kvq_prefill_workspace_bytes(...)."""
    _, Hq, _ = q.shape
    B = context_lens.numel()
    _check("kvq_prefill_attention", _lib.kvq_prefill_attention(
        C.byref(layout), C.byref(cache.struct), _ptr(q), DTYPES[q.dtype], B, Hq,
        _ptr(query_start), int(max_query_len), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), int(max_context_len), float(sm_scale), int(window), int(sink),
        int(split_blocks), _ptr(out), DTYPES[out.dtype], _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def kvq_pool_init(free_stack, free_top, initial_order=None, stream=None):
    _check("kvq_pool_init", _lib.kvq_pool_init(
        _ptr(free_stack), _ptr(free_top), _ptr(initial_order), free_stack.numel(),
        _stream(stream)))


def kvq_blocks_reserve(free_stack, free_top, block_tables, context_lens, new_tokens,
                       block_size, slot_mapping_out, status_flag,
                       context_lens_out=None, stream=None):
    _check("kvq_blocks_reserve", _lib.kvq_blocks_reserve(
        _ptr(free_stack), _ptr(free_top), free_stack.numel(), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), _ptr(new_tokens),
        context_lens.numel(), block_size, _ptr(slot_mapping_out),
        _ptr(context_lens_out), _ptr(status_flag), _stream(stream)))


def kvq_blocks_release(free_stack, free_top, block_tables, context_lens, release_mask,
                       block_size, status_flag, context_lens_out=None, stream=None):
    _check("kvq_blocks_release", _lib.kvq_blocks_release(
        _ptr(free_stack), _ptr(free_top), free_stack.numel(), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), _ptr(release_mask),
        context_lens.numel(), block_size, _ptr(context_lens_out), _ptr(status_flag),
        _stream(stream)))


def kvq_blocks_fork(refcount, block_tables, context_lens, src_rows, dst_rows, block_size,
                    stream=None):
    """Rows dst_rows[k] take rows src_rows[k]'s blocks (device int32 tensors)."""
    _check("kvq_blocks_fork", _lib.kvq_blocks_fork(
        _ptr(refcount), refcount.numel(), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), context_lens.numel(), _ptr(src_rows), _ptr(dst_rows),
        src_rows.numel(), block_size, _stream(stream)))


def kvq_blocks_reserve_shared(free_stack, free_top, refcount, block_tables, context_lens,
                              new_tokens, block_size, slot_mapping_out, cow_src, cow_dst,
                              cow_count, status_flag, context_lens_out=None, stream=None):
    _check("kvq_blocks_reserve_shared", _lib.kvq_blocks_reserve_shared(
        _ptr(free_stack), _ptr(free_top), free_stack.numel(), _ptr(refcount),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), _ptr(new_tokens),
        context_lens.numel(), block_size, _ptr(slot_mapping_out), _ptr(context_lens_out),
        _ptr(cow_src), _ptr(cow_dst), _ptr(cow_count), _ptr(status_flag), _stream(stream)))


def kvq_blocks_release_shared(free_stack, free_top, refcount, block_tables, context_lens,
                              release_mask, block_size, status_flag, context_lens_out=None,
                              stream=None):
    _check("kvq_blocks_release_shared", _lib.kvq_blocks_release_shared(
        _ptr(free_stack), _ptr(free_top), free_stack.numel(), _ptr(refcount),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), _ptr(release_mask),
        context_lens.numel(), block_size, _ptr(context_lens_out), _ptr(status_flag),
        _stream(stream)))


def kvq_copy_blocks(layout, cache: PagedCache, src_ids, dst_ids, count, max_pairs=None,
                    stream=None):
    """Copy block src_ids[k] onto dst_ids[k] in one layer, k < count[0] (device)."""
    _check("kvq_copy_blocks", _lib.kvq_copy_blocks(
        C.byref(layout), C.byref(cache.struct), _ptr(src_ids), _ptr(dst_ids), _ptr(count),
        src_ids.numel() if max_pairs is None else max_pairs, _stream(stream)))


def kvq_blocks_trim(free_stack, free_top, block_tables, context_lens, window, sink, block_size,
                    status_flag, stream=None):
    """Return the blocks no query past context_lens can see under the window."""
    _check("kvq_blocks_trim", _lib.kvq_blocks_trim(
        _ptr(free_stack), _ptr(free_top), free_stack.numel(), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), int(window), int(sink),
        context_lens.numel(), block_size, _ptr(status_flag), _stream(stream)))


def kvq_block_pack_bytes(layout) -> int:
    n = _lib.kvq_block_pack_bytes(C.byref(layout))
    if n < 0:
        raise KvqError("kvq_block_pack_bytes", n)
    return n


def kvq_pack_blocks(layout, cache: PagedCache, ids, dst, stream=None):
    """Pack blocks ids (device int32) of one layer into dst (uint8 tensor)."""
    _check("kvq_pack_blocks", _lib.kvq_pack_blocks(
        C.byref(layout), C.byref(cache.struct), _ptr(ids), ids.numel(), _ptr(dst),
        _stream(stream)))


def kvq_unpack_blocks(layout, cache: PagedCache, src, ids, stream=None):
    _check("kvq_unpack_blocks", _lib.kvq_unpack_blocks(
        C.byref(layout), C.byref(cache.struct), _ptr(src), _ptr(ids), ids.numel(),
        _stream(stream)))
