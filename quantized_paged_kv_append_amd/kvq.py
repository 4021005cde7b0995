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
KVQ_DECODE_SCRATCH_BYTES = 134217728   # the allocation-free decode's per-GPU array

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
    "kvq_append_decode_attention": (_i32, [_LP, _CP, _vp, _vp, _i64, _i64, _vp, _i32, _i32,
                                           _i32, _vp, _i32, _vp, _i32, _f32, _i32, _vp, _i32,
                                           _vp, _i64, _vp]),
    "kvq_decode_attention_noalloc": (_i32, [_LP, _CP, _vp, _i32, _i32, _i32, _vp, _i32, _vp,
                                            _i32, _f32, _i32, _vp, _i32, _vp]),
    "kvq_prefill_workspace_bytes": (_i64, [_LP, _i32, _i32, _i32, _i32, _i32]),
    "kvq_prefill_attention": (_i32, [_LP, _CP, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _i32,
                                     _vp, _i32, _f32, _i32, _i32, _i32, _vp, _i32, _vp, _i64,
                                     _vp]),
    "kvq_blocks_trim": (_i32, [_vp, _vp, _i64, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp,
                               _vp]),
    "kvq_pool_init": (_i32, [_vp, _vp, _vp, _i64, _vp]),
    "kvq_blocks_fork": (_i32, [_vp, _i64, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _vp]),
    "kvq_blocks_reserve_shared": (_i32, [_vp, _vp, _i64, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                         _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "kvq_blocks_release_shared": (_i32, [_vp, _vp, _i64, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                         _vp, _vp, _vp]),
    "kvq_copy_blocks": (_i32, [_LP, _CP, _vp, _vp, _vp, _i32, _vp]),
    "kvq_block_pack_bytes": (_i64, [_LP]),
    "kvq_pack_blocks": (_i32, [_LP, _CP, _vp, _i32, _vp, _vp]),
    "kvq_unpack_blocks": (_i32, [_LP, _CP, _vp, _vp, _i32, _vp]),
    "kvq_blocks_reserve": (_i32, [_vp, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _i32,
                                  _vp, _i64, _vp, _vp, _vp]),
    "kvq_blocks_release": (_i32, [_vp, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _i32,
                                  _vp, _vp, _vp]),
    "kvq_check_block_tables": (_i32, [_vp, _i32, _vp, _i32, _i32, _i64, _vp, _vp, _vp]),
    "kvq_check_slots": (_i32, [_vp, _i64, _i64, _i32, _vp, _vp, _vp]),
    "kvq_read_probe": (_i32, [_vp, _i64, _vp, _vp]),
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


# ---- argument validation ----------------------------------------------------
# The C ABI sees raw pointers only: a tensor of the wrong dtype, on the host,
# too small or with a strided inner dimension would be read or written as if
# it were right. Every entry point below checks its tensors first, in the
# order dtype, shape and size, layout in memory, then device, and raises
# ValueError naming the argument before anything reaches the library.

_SRC_DTYPES = {KVQ_F16: torch.float16, KVQ_BF16: torch.bfloat16}


def _need(t, name, dtypes, numel=None, min_numel=None, ndim=None, contiguous=True,
          optional=False):
    """Check one tensor argument; returns it unchanged."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name}: a tensor is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        want = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name}: dtype {str(t.dtype).replace('torch.', '')}, expected {want}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: {t.dim()}-D, expected {ndim}-D")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {min_numel} needed")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _on_device(**tensors):
    """Last check of every entry point: all tensor arguments on the GPU."""
    for name, t in tensors.items():
        if isinstance(t, PagedCache):
            for n, p in t.planes.items():
                if p is not None and not p.is_cuda:
                    raise ValueError(f"{name} plane {n}: must be a CUDA (HIP) device tensor")
        elif t is not None and not t.is_cuda:
            raise ValueError(f"{name}: must be a CUDA (HIP) device tensor")


_LAYOUT_FIELDS = ("num_kv_heads", "head_dim", "block_size", "group_size", "k_code", "v_code",
                  "k_mode", "v_mode", "src_dtype")


def _need_cache(layout, cache):
    """The cache's planes were sized for this layout."""
    if not isinstance(cache, PagedCache):
        raise ValueError(f"cache: expected a PagedCache, got {type(cache).__name__}")
    for f in _LAYOUT_FIELDS:
        if getattr(cache.layout, f) != getattr(layout, f):
            raise ValueError(f"cache: made for a layout with {f} = "
                             f"{getattr(cache.layout, f)}, called with {getattr(layout, f)}")


def _need_rows(t, name, layout, T=None):
    """K or V rows: [T][H][d] or [T][H*d] in the layout's source dtype, each
    row's H*d elements contiguous (rows themselves may be strided)."""
    H, d = layout.num_kv_heads, layout.head_dim
    want = _SRC_DTYPES.get(layout.src_dtype)
    if want is None:
        raise ValueError(f"layout.src_dtype {layout.src_dtype} is not F16 or BF16")
    _need(t, name, want, contiguous=False)
    if t.dim() == 3:
        if tuple(t.shape[1:]) != (H, d) or t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError(f"{name}: shape {tuple(t.shape)} strides {t.stride()}, expected "
                             f"[T][{H}][{d}] with contiguous rows")
    elif t.dim() == 2:
        if t.shape[1] != H * d or t.stride(1) != 1:
            raise ValueError(f"{name}: shape {tuple(t.shape)} strides {t.stride()}, expected "
                             f"[T][{H * d}] with contiguous rows")
    else:
        raise ValueError(f"{name}: {t.dim()}-D, expected [T][H][d] or [T][H*d]")
    if T is not None and t.shape[0] != T:
        raise ValueError(f"{name}: {t.shape[0]} rows, expected {T} (as k)")
    if t.shape[0] > 1 and t.stride(0) < H * d:
        raise ValueError(f"{name}: row stride {t.stride(0)} below H*d = {H * d}")
    return t


def _nbytes(t):
    return t.numel() * t.element_size()


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
    _need_rows(k, "k", layout)
    T = k.shape[0]
    _need_rows(v, "v", layout, T)
    _need(slot_mapping, "slot_mapping", torch.int64, numel=T)
    chan = layout.k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM
    _need(stage_rows, "stage_rows", torch.int32, numel=T, optional=not chan)
    if not chan and stage_rows is not None:
        raise ValueError("stage_rows: only for per-channel keys (channel_block)")
    _need_cache(layout, cache)
    _on_device(cache=cache, k=k, v=v, slot_mapping=slot_mapping, stage_rows=stage_rows)
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
    _need_rows(k, "k", layout)
    T = k.shape[0]
    _need_rows(v, "v", layout, T)
    _need(slot_mapping, "slot_mapping", torch.int64, numel=T)
    chan = layout.k_mode == KVQ_SCALE_CHANNEL_BLOCK_SYM
    _need(stage_rows, "stage_rows", torch.int32, numel=T, optional=not chan)
    if not chan and stage_rows is not None:
        raise ValueError("stage_rows: only for per-channel keys (channel_block)")
    H, d, gs = layout.num_kv_heads, layout.head_dim, layout.group_size
    for side, sc, zp in (("k", k_scales, k_zeros), ("v", v_scales, v_zeros)):
        code = layout.k_code if side == "k" else layout.v_code
        mode = layout.k_mode if side == "k" else layout.v_mode
        if code == KVQ_CODE_NONE16:
            n = 0
        elif mode == KVQ_SCALE_TOKEN_SYM:
            n = H
        elif mode == KVQ_SCALE_GROUP_ASYM:
            n = H * (d // gs if gs else 0)
        else:
            n = H * d
        _need(sc, f"{side}_scales", torch.float32, numel=n, optional=n == 0)
        asym = code != KVQ_CODE_NONE16 and mode == KVQ_SCALE_GROUP_ASYM
        _need(zp, f"{side}_zeros", torch.uint8, numel=n, optional=not asym)
    _need_cache(layout, cache)
    _on_device(cache=cache, k=k, v=v, slot_mapping=slot_mapping, stage_rows=stage_rows, k_scales=k_scales,
               k_zeros=k_zeros, v_scales=v_scales, v_zeros=v_zeros)
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


def _decode_checks(layout, q, block_tables, context_lens, out, workspace, rows=None):
    """Shared checks of decode and multi-query attention: q [rows][Hq][d]
    fp16/bf16, out of q's shape in fp32/fp16/bf16, int32 tables [B][max] and
    lengths [B], a workspace of bytes. Returns (B, Hq)."""
    _need(q, "q", (torch.float16, torch.bfloat16), ndim=3)
    if q.shape[2] != layout.head_dim:
        raise ValueError(f"q: head dim {q.shape[2]}, layout has {layout.head_dim}")
    Hq = q.shape[1]
    _need(context_lens, "context_lens", torch.int32, ndim=1)
    B = context_lens.numel()
    if rows is None and q.shape[0] != B:
        raise ValueError(f"q: {q.shape[0]} rows, context_lens has {B}")
    _need(block_tables, "block_tables", torch.int32, ndim=2)
    if block_tables.shape[0] < B:
        raise ValueError(f"block_tables: {block_tables.shape[0]} rows, batch is {B}")
    _need(out, "out", (torch.float32, torch.float16, torch.bfloat16), ndim=3)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out: shape {tuple(out.shape)}, expected {tuple(q.shape)} (as q)")
    if workspace is not None:
        _need(workspace, "workspace", tuple(DTYPES) + (torch.uint8, torch.int32, torch.int64))
    return B, Hq


def kvq_decode_attention(layout, cache: PagedCache, q, block_tables, context_lens,
                         max_context_len, out, workspace, sm_scale=0.0,
                         split_blocks=0, stream=None):
    """q: device [B][Hq][d] fp16/bf16; block_tables: int32 [B][max_blocks];
    context_lens: int32 [B]; out: device [B][Hq][d] fp32/fp16/bf16;
    workspace: device uint8 tensor of kvq_decode_workspace_bytes(...)."""
    B, Hq = _decode_checks(layout, q, block_tables, context_lens, out, workspace)
    _need_cache(layout, cache)
    _on_device(cache=cache, q=q, block_tables=block_tables, context_lens=context_lens, out=out,
               workspace=workspace)
    _check("kvq_decode_attention", _lib.kvq_decode_attention(
        C.byref(layout), C.byref(cache.struct), _ptr(q), DTYPES[q.dtype], B, Hq,
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        int(max_context_len), float(sm_scale), int(split_blocks), _ptr(out),
        DTYPES[out.dtype], _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def kvq_append_decode_attention(layout, cache: PagedCache, k, v, q, block_tables,
                                context_lens, max_context_len, out, workspace, sm_scale=0.0,
                                split_blocks=0, stream=None):
    """kvq_append of one new token per sequence (rows k[b], v[b]: device
    [B][H][d] or [B][H*d] in the layout's source dtype) into position
    context_lens[b] - 1, then kvq_decode_attention, in one launch. The other
    arguments are kvq_decode_attention's."""
    B, Hq = _decode_checks(layout, q, block_tables, context_lens, out, workspace)
    _need_rows(k, "k", layout, B)
    _need_rows(v, "v", layout, B)
    _need_cache(layout, cache)
    _on_device(cache=cache, k=k, v=v, q=q, block_tables=block_tables,
               context_lens=context_lens, out=out, workspace=workspace)
    _check("kvq_append_decode_attention", _lib.kvq_append_decode_attention(
        C.byref(layout), C.byref(cache.struct), _ptr(k), _ptr(v),
        k.stride(0) if B else 0, v.stride(0) if B else 0, _ptr(q), DTYPES[q.dtype], B, Hq,
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        int(max_context_len), float(sm_scale), int(split_blocks), _ptr(out),
        DTYPES[out.dtype], _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def kvq_decode_attention_noalloc(layout, cache: PagedCache, q, block_tables, context_lens,
                                 max_context_len, out, sm_scale=0.0, split_blocks=0,
                                 stream=None):
    """kvq_decode_attention without a workspace argument: the library's fixed
    per-GPU array (KVQ_DECODE_SCRATCH_BYTES) holds the partials, and the call
    allocates nothing. Calls that overlap on one GPU race on that array."""
    B, Hq = _decode_checks(layout, q, block_tables, context_lens, out, None)
    _need_cache(layout, cache)
    _on_device(cache=cache, q=q, block_tables=block_tables, context_lens=context_lens, out=out)
    _check("kvq_decode_attention_noalloc", _lib.kvq_decode_attention_noalloc(
        C.byref(layout), C.byref(cache.struct), _ptr(q), DTYPES[q.dtype], B, Hq,
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        int(max_context_len), float(sm_scale), int(split_blocks), _ptr(out),
        DTYPES[out.dtype], _stream(stream)))


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
    B, Hq = _decode_checks(layout, q, block_tables, context_lens, out, workspace, rows=True)
    _need(query_start, "query_start", torch.int32, numel=B + 1)
    _need_cache(layout, cache)
    _on_device(cache=cache, q=q, query_start=query_start, block_tables=block_tables,
               context_lens=context_lens, out=out, workspace=workspace)
    _check("kvq_prefill_attention", _lib.kvq_prefill_attention(
        C.byref(layout), C.byref(cache.struct), _ptr(q), DTYPES[q.dtype], B, Hq,
        _ptr(query_start), int(max_query_len), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), int(max_context_len), float(sm_scale), int(window), int(sink),
        int(split_blocks), _ptr(out), DTYPES[out.dtype], _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def _need_pool(free_stack, free_top):
    _need(free_stack, "free_stack", torch.int32, ndim=1)
    _need(free_top, "free_top", torch.int32, min_numel=1)


def _need_status(status_flag):
    _need(status_flag, "status_flag", torch.int32, min_numel=1)


def _need_lens_out(context_lens_out, B):
    _need(context_lens_out, "context_lens_out", torch.int32, numel=B, optional=True)


def kvq_pool_init(free_stack, free_top, initial_order=None, stream=None):
    _need_pool(free_stack, free_top)
    _need(initial_order, "initial_order", torch.int32, numel=free_stack.numel(), optional=True)
    _on_device(free_stack=free_stack, free_top=free_top, initial_order=initial_order)
    _check("kvq_pool_init", _lib.kvq_pool_init(
        _ptr(free_stack), _ptr(free_top), _ptr(initial_order), free_stack.numel(),
        _stream(stream)))


def kvq_blocks_reserve(free_stack, free_top, block_tables, context_lens, new_tokens,
                       block_size, slot_mapping_out, status_flag,
                       context_lens_out=None, stream=None):
    """slot_mapping_out: int64, at least sum(new_tokens) entries. Its length
    goes to the library, which checks the count on the device: a short
    buffer leaves everything unwritten and sets status_flag to
    KVQ_ERR_INVALID_ARGUMENT (no host read of new_tokens, so no wait for the
    device here)."""
    _need_pool(free_stack, free_top)
    _need(context_lens, "context_lens", torch.int32, ndim=1)
    B = context_lens.numel()
    _need(block_tables, "block_tables", torch.int32, ndim=2)
    if block_tables.shape[0] < B:
        raise ValueError(f"block_tables: {block_tables.shape[0]} rows, batch is {B}")
    _need(new_tokens, "new_tokens", torch.int32, numel=B)
    _need(slot_mapping_out, "slot_mapping_out", torch.int64, ndim=1)
    _need_status(status_flag)
    _need_lens_out(context_lens_out, B)
    _on_device(free_stack=free_stack, free_top=free_top, block_tables=block_tables,
               context_lens=context_lens, new_tokens=new_tokens,
               slot_mapping_out=slot_mapping_out, status_flag=status_flag,
               context_lens_out=context_lens_out)
    _check("kvq_blocks_reserve", _lib.kvq_blocks_reserve(
        _ptr(free_stack), _ptr(free_top), free_stack.numel(), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), _ptr(new_tokens),
        context_lens.numel(), block_size, _ptr(slot_mapping_out), slot_mapping_out.numel(),
        _ptr(context_lens_out), _ptr(status_flag), _stream(stream)))


def kvq_blocks_release(free_stack, free_top, block_tables, context_lens, release_mask,
                       block_size, status_flag, context_lens_out=None, stream=None):
    _need_pool(free_stack, free_top)
    _need(context_lens, "context_lens", torch.int32, ndim=1)
    B = context_lens.numel()
    _need(block_tables, "block_tables", torch.int32, ndim=2)
    if block_tables.shape[0] < B:
        raise ValueError(f"block_tables: {block_tables.shape[0]} rows, batch is {B}")
    _need(release_mask, "release_mask", torch.int32, numel=B)
    _need_status(status_flag)
    _need_lens_out(context_lens_out, B)
    _on_device(free_stack=free_stack, free_top=free_top, block_tables=block_tables,
               context_lens=context_lens, release_mask=release_mask, status_flag=status_flag,
               context_lens_out=context_lens_out)
    _check("kvq_blocks_release", _lib.kvq_blocks_release(
        _ptr(free_stack), _ptr(free_top), free_stack.numel(), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), _ptr(release_mask),
        context_lens.numel(), block_size, _ptr(context_lens_out), _ptr(status_flag),
        _stream(stream)))


def kvq_blocks_fork(refcount, block_tables, context_lens, src_rows, dst_rows, block_size,
                    stream=None):
    """Rows dst_rows[k] take rows src_rows[k]'s blocks (device int32 tensors)."""
    _need(refcount, "refcount", torch.int32, ndim=1)
    _need(context_lens, "context_lens", torch.int32, ndim=1)
    _need(block_tables, "block_tables", torch.int32, ndim=2)
    if block_tables.shape[0] < context_lens.numel():
        raise ValueError("block_tables: fewer rows than context_lens")
    _need(src_rows, "src_rows", torch.int32, ndim=1)
    _need(dst_rows, "dst_rows", torch.int32, numel=src_rows.numel())
    _on_device(refcount=refcount, block_tables=block_tables, context_lens=context_lens,
               src_rows=src_rows, dst_rows=dst_rows)
    _check("kvq_blocks_fork", _lib.kvq_blocks_fork(
        _ptr(refcount), refcount.numel(), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), context_lens.numel(), _ptr(src_rows), _ptr(dst_rows),
        src_rows.numel(), block_size, _stream(stream)))


def kvq_blocks_reserve_shared(free_stack, free_top, refcount, block_tables, context_lens,
                              new_tokens, block_size, slot_mapping_out, cow_src, cow_dst,
                              cow_count, status_flag, context_lens_out=None, stream=None):
    _need_pool(free_stack, free_top)
    _need(refcount, "refcount", torch.int32, numel=free_stack.numel())
    _need(context_lens, "context_lens", torch.int32, ndim=1)
    B = context_lens.numel()
    _need(block_tables, "block_tables", torch.int32, ndim=2)
    if block_tables.shape[0] < B:
        raise ValueError(f"block_tables: {block_tables.shape[0]} rows, batch is {B}")
    _need(new_tokens, "new_tokens", torch.int32, numel=B)
    _need(slot_mapping_out, "slot_mapping_out", torch.int64, ndim=1)
    _need(cow_src, "cow_src", torch.int32, min_numel=B)
    _need(cow_dst, "cow_dst", torch.int32, min_numel=B)
    _need(cow_count, "cow_count", torch.int32, min_numel=1)
    _need_status(status_flag)
    _need_lens_out(context_lens_out, B)
    _on_device(free_stack=free_stack, free_top=free_top, refcount=refcount,
               block_tables=block_tables, context_lens=context_lens, new_tokens=new_tokens,
               slot_mapping_out=slot_mapping_out, cow_src=cow_src, cow_dst=cow_dst,
               cow_count=cow_count, status_flag=status_flag, context_lens_out=context_lens_out)
    _check("kvq_blocks_reserve_shared", _lib.kvq_blocks_reserve_shared(
        _ptr(free_stack), _ptr(free_top), free_stack.numel(), _ptr(refcount),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), _ptr(new_tokens),
        context_lens.numel(), block_size, _ptr(slot_mapping_out), slot_mapping_out.numel(),
        _ptr(context_lens_out), _ptr(cow_src), _ptr(cow_dst), _ptr(cow_count),
        _ptr(status_flag), _stream(stream)))


def kvq_blocks_release_shared(free_stack, free_top, refcount, block_tables, context_lens,
                              release_mask, block_size, status_flag, context_lens_out=None,
                              stream=None):
    _need_pool(free_stack, free_top)
    _need(refcount, "refcount", torch.int32, numel=free_stack.numel())
    _need(context_lens, "context_lens", torch.int32, ndim=1)
    B = context_lens.numel()
    _need(block_tables, "block_tables", torch.int32, ndim=2)
    if block_tables.shape[0] < B:
        raise ValueError(f"block_tables: {block_tables.shape[0]} rows, batch is {B}")
    _need(release_mask, "release_mask", torch.int32, numel=B)
    _need_status(status_flag)
    _need_lens_out(context_lens_out, B)
    _on_device(free_stack=free_stack, free_top=free_top, refcount=refcount,
               block_tables=block_tables, context_lens=context_lens, release_mask=release_mask,
               status_flag=status_flag, context_lens_out=context_lens_out)
    _check("kvq_blocks_release_shared", _lib.kvq_blocks_release_shared(
        _ptr(free_stack), _ptr(free_top), free_stack.numel(), _ptr(refcount),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), _ptr(release_mask),
        context_lens.numel(), block_size, _ptr(context_lens_out), _ptr(status_flag),
        _stream(stream)))


def kvq_copy_blocks(layout, cache: PagedCache, src_ids, dst_ids, count, max_pairs=None,
                    stream=None):
    """Copy block src_ids[k] onto dst_ids[k] in one layer, k < count[0] (device)."""
    n = src_ids.numel() if max_pairs is None else max_pairs
    _need(src_ids, "src_ids", torch.int32, min_numel=n)
    _need(dst_ids, "dst_ids", torch.int32, min_numel=n)
    _need(count, "count", torch.int32, min_numel=1)
    _need_cache(layout, cache)
    _on_device(cache=cache, src_ids=src_ids, dst_ids=dst_ids, count=count)
    _check("kvq_copy_blocks", _lib.kvq_copy_blocks(
        C.byref(layout), C.byref(cache.struct), _ptr(src_ids), _ptr(dst_ids), _ptr(count),
        src_ids.numel() if max_pairs is None else max_pairs, _stream(stream)))


def kvq_blocks_trim(free_stack, free_top, block_tables, context_lens, window, sink, block_size,
                    status_flag, stream=None):
    """Return the blocks no query past context_lens can see under the window."""
    _need_pool(free_stack, free_top)
    _need(context_lens, "context_lens", torch.int32, ndim=1)
    _need(block_tables, "block_tables", torch.int32, ndim=2)
    if block_tables.shape[0] < context_lens.numel():
        raise ValueError("block_tables: fewer rows than context_lens")
    _need_status(status_flag)
    _on_device(free_stack=free_stack, free_top=free_top, block_tables=block_tables,
               context_lens=context_lens, status_flag=status_flag)
    _check("kvq_blocks_trim", _lib.kvq_blocks_trim(
        _ptr(free_stack), _ptr(free_top), free_stack.numel(), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), int(window), int(sink),
        context_lens.numel(), block_size, _ptr(status_flag), _stream(stream)))


def kvq_check_block_tables(block_tables, context_lens, block_size, num_blocks, first_bad,
                           status_flag, stream=None):
    """Debugging aid: status_flag (device int32 [1]) gets KVQ_OK, or
    KVQ_ERR_INVALID_ARGUMENT when a table entry a context uses lies outside
    [0, num_blocks) or a length outside [0, max_blocks * block_size];
    first_bad (device int64 [1]) gets the smallest flat index b * max_blocks
    + k of such an entry, or -1."""
    _need(context_lens, "context_lens", torch.int32, ndim=1)
    _need(block_tables, "block_tables", torch.int32, ndim=2)
    if block_tables.shape[0] < context_lens.numel():
        raise ValueError("block_tables: fewer rows than context_lens")
    _need(first_bad, "first_bad", torch.int64, numel=1)
    _need_status(status_flag)
    _on_device(block_tables=block_tables, context_lens=context_lens, first_bad=first_bad,
               status_flag=status_flag)
    _check("kvq_check_block_tables", _lib.kvq_check_block_tables(
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), context_lens.numel(),
        block_size, int(num_blocks), _ptr(first_bad), _ptr(status_flag), _stream(stream)))


def kvq_check_slots(slot_mapping, num_blocks, block_size, first_bad, status_flag, stream=None):
    """Debugging aid: every slot must be -1 or lie in [0, num_blocks *
    block_size); reports as kvq_check_block_tables (first_bad = the smallest
    bad token index, or -1)."""
    _need(slot_mapping, "slot_mapping", torch.int64, ndim=1)
    _need(first_bad, "first_bad", torch.int64, numel=1)
    _need_status(status_flag)
    _on_device(slot_mapping=slot_mapping, first_bad=first_bad, status_flag=status_flag)
    _check("kvq_check_slots", _lib.kvq_check_slots(
        _ptr(slot_mapping), slot_mapping.numel(), int(num_blocks), block_size, _ptr(first_bad),
        _ptr(status_flag), _stream(stream)))


def kvq_read_probe(buf, sink, stream=None):
    """Measurement aid: read every byte of buf (a device tensor, 16-byte
    aligned, nbytes a multiple of 16) once with non-temporal loads; sink is a
    device int32 [1] that is written only in a practically impossible case.
    Time the call with events on the stream to get the read rate."""
    _need(sink, "sink", torch.int32, numel=1)
    _on_device(buf=buf, sink=sink)
    if not buf.is_contiguous():
        raise ValueError("buf: must be contiguous")
    _check("kvq_read_probe", _lib.kvq_read_probe(_ptr(buf), _nbytes(buf), _ptr(sink),
                                                 _stream(stream)))


def kvq_block_pack_bytes(layout) -> int:
    n = _lib.kvq_block_pack_bytes(C.byref(layout))
    if n < 0:
        raise KvqError("kvq_block_pack_bytes", n)
    return n


def kvq_pack_blocks(layout, cache: PagedCache, ids, dst, stream=None):
    """Pack blocks ids (device int32) of one layer into dst (uint8 tensor)."""
    _need(ids, "ids", torch.int32, ndim=1)
    _need(dst, "dst", (torch.uint8, torch.int8), ndim=1, contiguous=True)
    if _nbytes(dst) < ids.numel() * kvq_block_pack_bytes(layout):
        raise ValueError(f"dst: {_nbytes(dst)} bytes, {ids.numel()} packed blocks need "
                         f"{ids.numel() * kvq_block_pack_bytes(layout)}")
    _need_cache(layout, cache)
    _on_device(cache=cache, ids=ids, dst=dst)
    _check("kvq_pack_blocks", _lib.kvq_pack_blocks(
        C.byref(layout), C.byref(cache.struct), _ptr(ids), ids.numel(), _ptr(dst),
        _stream(stream)))


def kvq_unpack_blocks(layout, cache: PagedCache, src, ids, stream=None):
    _need(ids, "ids", torch.int32, ndim=1)
    _need(src, "src", (torch.uint8, torch.int8), ndim=1)
    if _nbytes(src) < ids.numel() * kvq_block_pack_bytes(layout):
        raise ValueError(f"src: {_nbytes(src)} bytes, {ids.numel()} packed blocks need "
                         f"{ids.numel() * kvq_block_pack_bytes(layout)}")
    _need_cache(layout, cache)
    _on_device(cache=cache, src=src, ids=ids)
    _check("kvq_unpack_blocks", _lib.kvq_unpack_blocks(
        C.byref(layout), C.byref(cache.struct), _ptr(src), _ptr(ids), ids.numel(),
        _stream(stream)))
