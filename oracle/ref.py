"""ctypes front end of the CPU oracle (oracle/kvq_oracle.c).

TEST INFRASTRUCTURE: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It loads nothing from the
GPU library and the GPU library never imports it.

Arrays are numpy, on the host. 16-bit floating inputs (fp16 or bf16) are passed
as their raw uint16 bit patterns, so bf16 needs no numpy dtype.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

F16, BF16, F32 = 0, 1, 2
CODE_NONE16, CODE_INT8, CODE_FP8, CODE_INT4 = 0, 1, 2, 3
TOKEN_SYM, GROUP_ASYM, CHANNEL_BLOCK = 0, 1, 2
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_OUT_OF_BLOCKS = 0, -1, -2, -5


class Layout(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "num_kv_heads", "head_dim", "block_size", "group_size", "k_code",
        "v_code", "k_mode", "v_mode", "src_dtype", "reserved")]


class _Cache(C.Structure):
    _fields_ = [("k_codes", C.c_void_p), ("v_codes", C.c_void_p),
                ("k_scale", C.c_void_p), ("v_scale", C.c_void_p),
                ("k_zero", C.c_void_p), ("v_zero", C.c_void_p),
                ("k_stage", C.c_void_p), ("num_blocks", C.c_int64),
                ("max_seqs", C.c_int32), ("reserved", C.c_int32)]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _load():
    # KVQ_ORACLE_LIB names another build of the oracle (the mutation test
    # loads copies with planted mistakes this way); otherwise the oracle's
    # own library, rebuilt when its source is newer
    path = os.environ.get("KVQ_ORACLE_LIB")
    if not path:
        path = _build.LIB
        if not os.path.exists(path) or \
                os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
    lib = C.CDLL(path)
    vp, i32, i64, f32, f64 = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_double
    sig = {
        "orc_f16_to_f32": (f32, [C.c_uint16]),
        "orc_bf16_to_f32": (f32, [C.c_uint16]),
        "orc_e4m3_value": (f32, [C.c_uint8]),
        "orc_e4m3_encode": (C.c_uint8, [f32]),
        "orc_quant_sym": (None, [vp, C.c_int, C.c_int, vp, vp]),
        "orc_quant_fp8": (None, [vp, C.c_int, vp, vp]),
        "orc_quant_asym4": (None, [vp, C.c_int, vp, vp, vp]),
        "orc_quant_channel_block": (None, [vp, C.c_int, C.c_int, vp, vp]),
        "orc_quant_sym_static": (None, [vp, C.c_int, C.c_int, f32, vp]),
        "orc_quant_fp8_static": (None, [vp, C.c_int, f32, vp]),
        "orc_quant_asym4_static": (None, [vp, C.c_int, f32, C.c_uint8, vp]),
        "orc_prefill": (C.c_int, [vp, vp, vp, i32, i32, i32, vp, vp, i32, vp, i32, i32, f64, vp,
                                 i32]),
        "orc_blocks_trim": (C.c_int, [vp, vp, i64, vp, i32, vp, i32, i32, i32, i32, vp]),
        "orc_append_static": (C.c_int, [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]),
        "orc_int4_pack": (None, [vp, C.c_int, vp]),
        "orc_int4_unpack": (None, [vp, C.c_int, vp]),
        "orc_bytes_per_token": (i64, [vp, i32, i32]),
        "orc_plane_bytes": (C.c_int, [vp, i64, i32, vp]),
        "orc_append": (C.c_int, [vp, vp, vp, vp, i64, i64, i64, vp, vp]),
        "orc_dequant_token": (C.c_int, [vp, vp, C.c_int, vp, i32, i32, i32, i32, vp]),
        "orc_decode": (C.c_int, [vp, vp, vp, i32, i32, i32, vp, i32, vp, f64, vp, i32]),
        "orc_decode_range": (C.c_int, [vp, vp, vp, i32, i32, i32, i32, vp, i32,
                                        i32, i32, f64, vp, vp, vp]),
        "orc_pool_init": (C.c_int, [vp, vp, vp, i64]),
        "orc_blocks_fork": (C.c_int, [vp, vp, i32, vp, vp, vp, i32, i32]),
        "orc_blocks_reserve_shared": (C.c_int, [vp, vp, i64, vp, vp, i32, vp, vp, i32, i32,
                                                vp, vp, vp, vp, vp, vp]),
        "orc_blocks_release_shared": (C.c_int, [vp, vp, i64, vp, vp, i32, vp, vp, i32, i32,
                                                vp, vp]),
        "orc_copy_blocks": (C.c_int, [vp, vp, vp, vp, i32]),
        "orc_block_pack_bytes": (i64, [vp]),
        "orc_pack_blocks": (C.c_int, [vp, vp, vp, i32, vp]),
        "orc_unpack_blocks": (C.c_int, [vp, vp, vp, vp, i32]),
        "orc_blocks_reserve": (C.c_int, [vp, vp, i64, vp, i32, vp, vp, i32, i32,
                                          vp, vp, vp]),
        "orc_blocks_release": (C.c_int, [vp, vp, i64, vp, i32, vp, vp, i32, i32,
                                          vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def layout(num_kv_heads, head_dim, block_size, k_code, v_code=None,
           k_mode=TOKEN_SYM, v_mode=None, group_size=0, src_dtype=BF16):
    v_code = k_code if v_code is None else v_code
    v_mode = (TOKEN_SYM if k_mode == CHANNEL_BLOCK else k_mode) \
        if v_mode is None else v_mode
    return Layout(num_kv_heads, head_dim, block_size, group_size, k_code,
                  v_code, k_mode, v_mode, src_dtype, 0)


def plane_bytes(L, num_blocks, max_seqs=0):
    out = np.zeros(7, np.int64)
    rc = lib.orc_plane_bytes(C.byref(L), num_blocks, max_seqs, _ptr(out))
    if rc:
        raise ValueError(f"orc_plane_bytes: {rc}")
    return [int(x) for x in out]


class HostCache:
    """Host planes of one layer, shaped as the library's cache (bytes)."""

    NAMES = ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero",
             "k_stage")

    def __init__(self, L, num_blocks, max_seqs=0, fill=0):
        self.L, self.num_blocks, self.max_seqs = L, num_blocks, max_seqs
        sizes = plane_bytes(L, num_blocks, max_seqs)
        self.planes = {}
        for name, n in zip(self.NAMES, sizes):
            self.planes[name] = np.full(n, fill, np.uint8) if n else None
        self._keep = None

    def struct(self):
        p = self.planes
        s = _Cache(*(None if p[n] is None else p[n].ctypes.data for n in self.NAMES),
                   self.num_blocks, self.max_seqs, 0)
        return s

    def scale(self, side):
        a = self.planes["v_scale" if side else "k_scale"]
        return None if a is None else a.view(np.float32)


def bytes_per_token(L, num_layers, include_metadata=0):
    return int(lib.orc_bytes_per_token(C.byref(L), num_layers, include_metadata))


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def append(L, cache, k_bits, v_bits, slots, stage_rows=None,
           k_row_stride=None, v_row_stride=None):
    """k_bits, v_bits: uint16 [T][...] bit patterns of src_dtype rows."""
    k_bits, v_bits = _u16(k_bits), _u16(v_bits)
    T = k_bits.shape[0]
    ks = k_row_stride if k_row_stride is not None else k_bits.size // max(T, 1)
    vs = v_row_stride if v_row_stride is not None else v_bits.size // max(T, 1)
    slots = np.ascontiguousarray(slots, np.int64)
    sr = None if stage_rows is None else np.ascontiguousarray(stage_rows, np.int32)
    cs = cache.struct()
    rc = lib.orc_append(C.byref(L), C.byref(cs), _ptr(k_bits), _ptr(v_bits),
                        ks, vs, T, _ptr(slots), _ptr(sr))
    if rc:
        raise ValueError(f"orc_append: {rc}")


def append_static(L, cache, k_bits, v_bits, slots, k_scale, v_scale, k_zero=None,
                  v_zero=None, stage_rows=None):
    """Append with static scales: k_scale / v_scale float32 [H] (TOKEN_SYM),
    [H][d/gs] (GROUP_ASYM, with uint8 zero points of the same shape) or
    [H][d] (CHANNEL_BLOCK keys, with stage_rows as for append)."""
    k_bits, v_bits = _u16(k_bits), _u16(v_bits)
    T = k_bits.shape[0]
    ks, vs = k_bits.size // max(T, 1), v_bits.size // max(T, 1)
    slots = np.ascontiguousarray(slots, np.int64)
    arr = lambda a, t: None if a is None else np.ascontiguousarray(a, t)
    k_scale, v_scale = arr(k_scale, np.float32), arr(v_scale, np.float32)
    k_zero, v_zero = arr(k_zero, np.uint8), arr(v_zero, np.uint8)
    rows = None if stage_rows is None else np.ascontiguousarray(stage_rows, np.int32)
    cs = cache.struct()
    rc = lib.orc_append_static(C.byref(L), C.byref(cs), _ptr(k_bits), _ptr(v_bits),
                               ks, vs, T, _ptr(slots), _ptr(rows), _ptr(k_scale),
                               _ptr(k_zero), _ptr(v_scale), _ptr(v_zero))
    if rc:
        raise ValueError(f"orc_append_static: {rc}")


def quant_sym_static(x, qmax, s):
    x = np.ascontiguousarray(x, np.float32)
    q = np.zeros(x.size, np.int8)
    lib.orc_quant_sym_static(_ptr(x), x.size, qmax, s, _ptr(q))
    return q


def quant_fp8_static(x, s):
    x = np.ascontiguousarray(x, np.float32)
    q = np.zeros(x.size, np.uint8)
    lib.orc_quant_fp8_static(_ptr(x), x.size, s, _ptr(q))
    return q


def quant_asym4_static(x, s, z):
    x = np.ascontiguousarray(x, np.float32)
    q = np.zeros(x.size, np.uint8)
    lib.orc_quant_asym4_static(_ptr(x), x.size, s, z, _ptr(q))
    return q


def dequant_token(L, cache, side, table_row, context_len, stage_row, pos, head):
    out = np.zeros(L.head_dim, np.float32)
    tr = np.ascontiguousarray(table_row, np.int32)
    cs = cache.struct()
    rc = lib.orc_dequant_token(C.byref(L), C.byref(cs), side, _ptr(tr),
                               context_len, stage_row, pos, head, _ptr(out))
    if rc:
        raise ValueError(f"orc_dequant_token: {rc}")
    return out


def decode(L, cache, q, q_dtype, block_tables, context_lens, sm_scale=0.0,
           threads=1):
    """q: uint16 bits [B][Hq][d] (F16/BF16) or float32 (F32). Returns fp64."""
    q = np.ascontiguousarray(q)
    B, Hq, d = q.shape
    tables = np.ascontiguousarray(block_tables, np.int32)
    lens = np.ascontiguousarray(context_lens, np.int32)
    out = np.zeros((B, Hq, d), np.float64)
    cs = cache.struct()
    rc = lib.orc_decode(C.byref(L), C.byref(cs), _ptr(q), q_dtype, B, Hq,
                        _ptr(tables), tables.shape[1], _ptr(lens), sm_scale,
                        _ptr(out), threads)
    if rc:
        raise ValueError(f"orc_decode: {rc}")
    return out


def prefill(L, cache, q, q_dtype, query_start, block_tables, context_lens, sm_scale=0.0,
            threads=1, window=0, sink=0):
    """Multi-query attention: q uint16 bits [Tq][Hq][d], query_start int32
    [B+1] (sequence b's queries are its last query_start[b+1]-query_start[b]
    positions); window > 0 limits each query to its last `window` positions
    plus the first `sink`. Returns fp64 [Tq][Hq][d]."""
    q = np.ascontiguousarray(q)
    Tq, Hq, d = q.shape
    qs = np.ascontiguousarray(query_start, np.int32)
    tables = np.ascontiguousarray(block_tables, np.int32)
    lens = np.ascontiguousarray(context_lens, np.int32)
    assert qs[-1] == Tq
    out = np.zeros((Tq, Hq, d), np.float64)
    cs = cache.struct()
    rc = lib.orc_prefill(C.byref(L), C.byref(cs), _ptr(q), q_dtype, len(lens), Hq, _ptr(qs),
                         _ptr(tables), tables.shape[1], _ptr(lens), window, sink, sm_scale,
                         _ptr(out), threads)
    if rc:
        raise ValueError(f"orc_prefill: {rc}")
    return out


def decode_range(L, cache, q, q_dtype, b, h, table_row, context_len, t0, t1,
                 sm_scale=0.0):
    q = np.ascontiguousarray(q)
    Hq = q.shape[1]
    tr = np.ascontiguousarray(table_row, np.int32)
    m, l = C.c_double(), C.c_double()
    acc = np.zeros(L.head_dim, np.float64)
    cs = cache.struct()
    sm = sm_scale if sm_scale else 1.0 / np.sqrt(L.head_dim)
    rc = lib.orc_decode_range(C.byref(L), C.byref(cs), _ptr(q), q_dtype, Hq,
                              b, h, _ptr(tr), context_len, t0, t1, sm,
                              C.byref(m), C.byref(l), _ptr(acc))
    if rc:
        raise ValueError(f"orc_decode_range: {rc}")
    return m.value, l.value, acc


def quant_sym(x, qmax):
    x = np.ascontiguousarray(x, np.float32)
    q = np.zeros(x.size, np.int8)
    s = C.c_float()
    lib.orc_quant_sym(_ptr(x), x.size, qmax, _ptr(q), C.byref(s))
    return q, np.float32(s.value)


def quant_fp8(x):
    x = np.ascontiguousarray(x, np.float32)
    q = np.zeros(x.size, np.uint8)
    s = C.c_float()
    lib.orc_quant_fp8(_ptr(x), x.size, _ptr(q), C.byref(s))
    return q, np.float32(s.value)


def quant_asym4(x):
    x = np.ascontiguousarray(x, np.float32)
    q = np.zeros(x.size, np.uint8)
    s, z = C.c_float(), C.c_uint8()
    lib.orc_quant_asym4(_ptr(x), x.size, _ptr(q), C.byref(s), C.byref(z))
    return q, np.float32(s.value), int(z.value)


def quant_channel_block(x):
    x = np.ascontiguousarray(x, np.float32)
    bs, d = x.shape
    q = np.zeros((bs, d), np.int8)
    s = np.zeros(d, np.float32)
    lib.orc_quant_channel_block(_ptr(x), bs, d, _ptr(q), _ptr(s))
    return q, s


def int4_pack(nib):
    nib = np.ascontiguousarray(nib, np.uint8)
    out = np.zeros(nib.size // 2, np.uint8)
    lib.orc_int4_pack(_ptr(nib), nib.size, _ptr(out))
    return out


def int4_unpack(packed, d):
    packed = np.ascontiguousarray(packed, np.uint8)
    out = np.zeros(d, np.uint8)
    lib.orc_int4_unpack(_ptr(packed), d, _ptr(out))
    return out


def e4m3_value(code):
    return float(lib.orc_e4m3_value(int(code)))


def e4m3_encode(y):
    return int(lib.orc_e4m3_encode(float(y)))


def f16_to_f32(bits):
    return float(lib.orc_f16_to_f32(int(bits)))


def bf16_to_f32(bits):
    return float(lib.orc_bf16_to_f32(int(bits)))


def pool_init(num_blocks, order=None):
    stack = np.zeros(num_blocks, np.int32)
    top = np.zeros(1, np.int32)
    o = None if order is None else np.ascontiguousarray(order, np.int32)
    lib.orc_pool_init(_ptr(stack), _ptr(top), _ptr(o), num_blocks)
    return stack, top


def blocks_reserve(stack, top, tables, lens, new_tokens, bs, lens_out=None):
    """Mutates stack, top, tables (numpy) in place; returns (slots, status)."""
    lens = np.ascontiguousarray(lens, np.int32)
    new_tokens = np.ascontiguousarray(new_tokens, np.int32)
    slots = np.full(int(new_tokens.sum()), -7, np.int64)
    status = np.zeros(1, np.int32)
    rc = lib.orc_blocks_reserve(_ptr(stack), _ptr(top), stack.size, _ptr(tables),
                                tables.shape[1], _ptr(lens), _ptr(new_tokens),
                                lens.size, bs, _ptr(slots), _ptr(lens_out),
                                _ptr(status))
    assert rc == 0
    return slots, int(status[0])


def blocks_release(stack, top, tables, lens, mask, bs, lens_out=None):
    lens = np.ascontiguousarray(lens, np.int32)
    mask = np.ascontiguousarray(mask, np.int32)
    status = np.zeros(1, np.int32)
    rc = lib.orc_blocks_release(_ptr(stack), _ptr(top), stack.size, _ptr(tables),
                                tables.shape[1], _ptr(lens), _ptr(mask), lens.size,
                                bs, _ptr(lens_out), _ptr(status))
    assert rc == 0
    return int(status[0])


# ---- prefix sharing (block reference counts) ---------------------------------

def blocks_fork(refcount, tables, lens, src, dst, bs):
    """Mutates refcount, tables and lens (int32 numpy, in place)."""
    src = np.ascontiguousarray(src, np.int32)
    dst = np.ascontiguousarray(dst, np.int32)
    assert lens.dtype == np.int32 and lens.flags.c_contiguous
    rc = lib.orc_blocks_fork(_ptr(refcount), _ptr(tables), tables.shape[1], _ptr(lens),
                             _ptr(src), _ptr(dst), src.size, bs)
    assert rc == 0


def blocks_reserve_shared(stack, top, refcount, tables, lens, new_tokens, bs, lens_out=None):
    """Mutates stack, top, refcount, tables in place; returns (slots, status,
    cow_src, cow_dst) with the copy-on-write pairs in batch order."""
    lens = np.ascontiguousarray(lens, np.int32)
    new_tokens = np.ascontiguousarray(new_tokens, np.int32)
    slots = np.full(int(new_tokens.sum()), -7, np.int64)
    status = np.zeros(1, np.int32)
    cs = np.full(max(lens.size, 1), -7, np.int32)
    cd = np.full(max(lens.size, 1), -7, np.int32)
    cnt = np.zeros(1, np.int32)
    rc = lib.orc_blocks_reserve_shared(_ptr(stack), _ptr(top), stack.size, _ptr(refcount),
                                       _ptr(tables), tables.shape[1], _ptr(lens),
                                       _ptr(new_tokens), lens.size, bs, _ptr(slots),
                                       _ptr(lens_out), _ptr(cs), _ptr(cd), _ptr(cnt),
                                       _ptr(status))
    assert rc == 0
    n = int(cnt[0]) if status[0] == 0 else 0
    return slots, int(status[0]), cs[:n].copy(), cd[:n].copy()


def blocks_release_shared(stack, top, refcount, tables, lens, mask, bs, lens_out=None):
    lens = np.ascontiguousarray(lens, np.int32)
    mask = np.ascontiguousarray(mask, np.int32)
    status = np.zeros(1, np.int32)
    rc = lib.orc_blocks_release_shared(_ptr(stack), _ptr(top), stack.size, _ptr(refcount),
                                       _ptr(tables), tables.shape[1], _ptr(lens), _ptr(mask),
                                       lens.size, bs, _ptr(lens_out), _ptr(status))
    assert rc == 0
    return int(status[0])


def copy_blocks(L, cache, src, dst):
    src = np.ascontiguousarray(src, np.int32)
    dst = np.ascontiguousarray(dst, np.int32)
    cs = cache.struct()
    rc = lib.orc_copy_blocks(C.byref(L), C.byref(cs), _ptr(src), _ptr(dst), src.size)
    assert rc == 0


def blocks_trim(stack, top, tables, lens, window, sink, bs):
    """Mutates stack, top, tables in place; returns the status."""
    lens = np.ascontiguousarray(lens, np.int32)
    status = np.zeros(1, np.int32)
    rc = lib.orc_blocks_trim(_ptr(stack), _ptr(top), stack.size, _ptr(tables), tables.shape[1],
                             _ptr(lens), window, sink, lens.size, bs, _ptr(status))
    assert rc == 0
    return int(status[0])


def block_pack_bytes(L):
    return int(lib.orc_block_pack_bytes(C.byref(L)))


def pack_blocks(L, cache, ids):
    ids = np.ascontiguousarray(ids, np.int32)
    out = np.zeros(block_pack_bytes(L) * ids.size, np.uint8)
    cs = cache.struct()
    rc = lib.orc_pack_blocks(C.byref(L), C.byref(cs), _ptr(ids), ids.size, _ptr(out))
    if rc:
        raise ValueError(f"orc_pack_blocks: {rc}")
    return out


def unpack_blocks(L, cache, packed, ids):
    ids = np.ascontiguousarray(ids, np.int32)
    packed = np.ascontiguousarray(packed, np.uint8)
    cs = cache.struct()
    rc = lib.orc_unpack_blocks(C.byref(L), C.byref(cs), _ptr(packed), _ptr(ids), ids.size)
    if rc:
        raise ValueError(f"orc_unpack_blocks: {rc}")
