"""The Python binding checks every tensor before a pointer reaches the C ABI:
dtype, shape, size and inner contiguity first, device last. Each case below
breaks exactly one property of an otherwise valid call and expects the
ValueError that names the argument; no call here reaches the library's
kernels (host-side only, no GPU needed)."""
import pytest
import torch

kq = pytest.importorskip("quantized_paged_kv_append_amd")

H, D, BS = 2, 64, 16


def _layout(k_mode="token_sym", k_code="int8", dtype=torch.float16):
    return kq.make_layout(H, D, BS, k_code, k_mode=k_mode, src_dtype=dtype)


class _HostCache(kq.PagedCache):
    """A PagedCache whose planes live on the host: its layout fields are real,
    so every check before the device check can be reached."""

    def __init__(self, layout, num_blocks=8, max_seqs=0):
        super().__init__(layout, num_blocks, max_seqs, device="cpu")


def _append_args(T=4, dtype=torch.float16):
    k = torch.zeros(T, H, D, dtype=dtype)
    v = torch.zeros(T, H, D, dtype=dtype)
    slots = torch.arange(T, dtype=torch.int64)
    return k, v, slots


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_append_checks():
    L = _layout()
    c = _HostCache(L)
    k, v, slots = _append_args()
    _raises("^k: dtype bfloat16", kq.kvq_append, L, c, k.bfloat16(), v, slots)
    _raises("^v: dtype float32", kq.kvq_append, L, c, k, v.float(), slots)
    _raises("^slot_mapping: dtype int32", kq.kvq_append, L, c, k, v, slots.int())
    _raises("^slot_mapping: 3 elements", kq.kvq_append, L, c, k, v, slots[:3])
    _raises(r"^k: shape \(4, 2, 32\)", kq.kvq_append, L, c, k[:, :, :32], v, slots)
    # a strided inner dimension is refused; strided rows are fine up to the device check
    _raises(r"^k: shape \(4, 2, 64\) strides", kq.kvq_append, L, c, k.transpose(1, 2)
            .contiguous().transpose(1, 2), v, slots)
    wide = torch.zeros(4, 3 * H * D, dtype=torch.float16)
    _raises("^cache plane k_codes: must be a CUDA", kq.kvq_append, L, c, wide[:, :H * D], v, slots)
    _raises("^v: 3 rows, expected 4", kq.kvq_append, L, c, k, v[:3], slots)
    _raises("^stage_rows: only for per-channel", kq.kvq_append, L, c, k, v, slots,
            torch.zeros(4, dtype=torch.int32))
    # a cache made for another layout
    c8 = _HostCache(_layout(k_code="fp8"))
    _raises("^cache: made for a layout with k_code", kq.kvq_append, L, c8, k, v, slots)
    # everything right but on the host
    _raises("^cache plane k_codes: must be a CUDA", kq.kvq_append, L, c, k, v, slots)


def test_append_channel_keys_need_stage_rows():
    L = _layout(k_mode="channel_block")
    c = _HostCache(L, max_seqs=2)
    k, v, slots = _append_args()
    _raises("^stage_rows: a tensor is required", kq.kvq_append, L, c, k, v, slots)
    _raises("^stage_rows: dtype int64", kq.kvq_append, L, c, k, v, slots,
            torch.zeros(4, dtype=torch.int64))
    _raises("^stage_rows: 2 elements", kq.kvq_append, L, c, k, v, slots,
            torch.zeros(2, dtype=torch.int32))


def test_append_static_checks():
    L = _layout()
    c = _HostCache(L)
    k, v, slots = _append_args()
    ks = torch.ones(H)
    _raises("^k_scales: dtype float16", kq.kvq_append_static, L, c, k, v, slots, ks.half(), ks)
    _raises("^v_scales: 3 elements", kq.kvq_append_static, L, c, k, v, slots, ks,
            torch.ones(3))
    _raises("^k_zeros: a tensor is required", kq.kvq_append_static,
            kq.make_layout(H, D, BS, "int4", k_mode="group_asym", group_size=32,
                           src_dtype=torch.float16),
            _HostCache(kq.make_layout(H, D, BS, "int4", k_mode="group_asym", group_size=32,
                                      src_dtype=torch.float16)),
            k, v, slots, torch.ones(H * 2), torch.ones(H * 2))


def _decode_args(B=2, Hq=4):
    q = torch.zeros(B, Hq, D, dtype=torch.float16)
    tables = torch.zeros(B, 8, dtype=torch.int32)
    lens = torch.zeros(B, dtype=torch.int32)
    out = torch.zeros(B, Hq, D, dtype=torch.float32)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    return q, tables, lens, out, ws


def test_decode_checks():
    L = _layout()
    c = _HostCache(L)
    q, tables, lens, out, ws = _decode_args()
    call = kq.kvq_decode_attention
    _raises("^q: dtype float32", call, L, c, q.float(), tables, lens, 16, out, ws)
    _raises("^q: head dim 32", call, L, c, q[:, :, :32].contiguous(), tables, lens, 16,
            out[:, :, :32].contiguous(), ws)
    _raises("^q: must be contiguous", call, L, c, q.transpose(0, 1), tables, lens, 16, out, ws)
    _raises("^context_lens: dtype int64", call, L, c, q, tables, lens.long(), 16, out, ws)
    _raises("^q: 2 rows, context_lens has 3", call, L, c, q, tables,
            torch.zeros(3, dtype=torch.int32), 16, out, ws)
    _raises("^block_tables: dtype int64", call, L, c, q, tables.long(), lens, 16, out, ws)
    _raises("^block_tables: 1 rows", call, L, c, q, tables[:1], lens, 16, out, ws)
    _raises("^out: dtype int32", call, L, c, q, tables, lens, 16, out.int(), ws)
    _raises(r"^out: shape \(2, 4, 32\)", call, L, c, q, tables, lens, 16,
            out[:, :, :32].contiguous(), ws)
    _raises("^cache plane k_codes: must be a CUDA", call, L, c, q, tables, lens, 16, out, ws)


def test_prefill_checks():
    L = _layout()
    c = _HostCache(L)
    q, tables, lens, out, ws = _decode_args()
    qs = torch.tensor([0, 1, 2], dtype=torch.int32)
    call = kq.kvq_prefill_attention
    _raises("^query_start: dtype int64", call, L, c, q, qs.long(), 1, tables, lens, 16, out, ws)
    _raises("^query_start: 2 elements", call, L, c, q, qs[:2], 1, tables, lens, 16, out, ws)
    _raises("^cache plane k_codes: must be a CUDA", call, L, c, q, qs, 1, tables, lens, 16, out, ws)


def test_pool_checks():
    stack = torch.zeros(16, dtype=torch.int32)
    top = torch.zeros(1, dtype=torch.int32)
    _raises("^free_stack: dtype int64", kq.kvq_pool_init, stack.long(), top)
    _raises("^initial_order: 15 elements", kq.kvq_pool_init, stack, top,
            torch.zeros(15, dtype=torch.int32))
    tables = torch.zeros(2, 4, dtype=torch.int32)
    lens = torch.zeros(2, dtype=torch.int32)
    new = torch.tensor([3, 5], dtype=torch.int32)
    status = torch.zeros(1, dtype=torch.int32)
    res = kq.kvq_blocks_reserve
    _raises("^slot_mapping_out: dtype int32", res, stack, top, tables, lens, new, BS,
            torch.zeros(8, dtype=torch.int32), status)
    # a slot_mapping_out shorter than sum(new_tokens) is refused on the device
    # (status flag), not here: test_gpu_pool.py
    _raises("^new_tokens: 1 elements", res, stack, top, tables, lens, new[:1], BS,
            torch.zeros(8, dtype=torch.int64), status)
    _raises("^status_flag: dtype int64", res, stack, top, tables, lens, new, BS,
            torch.zeros(8, dtype=torch.int64), status.long())
    _raises("^free_stack: must be a CUDA", res, stack, top, tables, lens, new, BS,
            torch.zeros(8, dtype=torch.int64), status)
    rel = kq.kvq_blocks_release
    _raises("^release_mask: dtype bool", rel, stack, top, tables, lens,
            torch.zeros(2, dtype=torch.bool), BS, status)


def test_offload_checks():
    L = _layout()
    c = _HostCache(L)
    per = kq.kvq_block_pack_bytes(L)
    ids = torch.arange(3, dtype=torch.int32)
    _raises("^ids: dtype int64", kq.kvq_pack_blocks, L, c, ids.long(),
            torch.zeros(3 * per, dtype=torch.uint8))
    _raises(f"^dst: {3 * per - 1} bytes", kq.kvq_pack_blocks, L, c, ids,
            torch.zeros(3 * per - 1, dtype=torch.uint8))
    _raises(f"^src: {2 * per} bytes", kq.kvq_unpack_blocks, L, c,
            torch.zeros(2 * per, dtype=torch.uint8), ids)
    _raises("^cache plane k_codes: must be a CUDA", kq.kvq_pack_blocks, L, c, ids,
            torch.zeros(3 * per, dtype=torch.uint8))
