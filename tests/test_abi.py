"""The C-ABI library loads, exports every symbol include/kvq.h declares, and
its host-only entry points agree with the oracle and the pages' closed forms.
Argument errors are caught on the host before any launch, so these run
without a GPU."""
import ctypes as C
import json
import re
from pathlib import Path

import pytest
import torch

from oracle import ref

ROOT = Path(__file__).resolve().parents[1]
kq = pytest.importorskip("quantized_paged_kv_append_amd.kvq")


def _declared():
    text = (ROOT / "include" / "kvq.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 10
    lib = C.CDLL(kq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kq._SIGS), "binding must cover the header exactly"


def test_binding_constants_match_header():
    text = (ROOT / "include" / "kvq.h").read_text()
    for name, value in re.findall(r"#define\s+(KVQ_\w+)\s+\(?(-?\d+)\)?", text):
        assert getattr(kq, name) == int(value), name


def test_bytes_per_token_printed_and_oracle():
    g = json.loads((ROOT / "tests" / "golden" / "bytes_per_token.json").read_text())
    for bits, code in (("16", "none16"), ("8", "int8"), ("8", "fp8"), ("4", "int4")):
        L = kq.make_layout(8, 128, 16, code)
        assert kq.kvq_bytes_per_token(L, 80) == g["bytes_per_token"][bits]
    combos = [("int8", "token_sym", 16, 0), ("fp8", "token_sym", 32, 0),
              ("int4", "group_asym", 32, 32), ("int4", "token_sym", 16, 0),
              ("int8", "channel_block", 16, 0), ("none16", "token_sym", 16, 0)]
    cmap = {"none16": ref.CODE_NONE16, "int8": ref.CODE_INT8, "fp8": ref.CODE_FP8,
            "int4": ref.CODE_INT4}
    mmap = {"token_sym": ref.TOKEN_SYM, "group_asym": ref.GROUP_ASYM,
            "channel_block": ref.CHANNEL_BLOCK}
    for code, mode, bs, gs in combos:
        for H, d in ((8, 128), (2, 64), (5, 64)):
            L = kq.make_layout(H, d, bs, code, k_mode=mode, group_size=gs)
            OL = ref.layout(H, d, bs, cmap[code], k_mode=mmap[mode], group_size=gs)
            for layers in (1, 32, 80):
                for meta in (0, 1):
                    assert kq.kvq_bytes_per_token(L, layers, meta) == \
                        ref.bytes_per_token(OL, layers, meta)
            for nb, ms in ((1, 0), (37, 3)):
                assert kq.kvq_cache_plane_bytes(L, nb, ms) == ref.plane_bytes(OL, nb, ms)


def test_layout_check_errors():
    ok = kq.make_layout(8, 128, 16, "int8")
    assert kq.kvq_layout_check(ok) == kq.KVQ_OK
    bad = [kq.make_layout(0, 128, 16, "int8"), kq.make_layout(8, 96, 16, "int8"),
           kq.make_layout(8, 128, 24, "int8")]
    for L in bad:
        assert kq.kvq_layout_check(L) == kq.KVQ_ERR_INVALID_ARGUMENT
    L = kq.make_layout(8, 128, 16, "int8")
    L.reserved = 1
    assert kq.kvq_layout_check(L) == kq.KVQ_ERR_INVALID_ARGUMENT
    L = kq.make_layout(8, 128, 16, "int8")
    L.k_code = 9
    assert kq.kvq_layout_check(L) == kq.KVQ_ERR_INVALID_ARGUMENT
    unsupported = [kq.make_layout(8, 128, 16, "fp8", k_mode="group_asym", group_size=32),
                   kq.make_layout(8, 128, 16, "int4", k_mode="group_asym", group_size=64),
                   kq.make_layout(8, 128, 16, "int8", k_mode="token_sym", v_mode="channel_block"),
                   kq.make_layout(8, 128, 16, "fp8", k_mode="channel_block")]
    for L in unsupported:
        assert kq.kvq_layout_check(L) == kq.KVQ_ERR_UNSUPPORTED
    with pytest.raises(kq.KvqError):
        kq.kvq_bytes_per_token(ok, 0)
    assert kq.kvq_status_string(-5) == "KVQ_ERR_OUT_OF_BLOCKS"
    assert kq.kvq_status_string(42) == "KVQ_UNKNOWN_STATUS"


def test_workspace_size_is_pure_and_positive():
    L = kq.make_layout(8, 128, 16, "fp8")
    a = kq.kvq_decode_workspace_bytes(L, 16, 64, 32768)
    assert a == kq.kvq_decode_workspace_bytes(L, 16, 64, 32768) and a > 0
    assert kq.kvq_decode_workspace_bytes(L, 16, 64, 32768, 8) > a
    assert kq._lib.kvq_decode_workspace_bytes(C.byref(L), 16, 64, 32768, 257) == \
        kq.KVQ_ERR_INVALID_ARGUMENT
    assert kq._lib.kvq_decode_workspace_bytes(C.byref(L), -1, 64, 32768, 0) == \
        kq.KVQ_ERR_INVALID_ARGUMENT


def _fake_cache(L, nb=4):
    base = 1 << 20  # never dereferenced: the calls below fail their checks first
    s = kq.kvq_cache()
    s.k_codes, s.v_codes, s.k_scale, s.v_scale = base, base + 4096, base + 8192, base + 12288
    s.num_blocks = nb
    return s


def test_append_and_decode_reject_bad_arguments_on_host():
    L = kq.make_layout(8, 128, 16, "int8")
    cs = _fake_cache(L)
    lib = kq._lib
    p = C.c_void_p(1 << 21)
    # misaligned input
    assert lib.kvq_append(C.byref(L), C.byref(cs), C.c_void_p((1 << 21) + 2), p, 1024, 1024,
                          4, p, None, None) == kq.KVQ_ERR_INVALID_ARGUMENT
    # stride shorter than a row
    assert lib.kvq_append(C.byref(L), C.byref(cs), p, p, 512, 1024, 4, p, None,
                          None) == kq.KVQ_ERR_INVALID_ARGUMENT
    # stage rows given for a layout without per-channel keys
    assert lib.kvq_append(C.byref(L), C.byref(cs), p, p, 1024, 1024, 4, p, p,
                          None) == kq.KVQ_ERR_INVALID_ARGUMENT
    # a zero-point plane the layout does not use
    cz = _fake_cache(L)
    cz.k_zero = 1 << 22
    assert lib.kvq_append(C.byref(L), C.byref(cz), p, p, 1024, 1024, 4, p, None,
                          None) == kq.KVQ_ERR_INVALID_ARGUMENT
    # nothing to do
    assert lib.kvq_append(C.byref(L), C.byref(cs), None, None, 0, 0, 0, None, None,
                          None) == kq.KVQ_OK

    def dec(**kw):
        a = dict(q=p, q_dtype=kq.KVQ_BF16, batch=2, hq=32, tables=p, maxb=4, lens=p,
                 maxlen=64, sm=0.0, split=0, out=p, out_dtype=kq.KVQ_F32, ws=p,
                 wsb=1 << 30)
        a.update(kw)
        return lib.kvq_decode_attention(C.byref(L), C.byref(cs), a["q"], a["q_dtype"],
                                        a["batch"], a["hq"], a["tables"], a["maxb"],
                                        a["lens"], a["maxlen"], a["sm"], a["split"],
                                        a["out"], a["out_dtype"], a["ws"], a["wsb"], None)
    assert dec(hq=30) == kq.KVQ_ERR_INVALID_ARGUMENT           # Hq % H != 0
    assert dec(hq=8 * 17) == kq.KVQ_ERR_UNSUPPORTED             # group > 16
    assert dec(q_dtype=kq.KVQ_F32) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert dec(out_dtype=7) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert dec(maxlen=65) == kq.KVQ_ERR_INVALID_ARGUMENT        # > maxb * bs
    assert dec(split=257) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert dec(sm=float("nan")) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert dec(wsb=16) == kq.KVQ_ERR_WORKSPACE_TOO_SMALL
    assert dec(tables=None) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert dec(batch=0) == kq.KVQ_OK
    # a valid layout whose decode this library does not build: FP8 keys with
    # INT8 values
    Lmix = kq.make_layout(8, 128, 16, "fp8", v_code="int8")
    assert kq.kvq_layout_check(Lmix) == kq.KVQ_OK
    cmix = _fake_cache(Lmix)
    assert lib.kvq_decode_attention(C.byref(Lmix), C.byref(cmix), p, kq.KVQ_BF16, 2, 32, p, 4,
                                    p, 64, 0.0, 0, p, kq.KVQ_F32, p, 1 << 30,
                                    None) == kq.KVQ_ERR_UNSUPPORTED


def test_decode_noalloc_rejects_bad_arguments_on_host():
    """The allocation-free decode takes kvq_decode_attention's checks, and
    refuses sizes whose workspace exceeds its fixed per-GPU array before it
    touches the device."""
    L = kq.make_layout(8, 128, 16, "int8")
    lib = kq._lib
    p = C.c_void_p(1 << 21)

    def dec(**kw):
        a = dict(batch=2, hq=32, maxb=4, maxlen=64, tables=p)
        a.update(kw)
        cs = _fake_cache(L)
        return lib.kvq_decode_attention_noalloc(C.byref(L), C.byref(cs), p, kq.KVQ_BF16,
                                                a["batch"], a["hq"], a["tables"], a["maxb"], p,
                                                a["maxlen"], 0.0, 0, p, kq.KVQ_F32, None)
    assert dec(hq=30) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert dec(tables=None) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert dec(batch=0) == kq.KVQ_OK
    # a batch whose workspace bound is past KVQ_DECODE_SCRATCH_BYTES
    big_b, big_len = 4096, 1 << 20
    need = kq.kvq_decode_workspace_bytes(L, big_b, 32, big_len)
    assert need > kq.KVQ_DECODE_SCRATCH_BYTES
    assert dec(batch=big_b, maxb=big_len // 16, maxlen=big_len) == \
        kq.KVQ_ERR_WORKSPACE_TOO_SMALL
    # the workloads' shapes fit (the mixed step's 256 sequences of up to 32K
    # tokens is the largest)
    assert kq.kvq_decode_workspace_bytes(L, 256, 32, 33000) <= kq.KVQ_DECODE_SCRATCH_BYTES


def test_append_decode_rejects_bad_arguments_on_host():
    """The fused append + decode takes decode's checks, then its own: byte
    codes with per-token scales or 16-bit rows only, aligned new rows with
    strides of at least H * d elements, and room for the new token. Every
    call here fails, or returns for an empty batch, before touching the
    device."""
    lib = kq._lib
    p = C.c_void_p(1 << 21)

    def fused(L, batch=2, k=p, v=p, ks=1024, vs=1024, maxlen=64, hq=32, ws_bytes=1 << 30):
        cs = _fake_cache(L)
        if L.k_mode == kq.KVQ_SCALE_GROUP_ASYM:
            cs.k_zero, cs.v_zero = 1 << 22, 1 << 23
        if L.k_mode == kq.KVQ_SCALE_CHANNEL_BLOCK_SYM:
            cs.k_stage, cs.max_seqs = 1 << 24, 4
        return lib.kvq_append_decode_attention(C.byref(L), C.byref(cs), k, v, ks, vs, p,
                                               kq.KVQ_BF16, batch, hq, p, 4, p, maxlen, 0.0, 0,
                                               p, kq.KVQ_F32, p, ws_bytes, None)
    L8 = kq.make_layout(8, 128, 16, "int8")
    assert fused(L8, batch=0) == kq.KVQ_OK
    assert fused(L8, k=None) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert fused(L8, v=C.c_void_p((1 << 21) + 8)) == kq.KVQ_ERR_INVALID_ARGUMENT  # misaligned
    assert fused(L8, ks=8 * 128 - 8) == kq.KVQ_ERR_INVALID_ARGUMENT     # stride below H*d
    assert fused(L8, vs=1028) == kq.KVQ_ERR_INVALID_ARGUMENT            # not 16-byte rows
    assert fused(L8, maxlen=0) == kq.KVQ_ERR_INVALID_ARGUMENT           # no new token fits
    assert fused(L8, hq=30) == kq.KVQ_ERR_INVALID_ARGUMENT              # decode's own check
    assert fused(L8, ws_bytes=16) == kq.KVQ_ERR_WORKSPACE_TOO_SMALL
    # layouts the one-launch path does not code: 4-bit, per-channel keys
    for L in (kq.make_layout(8, 128, 32, "int4", k_mode="group_asym", group_size=32),
              kq.make_layout(8, 128, 16, "int4"),
              kq.make_layout(8, 128, 16, "int8", k_mode="channel_block", v_mode="token_sym")):
        assert kq.kvq_layout_check(L) == kq.KVQ_OK
        assert fused(L) == kq.KVQ_ERR_UNSUPPORTED


def test_append_static_rejects_bad_arguments_on_host():
    lib = kq._lib
    p = C.c_void_p(1 << 21)
    sc, zp = C.c_void_p(1 << 23), C.c_void_p(1 << 24)

    def app(L, cs, ks, kz, vs, vz, T=4, rows=None):
        return lib.kvq_append_static(C.byref(L), C.byref(cs), p, p, 1024, 1024, T, p,
                                     rows, ks, kz, vs, vz, None)
    L = kq.make_layout(8, 128, 16, "int8")
    cs = _fake_cache(L)
    assert app(L, cs, sc, None, sc, None, T=0) == kq.KVQ_OK
    assert app(L, cs, None, None, sc, None) == kq.KVQ_ERR_INVALID_ARGUMENT   # no key scales
    assert app(L, cs, sc, zp, sc, None) == kq.KVQ_ERR_INVALID_ARGUMENT       # zero for symmetric
    assert app(L, cs, C.c_void_p((1 << 23) + 2), None, sc, None) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert app(L, cs, sc, None, sc, None, T=-1) == kq.KVQ_ERR_INVALID_ARGUMENT
    La = kq.make_layout(8, 128, 32, "int4", k_mode="group_asym", group_size=32)
    ca = _fake_cache(La)
    ca.k_zero, ca.v_zero = 1 << 25, (1 << 25) + 4096
    assert app(La, ca, sc, zp, sc, zp, T=0) == kq.KVQ_OK
    assert app(La, ca, sc, None, sc, zp) == kq.KVQ_ERR_INVALID_ARGUMENT      # asym needs zeros
    # a 16-bit side takes no parameters
    Ln = kq.make_layout(8, 128, 16, "fp8", v_code="none16")
    cn = _fake_cache(Ln)
    cn.v_scale = None
    assert app(Ln, cn, sc, None, None, None, T=0) == kq.KVQ_OK
    assert app(Ln, cn, sc, None, sc, None) == kq.KVQ_ERR_INVALID_ARGUMENT
    # per-channel keys: stage rows required, [H][d] scales 16-byte aligned
    Lc = kq.make_layout(8, 128, 16, "int8", k_mode="channel_block")
    cc = _fake_cache(Lc)
    cc.k_stage, cc.max_seqs = 1 << 26, 4
    assert app(Lc, cc, sc, None, sc, None, T=0, rows=p) == kq.KVQ_OK
    assert app(Lc, cc, sc, None, sc, None) == kq.KVQ_ERR_INVALID_ARGUMENT          # no rows
    assert app(Lc, cc, C.c_void_p((1 << 23) + 4), None, sc, None,
               rows=p) == kq.KVQ_ERR_INVALID_ARGUMENT                              # alignment
    assert app(L, cs, sc, None, sc, None, rows=p) == kq.KVQ_ERR_INVALID_ARGUMENT   # rows unused


def test_prefill_rejects_bad_arguments_on_host():
    L = kq.make_layout(8, 128, 16, "int8")
    cs = _fake_cache(L)
    lib = kq._lib
    p = C.c_void_p(1 << 21)

    def pre(**kw):
        a = dict(q=p, q_dtype=kq.KVQ_BF16, batch=2, hq=32, qs=p, maxq=8, tables=p, maxb=4,
                 lens=p, maxlen=64, sm=0.0, split=0, out=p, out_dtype=kq.KVQ_F32, ws=p,
                 wsb=1 << 30, L=L, cs=cs)
        a.update(kw)
        return lib.kvq_prefill_attention(C.byref(a["L"]), C.byref(a["cs"]), a["q"], a["q_dtype"],
                                         a["batch"], a["hq"], a["qs"], a["maxq"], a["tables"],
                                         a["maxb"], a["lens"], a["maxlen"], a["sm"],
                                         a.get("window", 0), a.get("sink", 0), a["split"],
                                         a["out"], a["out_dtype"], a["ws"], a["wsb"], None)
    assert pre(hq=30) == kq.KVQ_ERR_INVALID_ARGUMENT            # Hq % H
    assert pre(maxq=65) == kq.KVQ_ERR_INVALID_ARGUMENT          # more queries than context
    assert pre(maxlen=65) == kq.KVQ_ERR_INVALID_ARGUMENT        # > maxb * bs
    assert pre(split=-1) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert pre(split=257) == kq.KVQ_ERR_INVALID_ARGUMENT        # a split's ids fit in LDS
    with pytest.raises(kq.KvqError):
        kq.kvq_prefill_workspace_bytes(L, 2, 32, 8, 4096, 257)
    assert pre(qs=None) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert pre(q=C.c_void_p((1 << 21) + 2)) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert pre(wsb=16) == kq.KVQ_ERR_WORKSPACE_TOO_SMALL
    assert pre(sm=float("inf")) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert pre(batch=0) == kq.KVQ_OK and pre(maxq=0) == kq.KVQ_OK
    assert pre(window=-1) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert pre(window=8, sink=-2) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert lib.kvq_blocks_trim(p, p, 64, p, 4, p, -1, 0, 2, 16, p, None) == \
        kq.KVQ_ERR_INVALID_ARGUMENT
    Lm = kq.make_layout(8, 128, 16, "int8", v_code="fp8")   # mixed codes: no kernel
    assert kq.kvq_layout_check(Lm) == kq.KVQ_OK
    assert pre(L=Lm, cs=_fake_cache(Lm)) == kq.KVQ_ERR_UNSUPPORTED
    # workspace grows with the query count and shrinks with longer splits
    w1 = kq.kvq_prefill_workspace_bytes(L, 2, 32, 8, 4096, 0)
    assert kq.kvq_prefill_workspace_bytes(L, 2, 32, 16, 4096, 0) > w1
    assert kq.kvq_prefill_workspace_bytes(L, 2, 32, 8, 4096, 256) < w1


def test_sharing_calls_reject_bad_arguments_on_host():
    lib = kq._lib
    p = C.c_void_p(1 << 21)
    assert lib.kvq_blocks_fork(None, 64, p, 4, p, 2, p, p, 1, 16, None) == \
        kq.KVQ_ERR_INVALID_ARGUMENT                                  # no counts
    assert lib.kvq_blocks_fork(p, 64, p, 4, p, 2, p, p, 0, 16, None) == kq.KVQ_OK
    assert lib.kvq_blocks_fork(p, 64, None, 4, p, 2, p, p, 1, 16, None) == \
        kq.KVQ_ERR_INVALID_ARGUMENT
    assert lib.kvq_blocks_reserve_shared(p, p, 64, p, p, 4, p, p, 2, 16, p, 8, None, None, p, p,
                                         p, None) == kq.KVQ_ERR_INVALID_ARGUMENT   # no copy pairs
    assert lib.kvq_blocks_reserve_shared(p, p, 64, None, p, 4, p, p, 2, 16, p, 8, None, p, p, p,
                                         p, None) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert lib.kvq_blocks_reserve_shared(p, p, 64, p, p, 4, p, p, 2, 16, p, -1, None, p, p, p,
                                         p, None) == kq.KVQ_ERR_INVALID_ARGUMENT   # slot count
    assert lib.kvq_blocks_release_shared(p, p, 0, p, p, 4, p, p, 2, 16, None, p, None) == \
        kq.KVQ_ERR_INVALID_ARGUMENT                                  # empty pool
    L = kq.make_layout(8, 128, 16, "int8")
    cs = _fake_cache(L)
    assert lib.kvq_copy_blocks(C.byref(L), C.byref(cs), p, p, p, 0, None) == kq.KVQ_OK
    assert lib.kvq_copy_blocks(C.byref(L), C.byref(cs), None, p, p, 4, None) == \
        kq.KVQ_ERR_INVALID_ARGUMENT


def test_block_pack_bytes_match_oracle():
    from itertools import product
    for code, mode, bs, d in product(["none16", "int8", "fp8", "int4"],
                                     ["token_sym", "group_asym", "channel_block"], [16, 32],
                                     [64, 128]):
        if mode == "group_asym" and code != "int4":
            continue
        if mode == "channel_block" and code != "int8":
            continue
        vmode = "token_sym" if mode == "channel_block" else mode
        L = kq.make_layout(4, d, bs, code, k_mode=mode, v_mode=vmode,
                           group_size=32 if mode == "group_asym" else 0)
        OL = ref.layout(4, d, bs, {"none16": 0, "int8": 1, "fp8": 2, "int4": 3}[code],
                        None, {"token_sym": 0, "group_asym": 1, "channel_block": 2}[mode],
                        {"token_sym": 0, "group_asym": 1}[vmode],
                        32 if mode == "group_asym" else 0, ref.BF16)
        assert kq.kvq_block_pack_bytes(L) == ref.block_pack_bytes(OL), (code, mode, bs, d)


def test_pool_calls_reject_bad_arguments_on_host():
    lib = kq._lib
    p = C.c_void_p(1 << 21)
    assert lib.kvq_pool_init(None, p, None, 16, None) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert lib.kvq_pool_init(p, p, None, 0, None) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert lib.kvq_blocks_reserve(p, p, 16, p, 4, p, p, 2, 16, p, 8, None, None,
                                  None) == kq.KVQ_ERR_INVALID_ARGUMENT   # no status
    assert lib.kvq_blocks_reserve(p, p, 16, None, 4, p, p, 2, 16, p, 8, None, p,
                                  None) == kq.KVQ_ERR_INVALID_ARGUMENT
    assert lib.kvq_blocks_reserve(p, p, 16, p, 4, p, p, 2, 16, p, -1, None, p,
                                  None) == kq.KVQ_ERR_INVALID_ARGUMENT   # negative slot count
    assert lib.kvq_blocks_reserve(p, p, 16, p, 4, p, p, 2, 16, None, 8, None, p,
                                  None) == kq.KVQ_ERR_INVALID_ARGUMENT   # slots without buffer
    assert lib.kvq_blocks_release(p, p, 16, p, 4, p, None, 2, 16, None, p,
                                  None) == kq.KVQ_ERR_INVALID_ARGUMENT


def test_check_calls_reject_bad_arguments_on_host():
    lib = kq._lib
    p = C.c_void_p(1 << 21)
    bad = kq.KVQ_ERR_INVALID_ARGUMENT
    assert lib.kvq_check_block_tables(p, 4, p, 2, 16, 100, None, p, None) == bad   # no first_bad
    assert lib.kvq_check_block_tables(p, 4, p, 2, 16, 100, p, None, None) == bad   # no status
    assert lib.kvq_check_block_tables(p, 4, p, 2, 16, 0, p, p, None) == bad        # empty pool
    assert lib.kvq_check_block_tables(None, 4, p, 2, 16, 100, p, p, None) == bad
    assert lib.kvq_check_block_tables(p, 0, p, 2, 16, 100, p, p, None) == bad
    assert lib.kvq_check_slots(p, 8, 100, 16, p, None, None) == bad
    assert lib.kvq_check_slots(None, 8, 100, 16, p, p, None) == bad
    assert lib.kvq_check_slots(p, -1, 100, 16, p, p, None) == bad
    assert lib.kvq_check_slots(p, 8, 100, 0, p, p, None) == bad


def test_read_probe_rejects_bad_arguments_on_host():
    lib = kq._lib
    p = C.c_void_p(1 << 21)
    bad = kq.KVQ_ERR_INVALID_ARGUMENT
    assert lib.kvq_read_probe(None, 1 << 20, p, None) == bad            # no buffer
    assert lib.kvq_read_probe(p, 1 << 20, None, None) == bad            # no sink
    assert lib.kvq_read_probe(p, 0, p, None) == bad                     # nothing to read
    assert lib.kvq_read_probe(p, 24, p, None) == bad                    # not whole words
    assert lib.kvq_read_probe(C.c_void_p((1 << 21) + 8), 64, p, None) == bad  # misaligned
