"""Pins of the oracle's block pack / unpack (the offload format): the packed
size against the pages' bytes-per-token closed form (a block holds bs
tokens), 2x and 4x fewer bytes than the 16-bit cache for 8- and 4-bit codes,
the packed layout by brute force, and a round trip through a pack that
restores a cache into other blocks with decode unchanged. No GPU."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import CODE, MODE, DT, OracleSeqs, bits, oracle_layout


def _layout(code, mode, bs=16, H=8, d=128, vcode=None, vmode=None):
    return ref.layout(H, d, bs, CODE[code], CODE[vcode or code], MODE[mode],
                      MODE[vmode or mode], 32 if mode == "group_asym" else 0, ref.BF16)


@pytest.mark.parametrize("code,mode,bs", [("none16", "token_sym", 16), ("int8", "token_sym", 16),
                                          ("fp8", "token_sym", 32), ("int4", "token_sym", 16),
                                          ("int4", "group_asym", 32)])
def test_pack_size_is_bytes_per_token_times_block(code, mode, bs):
    L = _layout(code, mode, bs)
    assert ref.block_pack_bytes(L) == ref.bytes_per_token(L, 1, include_metadata=1) * bs


def test_pack_size_per_channel_keys_and_ratios():
    Lc = _layout("int8", "channel_block", 16, vcode="int8", vmode="token_sym")
    # per-channel key scales: one float per (head, channel) per block
    assert ref.block_pack_bytes(Lc) == 8 * 16 * 128 * 2 + 8 * 128 * 4 + 8 * 16 * 4
    b16 = ref.block_pack_bytes(_layout("none16", "token_sym"))
    assert b16 == 2 * 8 * 16 * 128 * 2
    r8 = b16 / ref.block_pack_bytes(_layout("fp8", "token_sym"))
    r4 = b16 / ref.block_pack_bytes(_layout("int4", "group_asym", 16))
    assert 1.9 < r8 < 2.0 and 3.0 < r4 < 4.0


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("int4", "group_asym"),
                                       ("int8", "channel_block")])
def test_pack_layout_and_round_trip(code, mode):
    bs = 16
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode,
                      v_mode="token_sym" if mode == "channel_block" else mode,
                      group_size=32 if mode == "group_asym" else 0, block_size=bs, head_dim=64,
                      num_kv_heads=2, num_q_heads=8, batch=2, src_dtype="bfloat16")
    L = oracle_layout(w)
    lens = np.array([40, 37], np.int32)
    s = OracleSeqs(L, 12, 2, 4, order=np.random.default_rng(2).permutation(12).astype(np.int32),
                   max_seqs=2)
    k, v = workloads.kv_rows(w, int(lens.sum()), seed=1)
    s.append(k, v, lens)
    ids = s.tables[:, :3].reshape(-1)
    ids = ids[ids >= 0]
    packed = ref.pack_blocks(L, s.cache, ids)
    per = ref.block_pack_bytes(L)
    assert packed.size == per * len(ids)
    # brute force: block k's slice of each plane, in plane order
    H = 2
    for kk, bid in enumerate(ids):
        off = kk * per
        for name in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
            plane = s.cache.planes[name]
            if plane is None:
                continue
            nbytes = plane.size // s.cache.num_blocks
            assert np.array_equal(packed[off:off + nbytes], plane[bid * nbytes:(bid + 1) * nbytes])
            off += nbytes
        assert off == (kk + 1) * per
    # restore into a fresh cache at other block ids: decode is unchanged
    fresh = ref.HostCache(L, 12, 2, fill=0xFF)
    fresh.planes["k_stage"] = s.cache.planes["k_stage"]
    new_ids = (ids + 5) % 12
    ref.unpack_blocks(L, fresh, packed, new_ids)
    remap = dict(zip(ids.tolist(), new_ids.tolist()))
    tables = np.vectorize(lambda x: remap.get(x, x))(s.tables).astype(np.int32)
    q = workloads.queries(w, seed=1)
    a = ref.decode(L, s.cache, bits(q), ref.BF16, s.tables, s.lens)
    b = ref.decode(L, fresh, bits(q), ref.BF16, tables, s.lens)
    assert np.array_equal(a, b)
