"""Pins of the oracle's multi-query (prefill) attention: the 16-bit cache
against torch's scaled_dot_product_attention in fp64 with an explicit causal
mask (a library routine), quantized caches against the same routine over the
dequantized rows, one query per sequence against decode, and each query
against decode over its own prefix. No GPU."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads
from oracle import ref
from _util import DT, OracleSeqs, bits, oracle_layout


def _case(code="int8", mode="token_sym", lens=(37, 80, 5, 17), nq=(5, 16, 5, 1), Hq=8, H=2,
          d=64, bs=16, src="bfloat16", seed=0):
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode,
                      v_mode="token_sym" if mode == "channel_block" else mode,
                      group_size=32 if mode == "group_asym" else 0, block_size=bs,
                      src_dtype=src, num_q_heads=Hq, num_kv_heads=H, head_dim=d,
                      batch=len(lens))
    L = oracle_layout(w)
    lens = np.asarray(lens, np.int32)
    T = int(lens.sum())
    g = torch.Generator().manual_seed(seed)
    k = (torch.randn((T, H, d), generator=g) * 3).to(w.torch_dtype)
    v = torch.randn((T, H, d), generator=g).to(w.torch_dtype)
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = torch.randn((int(qs[-1]), Hq, d), generator=g).to(w.torch_dtype)
    s = OracleSeqs(L, workloads.pool_blocks(lens, bs) + 3, len(lens), int(lens.max()) // bs + 2,
                   max_seqs=len(lens))
    s.append(k, v, lens)
    return w, L, s, k, v, q, qs


def _rows(L, s, side, b, h):
    """Dequantized rows of sequence b, KV head h (the oracle's own reading)."""
    Lb = int(s.lens[b])
    return np.stack([ref.dequant_token(L, s.cache, side, s.tables[b], Lb, b, t, h)
                     for t in range(Lb)]) if Lb else np.zeros((0, L.head_dim), np.float32)


def _sdpa_causal(q, K, V, qs, lens, Hq, H):
    """SDPA in fp64 per sequence; K[b], V[b]: [H][L][d]. Query i of sequence
    b sees positions 0 .. L - nq + i."""
    out = np.zeros((q.shape[0], Hq, q.shape[2]))
    G = Hq // H
    for b, Lb in enumerate(lens):
        nq = qs[b + 1] - qs[b]
        if nq == 0:
            continue
        kk = torch.from_numpy(K[b]).double().repeat_interleave(G, 0).contiguous()
        vv = torch.from_numpy(V[b]).double().repeat_interleave(G, 0).contiguous()
        qq = q[qs[b]:qs[b + 1]].double().transpose(0, 1).contiguous()   # [Hq][nq][d]
        pos = torch.arange(Lb)
        qpos = Lb - nq + torch.arange(nq)
        mask = pos[None, :] <= qpos[:, None]                            # [nq][L]
        o = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
        out[qs[b]:qs[b + 1]] = o.transpose(0, 1).numpy()
    return out


@pytest.mark.parametrize("src", ["float16", "bfloat16"])
@pytest.mark.parametrize("Hq,H", [(8, 2), (4, 4)])
def test_passthrough_prefill_equals_causal_sdpa(src, Hq, H):
    w, L, s, k, v, q, qs = _case("none16", src=src, Hq=Hq, H=H)
    got = ref.prefill(L, s.cache, bits(q), DT[src], qs, s.tables, s.lens, threads=4)
    K, V, start = [], [], 0
    for Lb in s.lens:
        K.append(k[start:start + Lb].double().transpose(0, 1).numpy())
        V.append(v[start:start + Lb].double().transpose(0, 1).numpy())
        start += Lb
    exp = _sdpa_causal(q, K, V, qs, s.lens, Hq, H)
    assert np.abs(got - exp).max() < 1e-12


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("fp8", "token_sym"),
                                       ("int4", "group_asym"), ("int8", "channel_block")])
def test_quantized_prefill_equals_causal_sdpa_on_dequantized_rows(code, mode):
    w, L, s, k, v, q, qs = _case(code, mode, bs=32 if mode == "group_asym" else 16)
    got = ref.prefill(L, s.cache, bits(q), ref.BF16, qs, s.tables, s.lens, threads=4)
    K = [np.stack([_rows(L, s, 0, b, h) for h in range(2)]) for b in range(len(s.lens))]
    V = [np.stack([_rows(L, s, 1, b, h) for h in range(2)]) for b in range(len(s.lens))]
    exp = _sdpa_causal(q, K, V, qs, s.lens, 8, 2)
    assert np.abs(got - exp).max() < 1e-12


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("int8", "channel_block")])
def test_one_query_per_sequence_is_decode(code, mode):
    w, L, s, k, v, q, qs = _case(code, mode, nq=(1, 1, 1, 1))
    got = ref.prefill(L, s.cache, bits(q), ref.BF16, qs, s.tables, s.lens, threads=2)
    exp = ref.decode(L, s.cache, bits(q), ref.BF16, s.tables, s.lens, threads=2)
    assert np.array_equal(got, exp)


def test_each_query_is_decode_over_its_prefix():
    # Per-token scales: dequantized values do not depend on the length, so
    # query i equals decode over the first L - nq + i + 1 positions.
    w, L, s, k, v, q, qs = _case("fp8", lens=(40, 21), nq=(9, 21))
    got = ref.prefill(L, s.cache, bits(q), ref.BF16, qs, s.tables, s.lens, threads=2)
    for b in range(2):
        nq = qs[b + 1] - qs[b]
        for i in range(nq):
            r = qs[b] + i
            lens = s.lens.copy()
            lens[b] = s.lens[b] - nq + i + 1
            qb = np.repeat(bits(q[r:r + 1]), 2, 0)
            exp = ref.decode(L, s.cache, qb, ref.BF16, s.tables, lens)
            assert np.array_equal(got[r], exp[b]), (b, i)


def test_sequences_without_queries_and_bad_counts():
    w, L, s, k, v, q, qs = _case("int8", nq=(0, 3, 0, 2))
    got = ref.prefill(L, s.cache, bits(q), ref.BF16, qs, s.tables, s.lens)
    w2, L2, s2, k2, v2, q2, qs2 = _case("int8", nq=(1, 3, 1, 2))
    # rows of sequences 1 and 3 are the same queries in both calls
    q2 = q2.clone()
    q2[1:4] = q[0:3]
    q2[5:7] = q[3:5]
    got2 = ref.prefill(L2, s2.cache, bits(q2), ref.BF16, qs2, s2.tables, s2.lens)
    assert np.array_equal(got[0:3], got2[1:4]) and np.array_equal(got[3:5], got2[5:7])
    with pytest.raises(ValueError):   # more queries than cached tokens
        ref.prefill(L, s.cache, bits(torch.zeros((6, 8, 64), dtype=torch.bfloat16)),
                    ref.BF16, np.array([0, 0, 0, 6, 6], np.int32), s.tables, s.lens)
