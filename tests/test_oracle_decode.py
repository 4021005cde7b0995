"""Pins of the oracle's decode attention: the 16-bit passthrough case against
torch's scaled_dot_product_attention in fp64 (a library routine), exact special
cases (one token, identical keys, a dominant key, empty context), GQA against
MHA with duplicated KV heads, split-K merging, and block-permutation
invariance. No GPU."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads
from oracle import ref
from _util import DT, OracleSeqs, bits, oracle_layout

rng = np.random.default_rng(7)


def _case(code="int8", mode="token_sym", lens=(37, 80, 5, 1), Hq=8, H=2, d=64,
          bs=16, src="bfloat16", seed=0, order=None, kscale=3.0):
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode,
                      v_mode="token_sym" if mode == "channel_block" else mode,
                      group_size=32 if mode == "group_asym" else 0,
                      block_size=bs, src_dtype=src, num_q_heads=Hq,
                      num_kv_heads=H, head_dim=d, batch=len(lens))
    L = oracle_layout(w)
    lens = np.asarray(lens, np.int32)
    T = int(lens.sum())
    g = torch.Generator().manual_seed(seed)
    k = (torch.randn((T, H, d), generator=g) * kscale).to(w.torch_dtype)
    v = torch.randn((T, H, d), generator=g).to(w.torch_dtype)
    q = torch.randn((len(lens), Hq, d), generator=g).to(w.torch_dtype)
    nb = len(order) if order is not None else workloads.pool_blocks(lens, bs) + 4
    s = OracleSeqs(L, nb, len(lens), int(lens.max()) // bs + 2, order=order)
    s.append(k, v, lens)
    return w, L, s, k, v, q


def _sdpa(q, k_rows, v_rows, lens, Hq, scale=None):
    """Reference attention with torch SDPA in fp64, per sequence; KV head of
    query head h is h // (Hq / H) (repeat_interleave)."""
    B, _, d = q.shape
    out = torch.zeros((B, Hq, d), dtype=torch.float64)
    start = 0
    for b, Lb in enumerate(lens):
        if Lb == 0:
            continue
        kk = k_rows[start:start + Lb].double().transpose(0, 1)   # [H][L][d]
        vv = v_rows[start:start + Lb].double().transpose(0, 1)
        G = Hq // kk.shape[0]
        kk = kk.repeat_interleave(G, 0).contiguous()
        vv = vv.repeat_interleave(G, 0).contiguous()
        qq = q[b].double().unsqueeze(1)                           # [Hq][1][d]
        out[b] = F.scaled_dot_product_attention(qq, kk, vv, scale=scale).squeeze(1)
        start += Lb
    return out.numpy()


@pytest.mark.parametrize("src", ["float16", "bfloat16"])
@pytest.mark.parametrize("Hq,H", [(8, 2), (4, 4), (16, 2)])
def test_passthrough_cache_equals_sdpa(src, Hq, H):
    lens = (37, 80, 5, 1, 16)
    w, L, s, k, v, q = _case("none16", lens=lens, Hq=Hq, H=H, src=src,
                             order=rng.permutation(60).astype(np.int32))
    out = ref.decode(L, s.cache, bits(q), DT[src], s.tables, s.lens)
    exp = _sdpa(q, k, v, lens, Hq)
    np.testing.assert_allclose(out, exp, rtol=1e-12, atol=1e-13)
    out2 = ref.decode(L, s.cache, bits(q), DT[src], s.tables, s.lens, sm_scale=0.37)
    np.testing.assert_allclose(out2, _sdpa(q, k, v, lens, Hq, scale=0.37),
                               rtol=1e-12, atol=1e-13)


def _deq_rows(L, s, side, lens, head):
    rows = []
    for b, Lb in enumerate(lens):
        for pos in range(Lb):
            rows.append(ref.dequant_token(L, s.cache, side, s.tables[b], Lb, b, pos, head))
    return np.array(rows, np.float64)


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("fp8", "token_sym"),
                                       ("int4", "group_asym"), ("int4", "token_sym")])
def test_quantized_cache_equals_sdpa_on_dequantized_rows(code, mode):
    lens = (37, 80, 5, 1)
    w, L, s, k, v, q = _case(code, mode, lens=lens)
    out = ref.decode(L, s.cache, bits(q), DT[w.src_dtype], s.tables, s.lens)
    kd = torch.from_numpy(np.stack([_deq_rows(L, s, 0, lens, h) for h in range(2)], 1))
    vd = torch.from_numpy(np.stack([_deq_rows(L, s, 1, lens, h) for h in range(2)], 1))
    np.testing.assert_allclose(out, _sdpa(q, kd, vd, lens, 8), rtol=1e-12, atol=1e-13)
    # and the dequantized rows are within the codec's bound of the inputs
    assert np.abs(kd.numpy() - k.double().numpy()).max() <= np.abs(k.double().numpy()).max() / 2
    # quantization error only (4-bit codes are coarse on keys scaled by 3)
    tol = {"int8": 0.1, "fp8": 0.25, "int4": 1.5}[code]
    np.testing.assert_allclose(out, _sdpa(q, k, v, lens, 8), atol=tol)


def test_single_token_returns_its_value_row():
    w, L, s, k, v, q = _case("int8", lens=(1, 1, 1))
    out = ref.decode(L, s.cache, bits(q), DT[w.src_dtype], s.tables, s.lens)
    for b in range(3):
        for h in range(8):
            vr = ref.dequant_token(L, s.cache, 1, s.tables[b], 1, b, 0, h // 4)
            assert (out[b, h] == vr.astype(np.float64)).all()
            # and that row is the input value row within half a scale step
            assert np.abs(vr - v[b, h // 4].float().numpy()).max() <= \
                np.abs(v[b, h // 4].float().numpy()).max() / 127 * 0.51


def test_identical_keys_give_the_mean_value():
    lens = (48,)
    w, L, s, k, v, q = _case("int8", lens=lens)
    same = torch.randn((1, 2, 64)).to(torch.bfloat16).expand(48, 2, 64).contiguous()
    s2 = OracleSeqs(L, 10, 1, 4)
    s2.append(same, v, np.array(lens, np.int32))
    out = ref.decode(L, s2.cache, bits(q), DT[w.src_dtype], s2.tables, s2.lens)
    for h in range(8):
        vd = np.array([ref.dequant_token(L, s2.cache, 1, s2.tables[0], 48, 0, p, h // 4)
                       for p in range(48)], np.float64)
        np.testing.assert_allclose(out[0, h], vd.mean(0), rtol=1e-13, atol=1e-15)


def test_dominant_key_selects_its_value():
    lens = (64,)
    w, L, s, k, v, q = _case("none16", lens=lens, src="float16")
    kk = k.clone()
    kk[17] = (q[0, ::4].float() * 8).to(torch.float16)   # KV head g gets q head 4g
    s2 = OracleSeqs(L, 10, 1, 8)
    s2.append(kk, v, np.array(lens, np.int32))
    out = ref.decode(L, s2.cache, bits(q), ref.F16, s2.tables, s2.lens, sm_scale=4.0)
    for g in range(2):
        np.testing.assert_allclose(out[0, 4 * g], v[17, g].double().numpy(), atol=1e-9)


def test_gqa_equals_mha_with_duplicated_kv_heads():
    lens = (37, 80, 5)
    w, L, s, k, v, q = _case("int8", lens=lens, Hq=8, H=2, seed=3)
    out_gqa = ref.decode(L, s.cache, bits(q), DT[w.src_dtype], s.tables, s.lens)
    L8 = ref.layout(8, 64, 16, ref.CODE_INT8, src_dtype=ref.BF16)
    s8 = OracleSeqs(L8, 30, 3, 8)
    s8.append(k.repeat_interleave(4, 1), v.repeat_interleave(4, 1), np.array(lens, np.int32))
    out_mha = ref.decode(L8, s8.cache, bits(q), ref.BF16, s8.tables, s8.lens)
    assert (out_gqa == out_mha).all()


def test_split_merge_equals_full():
    lens = (200, 33)
    w, L, s, k, v, q = _case("fp8", lens=lens)
    full = ref.decode(L, s.cache, bits(q), DT[w.src_dtype], s.tables, s.lens)
    qb = bits(q)
    for b, Lb in enumerate(lens):
        cuts = sorted(set([0, Lb] + rng.integers(0, Lb, 4).tolist()))
        for h in range(8):
            parts = [ref.decode_range(L, s.cache, qb, ref.BF16, b, h, s.tables[b], Lb, a, c)
                     for a, c in zip(cuts, cuts[1:])]
            M = max(p[0] for p in parts)
            num = sum(np.exp(m - M) * acc for m, l, acc in parts if l > 0)
            den = sum(np.exp(m - M) * l for m, l, acc in parts if l > 0)
            np.testing.assert_allclose(num / den, full[b, h], rtol=1e-12, atol=1e-14)


def test_block_permutation_is_bit_invariant_and_empty_context_is_zero():
    lens = (37, 0, 80)
    outs = []
    for order in (None, rng.permutation(40).astype(np.int32)):
        w, L, s, k, v, q = _case("int8", lens=lens, order=order)
        outs.append(ref.decode(L, s.cache, bits(q), DT[w.src_dtype], s.tables, s.lens))
    assert (outs[0] == outs[1]).all()
    assert (outs[0][1] == 0).all()


def test_channel_block_keys_decode_with_raw_tail():
    lens = (40, 19, 16)
    w, L, s, k, v, q = _case("int8", "channel_block", lens=lens, H=2, Hq=8)
    out = ref.decode(L, s.cache, bits(q), DT[w.src_dtype], s.tables, s.lens)
    kd = torch.from_numpy(np.stack([_deq_rows(L, s, 0, lens, h) for h in range(2)], 1))
    vd = torch.from_numpy(np.stack([_deq_rows(L, s, 1, lens, h) for h in range(2)], 1))
    np.testing.assert_allclose(out, _sdpa(q, kd, vd, lens, 8), rtol=1e-12, atol=1e-13)
    # tail rows (positions 32..39 of seq 0, 16..18 of seq 1) are the raw inputs
    assert (kd[32:40].numpy() == k[32:40].double().numpy()).all()
    assert (kd[40 + 16:40 + 19].numpy() == k[40 + 16:40 + 19].double().numpy()).all()
