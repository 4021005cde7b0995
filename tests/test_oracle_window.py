"""Pins of the oracle's sliding-window / attention-sink attention and of block
recycling under a window: torch SDPA in fp64 with the explicit window mask
(a library routine), exact special cases (a window of one is the query's own
value row; a window as long as the context is full attention), a
hand-worked trim, and windowed attention after trimming (the dropped blocks
are never read again). No GPU."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads
from oracle import ref
from _util import DT, OracleSeqs, bits, oracle_layout


def _case(code="none16", lens=(70, 33, 5), nq=(6, 33, 1), bs=16, seed=0, src="bfloat16"):
    w = workloads.get("tiny", k_code=code, v_code=code, block_size=bs, src_dtype=src,
                      num_q_heads=4, num_kv_heads=2, head_dim=64, batch=len(lens))
    L = oracle_layout(w)
    lens = np.asarray(lens, np.int32)
    g = torch.Generator().manual_seed(seed)
    T = int(lens.sum())
    k = (torch.randn((T, 2, 64), generator=g) * 3).to(w.torch_dtype)
    v = torch.randn((T, 2, 64), generator=g).to(w.torch_dtype)
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = torch.randn((int(qs[-1]), 4, 64), generator=g).to(w.torch_dtype)
    s = OracleSeqs(L, workloads.pool_blocks(lens, bs) + 4, len(lens), int(lens.max()) // bs + 3)
    s.append(k, v, lens)
    return w, L, s, k, v, q, qs


def _sdpa_window(q, k, v, qs, lens, window, sink):
    out = np.zeros((q.shape[0], 4, 64))
    start = 0
    for b, Lb in enumerate(lens):
        nq = qs[b + 1] - qs[b]
        kk = k[start:start + Lb].double().transpose(0, 1).repeat_interleave(2, 0).contiguous()
        vv = v[start:start + Lb].double().transpose(0, 1).repeat_interleave(2, 0).contiguous()
        start += Lb
        if nq == 0:
            continue
        qq = q[qs[b]:qs[b + 1]].double().transpose(0, 1).contiguous()
        t = torch.arange(Lb)[None, :]
        p = (Lb - nq + torch.arange(nq))[:, None]
        mask = (t <= p) & ((t >= p + 1 - window) | (t < sink))
        out[qs[b]:qs[b + 1]] = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask) \
            .transpose(0, 1).numpy()
    return out


@pytest.mark.parametrize("window,sink", [(1, 0), (7, 0), (16, 4), (20, 1), (33, 16), (100, 3)])
def test_window_equals_masked_sdpa(window, sink):
    w, L, s, k, v, q, qs = _case()
    got = ref.prefill(L, s.cache, bits(q), ref.BF16, qs, s.tables, s.lens, window=window,
                      sink=sink)
    exp = _sdpa_window(q, k, v, qs, s.lens, window, sink)
    assert np.abs(got - exp).max() < 1e-12


def test_window_special_cases():
    w, L, s, k, v, q, qs = _case("int8")
    full = ref.prefill(L, s.cache, bits(q), ref.BF16, qs, s.tables, s.lens)
    wide = ref.prefill(L, s.cache, bits(q), ref.BF16, qs, s.tables, s.lens, window=70, sink=5)
    assert np.array_equal(full, wide)
    one = ref.prefill(L, s.cache, bits(q), ref.BF16, qs, s.tables, s.lens, window=1)
    for b in range(3):
        nq = qs[b + 1] - qs[b]
        for i in range(nq):
            pos = s.lens[b] - nq + i
            for h in range(4):
                row = ref.dequant_token(L, s.cache, 1, s.tables[b], s.lens[b], b, pos, h // 2)
                assert np.array_equal(one[qs[b] + i, h], row.astype(np.float64))


def test_trim_hand_worked():
    stack, top = ref.pool_init(16)
    tables = np.full((2, 8), -1, np.int32)
    lens = np.zeros(2, np.int32)
    ref.blocks_reserve(stack, top, tables, lens, [20, 5], 4, lens)
    assert tables[0, :5].tolist() == [11, 12, 13, 14, 15] and top[0] == 9
    # window 6, sink 2, length 20: later queries see t >= 15 and t < 2
    assert ref.blocks_trim(stack, top, tables, lens, 6, 2, 4) == 0
    assert tables[0, :5].tolist() == [11, -1, -1, 14, 15] and top[0] == 11
    assert stack[9:11].tolist() == [12, 13]
    assert tables[1, :2].tolist() == [9, 10]        # length 5 keeps everything
    # trimming again changes nothing; window 0 never trims
    assert ref.blocks_trim(stack, top, tables, lens, 6, 2, 4) == 0 and top[0] == 11
    assert ref.blocks_trim(stack, top, tables, lens, 0, 0, 4) == 0 and top[0] == 11


@pytest.mark.parametrize("code", ["int8", "fp8"])
def test_windowed_steps_after_trimming(code):
    """A windowed stream: at every step each sequence appends its new tokens,
    attends with them through the window, then drops the blocks no later
    query can see. The answers equal the same steps on a cache that never
    drops anything, and the dropped blocks (overwritten by other sequences'
    later appends) are never read."""
    bs, window, sink = 16, 40, 3
    w = workloads.get("tiny", k_code=code, v_code=code, block_size=bs, src_dtype="bfloat16",
                      num_q_heads=4, num_kv_heads=2, head_dim=64, batch=3)
    L = oracle_layout(w)
    n = 40
    trim = OracleSeqs(L, n, 3, 16, order=np.random.default_rng(1).permutation(n).astype(np.int32))
    keep = OracleSeqs(L, 64, 3, 16)
    rng = np.random.default_rng(5)
    for step in range(6):
        new = rng.integers(1, 30, 3).astype(np.int32)
        k, v = workloads.kv_rows(w, int(new.sum()), seed=step)
        trim.append(k, v, new)
        keep.append(k, v, new)
        qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
        q = workloads.query_rows(w, int(new.sum()), step=step)
        a = ref.prefill(L, trim.cache, bits(q), ref.BF16, qs, trim.tables, trim.lens,
                        window=window, sink=sink)
        b = ref.prefill(L, keep.cache, bits(q), ref.BF16, qs, keep.tables, keep.lens,
                        window=window, sink=sink)
        assert np.array_equal(a, b), step
        assert ref.blocks_trim(trim.stack, trim.top, trim.tables, trim.lens, window, sink, bs) == 0
    assert (trim.tables == -1).any()
