"""kvq_append on the GPU against the oracle: every byte of every plane equal
(codes, fp32 scales, zero points, staged rows, and untouched bytes)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import OracleSeqs, bits, oracle_layout
from _gpu_util import DEV, gpu_cache, lib_layout, need_gpu, planes_equal, kq

pytestmark = pytest.mark.gpu

CASES = [  # code, mode, group, src, d, bs
    ("int8", "token_sym", 0, "bfloat16", 128, 16),
    ("int8", "token_sym", 0, "float16", 64, 16),
    ("int8", "token_sym", 0, "bfloat16", 64, 32),
    ("fp8", "token_sym", 0, "bfloat16", 128, 16),
    ("fp8", "token_sym", 0, "float16", 128, 32),
    ("fp8", "token_sym", 0, "float16", 64, 16),
    ("int4", "token_sym", 0, "bfloat16", 128, 16),
    ("int4", "token_sym", 0, "float16", 64, 32),
    ("int4", "group_asym", 32, "bfloat16", 128, 32),
    ("int4", "group_asym", 32, "float16", 64, 16),
    ("none16", "token_sym", 0, "bfloat16", 128, 16),
    ("none16", "token_sym", 0, "float16", 64, 32),
]


def _workload(code, mode, gs, src, d, bs, H=3, batch=7):
    return workloads.get("tiny", k_code=code, v_code=code, k_mode=mode, v_mode=mode,
                         group_size=gs, src_dtype=src, head_dim=d, block_size=bs,
                         num_kv_heads=H, num_q_heads=H, batch=batch)


def _edge_rows(n, H, d, dtype, g):
    """Rows that exercise the codec's special cases: zero rows, a single
    non-zero, -0, the largest finite input, tiny magnitudes, exact ties at
    unit scale (max |x| = 127 or 448), and all-negative / all-positive groups."""
    big = 65504.0 if dtype == torch.float16 else 3.0e38
    tiny = 6e-8 if dtype == torch.float16 else 1e-38
    rows = torch.randn((n, H, d), generator=g) * 3
    rows[0] = 0.0
    rows[1] = 0.0
    rows[1, :, 5] = -2.5
    rows[2] = -0.0
    rows[3, :, :] = big * torch.sign(torch.randn((H, d), generator=g))
    rows[4] = tiny * torch.randn((H, d), generator=g)
    rows[5] = (torch.randint(-254, 255, (H, d), generator=g) / 2.0)   # halves
    rows[5, :, 0] = 127.0
    rows[6] = (torch.randint(-896, 897, (H, d), generator=g) / 2.0)
    rows[6, :, 0] = 448.0
    rows[7] = torch.rand((H, d), generator=g) * 5 + 0.1                # all positive
    rows[8] = -torch.rand((H, d), generator=g) * 5 - 0.1               # all negative
    rows[9] = torch.randn((H, d), generator=g) * 1e-3
    return rows.to(dtype)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_append_matches_oracle_bytewise(case):
    need_gpu()
    code, mode, gs, src, d, bs = case
    w = _workload(*case)
    L = oracle_layout(w)
    LL = lib_layout(w)
    lens = np.array([37, 80, 5, 1, 16, 0, 33], np.int32)
    T = int(lens.sum())
    g = torch.Generator().manual_seed(11)
    k, v = workloads.kv_rows(w, T, seed=3)
    k[:10] = _edge_rows(10, w.num_kv_heads, d, w.torch_dtype, g)
    v[10:20] = _edge_rows(10, w.num_kv_heads, d, w.torch_dtype, g)
    nb = workloads.pool_blocks(lens, bs) + 5
    order = workloads.pool_order(nb, seed=1)
    seqs = OracleSeqs(L, nb, len(lens), 16, order=order)
    seqs.cache = ref.HostCache(L, nb, fill=0xA5)
    slots, _ = seqs.grow(lens)
    slots[[3, 50, 120]] = -1                                   # skipped tokens
    ref.append(L, seqs.cache, bits(k).reshape(T, -1), bits(v).reshape(T, -1), slots)
    gc = gpu_cache(LL, nb)
    kq.kvq_append(LL, gc, k.to(DEV), v.to(DEV), torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert planes_equal(gc, seqs.cache) == []


def _unit_scale_rows(values, anchor, H, d):
    """Pack every value into rows whose first element is the anchor (max |x|),
    so the scale is exactly 1 and every code is the encoding of x itself."""
    per = d - 1
    n = (len(values) + per - 1) // per
    pad = np.concatenate([values, np.zeros(n * per - len(values), values.dtype)])
    rows = np.concatenate([np.full((n, 1), anchor, values.dtype), pad.reshape(n, per)], 1)
    rows = np.repeat(rows[:, None, :], H, 1)
    return torch.from_numpy(rows.astype(np.float32))


@pytest.mark.parametrize("code,anchor", [("int8", 127.0), ("fp8", 448.0), ("int4", 7.0)])
@pytest.mark.parametrize("src", ["float16", "bfloat16"])
def test_append_every_16bit_input_at_unit_scale(code, anchor, src):
    """Exhaustive over the source format: every finite 16-bit value with
    |x| <= anchor, quantized at scale exactly 1 (covers every rounding tie)."""
    need_gpu()
    dt = torch.float16 if src == "float16" else torch.bfloat16
    allbits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(dt).float()
    vals = allbits[torch.isfinite(allbits) & (allbits.abs() <= anchor)].numpy()
    w = _workload(code, "token_sym", 0, src, 128, 16, H=2, batch=1)
    L, LL = oracle_layout(w), lib_layout(w)
    k = _unit_scale_rows(vals, anchor, 2, 128).to(dt)
    v = _unit_scale_rows(vals[::-1].copy(), -anchor, 2, 128).to(dt)
    T = k.shape[0]
    nb = (T + 15) // 16
    slots = np.arange(T, dtype=np.int64)
    hc = ref.HostCache(L, nb, fill=0)
    ref.append(L, hc, bits(k).reshape(T, -1), bits(v).reshape(T, -1), slots)
    gc = gpu_cache(LL, nb, fill=0)
    kq.kvq_append(LL, gc, k.to(DEV), v.to(DEV), torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert planes_equal(gc, hc) == []
    s = gc.planes["k_scale"].view(torch.float32).cpu().reshape(nb, 2, 16)
    s = s.permute(0, 2, 1).reshape(-1, 2)[:T]        # slot order, both heads
    assert (s == 1.0).all()


def test_append_strided_rows_and_large_batch():
    """Rows with a stride larger than H*d (e.g. a fused QKV buffer) and a
    token count that spans many waves."""
    need_gpu()
    w = workloads.get("llama3_8b")
    L, LL = oracle_layout(w), lib_layout(w)
    T = 5000
    fused = torch.randn((T, 3 * w.num_kv_heads * w.head_dim)).to(torch.bfloat16)
    row = w.num_kv_heads * w.head_dim
    k, v = fused[:, row:2 * row], fused[:, 2 * row:]
    nb = (T + 15) // 16 + 3
    slots = np.random.default_rng(5).permutation(nb * 16)[:T].astype(np.int64)
    hc = ref.HostCache(L, nb, fill=0x5A)
    ref.append(L, hc, bits(k.contiguous()), bits(v.contiguous()), slots)
    gc = gpu_cache(LL, nb, fill=0x5A)
    fd = fused.to(DEV)
    kq.kvq_append(LL, gc, fd[:, row:2 * row], fd[:, 2 * row:], torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert planes_equal(gc, hc) == []


def test_append_channel_block_keys_in_chunks():
    """Per-channel keys: the same token stream appended in different chunkings
    gives the oracle's bytes (completed blocks, value planes, staged rows)."""
    need_gpu()
    w = workloads.get("mixed", batch=5)
    L, LL = oracle_layout(w), lib_layout(w)
    lens_final = np.array([40, 19, 16, 3, 77], np.int32)
    starts = np.concatenate([[0], np.cumsum(lens_final)[:-1]])
    k, v = workloads.kv_rows(w, int(lens_final.sum()), seed=9)
    chunks = [[1, 1, 1, 1, 1], [8, 0, 15, 2, 8], [31, 18, 0, 0, 60], [0, 0, 0, 0, 8]]
    nb = 40
    seqs = OracleSeqs(L, nb, 5, 8, order=workloads.pool_order(nb, seed=2), max_seqs=5)
    seqs.cache = ref.HostCache(L, nb, 5, fill=0)
    gc = gpu_cache(LL, nb, 5, fill=0)
    done = np.zeros(5, np.int64)
    for ch in chunks:
        ch = np.asarray(ch, np.int32)
        idx = np.concatenate([starts[b] + done[b] + np.arange(ch[b]) for b in range(5)]).astype(np.int64)
        slots, rows = seqs.grow(ch)
        kk, vv = k[idx], v[idx]
        ref.append(L, seqs.cache, bits(kk).reshape(len(idx), -1), bits(vv).reshape(len(idx), -1),
                   slots, rows)
        kq.kvq_append(LL, gc, kk.to(DEV), vv.to(DEV), torch.from_numpy(slots).to(DEV),
                      stage_rows=torch.from_numpy(rows).to(DEV))
        done += ch
    torch.cuda.synchronize()
    assert planes_equal(gc, seqs.cache, ["k_codes", "k_scale", "v_codes", "v_scale"]) == []
    st_g = gc.planes["k_stage"].cpu().numpy().reshape(5, 8, 16, 256)
    st_h = seqs.cache.planes["k_stage"].reshape(5, 8, 16, 256)
    for b, Lb in enumerate(lens_final):
        tail = Lb % 16
        assert np.array_equal(st_g[b, :, :tail], st_h[b, :, :tail]), b


def test_append_channel_block_keys_bulk_then_step():
    """Per-channel keys through both append paths: two bulk calls (more than
    131072 (token, head) items each, taken 64 tokens at a time per wave) that
    leave every sequence with a partial block, whose rows the second call and
    then a small call (one wave per (token, head)) complete; completed
    blocks, value planes and staged rows equal the oracle's."""
    need_gpu()
    B = 48
    w = workloads.get("mixed", batch=B)
    L, LL = oracle_layout(w), lib_layout(w)
    g = np.random.default_rng(21)
    lens_final = g.integers(500, 1500, B).astype(np.int32)
    c1 = (lens_final * g.uniform(0.45, 0.65, B)).astype(np.int32)
    c2 = ((lens_final - c1) * g.uniform(0.7, 0.95, B)).astype(np.int32)
    c3 = lens_final - c1 - c2
    assert c1.sum() * w.num_kv_heads > 131072 and c2.sum() * w.num_kv_heads > 131072
    starts = np.concatenate([[0], np.cumsum(lens_final)[:-1]])
    k, v = workloads.kv_rows(w, int(lens_final.sum()), seed=11)
    nb = workloads.pool_blocks(lens_final, 16) + 8
    maxb = int(lens_final.max()) // 16 + 2
    seqs = OracleSeqs(L, nb, B, maxb, order=workloads.pool_order(nb, seed=3), max_seqs=B)
    seqs.cache = ref.HostCache(L, nb, B, fill=0)
    gc = gpu_cache(LL, nb, B, fill=0)
    done = np.zeros(B, np.int64)
    for ch in (c1, c2, c3):
        idx = np.concatenate([starts[b] + done[b] + np.arange(ch[b]) for b in range(B)]).astype(np.int64)
        slots, rows = seqs.grow(ch)
        kk, vv = k[idx], v[idx]
        ref.append(L, seqs.cache, bits(kk).reshape(len(idx), -1), bits(vv).reshape(len(idx), -1),
                   slots, rows)
        kq.kvq_append(LL, gc, kk.to(DEV), vv.to(DEV), torch.from_numpy(slots).to(DEV),
                      stage_rows=torch.from_numpy(rows).to(DEV))
        done += ch
        torch.cuda.synchronize()
        assert planes_equal(gc, seqs.cache, ["k_codes", "k_scale", "v_codes", "v_scale"]) == []
        st_g = gc.planes["k_stage"].cpu().numpy().reshape(B, 8, 16, 256)
        st_h = seqs.cache.planes["k_stage"].reshape(B, 8, 16, 256)
        for b in range(B):
            tail = int(done[b]) % 16
            assert np.array_equal(st_g[b, :, :tail], st_h[b, :, :tail]), b
