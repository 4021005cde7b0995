"""kvq_prefill_attention (multi-query, causal) on the GPU against the oracle's
fp64 prefill attention: caches built by the oracle and copied to the device.
Tolerance |gpu - oracle| <= 2e-3 + 1e-3 |oracle| elementwise."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import DT, OracleSeqs, bits, oracle_layout
from _gpu_util import DEV, assert_decode_close, decode_gpu, lib_layout, need_gpu, upload, kq

pytestmark = pytest.mark.gpu

# context lengths and query counts: a whole prompt (nq = L), single queries,
# no queries, chunks across block and column-tile edges, an empty sequence
LENS = (37, 80, 5, 1, 16, 0, 300, 33)
NQ = (37, 8, 0, 1, 16, 0, 45, 3)


def _setup(code="int8", d=128, bs=16, G=4, H=2, src="bfloat16", lens=LENS, nq=NQ, seed=0,
           mode="token_sym", fill=0xFF):
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode,
                      v_mode="token_sym" if mode == "channel_block" else mode,
                      group_size=32 if mode == "group_asym" else 0,
                      src_dtype=src, head_dim=d, block_size=bs, num_kv_heads=H,
                      num_q_heads=G * H, batch=len(lens), n_outliers=2, outlier_factor=8.0)
    L, LL = oracle_layout(w), lib_layout(w)
    lens = np.asarray(lens, np.int32)
    nb = workloads.pool_blocks(lens, bs) + 3
    s = OracleSeqs(L, nb, len(lens), int(lens.max()) // bs + 2,
                   order=workloads.pool_order(nb, seed=seed), max_seqs=len(lens))
    s.cache = ref.HostCache(L, nb, len(lens), fill=fill)   # unwritten bytes are NaN
    k, v = workloads.kv_rows(w, int(lens.sum()), seed=seed)
    s.append(k, v, lens)
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    g = torch.Generator().manual_seed(seed + 100)
    q = torch.randn((int(qs[-1]), G * H, d), generator=g).to(w.torch_dtype)
    return w, L, LL, s, q, qs


def prefill_gpu(LL, gc, q, qs, tables, lens, max_q, max_len, out_dtype=torch.float32,
                split_blocks=0, sm_scale=0.0, window=0, sink=0):
    Tq, Hq, d = q.shape
    B = lens.numel()
    ws = torch.empty(kq.kvq_prefill_workspace_bytes(LL, B, Hq, max_q, max_len, split_blocks),
                     dtype=torch.uint8, device=DEV)
    out = torch.full((Tq, Hq, d), float("nan"), dtype=out_dtype, device=DEV)
    kq.kvq_prefill_attention(LL, gc, q, qs, max_q, tables, lens, max_len, out, ws,
                             sm_scale=sm_scale, split_blocks=split_blocks, window=window,
                             sink=sink)
    torch.cuda.synchronize()
    return out


def _run(w, L, LL, s, q, qs, split_blocks=0, out_dtype=torch.float32, sm_scale=0.0, window=0,
         sink=0):
    exp = ref.prefill(L, s.cache, bits(q), DT[w.src_dtype], qs, s.tables, s.lens,
                      sm_scale=sm_scale, threads=8, window=window, sink=sink)
    gc = upload(s.cache, LL)
    got = prefill_gpu(LL, gc, q.to(DEV), torch.from_numpy(qs).to(DEV),
                      torch.from_numpy(s.tables).to(DEV), torch.from_numpy(s.lens).to(DEV),
                      int(np.diff(qs).max()), int(s.lens.max()), out_dtype, split_blocks,
                      sm_scale, window, sink)
    return got, exp


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("fp8", "token_sym"),
                                       ("none16", "token_sym"), ("int8", "channel_block"),
                                       ("int4", "token_sym"), ("int4", "group_asym")])
@pytest.mark.parametrize("d,bs", [(128, 16), (64, 32), (128, 32)])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_prefill_matches_oracle(code, mode, d, bs, G):
    need_gpu()
    w, L, LL, s, q, qs = _setup(code, d, bs, G, mode=mode)
    got, exp = _run(w, L, LL, s, q, qs)
    assert_decode_close(got, exp, f"{code}/{mode} d{d} bs{bs} G{G}")


@pytest.mark.parametrize("split", [1, 2, 3, 7, 64])
@pytest.mark.parametrize("code,mode", [("fp8", "token_sym"), ("int8", "channel_block"),
                                       ("int4", "group_asym"), ("int4", "token_sym")])
def test_prefill_split_counts(split, code, mode):
    need_gpu()
    w, L, LL, s, q, qs = _setup(code, G=8, mode=mode, lens=(700, 1, 250, 64, 0, 413),
                                nq=(40, 1, 250, 9, 0, 17))
    got, exp = _run(w, L, LL, s, q, qs, split_blocks=split)
    assert_decode_close(got, exp, f"{code} split {split}")


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("src", ["float16", "bfloat16"])
def test_prefill_output_and_query_dtypes(out_dtype, src):
    need_gpu()
    w, L, LL, s, q, qs = _setup("int8", src=src)
    got, exp = _run(w, L, LL, s, q, qs, out_dtype=out_dtype, sm_scale=0.3)
    assert_decode_close(got, exp, f"{src}->{out_dtype}")


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("int8", "channel_block"),
                                       ("int4", "group_asym")])
def test_prefill_single_queries_match_decode(code, mode):
    """One query per sequence is decode: both GPU paths agree with each other
    and with the oracle."""
    need_gpu()
    lens = (37, 80, 5, 300, 16, 33)
    w, L, LL, s, q, qs = _setup(code, G=4, mode=mode, lens=lens, nq=(1,) * 6)
    got, exp = _run(w, L, LL, s, q, qs)
    assert_decode_close(got, exp, "nq=1")
    gc = upload(s.cache, LL)
    dec = decode_gpu(LL, gc, q.to(DEV), torch.from_numpy(s.tables).to(DEV),
                     torch.from_numpy(s.lens).to(DEV), int(s.lens.max()))
    assert torch.allclose(got, dec, atol=2e-3, rtol=1e-3)


@pytest.mark.parametrize("code", ["fp8", "int8"])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("split", [0, 2])
def test_prefill_checks_new_tokens_g8(code, bs, split):
    """The shape of checking several new tokens at once on the 70B model: 8
    queries per sequence, 8 query heads per KV head (4 column tiles, the
    two-wave LDS kernel), d 128, lengths across many 32-token chunks and
    the library's split rule or 2-block splits (an even split count, so the
    grid's extra split is there)."""
    need_gpu()
    lens = (1000, 333, 8, 2049, 64, 517)
    w, L, LL, s, q, qs = _setup(code, d=128, bs=bs, G=8, lens=lens, nq=(8,) * len(lens))
    got, exp = _run(w, L, LL, s, q, qs, split_blocks=split)
    assert_decode_close(got, exp, f"{code} bs{bs} split {split}")


def test_prefill_chunk_of_a_long_prompt_sampled():
    """A 512-token prompt chunk at the end of a 4096-token context, 64 query /
    8 KV heads, d 128, FP8: the whole GPU output, checked against the oracle
    on every 17th query row."""
    need_gpu()
    lens, nq = (4096,), (512,)
    w = workloads.get("llama3_70b", batch=1)
    L, LL = oracle_layout(w), lib_layout(w)
    lens_a = np.asarray(lens, np.int32)
    nb = workloads.pool_blocks(lens_a, 16) + 2
    s = OracleSeqs(L, nb, 1, 4096 // 16 + 2, order=workloads.pool_order(nb))
    k, v = workloads.kv_rows(w, 4096)
    s.append(k, v, lens_a)
    g = torch.Generator().manual_seed(5)
    q = torch.randn((512, w.num_q_heads, 128), generator=g).to(torch.bfloat16)
    qs = np.array([0, 512], np.int32)
    gc = upload(s.cache, LL)
    got = prefill_gpu(LL, gc, q.to(DEV), torch.from_numpy(qs).to(DEV),
                      torch.from_numpy(s.tables).to(DEV), torch.from_numpy(s.lens).to(DEV),
                      512, 4096).cpu()
    rows = np.arange(0, 512, 17)
    for r0 in rows:
        # query r0 alone: the oracle over the prefix it sees is decode
        ln = np.array([4096 - 512 + r0 + 1], np.int32)
        exp = ref.decode(L, s.cache, bits(q[r0:r0 + 1]), ref.BF16, s.tables, ln, threads=8)
        assert_decode_close(got[r0:r0 + 1], exp, f"row {r0}")


@pytest.mark.parametrize("window,sink", [(1, 0), (7, 3), (16, 16), (40, 20), (100, 1), (33, 0)])
@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("fp8", "token_sym"),
                                       ("none16", "token_sym"), ("int8", "channel_block"),
                                       ("int4", "group_asym")])
@pytest.mark.parametrize("G,bs", [(4, 16), (8, 32)])
def test_prefill_sliding_window_and_sinks(window, sink, code, mode, G, bs):
    need_gpu()
    w, L, LL, s, q, qs = _setup(code, 128, bs, G, mode=mode)
    got, exp = _run(w, L, LL, s, q, qs, window=window, sink=sink)
    assert_decode_close(got, exp, f"{code}/{mode} window {window} sink {sink}")


@pytest.mark.parametrize("split", [1, 5, 64])
def test_prefill_window_split_counts(split):
    need_gpu()
    w, L, LL, s, q, qs = _setup("fp8", G=8, lens=(700, 1, 250, 64, 0, 413),
                                nq=(40, 1, 250, 9, 0, 17))
    got, exp = _run(w, L, LL, s, q, qs, split_blocks=split, window=100, sink=4)
    assert_decode_close(got, exp, f"window split {split}")


@pytest.mark.parametrize("code", ["int8", "fp8"])
def test_windowed_stream_with_trimming(code):
    """Each step: reserve, append (GPU and oracle), windowed attention with
    the new tokens, then trim the blocks no later query sees. Pools and
    tables stay equal to the oracle's; the trimmed blocks are handed to
    other sequences and overwritten, and the answers still match."""
    need_gpu()
    bs, window, sink, B, n = 16, 40, 3, 3, 40
    w = workloads.get("tiny", k_code=code, v_code=code, block_size=bs, src_dtype="bfloat16",
                      num_q_heads=8, num_kv_heads=2, head_dim=128, batch=B)
    L, LL = oracle_layout(w), lib_layout(w)
    order = np.random.default_rng(1).permutation(n).astype(np.int32)
    s = OracleSeqs(L, n, B, 16, order=order)
    gstack = torch.empty(n, dtype=torch.int32, device=DEV)
    gtop = torch.empty(1, dtype=torch.int32, device=DEV)
    kq.kvq_pool_init(gstack, gtop, torch.from_numpy(order).to(DEV))
    gtab = torch.full((B, 16), -1, dtype=torch.int32, device=DEV)
    glens = torch.zeros(B, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gc = kq.PagedCache(LL, n, device=DEV)
    for t in gc.planes.values():
        if t is not None:
            t.fill_(0xFF)
    rng = np.random.default_rng(5)
    trimmed = 0
    for step in range(8):
        new = rng.integers(1, 30, B).astype(np.int32)
        k, v = workloads.kv_rows(w, int(new.sum()), seed=step)
        slots, _ = s.grow(new)
        ref.append(L, s.cache, bits(k).reshape(len(slots), -1), bits(v).reshape(len(slots), -1),
                   slots)
        gsl = torch.empty(int(new.sum()), dtype=torch.int64, device=DEV)
        kq.kvq_blocks_reserve(gstack, gtop, gtab, glens, torch.from_numpy(new).to(DEV), bs, gsl,
                              status, glens)
        kq.kvq_append(LL, gc, k.to(DEV), v.to(DEV), gsl)
        qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
        q = workloads.query_rows(w, int(new.sum()), step=step)
        exp = ref.prefill(L, s.cache, bits(q), ref.BF16, qs, s.tables, s.lens, threads=8,
                          window=window, sink=sink)
        got = prefill_gpu(LL, gc, q.to(DEV), torch.from_numpy(qs).to(DEV), gtab, glens,
                          int(new.max()), int(s.lens.max()), window=window, sink=sink)
        assert_decode_close(got, exp, f"windowed step {step}")
        before = int(s.top[0])
        assert ref.blocks_trim(s.stack, s.top, s.tables, s.lens, window, sink, bs) == 0
        trimmed += int(s.top[0]) - before
        kq.kvq_blocks_trim(gstack, gtop, gtab, glens, window, sink, bs, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert np.array_equal(gtab.cpu().numpy(), s.tables), step
        assert np.array_equal(gstack.cpu().numpy(), s.stack) and int(gtop.item()) == int(s.top[0])
    assert trimmed > 0
