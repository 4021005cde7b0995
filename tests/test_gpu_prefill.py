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
                split_blocks=0, sm_scale=0.0):
    Tq, Hq, d = q.shape
    B = lens.numel()
    ws = torch.empty(kq.kvq_prefill_workspace_bytes(LL, B, Hq, max_q, max_len, split_blocks),
                     dtype=torch.uint8, device=DEV)
    out = torch.full((Tq, Hq, d), float("nan"), dtype=out_dtype, device=DEV)
    kq.kvq_prefill_attention(LL, gc, q, qs, max_q, tables, lens, max_len, out, ws,
                             sm_scale=sm_scale, split_blocks=split_blocks)
    torch.cuda.synchronize()
    return out


def _run(w, L, LL, s, q, qs, split_blocks=0, out_dtype=torch.float32, sm_scale=0.0):
    exp = ref.prefill(L, s.cache, bits(q), DT[w.src_dtype], qs, s.tables, s.lens,
                      sm_scale=sm_scale, threads=8)
    gc = upload(s.cache, LL)
    got = prefill_gpu(LL, gc, q.to(DEV), torch.from_numpy(qs).to(DEV),
                      torch.from_numpy(s.tables).to(DEV), torch.from_numpy(s.lens).to(DEV),
                      int(np.diff(qs).max()), int(s.lens.max()), out_dtype, split_blocks,
                      sm_scale)
    return got, exp


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("fp8", "token_sym"),
                                       ("none16", "token_sym"), ("int8", "channel_block")])
@pytest.mark.parametrize("d,bs", [(128, 16), (64, 32), (128, 32)])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_prefill_matches_oracle(code, mode, d, bs, G):
    need_gpu()
    w, L, LL, s, q, qs = _setup(code, d, bs, G, mode=mode)
    got, exp = _run(w, L, LL, s, q, qs)
    assert_decode_close(got, exp, f"{code}/{mode} d{d} bs{bs} G{G}")


@pytest.mark.parametrize("split", [1, 2, 3, 7, 64])
@pytest.mark.parametrize("code,mode", [("fp8", "token_sym"), ("int8", "channel_block")])
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


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("int8", "channel_block")])
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
