"""Raw bf16 rows past fp16's range, on the GPU against the oracle.

The passthrough cache (NONE16) and the staged rows of per-channel keys hold
source rows as given. In bf16 they may lie far outside fp16's range: past
65504 or below 2^-14. Such rows must keep their values in attention, which
computes with the dequantized keys and values ("KV Cache Optimization:
Strategies for Faster LLM Inference", §KV Cache Quantization: When and How to
Compress -- the unquantized cache is the baseline the codes approximate).

Inputs: the seeded rows of workloads.kv_rows, with key channels KBIG scaled
by 1e5 and KTINY by 1e-7, and value channels VBIG by 2e5 and VTINY by 1e-7,
then rounded to bf16. sm_scale = 1e-5 keeps the softmax spread out (scores
of a few units, set by the 1e5 key channels). Outputs are fp32.

Tolerance: the usual |gpu - oracle| <= 2e-3 + 1e-3 |oracle| applied at each
value channel's own scale f: |gpu - oracle| <= 2e-3 f + 1e-3 |oracle|. At
f = 1e-7 that asks for a relative 2e-3, which an fp16 rounding of the
values (subnormal there) would miss."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import DT, OracleSeqs, bits, oracle_layout
from _gpu_util import DEV, decode_gpu, kq, lib_layout, need_gpu, upload

pytestmark = pytest.mark.gpu

LENS = (37, 80, 5, 1, 16, 0, 17, 300, 15, 33)
KBIG, KTINY = (3, 17, 40, 61), (5, 22)
VBIG, VTINY = (0, 9, 33, 50), (2, 13, 47)
SM = 1e-5


def _scaled(k, v):
    k, v = k.float(), v.float()
    k[..., list(KBIG)] *= 1e5
    k[..., list(KTINY)] *= 1e-7
    v[..., list(VBIG)] *= 2e5
    v[..., list(VTINY)] *= 1e-7
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def _setup(code, mode, d, bs, G, H=2, lens=LENS, seed=0):
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode,
                      v_mode="token_sym" if mode == "channel_block" else mode,
                      src_dtype="bfloat16", head_dim=d, block_size=bs, num_kv_heads=H,
                      num_q_heads=G * H, batch=len(lens), n_outliers=0)
    L, LL = oracle_layout(w), lib_layout(w)
    lens = np.asarray(lens, np.int32)
    nb = workloads.pool_blocks(lens, bs) + 3
    s = OracleSeqs(L, nb, len(lens), int(lens.max()) // bs + 2,
                   order=workloads.pool_order(nb, seed=seed), max_seqs=len(lens))
    s.cache = ref.HostCache(L, nb, len(lens), fill=0xFF)   # unwritten bytes are NaN
    k, v = _scaled(*workloads.kv_rows(w, int(lens.sum()), seed=seed))
    assert k.float().abs().max() > 65504 and v.float().abs().max() > 65504
    s.append(k, v, lens)
    return w, L, LL, s


def _close(got, exp, d, what):
    f = np.ones(d)
    f[list(VBIG)] = 2e5
    f[list(VTINY)] = 1e-7
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - exp)
    lim = 2e-3 * f + 1e-3 * np.abs(exp)
    bad = ~(err <= lim)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside; first at "
                           f"{np.argwhere(bad)[0].tolist()}: got {g[bad][0]!r} "
                           f"oracle {exp[bad][0]!r}")


@pytest.mark.parametrize("code,mode", [("none16", "token_sym"), ("int8", "channel_block")])
@pytest.mark.parametrize("d,bs", [(128, 16), (64, 32)])
@pytest.mark.parametrize("G", [1, 8])
def test_decode_keeps_bf16_range(code, mode, d, bs, G):
    need_gpu()
    w, L, LL, s = _setup(code, mode, d, bs, G)
    q = workloads.queries(w, seed=1)
    exp = ref.decode(L, s.cache, bits(q), DT[w.src_dtype], s.tables, s.lens, sm_scale=SM,
                     threads=8)
    gc = upload(s.cache, LL)
    got = decode_gpu(LL, gc, q.to(DEV), torch.from_numpy(s.tables).to(DEV),
                     torch.from_numpy(s.lens).to(DEV), int(s.lens.max()), torch.float32, SM)
    _close(got, exp, d, f"decode {code}/{mode} d{d} bs{bs} G{G}")
    assert (got[5] == 0).all()   # empty context


@pytest.mark.parametrize("code,mode", [("none16", "token_sym"), ("int8", "channel_block")])
@pytest.mark.parametrize("d,bs", [(128, 16), (64, 32)])
def test_prefill_keeps_bf16_range(code, mode, d, bs):
    need_gpu()
    lens, nq = (37, 80, 5, 1, 16, 0, 300, 33), (37, 8, 0, 1, 16, 0, 45, 3)
    w, L, LL, s = _setup(code, mode, d, bs, 4, lens=lens)
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    g = torch.Generator().manual_seed(101)
    q = torch.randn((int(qs[-1]), w.num_q_heads, d), generator=g).to(torch.bfloat16)
    exp = ref.prefill(L, s.cache, bits(q), DT[w.src_dtype], qs, s.tables, s.lens,
                      sm_scale=SM, threads=8)
    gc = upload(s.cache, LL)
    B, max_q, max_len = len(lens), int(max(nq)), int(s.lens.max())
    ws = torch.empty(kq.kvq_prefill_workspace_bytes(LL, B, w.num_q_heads, max_q, max_len, 0),
                     dtype=torch.uint8, device=DEV)
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=DEV)
    kq.kvq_prefill_attention(LL, gc, q.to(DEV), torch.from_numpy(qs).to(DEV), max_q,
                             torch.from_numpy(s.tables).to(DEV),
                             torch.from_numpy(s.lens).to(DEV), max_len, out, ws, sm_scale=SM)
    torch.cuda.synchronize()
    _close(out, exp, d, f"prefill {code}/{mode} d{d} bs{bs}")
