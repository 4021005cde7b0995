"""kvq_decode_attention_noalloc on the GPU: the allocation-free decode (its
partials in the library's fixed per-GPU array) gives the same output as
kvq_decode_attention with a caller workspace, bit for bit, and both are
within the oracle's tolerance. Two calls in a row, the second with a smaller
batch, shorter contexts and another layout, so the second call runs on what
the first left in the array."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import DT, OracleSeqs, bits, oracle_layout
from _gpu_util import DEV, assert_decode_close, decode_gpu, kq, lib_layout, need_gpu, upload

pytestmark = pytest.mark.gpu


def _case(code, mode, lens, G, bs, seed):
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode, v_mode=mode,
                      group_size=32 if mode == "group_asym" else 0, src_dtype="bfloat16",
                      head_dim=128, block_size=bs, num_kv_heads=4, num_q_heads=4 * G,
                      batch=len(lens), n_outliers=2, outlier_factor=8.0)
    L, LL = oracle_layout(w), lib_layout(w)
    lens = np.asarray(lens, np.int32)
    nb = workloads.pool_blocks(lens, bs) + 3
    s = OracleSeqs(L, nb, len(lens), int(lens.max()) // bs + 2,
                   order=workloads.pool_order(nb, seed=seed))
    k, v = workloads.kv_rows(w, int(lens.sum()), seed=seed)
    s.append(k, v, lens)
    q = workloads.queries(w, seed=seed)
    return w, L, LL, s, q


def _noalloc(LL, gc, q, tables, lens, max_len, split_blocks=0):
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    kq.kvq_decode_attention_noalloc(LL, gc, q, tables, lens, max_len, out,
                                    split_blocks=split_blocks)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("split_blocks", [0, 3])
def test_noalloc_equals_workspace_decode_twice(split_blocks):
    need_gpu()
    cases = [("fp8", "token_sym", (3000, 17, 900, 0, 2500, 64, 1, 1200), 8, 16, 0),
             ("int4", "group_asym", (700, 5, 33), 4, 32, 1)]
    for code, mode, lens, G, bs, seed in cases:   # the second call is the smaller one
        print(f"noalloc case {code}/{mode} batch {len(lens)} split {split_blocks}", flush=True)
        w, L, LL, s, q = _case(code, mode, lens, G, bs, seed)
        gc = upload(s.cache, LL)
        qd = q.to(DEV)
        tables = torch.from_numpy(s.tables).to(DEV)
        glens = torch.from_numpy(s.lens).to(DEV)
        max_len = int(s.lens.max())
        ref_out = decode_gpu(LL, gc, qd, tables, glens, max_len, split_blocks=split_blocks)
        got = _noalloc(LL, gc, qd, tables, glens, max_len, split_blocks)
        assert torch.equal(got, ref_out), f"{code}/{mode}: differs from the workspace decode"
        exp = ref.decode(L, s.cache, bits(q), DT[w.src_dtype], s.tables, s.lens, threads=8)
        assert_decode_close(got, exp, f"noalloc {code}/{mode}")
        assert (got[np.asarray(lens) == 0] == 0).all()


def test_noalloc_refuses_sizes_past_its_array():
    need_gpu()
    w, L, LL, s, q = _case("int8", "token_sym", (40, 9), 4, 16, 2)
    gc = upload(s.cache, LL)
    B, big = 256, 1 << 18
    assert kq.kvq_decode_workspace_bytes(LL, B, 16, big) > kq.KVQ_DECODE_SCRATCH_BYTES
    qd = torch.zeros((B, 16, 128), dtype=torch.bfloat16, device=DEV)
    tables = torch.zeros((B, big // 16), dtype=torch.int32, device=DEV)
    lens = torch.zeros(B, dtype=torch.int32, device=DEV)
    out = torch.zeros((B, 16, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(kq.KvqError, match="WORKSPACE_TOO_SMALL"):
        kq.kvq_decode_attention_noalloc(LL, gc, qd, tables, lens, big, out)
