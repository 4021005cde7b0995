"""Block offload on the GPU against the oracle: kvq_pack_blocks gives the
oracle's packed bytes, kvq_unpack_blocks restores them into other blocks
(every plane equal to the oracle's unpack), and a round trip through pinned
host memory leaves decode unchanged."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import OracleSeqs, bits, oracle_layout
from _gpu_util import DEV, assert_decode_close, decode_gpu, kq, lib_layout, need_gpu, planes_equal, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("code,mode,bs", [("int8", "token_sym", 16), ("fp8", "token_sym", 32),
                                          ("int4", "group_asym", 32), ("int4", "token_sym", 16),
                                          ("none16", "token_sym", 16),
                                          ("int8", "channel_block", 16)])
def test_pack_unpack_match_oracle_and_round_trip(code, mode, bs):
    need_gpu()
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode,
                      v_mode="token_sym" if mode == "channel_block" else mode,
                      group_size=32 if mode == "group_asym" else 0, block_size=bs,
                      head_dim=128, num_kv_heads=4, num_q_heads=16, batch=3,
                      src_dtype="bfloat16")
    L, LL = oracle_layout(w), lib_layout(w)
    lens = np.array([300, 77, 130], np.int32)
    n = workloads.pool_blocks(lens, bs) * 2 + 4
    s = OracleSeqs(L, n, 3, 32, order=np.random.default_rng(4).permutation(n).astype(np.int32),
                   max_seqs=3)
    k, v = workloads.kv_rows(w, int(lens.sum()), seed=2)
    s.append(k, v, lens)
    used = [int(x) for x in s.tables.reshape(-1) if x >= 0]
    free = [i for i in range(n) if i not in set(used)]
    ids = np.array(used, np.int32)
    gc = upload(s.cache, LL)
    per = kq.kvq_block_pack_bytes(LL)
    assert per == ref.block_pack_bytes(L)
    packed = torch.empty(per * len(ids), dtype=torch.uint8, device=DEV)
    kq.kvq_pack_blocks(LL, gc, torch.from_numpy(ids).to(DEV), packed)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), ref.pack_blocks(L, s.cache, ids))
    # through pinned host memory and back, into other blocks
    host = torch.empty(packed.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(packed, non_blocking=True)
    back = torch.empty_like(packed)
    back.copy_(host, non_blocking=True)
    new_ids = np.array(free[:len(ids)], np.int32)
    kq.kvq_unpack_blocks(LL, gc, back, torch.from_numpy(new_ids).to(DEV))
    ref.unpack_blocks(L, s.cache, ref.pack_blocks(L, s.cache, ids), new_ids)
    torch.cuda.synchronize()
    assert planes_equal(gc, s.cache) == []
    remap = dict(zip(ids.tolist(), new_ids.tolist()))
    tables = np.vectorize(lambda x: remap.get(x, x))(s.tables).astype(np.int32)
    q = workloads.queries(w, seed=2)
    exp = ref.decode(L, s.cache, bits(q), ref.BF16, tables, s.lens, threads=4)
    got = decode_gpu(LL, gc, q.to(DEV), torch.from_numpy(tables).to(DEV),
                     torch.from_numpy(s.lens).to(DEV), int(lens.max()))
    assert_decode_close(got, exp, f"unpacked {code}/{mode}")
