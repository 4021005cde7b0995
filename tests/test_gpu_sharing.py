"""Prefix sharing on the GPU against the oracle: forks, refcounted
reservations with copy on write, refcounted releases (identical stacks,
tops, counts, tables, slots, copy pairs and lengths, step after step), and
a forked cache built with kvq_copy_blocks, byte for byte, then decoded."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import bits, oracle_layout
from _gpu_util import DEV, assert_decode_close, decode_gpu, gpu_cache, kq, lib_layout, need_gpu, planes_equal

pytestmark = pytest.mark.gpu


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("B,bs,n", [(6, 4, 64), (300, 16, 6000), (1500, 16, 30000)])
def test_sharing_steps_match_oracle(B, bs, n):
    need_gpu()
    rng = np.random.default_rng(B + bs)
    maxb = 40
    order = rng.permutation(n).astype(np.int32)
    # oracle state
    ostack, otop = ref.pool_init(n, order)
    orc = np.zeros(n, np.int32)
    otab = np.full((B, maxb), -1, np.int32)
    lens = np.zeros(B, np.int32)
    # device state
    gstack = torch.empty(n, dtype=torch.int32, device=DEV)
    gtop = torch.empty(1, dtype=torch.int32, device=DEV)
    kq.kvq_pool_init(gstack, gtop, _t(order))
    grc = torch.zeros(n, dtype=torch.int32, device=DEV)
    gtab = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    glens = torch.zeros(B, dtype=torch.int32, device=DEV)
    status = torch.full((1,), 99, dtype=torch.int32, device=DEV)
    cs = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    cd = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    cows = forks = 0
    for step in range(40):
        op = step % 5
        if op in (0, 1, 3):
            hi = 3 * bs if step != 20 else 40 * bs     # step 20 exhausts the pool
            new = (rng.integers(0, hi, B) * (rng.random(B) < 0.7)).astype(np.int32)
            olens = lens.copy()
            oslots, ost, ocs, ocd = ref.blocks_reserve_shared(ostack, otop, orc, otab, lens, new,
                                                              bs, olens)
            gslots = torch.full((int(new.sum()),), -7, dtype=torch.int64, device=DEV)
            kq.kvq_blocks_reserve_shared(gstack, gtop, grc, gtab, glens, _t(new), bs, gslots,
                                         cs, cd, cnt, status, glens)
            torch.cuda.synchronize()
            assert int(status.item()) == ost, step
            assert np.array_equal(gslots.cpu().numpy(), oslots), step
            if ost == 0:
                k = int(cnt.item())
                assert k == len(ocs), step
                assert np.array_equal(cs[:k].cpu().numpy(), ocs), step
                assert np.array_equal(cd[:k].cpu().numpy(), ocd), step
                lens = olens
                cows += k
        elif op == 2:
            empty = np.flatnonzero(lens == 0)
            full = np.flatnonzero(lens > 0)
            k = min(len(empty), len(full), max(1, B // 4))
            if k:
                src = rng.choice(full, k, replace=True).astype(np.int32)   # shared sources
                dst = rng.choice(empty, k, replace=False).astype(np.int32)
                ref.blocks_fork(orc, otab, lens, src, dst, bs)
                kq.kvq_blocks_fork(grc, gtab, glens, _t(src), _t(dst), bs)
                forks += k
        else:
            mask = (rng.random(B) < 0.25).astype(np.int32)
            olens = lens.copy()
            ost = ref.blocks_release_shared(ostack, otop, orc, otab, lens, mask, bs, olens)
            kq.kvq_blocks_release_shared(gstack, gtop, grc, gtab, glens, _t(mask), bs, status,
                                         glens)
            torch.cuda.synchronize()
            assert int(status.item()) == ost, step
            lens = olens
        torch.cuda.synchronize()
        assert int(gtop.item()) == int(otop[0]), step
        assert np.array_equal(gstack.cpu().numpy(), ostack), step
        assert np.array_equal(grc.cpu().numpy(), orc), step
        assert np.array_equal(gtab.cpu().numpy(), otab), step
        assert np.array_equal(glens.cpu().numpy(), lens), step
    assert cows > 0 and forks > 0


@pytest.mark.parametrize("code,mode,bs", [("fp8", "token_sym", 16), ("int4", "group_asym", 32),
                                          ("none16", "token_sym", 16)])
def test_forked_cache_with_copy_on_write(code, mode, bs):
    """A 37-token prefix appended once and forked into two more sequences;
    two of the three then append into the shared, partly filled block, so it
    is copied (kvq_copy_blocks) before their tails land. Every plane equals
    the oracle's after the same steps, and decode matches the oracle."""
    need_gpu()
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode, v_mode=mode,
                      group_size=32 if mode == "group_asym" else 0, block_size=bs,
                      head_dim=128, num_kv_heads=2, num_q_heads=16, batch=3,
                      src_dtype="bfloat16")
    L, LL = oracle_layout(w), lib_layout(w)
    n, prefix, tails = 24, 37, (5, 11, 0)
    k, v = workloads.kv_rows(w, prefix + sum(tails), seed=4)
    order = np.random.default_rng(3).permutation(n).astype(np.int32)
    # oracle
    ostack, otop = ref.pool_init(n, order)
    orc = np.zeros(n, np.int32)
    otab = np.full((3, 8), -1, np.int32)
    lens = np.zeros(3, np.int32)
    hc = ref.HostCache(L, n, fill=0x33)
    s1, _, _, _ = ref.blocks_reserve_shared(ostack, otop, orc, otab, lens, [prefix, 0, 0], bs, lens)
    ref.append(L, hc, bits(k[:prefix]).reshape(prefix, -1), bits(v[:prefix]).reshape(prefix, -1), s1)
    ref.blocks_fork(orc, otab, lens, [0, 0], [1, 2], bs)
    s2, st, ocs, ocd = ref.blocks_reserve_shared(ostack, otop, orc, otab, lens, list(tails), bs,
                                                 lens)
    assert st == 0 and len(ocs) == 2
    ref.copy_blocks(L, hc, ocs, ocd)
    T = sum(tails)
    ref.append(L, hc, bits(k[prefix:]).reshape(T, -1), bits(v[prefix:]).reshape(T, -1), s2)
    # device
    gstack = torch.empty(n, dtype=torch.int32, device=DEV)
    gtop = torch.empty(1, dtype=torch.int32, device=DEV)
    kq.kvq_pool_init(gstack, gtop, _t(order))
    grc = torch.zeros(n, dtype=torch.int32, device=DEV)
    gtab = torch.full((3, 8), -1, dtype=torch.int32, device=DEV)
    glens = torch.zeros(3, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    cs = torch.full((3,), -7, dtype=torch.int32, device=DEV)
    cd = torch.full((3,), -7, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    gc = gpu_cache(LL, n, fill=0x33)
    sl = torch.empty(prefix, dtype=torch.int64, device=DEV)
    kq.kvq_blocks_reserve_shared(gstack, gtop, grc, gtab, glens, _t(np.array([prefix, 0, 0], np.int32)),
                                 bs, sl, cs, cd, cnt, status, glens)
    kq.kvq_append(LL, gc, k[:prefix].to(DEV), v[:prefix].to(DEV), sl)
    kq.kvq_blocks_fork(grc, gtab, glens, _t(np.array([0, 0], np.int32)),
                       _t(np.array([1, 2], np.int32)), bs)
    sl2 = torch.empty(T, dtype=torch.int64, device=DEV)
    kq.kvq_blocks_reserve_shared(gstack, gtop, grc, gtab, glens, _t(np.array(tails, np.int32)), bs,
                                 sl2, cs, cd, cnt, status, glens)
    kq.kvq_copy_blocks(LL, gc, cs, cd, cnt)
    kq.kvq_append(LL, gc, k[prefix:].to(DEV), v[prefix:].to(DEV), sl2)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and int(cnt.item()) == 2
    assert np.array_equal(gtab.cpu().numpy(), otab) and np.array_equal(glens.cpu().numpy(), lens)
    assert np.array_equal(grc.cpu().numpy(), orc)
    assert planes_equal(gc, hc) == []
    q = workloads.queries(w, seed=4)
    exp = ref.decode(L, hc, bits(q), ref.BF16, otab, lens, threads=4)
    got = decode_gpu(LL, gc, q.to(DEV), gtab, glens, int(lens.max()))
    assert_decode_close(got, exp, f"forked {code}")
