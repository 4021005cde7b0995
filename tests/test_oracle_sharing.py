"""Pins of the oracle's prefix sharing (block reference counts, fork, copy on
write, release): a hand-worked example, equivalence with the plain pool when
nothing is shared, invariants over a random walk, and decode of forked
sequences against the same sequences built without sharing. No GPU."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import bits, oracle_layout

rng = np.random.default_rng(2024)


def test_hand_worked_fork_copy_on_write_release():
    stack, top = ref.pool_init(8)                       # ids 0..7 in order
    rc = np.zeros(8, np.int32)
    tables = np.full((2, 4), -1, np.int32)
    lens = np.zeros(2, np.int32)
    slots, st, cs, cd = ref.blocks_reserve_shared(stack, top, rc, tables, lens, [6, 0], 4, lens)
    assert st == 0 and tables[0, :2].tolist() == [6, 7] and top[0] == 6
    assert slots.tolist() == [24, 25, 26, 27, 28, 29] and rc[6] == 1 and rc[7] == 1
    ref.blocks_fork(rc, tables, lens, [0], [1], 4)
    assert tables[1, :2].tolist() == [6, 7] and lens[1] == 6 and rc[6] == 2 and rc[7] == 2
    # both append into the shared, half-filled block 7: both copy it first
    slots, st, cs, cd = ref.blocks_reserve_shared(stack, top, rc, tables, lens, [1, 3], 4, lens)
    assert st == 0
    assert cs.tolist() == [7, 7] and cd.tolist() == [5, 3]
    assert tables[0, :2].tolist() == [6, 5] and tables[1, :3].tolist() == [6, 3, 4]
    assert slots.tolist() == [22, 14, 15, 16]
    # block 7 lost both references and went back to the stack
    assert top[0] == 4 and stack[3] == 7 and rc[7] == 0
    assert [rc[i] for i in (6, 5, 3, 4)] == [2, 1, 1, 1]
    assert lens.tolist() == [7, 9]
    st = ref.blocks_release_shared(stack, top, rc, tables, lens, [0, 1], 4, lens)
    assert st == 0 and top[0] == 6 and stack[4:6].tolist() == [3, 4] and rc[6] == 1
    st = ref.blocks_release_shared(stack, top, rc, tables, lens, [1, 0], 4, lens)
    assert st == 0 and top[0] == 8 and stack[6:8].tolist() == [6, 5] and not rc.any()
    assert sorted(stack.tolist()) == list(range(8))


def test_without_sharing_equals_the_plain_pool():
    n, B, bs = 64, 6, 16
    order = rng.permutation(n).astype(np.int32)
    sa, ta = ref.pool_init(n, order)
    sb, tb = ref.pool_init(n, order)
    rcb = np.zeros(n, np.int32)
    tab_a = np.full((B, 12), -1, np.int32)
    tab_b = tab_a.copy()
    la = np.zeros(B, np.int32)
    lb = la.copy()
    for step in range(12):
        new = rng.integers(0, 40, B).astype(np.int32)
        s1, st1 = ref.blocks_reserve(sa, ta, tab_a, la, new, bs, la)
        s2, st2, cs, cd = ref.blocks_reserve_shared(sb, tb, rcb, tab_b, lb, new, bs, lb)
        assert st1 == st2 and len(cs) == 0
        if st1 == 0:
            assert np.array_equal(s1, s2)
        if step % 4 == 3:
            mask = (rng.random(B) < 0.5).astype(np.int32)
            assert ref.blocks_release(sa, ta, tab_a, la, mask, bs, la) == \
                ref.blocks_release_shared(sb, tb, rcb, tab_b, lb, mask, bs, lb)
        assert np.array_equal(sa[:ta[0]], sb[:tb[0]]) and ta[0] == tb[0]
        assert np.array_equal(tab_a, tab_b) and np.array_equal(la, lb)


def _check_invariants(stack, top, rc, tables, lens, bs, n):
    held = np.zeros(n, np.int64)
    for b, L in enumerate(lens):
        for i in range((L + bs - 1) // bs):
            held[tables[b, i]] += 1
    assert np.array_equal(held, rc), "counts equal the table references"
    free = stack[:top[0]]
    assert len(set(free.tolist())) == len(free), "no block twice on the stack"
    assert not (rc[free] != 0).any(), "free blocks are unreferenced"
    assert len(free) + int((rc > 0).sum()) == n, "every block is free or referenced"


def test_random_walk_invariants_and_exclusive_writes():
    n, B, bs = 48, 8, 4
    stack, top = ref.pool_init(n, rng.permutation(n).astype(np.int32))
    rc = np.zeros(n, np.int32)
    tables = np.full((B, 24), -1, np.int32)
    lens = np.zeros(B, np.int32)
    cows = 0
    for step in range(300):
        op = rng.integers(0, 3)
        if op == 0:
            new = (rng.integers(0, 7, B) * (rng.random(B) < 0.6)).astype(np.int32)
            before = tables.copy()
            rc0 = rc.copy()
            slots, st, cs, cd = ref.blocks_reserve_shared(stack, top, rc, tables, lens, new, bs,
                                                          lens)
            if st == 0:
                cows += len(cs)
                # every written slot lies in a block this sequence alone holds
                owner = np.repeat(np.arange(B), new)
                for s_, b in zip(slots, owner):
                    assert rc[s_ // bs] == 1 and (tables[b] == s_ // bs).any()
                # a copied block's source held the sequence's old last block
                for a, c in zip(cs, cd):
                    assert rc0[a] > 1 and rc0[c] == 0
            else:
                assert np.array_equal(before, tables) and np.array_equal(rc0, rc)
        elif op == 1:
            empty = np.flatnonzero(lens == 0)
            full = np.flatnonzero(lens > 0)
            if len(empty) and len(full):
                k = min(len(empty), len(full), int(rng.integers(1, 3)))
                ref.blocks_fork(rc, tables, lens, rng.choice(full, k, replace=False),
                                rng.choice(empty, k, replace=False), bs)
        else:
            mask = (rng.random(B) < 0.3).astype(np.int32)
            assert ref.blocks_release_shared(stack, top, rc, tables, lens, mask, bs, lens) == 0
        _check_invariants(stack, top, rc, tables, lens, bs, n)
    assert cows > 5


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("int4", "group_asym"),
                                       ("none16", "token_sym")])
def test_forked_sequences_decode_as_if_built_apart(code, mode):
    bs = 16
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode, v_mode=mode,
                      group_size=32 if mode == "group_asym" else 0, block_size=bs,
                      head_dim=64, num_kv_heads=2, num_q_heads=8, batch=3, src_dtype="bfloat16")
    L = oracle_layout(w)
    n = 40
    prefix, tails = 37, (5, 11, 0)
    k, v = workloads.kv_rows(w, prefix + sum(tails), seed=4)
    # shared: one prefix, forked twice, then each sequence appends its tail
    stack, top = ref.pool_init(n, rng.permutation(n).astype(np.int32))
    rc = np.zeros(n, np.int32)
    tables = np.full((3, 8), -1, np.int32)
    lens = np.zeros(3, np.int32)
    cache = ref.HostCache(L, n)
    slots, st, _, _ = ref.blocks_reserve_shared(stack, top, rc, tables, lens, [prefix, 0, 0], bs,
                                                lens)
    ref.append(L, cache, bits(k[:prefix]).reshape(prefix, -1), bits(v[:prefix]).reshape(prefix, -1),
               slots)
    ref.blocks_fork(rc, tables, lens, [0, 0], [1, 2], bs)
    slots, st, cs, cd = ref.blocks_reserve_shared(stack, top, rc, tables, lens, list(tails), bs,
                                                  lens)
    assert st == 0 and len(cs) == 2                         # sequences 0 and 1 copy
    ref.copy_blocks(L, cache, cs, cd)
    T = sum(tails)
    ref.append(L, cache, bits(k[prefix:]).reshape(T, -1), bits(v[prefix:]).reshape(T, -1), slots)
    # apart: three sequences, each with its own copy of the prefix
    s2, t2 = ref.pool_init(n)
    tab2 = np.full((3, 8), -1, np.int32)
    l2 = np.zeros(3, np.int32)
    c2 = ref.HostCache(L, n)
    rows_k, rows_v = [], []
    for b in range(3):
        idx = np.r_[0:prefix, prefix + sum(tails[:b]) + np.arange(tails[b])].astype(np.int64)
        rows_k.append(k[idx])
        rows_v.append(v[idx])
    kk, vv = torch.cat(rows_k), torch.cat(rows_v)
    sl2, st2 = ref.blocks_reserve(s2, t2, tab2, l2, [prefix + t for t in tails], bs, l2)
    ref.append(L, c2, bits(kk).reshape(len(kk), -1), bits(vv).reshape(len(vv), -1), sl2)
    assert np.array_equal(lens, l2)
    q = workloads.queries(w, seed=4)
    a = ref.decode(L, cache, bits(q), ref.BF16, tables, lens)
    b = ref.decode(L, c2, bits(q), ref.BF16, tab2, l2)
    assert np.array_equal(a, b)
