"""The device block pool against the oracle's pool: identical stacks, tops,
block tables, slot mappings, lengths and status words, step after step."""
import numpy as np
import pytest
import torch

from oracle import ref
from _gpu_util import DEV, kq, need_gpu

pytestmark = pytest.mark.gpu


class GpuPool:
    def __init__(self, n, B, maxb, order):
        self.stack = torch.empty(n, dtype=torch.int32, device=DEV)
        self.top = torch.empty(1, dtype=torch.int32, device=DEV)
        kq.kvq_pool_init(self.stack, self.top,
                         None if order is None else torch.from_numpy(order).to(DEV))
        self.tables = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
        self.status = torch.full((1,), 99, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("B,bs,n", [(5, 16, 64), (300, 16, 5000), (2500, 32, 40000)])
def test_pool_steps_match_oracle(B, bs, n):
    need_gpu()
    rng = np.random.default_rng(B)
    maxb = 96
    order = rng.permutation(n).astype(np.int32)
    gp = GpuPool(n, B, maxb, order)
    ostack, otop = ref.pool_init(n, order)
    otables = np.full((B, maxb), -1, np.int32)
    lens = np.zeros(B, np.int32)
    glens = torch.zeros(B, dtype=torch.int32, device=DEV)
    saw_fail = False
    for step in range(12):
        if step % 4 == 3:
            mask = (rng.random(B) < 0.3).astype(np.int32)
            olens = lens.copy()
            ost = ref.blocks_release(ostack, otop, otables, olens, mask, bs, olens)
            kq.kvq_blocks_release(gp.stack, gp.top, gp.tables, glens,
                                  torch.from_numpy(mask).to(DEV), bs, gp.status, glens)
            lens = olens
        else:
            big = step == 2
            new = rng.integers(0, 200 if big else 40, size=B).astype(np.int32)
            if big and B < 100:
                new[:] = 500          # forces exhaustion of the small pool
            olens = np.zeros(B, np.int32)
            oslots, ost = ref.blocks_reserve(ostack, otop, otables, lens, new, bs, olens)
            gslots = torch.full((int(new.sum()),), -7, dtype=torch.int64, device=DEV)
            kq.kvq_blocks_reserve(gp.stack, gp.top, gp.tables, glens,
                                  torch.from_numpy(new).to(DEV), bs, gslots, gp.status, glens)
            torch.cuda.synchronize()
            assert np.array_equal(gslots.cpu().numpy(), oslots), step
            if ost == 0:
                lens = olens
            else:
                saw_fail = True
        torch.cuda.synchronize()
        assert int(gp.status.item()) == ost, step
        assert int(gp.top.item()) == int(otop[0]), step
        assert np.array_equal(gp.stack.cpu().numpy(), ostack), step
        assert np.array_equal(gp.tables.cpu().numpy(), otables), step
        assert np.array_equal(glens.cpu().numpy(), lens), step
    if B < 100:
        assert saw_fail


def test_pool_release_overflow_changes_nothing():
    need_gpu()
    gp = GpuPool(4, 1, 4, None)
    tables = torch.zeros((1, 4), dtype=torch.int32, device=DEV)
    lens = torch.full((1,), 16, dtype=torch.int32, device=DEV)
    kq.kvq_blocks_release(gp.stack, gp.top, tables, lens,
                          torch.ones(1, dtype=torch.int32, device=DEV), 16, gp.status, lens)
    torch.cuda.synchronize()
    assert int(gp.status.item()) == kq.kvq.KVQ_ERR_OUT_OF_BLOCKS
    assert int(gp.top.item()) == 4 and int(lens.item()) == 16


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("B", [7, 1500])
def test_reserve_short_slot_buffer_changes_nothing(shared, B):
    """A slot_mapping_out one entry short of sum(new_tokens) is refused on the
    device: status KVQ_ERR_INVALID_ARGUMENT and no other byte written (stack,
    top, tables, counts, lengths, slots, copy pairs), even when the pool is
    also too small; the same call with the full buffer then matches the
    oracle. B = 1500 spans two chunks of the kernel's scan."""
    need_gpu()
    rng = np.random.default_rng(B + 17 * shared)
    bs, maxb, n = 16, 8, 4 * B
    order = rng.permutation(n).astype(np.int32)
    gp = GpuPool(n, B, maxb, order)
    ostack, otop = ref.pool_init(n, order)
    otab = np.full((B, maxb), -1, np.int32)
    lens0 = np.zeros(B, np.int32)                    # empty sequences (valid tables)
    new = rng.integers(1, 30, B).astype(np.int32)
    total = int(new.sum())
    glens = torch.from_numpy(lens0).to(DEV)
    grc = torch.zeros(n, dtype=torch.int32, device=DEV)
    cs = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    cd = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((1,), -7, dtype=torch.int32, device=DEV)

    def call(slots, lens_dev, new_t):
        if shared:
            kq.kvq_blocks_reserve_shared(gp.stack, gp.top, grc, gp.tables, lens_dev, new_t, bs,
                                         slots, cs, cd, cnt, gp.status, lens_dev)
        else:
            kq.kvq_blocks_reserve(gp.stack, gp.top, gp.tables, lens_dev, new_t, bs, slots,
                                  gp.status, lens_dev)

    def snapshot():
        torch.cuda.synchronize()
        return [t.cpu().clone() for t in (gp.stack, gp.top, gp.tables, glens, grc, cs, cd, cnt)]

    before = snapshot()
    short = torch.full((total - 1,), -7, dtype=torch.int64, device=DEV)
    call(short, glens, torch.from_numpy(new).to(DEV))
    after = snapshot()
    assert int(gp.status.item()) == kq.kvq.KVQ_ERR_INVALID_ARGUMENT
    assert all(torch.equal(a, b) for a, b in zip(before, after))
    assert (short.cpu() == -7).all()
    # also too many blocks for the pool: the slot check still comes first
    big = torch.full((B,), 64 * bs, dtype=torch.int32, device=DEV)
    short2 = torch.full((64 * bs * B - 1,), -7, dtype=torch.int64, device=DEV)
    call(short2, glens, big)
    assert int(gp.status.item()) == kq.kvq.KVQ_ERR_INVALID_ARGUMENT
    assert all(torch.equal(a, b) for a, b in zip(before, snapshot()))
    # the full buffer: the reservation the oracle makes
    olens = np.zeros(B, np.int32)
    if shared:
        orc = np.zeros(n, np.int32)
        oslots, ost, _, _ = ref.blocks_reserve_shared(ostack, otop, orc, otab, lens0, new, bs,
                                                      olens)
    else:
        oslots, ost = ref.blocks_reserve(ostack, otop, otab, lens0, new, bs, olens)
    full = torch.full((total,), -7, dtype=torch.int64, device=DEV)
    call(full, glens, torch.from_numpy(new).to(DEV))
    torch.cuda.synchronize()
    assert ost == 0 and int(gp.status.item()) == 0
    assert np.array_equal(full.cpu().numpy(), oslots)
    assert np.array_equal(gp.stack.cpu().numpy(), ostack)
    assert int(gp.top.item()) == int(otop[0])


@pytest.mark.parametrize("B,window,sink", [(1500, 40, 20), (3, 70, 0), (1100, 1, 33)])
def test_trim_large_batches_match_oracle(B, window, sink):
    """Trim after placing long contexts: chunks of 1024 rows, many more
    entries per chunk than threads, rows partly trimmed already (a second
    trim after growth), and rows with nothing to trim; stack, top, tables and
    status equal to the oracle's."""
    need_gpu()
    bs = 16
    rng = np.random.default_rng(B + window)
    lens = rng.integers(0, 2000 if B > 10 else 30000, size=B).astype(np.int32)
    maxb = int(lens.max()) // bs + 40
    n = int(sum((int(x) + 200) // bs + 2 for x in lens))
    order = rng.permutation(n).astype(np.int32)
    gp = GpuPool(n, B, maxb, order)
    ostack, otop = ref.pool_init(n, order)
    otables = np.full((B, maxb), -1, np.int32)
    zero = np.zeros(B, np.int32)
    glens = torch.zeros(B, dtype=torch.int32, device=DEV)
    oslots, ost = ref.blocks_reserve(ostack, otop, otables, zero, lens, bs)
    assert ost == 0
    gslots = torch.empty(int(lens.sum()), dtype=torch.int64, device=DEV)
    kq.kvq_blocks_reserve(gp.stack, gp.top, gp.tables, glens, torch.from_numpy(lens).to(DEV),
                          bs, gslots, gp.status, glens)
    cur = lens.copy()
    for rnd in range(2):
        ost = ref.blocks_trim(ostack, otop, otables, cur, window, sink, bs)
        kq.kvq_blocks_trim(gp.stack, gp.top, gp.tables, torch.from_numpy(cur).to(DEV), window,
                           sink, bs, gp.status)
        torch.cuda.synchronize()
        assert int(gp.status.item()) == ost, rnd
        assert int(gp.top.item()) == int(otop[0]), rnd
        assert np.array_equal(gp.stack.cpu().numpy(), ostack), rnd
        assert np.array_equal(gp.tables.cpu().numpy(), otables), rnd
        # grow every row by up to 180 tokens, then trim again
        new = rng.integers(0, 180, size=B).astype(np.int32)
        olens = np.zeros(B, np.int32)
        _, ost = ref.blocks_reserve(ostack, otop, otables, cur, new, bs, olens)
        assert ost == 0
        gs = torch.empty(int(new.sum()), dtype=torch.int64, device=DEV)
        g_cur = torch.from_numpy(cur).to(DEV)
        kq.kvq_blocks_reserve(gp.stack, gp.top, gp.tables, g_cur, torch.from_numpy(new).to(DEV),
                              bs, gs, gp.status, g_cur)
        cur = olens
