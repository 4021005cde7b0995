"""The debugging checks of block tables and slot mappings on the GPU: valid
maps report KVQ_OK and -1; planted bad entries report
KVQ_ERR_INVALID_ARGUMENT and the smallest offending index (the rule of
include/kvq.h written out here with numpy), whatever else is wrong later
in the map. Entries past a context's blocks are not read."""
import numpy as np
import pytest
import torch

from _gpu_util import DEV, kq, need_gpu

pytestmark = pytest.mark.gpu


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _run_tables(tables, lens, bs, nb):
    fb = torch.full((1,), -7, dtype=torch.int64, device=DEV)
    st = torch.full((1,), 99, dtype=torch.int32, device=DEV)
    kq.kvq_check_block_tables(_t(tables), _t(lens), bs, nb, fb, st)
    torch.cuda.synchronize()
    return int(st.item()), int(fb.item())


def _first_bad_tables(tables, lens, bs, nb):
    B, M = tables.shape
    for b in range(B):
        L = int(lens[b])
        if L < 0 or L > M * bs:
            return b * M
        for k in range(-(-L // bs)):
            if not 0 <= tables[b, k] < nb:
                return b * M + k
    return -1


@pytest.mark.parametrize("B,M,bs", [(3, 5, 16), (1500, 40, 16), (700, 24, 32)])
def test_block_table_check(B, M, bs):
    need_gpu()
    rng = np.random.default_rng(B)
    nb = 4 * B * M
    lens = rng.integers(0, M * bs + 1, B).astype(np.int32)
    tables = np.full((B, M), -1, np.int32)
    for b in range(B):
        n = -(-int(lens[b]) // bs)
        tables[b, :n] = rng.integers(0, nb, n)
    assert _run_tables(tables, lens, bs, nb) == (kq.kvq.KVQ_OK, -1)
    # entries past a context's blocks are never read, whatever they hold
    t2 = tables.copy()
    for b in range(B):
        n = -(-int(lens[b]) // bs)
        t2[b, n:] = rng.integers(-5, 5, M - n) * nb
    assert _run_tables(t2, lens, bs, nb) == (kq.kvq.KVQ_OK, -1)
    # planted faults: an id past the pool, a negative id, a length past the table
    used = [(b, k) for b in range(B) for k in range(-(-int(lens[b]) // bs))]
    for trial in range(4):
        t3, l3 = tables.copy(), lens.copy()
        picks = [used[i] for i in rng.choice(len(used), size=min(3, len(used)), replace=False)]
        for i, (b, k) in enumerate(picks):
            t3[b, k] = nb + i if (trial + i) % 2 else -1 - i
        if trial == 3:
            l3[rng.integers(0, B)] = M * bs + 1
        exp = _first_bad_tables(t3, l3, bs, nb)
        assert exp >= 0
        assert _run_tables(t3, l3, bs, nb) == (kq.kvq.KVQ_ERR_INVALID_ARGUMENT, exp), trial


@pytest.mark.parametrize("n", [1, 100, 70000])
def test_slot_check(n):
    need_gpu()
    rng = np.random.default_rng(n)
    nb, bs = 5000, 16
    slots = rng.integers(-1, nb * bs, n).astype(np.int64)

    def run(s):
        fb = torch.full((1,), -7, dtype=torch.int64, device=DEV)
        st = torch.full((1,), 99, dtype=torch.int32, device=DEV)
        kq.kvq_check_slots(_t(s), nb, bs, fb, st)
        torch.cuda.synchronize()
        return int(st.item()), int(fb.item())

    assert run(slots) == (kq.kvq.KVQ_OK, -1)
    s2 = slots.copy()
    bad = sorted(set(rng.integers(0, n, 3).tolist()))
    for i, t in enumerate(bad):
        s2[t] = nb * bs if i % 2 else -2
    assert run(s2) == (kq.kvq.KVQ_ERR_INVALID_ARGUMENT, bad[0])
