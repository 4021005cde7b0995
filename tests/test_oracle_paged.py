"""Pins of the oracle's paged placement, staging and block pool: hand-worked
cases, invariants and brute force on small inputs. No GPU."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import OracleSeqs, bits, oracle_layout

rng = np.random.default_rng(99)


def _rows(T, H, d, dtype=torch.bfloat16, seed=0):
    g = torch.Generator().manual_seed(seed)
    k = (torch.randn((T, H, d), generator=g) * 3).to(dtype)
    v = torch.randn((T, H, d), generator=g).to(dtype)
    return k, v


# ---------------------------------------------------------------------------
# Block pool.
# ---------------------------------------------------------------------------

def test_pool_hand_worked_example():
    bs = 4
    stack, top = ref.pool_init(8)                       # stack 0..7, top 8
    tables = np.full((2, 4), -1, np.int32)
    lens = np.array([0, 0], np.int32)
    # need = [ceil(3/4), ceil(5/4)] = [1, 2]; seq 0 takes stack[7],
    # seq 1 takes stack[5], stack[6].
    slots, st = ref.blocks_reserve(stack, top, tables, lens, [3, 5], bs)
    assert st == 0 and top[0] == 5
    assert tables[0, :1].tolist() == [7] and tables[1, :2].tolist() == [5, 6]
    assert slots.tolist() == [28, 29, 30, 20, 21, 22, 23, 24]
    lens = np.array([3, 5], np.int32)
    # need = [ceil(5/4)-1, ceil(9/4)-2] = [1, 1]: seq 0 takes stack[4] = 4,
    # seq 1 takes stack[3] = 3.
    lens_out = np.zeros(2, np.int32)
    slots, st = ref.blocks_reserve(stack, top, tables, lens, [2, 4], bs, lens_out)
    assert st == 0 and top[0] == 3 and lens_out.tolist() == [5, 9]
    assert tables.tolist() == [[7, 4, -1, -1], [5, 6, 3, -1]]
    assert slots.tolist() == [31, 16, 25, 26, 27, 12]
    # release sequence 1 (9 tokens = 3 blocks): pushed in logical order
    st = ref.blocks_release(stack, top, tables, lens_out, [0, 1], bs, lens_out)
    assert st == 0 and top[0] == 6 and stack[3:6].tolist() == [5, 6, 3]
    assert lens_out.tolist() == [5, 0]


def test_pool_all_or_nothing():
    stack, top = ref.pool_init(5)
    tables = np.full((2, 8), -1, np.int32)
    before = (stack.copy(), top.copy(), tables.copy())
    slots, st = ref.blocks_reserve(stack, top, tables, [0, 0], [33, 64], 16)  # needs 3 + 4
    assert st == ref.ERR_OUT_OF_BLOCKS
    assert (stack == before[0]).all() and top == before[1] and (tables == before[2]).all()
    assert (slots == -7).all()                       # slot output untouched
    # a sequence that would outgrow its table row fails the same way
    stack, top = ref.pool_init(100)
    slots, st = ref.blocks_reserve(stack, top, np.full((1, 2), -1, np.int32), [0], [33], 16)
    assert st == ref.ERR_OUT_OF_BLOCKS and top[0] == 100
    # release that would overflow the stack changes nothing
    stack, top = ref.pool_init(4)
    st = ref.blocks_release(stack, top, np.zeros((1, 4), np.int32), [16], [1], 16)
    assert st == ref.ERR_OUT_OF_BLOCKS and top[0] == 4


def test_pool_invariants_random_walk():
    N, B, bs, maxb = 400, 12, 16, 64
    order = rng.permutation(N).astype(np.int32)
    stack, top = ref.pool_init(N, order)
    tables = np.full((B, maxb), -1, np.int32)
    lens = np.zeros(B, np.int32)
    for step in range(60):
        new = rng.integers(0, 40, size=B).astype(np.int32)
        lens_out = np.zeros(B, np.int32)
        slots, st = ref.blocks_reserve(stack, top, tables, lens, new, bs, lens_out)
        if st == 0:
            # slots agree with tables, in batch order
            o = 0
            for b in range(B):
                for kk in range(new[b]):
                    pos = lens[b] + kk
                    assert slots[o] == tables[b, pos // bs] * bs + pos % bs
                    o += 1
            lens = lens_out
        live = np.concatenate([tables[b, :(lens[b] + bs - 1) // bs] for b in range(B)])
        assert len(set(live.tolist())) == len(live)                 # distinct
        assert ((live >= 0) & (live < N)).all()
        free = stack[:top[0]]
        assert sorted(np.concatenate([live, free]).tolist()) == list(range(N))
        if step % 7 == 6:
            mask = (rng.random(B) < 0.4).astype(np.int32)
            assert ref.blocks_release(stack, top, tables, lens, mask, bs, lens) == 0


# ---------------------------------------------------------------------------
# Paged placement.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("fp8", "token_sym"),
                                       ("int4", "group_asym"), ("int4", "token_sym"),
                                       ("none16", "token_sym")])
def test_paged_equals_contiguous(code, mode):
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode, v_mode=mode,
                      group_size=32 if mode == "group_asym" else 0, block_size=16,
                      src_dtype="bfloat16")
    L = oracle_layout(w)
    lens = np.array([37, 80, 5], np.int32)
    nb = 30
    k, v = _rows(int(lens.sum()), w.num_kv_heads, w.head_dim)
    paged = OracleSeqs(L, nb, 3, 8, order=rng.permutation(nb).astype(np.int32))
    flat = OracleSeqs(L, nb, 3, 8, order=None)
    for s in (paged, flat):
        s.append(k, v, lens)
    assert not (paged.tables == flat.tables).all()
    H, bs = w.num_kv_heads, w.block_size
    rb = {"none16": 2 * w.head_dim, "int4": w.head_dim // 2}.get(code, w.head_dim)
    for side, name in ((0, "k_codes"), (1, "v_codes")):
        A = paged.cache.planes[name].reshape(nb, H, bs, rb)
        Bp = flat.cache.planes[name].reshape(nb, H, bs, rb)
        for b in range(3):
            for pos in range(lens[b]):
                pa, pb = paged.tables[b, pos // bs], flat.tables[b, pos // bs]
                assert (A[pa, :, pos % bs] == Bp[pb, :, pos % bs]).all()
                xa = ref.dequant_token(L, paged.cache, side, paged.tables[b], lens[b], b, pos, 1)
                xb = ref.dequant_token(L, flat.cache, side, flat.tables[b], lens[b], b, pos, 1)
                assert (xa == xb).all()


def test_append_places_each_token_at_its_slot():
    # Brute force: every appended row, read back through the table, is the
    # quantization of the input row of that (token, head).
    w = workloads.get("tiny", block_size=16, src_dtype="float16")
    L = oracle_layout(w)
    lens = np.array([21, 16], np.int32)
    k, v = _rows(int(lens.sum()), 2, 64, dtype=torch.float16)
    s = OracleSeqs(L, 10, 2, 4, order=rng.permutation(10).astype(np.int32))
    slots, _ = s.append(k, v, lens)
    codes = s.cache.planes["k_codes"].view(np.int8).reshape(10, 2, 16, 64)
    scales = s.cache.scale(0).reshape(10, 2, 16)
    for t, slot in enumerate(slots):
        for h in range(2):
            q, sc = ref.quant_sym(k[t, h].float().numpy(), 127)
            assert (codes[slot // 16, h, slot % 16] == q).all()
            assert scales[slot // 16, h, slot % 16] == sc
    # slot -1 writes nothing
    before = s.cache.planes["k_codes"].copy()
    ref.append(L, s.cache, bits(k[:1]).reshape(1, -1), bits(v[:1]).reshape(1, -1), [-1])
    assert (before == s.cache.planes["k_codes"]).all()


# ---------------------------------------------------------------------------
# Per-channel-per-block keys with staging.
# ---------------------------------------------------------------------------

def _channel_block_run(chunks, lens_final, seed=5):
    w = workloads.get("mixed", batch=len(lens_final))
    L = oracle_layout(w)
    B = len(lens_final)
    total = int(sum(lens_final))
    k, v = _rows(total, w.num_kv_heads, w.head_dim, seed=seed)
    # per-sequence token streams
    starts = np.concatenate([[0], np.cumsum(lens_final)[:-1]])
    s = OracleSeqs(L, 64, B, 16, order=np.arange(64, dtype=np.int32))
    done = np.zeros(B, np.int64)
    for chunk in chunks:                                   # chunk[b] tokens per seq
        idx = np.concatenate([starts[b] + done[b] + np.arange(chunk[b]) for b in range(B)]).astype(np.int64)
        s.append(k[idx], v[idx], np.asarray(chunk, np.int32))
        done += np.asarray(chunk)
    return s, k


def test_channel_block_append_order_invariance():
    lens = [40, 19]
    splits = [
        [[1, 1]] * 19 + [[1, 0]] * 21,
        [[8, 8], [8, 8], [8, 3], [8, 0], [8, 0]],
        [[40, 19]],
        [[16, 5], [16, 14], [8, 0]],
    ]
    runs = [_channel_block_run(c, lens)[0] for c in splits]
    ref0 = runs[0]
    bs, H, d = 16, 8, 128

    def logical(r):
        kc = r.cache.planes["k_codes"].reshape(64, H, bs * d)
        vc = r.cache.planes["v_codes"].reshape(64, H, bs * d)
        ks = r.cache.scale(0).reshape(64, H, d)
        vs = r.cache.scale(1).reshape(64, H, bs)
        st = r.cache.planes["k_stage"].reshape(len(lens), H, bs, d * 2)
        out = []
        for b, Lb in enumerate(lens):
            for blk in range(Lb // bs):                    # completed blocks
                p = r.tables[b, blk]
                out += [kc[p].tobytes(), ks[p].tobytes(), vc[p].tobytes(), vs[p].tobytes()]
            tail = Lb % bs
            if tail:                                       # partial block
                p = r.tables[b, Lb // bs]
                out += [vc[p].reshape(H, bs, d)[:, :tail].tobytes(),
                        vs[p][:, :tail].tobytes(), st[b, :, :tail].tobytes()]
        return out

    expect = logical(ref0)
    for r in runs[1:]:
        assert logical(r) == expect


def test_channel_block_completed_blocks_and_raw_tail():
    s, k = _channel_block_run([[40, 19]], [40, 19])
    L = s.L
    kf = k.float().numpy()
    starts = [0, 40]
    for b, Lb in enumerate([40, 19]):
        full = (Lb // 16) * 16
        for blk in range(Lb // 16):
            rows = kf[starts[b] + 16 * blk: starts[b] + 16 * blk + 16]   # [16][H][d]
            for h in range(8):
                q, sc = ref.quant_channel_block(rows[:, h, :])
                pb = s.tables[b, blk]
                codes = s.cache.planes["k_codes"].view(np.int8).reshape(64, 8, 16, 128)
                assert (codes[pb, h] == q).all()
                assert (s.cache.scale(0).reshape(64, 8, 128)[pb, h] == sc).all()
        for pos in range(full, Lb):        # tail is read back raw
            for h in range(8):
                x = ref.dequant_token(L, s.cache, 0, s.tables[b], Lb, b, pos, h)
                assert (x == kf[starts[b] + pos, h]).all()
