"""Full-size workloads in the benchmark's launch configuration: device pool ->
quantize-on-append -> decode, for one layer. The oracle runs its own pool
mirror from the same initial order (its tables are checked equal to the
device's, never read from it), appends the sampled sequences' rows and decodes
them; the device output and planes must match on those samples."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import DT, bits, oracle_layout
from _gpu_util import DEV, assert_decode_close, decode_gpu, kq, lib_layout, need_gpu

pytestmark = pytest.mark.gpu


def _populate(w, seed=0, chunk=1 << 20, layer=0):
    """What bench.py does for one layer: pool init (permuted order), one
    reservation for every sequence's context, K/V generated on the device and
    appended in chunks (layer selects that layer's draw)."""
    LL = lib_layout(w)
    lens = workloads.lengths(w, seed)
    nb = workloads.pool_blocks(lens, w.block_size, headroom_tokens=w.block_size)
    maxb = int(lens.max()) // w.block_size + 2
    order = workloads.pool_order(nb, seed)
    stack = torch.empty(nb, dtype=torch.int32, device=DEV)
    top = torch.empty(1, dtype=torch.int32, device=DEV)
    kq.kvq_pool_init(stack, top, torch.from_numpy(order).to(DEV))
    tables = torch.full((w.batch, maxb), -1, dtype=torch.int32, device=DEV)
    ctx = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    T = int(lens.sum())
    slots = torch.empty(T, dtype=torch.int64, device=DEV)
    status = torch.empty(1, dtype=torch.int32, device=DEV)
    kq.kvq_blocks_reserve(stack, top, tables, ctx, torch.from_numpy(lens).to(DEV),
                          w.block_size, slots, status, ctx)
    cache = kq.PagedCache(LL, nb, w.batch, device=DEV)
    k, v = workloads.kv_rows(w, T, seed=seed, device=DEV, layer=layer)
    rows = None
    if w.k_mode == "channel_block":   # stage row of each token: its sequence
        rows = torch.from_numpy(np.repeat(np.arange(w.batch, dtype=np.int32), lens)).to(DEV)
    for t0 in range(0, T, chunk):
        kq.kvq_append(LL, cache, k[t0:t0 + chunk], v[t0:t0 + chunk], slots[t0:t0 + chunk],
                      stage_rows=None if rows is None else rows[t0:t0 + chunk])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return dict(LL=LL, lens=lens, nb=nb, maxb=maxb, order=order, tables=tables, ctx=ctx,
                cache=cache, k=k, v=v, stack=stack, top=top)


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _check(w, P, sample=None, seed=0, layer=0):
    """sample: the sequences compared (None: every sequence)."""
    L = oracle_layout(w)
    lens, nb = P["lens"], P["nb"]
    if sample is None:
        sample = list(range(w.batch))
    # oracle pool mirror
    ostack, otop = ref.pool_init(nb, P["order"])
    otables = np.full((w.batch, P["maxb"]), -1, np.int32)
    oslots, st = ref.blocks_reserve(ostack, otop, otables, np.zeros(w.batch, np.int32),
                                    lens, w.block_size)
    assert st == 0
    assert np.array_equal(otables, P["tables"].cpu().numpy())
    # oracle append of the sampled sequences only (stage row = sequence), one
    # call per sequence on a thread pool: sequences own disjoint blocks and
    # stage rows, and the oracle's C code runs outside the interpreter lock
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    hc = ref.HostCache(L, nb, w.batch)

    def one(b):
        idx = (starts[b] + np.arange(lens[b])).astype(np.int64)
        ti = torch.from_numpy(idx).to(DEV)
        ki = bits(P["k"][ti]).reshape(len(idx), -1)
        vi = bits(P["v"][ti]).reshape(len(idx), -1)
        ref.append(L, hc, ki, vi, oslots[idx], np.full(lens[b], b, np.int32))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, sample))
    # planes of the sampled sequences' blocks, bytewise
    H, bs, d = w.num_kv_heads, w.block_size, w.head_dim
    chan = w.k_mode == "channel_block"
    blocks = np.concatenate([otables[b, :(lens[b] + bs - 1) // bs] for b in sample])
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
        g = P["cache"].planes[name]
        if g is None:
            continue
        per_block = g.numel() // nb
        gb = g.view(nb, per_block)[torch.from_numpy(blocks).long().to(DEV)].cpu().numpy()
        hb = hc.planes[name].reshape(nb, per_block)[blocks]
        # per-channel keys: a block's codes and scales exist once it is full
        chan_k = chan and name in ("k_codes", "k_scale")
        gb, hb = gb.reshape(len(blocks), H, bs, -1), hb.reshape(len(blocks), H, bs, -1)
        o = 0
        for b in sample:   # a partial last block: compare its written rows only
            n = (lens[b] + bs - 1) // bs
            tail = lens[b] - (n - 1) * bs
            full = n if tail == bs else n - 1
            assert np.array_equal(gb[o:o + full], hb[o:o + full]), (name, b)
            if full < n and not chan_k:
                assert np.array_equal(gb[o + n - 1, :, :tail], hb[o + n - 1, :, :tail]), (name, b)
            o += n
    if chan:   # staged rows of the partial last blocks
        gs = P["cache"].planes["k_stage"].cpu().numpy().reshape(w.batch, H, bs, d * 2)
        hs = hc.planes["k_stage"].reshape(w.batch, H, bs, d * 2)
        for b in sample:
            tail = lens[b] % bs
            assert np.array_equal(gs[b, :, :tail], hs[b, :, :tail]), ("k_stage", b)
    # decode: every query head of the sampled sequences (the oracle attends
    # over the sampled sequences only; the others get length 0)
    q = workloads.queries(w, seed=seed, device=DEV, layer=layer)
    got = decode_gpu(P["LL"], P["cache"], q, P["tables"], P["ctx"], int(lens.max()))
    olens = np.zeros_like(lens)
    olens[sample] = lens[sample]
    exp = ref.decode(L, hc, bits(q), DT[w.src_dtype], otables, olens, threads=_threads())
    P["oracle"] = dict(hc=hc, stack=ostack, top=otop, tables=otables)
    return assert_decode_close(got[torch.as_tensor(sample, device=DEV)], exp[sample], w.name)


def _multi_query(w, P, sample, nq=8, seed=0):
    """Multi-query attention over the populated layer, as `bench.py
    --prefill-queries` launches it: the last nq positions of each sampled
    sequence are its queries (the other sequences have none), compared with
    the oracle's multi-query attention over its cache of the same sequences
    (built by _check)."""
    L = oracle_layout(w)
    lens = P["lens"]
    counts = np.zeros(w.batch, np.int64)
    for b in sample:
        counts[b] = min(nq, int(lens[b]))
    qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    Tq, max_q, max_len = int(qs[-1]), int(counts.max()), int(lens.max())
    q = workloads.query_rows(w, Tq, seed=seed, device=DEV)
    ws = torch.empty(kq.kvq_prefill_workspace_bytes(P["LL"], w.batch, w.num_q_heads, max_q,
                                                    max_len, 0),
                     dtype=torch.uint8, device=DEV)
    out = torch.full((Tq, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32,
                     device=DEV)
    kq.kvq_prefill_attention(P["LL"], P["cache"], q, torch.from_numpy(qs).to(DEV), max_q,
                             P["tables"], P["ctx"], max_len, out, ws)
    torch.cuda.synchronize()
    o = P["oracle"]
    olens = np.zeros_like(lens)
    olens[sample] = lens[sample]
    exp = ref.prefill(L, o["hc"], bits(q), DT[w.src_dtype], qs, o["tables"], olens,
                      threads=_threads())
    return assert_decode_close(out, exp, f"{w.name} multi-query")


def _other_layers(w, n=2, seed=0):
    """Layer 1 and n seeded layers among the rest of the workload's layers."""
    g = np.random.default_rng([seed, 80])
    return [1] + sorted(int(x) for x in g.choice(np.arange(2, w.layers), n, replace=False))


@pytest.mark.parametrize("name", ["llama3_70b", "llama3_70b_int8"])
def test_llama3_70b_every_sequence_of_layer_0(name):
    """The 70B KV shape (16 x 32768 tokens, 64 q / 8 KV heads, block 16) with
    E4M3 or INT8 per-token codes: every sequence's planes and every query
    head's output of layer 0; then 8 queries at the end of three seeded
    sequences (the LDS-staged multi-query kernel over the whole layer)."""
    need_gpu()
    w = workloads.get(name)
    P = _populate(w)
    err = _check(w, P)
    print(f"{name} layer 0, all 16 sequences: max err {err:.2e}")
    sample = sorted(int(x) for x in np.random.default_rng([0, 83]).choice(w.batch, 3,
                                                                           replace=False))
    err = _multi_query(w, P, sample)
    print(f"{name} layer 0, 8 queries on sequences {sample}: max err {err:.2e}")


@pytest.mark.parametrize("name", ["llama3_70b", "llama3_70b_int8"])
def test_llama3_70b_seeded_rows_of_other_layers(name):
    """Layer 1 and two seeded layers of the 80 (each its own K/V/q draw): two
    seeded sequences each."""
    need_gpu()
    w = workloads.get(name)
    g = np.random.default_rng([0, 81])
    for layer in _other_layers(w):
        P = _populate(w, layer=layer)
        sample = sorted(int(x) for x in g.choice(w.batch, 2, replace=False))
        err = _check(w, P, sample=sample, layer=layer)
        print(f"{name} layer {layer}, sequences {sample}: max err {err:.2e}")
        del P
        torch.cuda.empty_cache()


def test_llama3_70b_one_layer_bf16_passthrough():
    """The 70B layer shape with the 16-bit passthrough cache."""
    need_gpu()
    w = workloads.get("llama3_70b_bf16")
    P = _populate(w)
    err = _check(w, P, sample=[0, 7, 15])
    print(f"llama3_70b_bf16 layer: max err {err:.2e}")


def test_llama3_8b_layer_int8():
    need_gpu()
    w = workloads.get("llama3_8b")
    P = _populate(w)
    lens = P["lens"]
    sample = [int(np.argmax(lens)), int(np.argmin(lens)), 7, 33]
    err = _check(w, P, sample=sample)
    print(f"llama3_8b: max err {err:.2e}")
    err = _multi_query(w, P, sample)
    print(f"llama3_8b, 8 queries: max err {err:.2e}")


def test_int4_long_context_one_layer():
    """One layer of the INT4 long-context workload: one 131072-token sequence,
    64 q / 8 KV heads, per-32-group scale and zero point, block 32; decode,
    then 8 queries at its end (64 columns per KV head: four column tiles,
    two per wave)."""
    need_gpu()
    w = workloads.get("int4_long")
    P = _populate(w)
    err = _check(w, P, sample=[0])
    print(f"int4_long layer: max err {err:.2e}")
    err = _multi_query(w, P, [0])
    print(f"int4_long layer, 8 queries: max err {err:.2e}")


def test_int4_batch_one_layer():
    """One layer of the INT4 batch workload: all 32 sequences (log-normal
    lengths, median 4096, cap 65536), decode and 8 queries per sequence, then
    seeded sequences of other layers."""
    need_gpu()
    w = workloads.get("int4_batch")
    P = _populate(w)
    err = _check(w, P)
    print(f"int4_batch layer 0, all 32 sequences: max err {err:.2e}")
    err = _multi_query(w, P, list(range(w.batch)))
    print(f"int4_batch layer 0, 8 queries per sequence: max err {err:.2e}")
    del P
    g = np.random.default_rng([0, 82])
    for layer in _other_layers(w, n=1):
        P = _populate(w, layer=layer)
        sample = sorted(int(x) for x in g.choice(w.batch, 3, replace=False))
        err = _check(w, P, sample=sample, layer=layer)
        print(f"int4_batch layer {layer}, sequences {sample}: max err {err:.2e}")
        del P


def test_mixed_continuous_step_one_layer():
    """The mixed workload at full size (256 sequences, log-normal lengths
    median 2048, cap 32768, INT8 per-channel-per-block keys with staging, INT8
    per-token values), then one continuous step: 8 new tokens per sequence
    reserved, appended and decoded, and the 8 tokens checked at once by
    multi-query attention."""
    need_gpu()
    w = workloads.get("mixed")
    P = _populate(w)
    lens = P["lens"]
    sample = [int(np.argmax(lens)), int(np.argmin(lens)), 3, 100, 255]
    err = _check(w, P, sample=sample)
    print(f"mixed populate: max err {err:.2e}")

    # one step: reserve, append (stage rows = sequence), decode
    B, n, bs = w.batch, w.new_tokens, w.block_size
    L = oracle_layout(w)
    O = P["oracle"]
    new_tok = np.full(B, n, np.int32)
    slots = torch.empty(B * n, dtype=torch.int64, device=DEV)
    status = torch.empty(1, dtype=torch.int32, device=DEV)
    kq.kvq_blocks_reserve(P["stack"], P["top"], P["tables"], P["ctx"],
                          torch.from_numpy(new_tok).to(DEV), bs, slots, status, P["ctx"])
    k2, v2 = workloads.kv_rows(w, B * n, seed=0, device=DEV, chunk=7)
    rows = torch.from_numpy(np.repeat(np.arange(B, dtype=np.int32), n)).to(DEV)
    kq.kvq_append(P["LL"], P["cache"], k2, v2, slots, stage_rows=rows)
    oslots, st = ref.blocks_reserve(O["stack"], O["top"], O["tables"], lens, new_tok, bs)
    torch.cuda.synchronize()
    assert st == 0 and int(status.item()) == 0
    assert np.array_equal(O["tables"], P["tables"].cpu().numpy())
    assert np.array_equal(oslots, slots.cpu().numpy())
    idx = np.concatenate([b * n + np.arange(n) for b in sample]).astype(np.int64)
    ref.append(L, O["hc"], bits(k2.cpu()[idx]).reshape(len(idx), -1),
               bits(v2.cpu()[idx]).reshape(len(idx), -1), oslots[idx],
               np.repeat(np.asarray(sample, np.int32), n))
    lens2 = lens + n
    q = workloads.queries(w, seed=0, device=DEV, step=1)
    got = decode_gpu(P["LL"], P["cache"], q, P["tables"], P["ctx"], int(lens2.max()))
    olens = np.zeros_like(lens2)
    olens[sample] = lens2[sample]
    exp = ref.decode(L, O["hc"], bits(q), DT[w.src_dtype], O["tables"], olens, threads=16)
    err = assert_decode_close(got[torch.as_tensor(sample, device=DEV)], exp[sample], "mixed step")
    print(f"mixed step: max err {err:.2e}")
    # the step's 8 new tokens as queries, checked at once (partial last blocks
    # read raw from the stage rows)
    P["lens"] = lens2
    err = _multi_query(w, P, sample)
    print(f"mixed step, 8 queries: max err {err:.2e}")
