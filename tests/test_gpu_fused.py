"""kvq_append_decode_attention (the step's new token coded into its slot by
the decode launch itself) against the two-call step it replaces: block
reservation, kvq_append, kvq_decode_attention. Two copies of one populated
state take the same steps, one per path; outputs, pool, tables, lengths and
every cache plane must agree bit for bit after each step, so the fused path
inherits the two-call path's parity with the oracle. Lengths put new tokens
at the first and last offset of a block and give one sequence its first
token; a graph replay of the fused step must equal it run eagerly."""
import numpy as np
import pytest
import torch

import workloads
from _gpu_util import DEV, kq, lib_layout, need_gpu
from test_gpu_graph import State

pytestmark = pytest.mark.gpu

LENS = np.array([0, 15, 16, 31, 1, 300, 47, 64], np.int32)


def _workload(code, d, bs, G, src):
    return workloads.get("llama3_8b", k_code=code, v_code=code, k_mode="token_sym",
                         v_mode="token_sym", src_dtype=src, head_dim=d, block_size=bs,
                         num_kv_heads=2, num_q_heads=2 * G, batch=len(LENS),
                         lengths=("fixed", 0), new_tokens=1)


def _inputs(w, s, layers):
    kv = [workloads.kv_rows(w, w.batch, layer=layer, device=DEV, chunk=200 + s)
          for layer in range(layers)]
    q = [workloads.queries(w, device=DEV, step=s, layer=layer) for layer in range(layers)]
    return kv, q


def _fused_step(st, LL, bs, kv, q, split):
    kq.kvq_blocks_reserve(st.stack, st.top, st.tables, st.ctx, st.new_tok, bs, st.slots,
                          st.status, st.ctx)
    for layer, c in enumerate(st.caches):
        k, v = kv[layer]
        kq.kvq_append_decode_attention(LL, c, k, v, q[layer], st.tables, st.ctx, st.max_ctx,
                                       st.out[layer], st.ws, split_blocks=split)


def _two_call_step(st, LL, bs, kv, q, split):
    kq.kvq_blocks_reserve(st.stack, st.top, st.tables, st.ctx, st.new_tok, bs, st.slots,
                          st.status, st.ctx)
    for layer, c in enumerate(st.caches):
        k, v = kv[layer]
        kq.kvq_append(LL, c, k, v, st.slots)
        kq.kvq_decode_attention(LL, c, q[layer], st.tables, st.ctx, st.max_ctx, st.out[layer],
                                st.ws, split_blocks=split)


def _same(a, b, what):
    for i, (x, y) in enumerate(zip(a.snapshot(), b.snapshot())):
        assert torch.equal(x, y), f"{what}: buffer {i} differs"


@pytest.mark.parametrize("code,d,bs,G,src,split", [
    ("fp8", 128, 16, 8, "bfloat16", 0),
    ("fp8", 64, 32, 1, "float16", 1),
    ("int8", 128, 16, 4, "bfloat16", 3),
    ("int8", 64, 16, 2, "float16", 0),
    ("int8", 128, 32, 16, "bfloat16", 0),
    ("none16", 128, 16, 8, "bfloat16", 0),
    ("none16", 64, 32, 4, "float16", 2),
])
def test_fused_step_equals_append_then_decode(code, d, bs, G, src, split):
    need_gpu()
    layers, steps = 2, 4
    w = _workload(code, d, bs, G, src)
    LL = lib_layout(w)
    fused = State(w, LL, LENS, layers, 1, steps)
    ref = State(w, LL, LENS, layers, 1, steps)
    for st in (fused, ref):   # the workspace for this split size
        st.ws = torch.zeros(kq.kvq_decode_workspace_bytes(LL, w.batch, w.num_q_heads, st.max_ctx,
                                                          split), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    for s in range(steps):
        kv, q = _inputs(w, s, layers)
        _two_call_step(ref, LL, bs, kv, q, split)
        _fused_step(fused, LL, bs, kv, q, split)
        torch.cuda.synchronize()
        assert int(ref.status.item()) == 0
        # the fused path leaves the reservation's slots as they were; compare
        # every buffer, slots included (both ran the same reservation)
        _same(ref, fused, f"{code} d{d} bs{bs} G{G} step {s}")
        assert bool(torch.isfinite(fused.out).all())
        assert (fused.ctx.cpu().numpy() == LENS + s + 1).all()


def test_fused_step_graph_replays_equal_eager():
    need_gpu()
    layers, steps = 2, 3
    w = _workload("fp8", 128, 16, 8, "bfloat16")
    LL = lib_layout(w)
    eager = State(w, LL, LENS, layers, 1, steps)
    graphed = State(w, LL, LENS, layers, 1, steps)
    k_in = [torch.empty((w.batch, w.num_kv_heads, w.head_dim), dtype=w.torch_dtype, device=DEV)
            for _ in range(layers)]
    v_in = [torch.empty_like(t) for t in k_in]
    q_in = [torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=w.torch_dtype, device=DEV)
            for _ in range(layers)]
    kv_in = list(zip(k_in, v_in))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            _fused_step(graphed, LL, w.block_size, kv_in, q_in, 0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for s in range(steps):
        kv, q = _inputs(w, s, layers)
        for layer in range(layers):
            k_in[layer].copy_(kv[layer][0].view(k_in[layer].shape))
            v_in[layer].copy_(kv[layer][1].view(v_in[layer].shape))
            q_in[layer].copy_(q[layer])
        _fused_step(eager, LL, w.block_size, kv_in, q_in, 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(eager, graphed, f"graph step {s}")


def test_fused_step_skips_a_length_past_max_context_len():
    """A length above max_context_len (a broken precondition) is cut to it by
    the decode; the fused call then codes no row for that sequence rather than
    one over a cached token. Equal, bit for bit, to kvq_append with that
    sequence's slot set to -1, then decode with the same cut."""
    need_gpu()
    w = _workload("int8", 128, 16, 4, "bfloat16")
    LL = lib_layout(w)
    fused = State(w, LL, LENS, 1, 1, 1)
    ref = State(w, LL, LENS, 1, 1, 1)
    long_b = int(np.argmax(LENS))
    cut = int(LENS[long_b])          # after the reservation that sequence holds cut + 1
    kv, q = _inputs(w, 0, 1)
    k, v = kv[0]
    for st in (fused, ref):
        kq.kvq_blocks_reserve(st.stack, st.top, st.tables, st.ctx, st.new_tok, w.block_size,
                              st.slots, st.status, st.ctx)
    skip = ref.slots.clone()
    skip[long_b] = -1
    kq.kvq_append(LL, ref.caches[0], k, v, skip)
    kq.kvq_decode_attention(LL, ref.caches[0], q[0], ref.tables, ref.ctx, cut, ref.out[0], ref.ws)
    kq.kvq_append_decode_attention(LL, fused.caches[0], k, v, q[0], fused.tables, fused.ctx, cut,
                                   fused.out[0], fused.ws)
    torch.cuda.synchronize()
    assert int(ref.status.item()) == 0
    _same(ref, fused, "cut length")
