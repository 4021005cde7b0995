"""One decode step -- block reservation, quantize-on-append of the new
tokens, decode attention over the whole context, for two layers -- captured
once in a HIP graph and replayed step after step. Every replay, with the
program's own eager work (new inputs copied in) and synchronizations between
replays, must equal the same step run eagerly on an identical copy of the
state, bit for bit: outputs, pool, tables, lengths, slots and cache planes.
The library issues no memset, allocation or host synchronization, so the
graph holds only its kernels."""
import numpy as np
import pytest
import torch

import workloads
from _gpu_util import DEV, kq, lib_layout, need_gpu

pytestmark = pytest.mark.gpu


class State:
    """A pool, tables, lengths and per-layer caches, populated with the same
    prompt (same seeded rows, same slots) for every copy."""

    def __init__(self, w, LL, lens, layers, new_per_step, steps):
        B, bs = w.batch, w.block_size
        nb = workloads.pool_blocks(lens, bs, headroom_tokens=new_per_step * steps + bs)
        maxb = (int(lens.max()) + new_per_step * steps) // bs + 2
        self.max_ctx = int(lens.max()) + new_per_step * steps
        self.stack = torch.empty(nb, dtype=torch.int32, device=DEV)
        self.top = torch.empty(1, dtype=torch.int32, device=DEV)
        kq.kvq_pool_init(self.stack, self.top, torch.from_numpy(workloads.pool_order(nb)).to(DEV))
        self.tables = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
        self.ctx = torch.zeros(B, dtype=torch.int32, device=DEV)
        self.status = torch.zeros(1, dtype=torch.int32, device=DEV)
        T0 = int(lens.sum())
        slots0 = torch.empty(T0, dtype=torch.int64, device=DEV)
        kq.kvq_blocks_reserve(self.stack, self.top, self.tables, self.ctx,
                              torch.from_numpy(lens).to(DEV), bs, slots0, self.status, self.ctx)
        cb = w.k_mode == "channel_block"
        self.stage_rows = (torch.from_numpy(np.repeat(np.arange(B, dtype=np.int32), new_per_step))
                           .to(DEV) if cb else None)
        rows0 = (torch.from_numpy(np.repeat(np.arange(B, dtype=np.int32), lens)).to(DEV)
                 if cb else None)
        self.caches = []
        for layer in range(layers):
            c = kq.PagedCache(LL, nb, B if cb else 0, device=DEV)
            for t in c.planes.values():
                if t is not None:
                    t.fill_(0x5A)
            k, v = workloads.kv_rows(w, T0, layer=layer, device=DEV)
            kq.kvq_append(LL, c, k, v, slots0, rows0)
            self.caches.append(c)
        Tn = B * new_per_step
        self.slots = torch.full((Tn,), -3, dtype=torch.int64, device=DEV)
        self.new_tok = torch.full((B,), new_per_step, dtype=torch.int32, device=DEV)
        self.out = torch.zeros((layers, B, w.num_q_heads, w.head_dim), dtype=torch.float32,
                               device=DEV)
        self.ws = torch.zeros(kq.kvq_decode_workspace_bytes(LL, B, w.num_q_heads, self.max_ctx),
                              dtype=torch.uint8, device=DEV)

    def step(self, LL, bs, k_in, v_in, q_in):
        kq.kvq_blocks_reserve(self.stack, self.top, self.tables, self.ctx, self.new_tok, bs,
                              self.slots, self.status, self.ctx)
        for layer, c in enumerate(self.caches):
            kq.kvq_append(LL, c, k_in[layer], v_in[layer], self.slots, self.stage_rows)
            kq.kvq_decode_attention(LL, c, q_in[layer], self.tables, self.ctx, self.max_ctx,
                                    self.out[layer], self.ws)

    def snapshot(self):
        planes = [t.clone() for c in self.caches for t in c.planes.values() if t is not None]
        return [self.stack.clone(), self.top.clone(), self.tables.clone(), self.ctx.clone(),
                self.status.clone(), self.slots.clone(), self.out.clone()] + planes


@pytest.mark.parametrize("code,kmode,vmode,new_per_step", [
    ("fp8", "token_sym", "token_sym", 1),
    ("int4", "group_asym", "group_asym", 1),
    ("int8", "channel_block", "token_sym", 3),
])
def test_graph_replays_equal_eager_steps(code, kmode, vmode, new_per_step):
    need_gpu()
    layers, steps = 2, 5
    w = workloads.get("llama3_8b", k_code=code, v_code=code, k_mode=kmode, v_mode=vmode,
                      group_size=32 if kmode == "group_asym" else 0,
                      block_size=32 if code == "int4" else 16, batch=6,
                      lengths=("fixed", 0), new_tokens=new_per_step)
    lens = np.array([33, 300, 1, 17, 130, 64], np.int32)
    LL = lib_layout(w)
    eager = State(w, LL, lens, layers, new_per_step, steps)
    graphed = State(w, LL, lens, layers, new_per_step, steps)
    Tn = w.batch * new_per_step
    # graph inputs: fixed buffers that the program refills before each replay
    k_in = [torch.empty((Tn, w.num_kv_heads, w.head_dim), dtype=w.torch_dtype, device=DEV)
            for _ in range(layers)]
    v_in = [torch.empty_like(t) for t in k_in]
    q_in = [torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=w.torch_dtype, device=DEV)
            for _ in range(layers)]
    torch.cuda.synchronize()

    def load_inputs(s):
        for layer in range(layers):
            k, v = workloads.kv_rows(w, Tn, layer=layer, device=DEV, chunk=100 + s)
            k_in[layer].copy_(k.view(k_in[layer].shape))
            v_in[layer].copy_(v.view(v_in[layer].shape))
            q_in[layer].copy_(workloads.queries(w, device=DEV, step=s, layer=layer))

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            graphed.step(LL, w.block_size, k_in, v_in, q_in)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture ran nothing: the graphed state is still the populated prompt
    assert torch.equal(graphed.ctx, eager.ctx)
    for s in range(steps):
        load_inputs(s)
        eager.step(LL, w.block_size, k_in, v_in, q_in)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = eager.snapshot(), graphed.snapshot()
        assert int(eager.status.item()) == 0
        for i, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), f"step {s}: buffer {i} differs"
        assert bool(torch.isfinite(eager.out).all())
