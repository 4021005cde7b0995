"""Decode-step benchmark of the quantized paged KV cache on one MI355X.

One step is one pass of the whole hot path over a batch: the device pool
reserves a slot for one new token per sequence, then for every layer the new
token's K/V rows are quantized into the cache and decode attention runs over
the whole quantized context, the new token included: one
kvq_append_decode_attention launch (split kernel, which also codes the new
rows, + cross-split reduce) where the layout allows it, else kvq_append then
kvq_decode_attention (--two-call forces the latter). The default workload is the Llama-3-70B KV shape
with all 80 layers resident: 16 sequences x 32768 tokens, 64 query / 8 KV
heads, d = 128, FP8 E4M3 codes with fp32 per-token-per-head scales, block 16,
bf16 inputs (synthetic, seeded; see workloads.py).

Printed: one JSON line with the decode KV GB/s over the step (value), the
split+reduce launch durations measured with HIP events on the launch stream
(roofline), the bulk-append throughput measured while the cache is populated,
and the CPU oracle timed on a bounded sample of the same workload
(cpu_baseline).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_F16_TFLOPS = 2500.0   # dense fp16 MFMA, MI355X
HERE = os.path.dirname(os.path.abspath(__file__))
# sources whose change invalidates committed decode counters
DECODE_SOURCES = ("kvq_decode.hip", "kvq_attn_tiles.h", "kvq_int4_tiles.h", "kvq_device.h",
                  "kvq_encode.h",
                  "kvq_internal.h", "kvq_api.cpp")


def decode_source_hash():
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(HERE, "quantized_paged_kv_append_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """HBM bytes per kvq_decode_attention launch (split + reduce kernels)
    from the committed rocprofv3 counter summary of this workload, when it
    was taken on the current decode sources; None otherwise."""
    path = os.path.join(HERE, "profiles", f"decode_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            key, sep, val = line.strip().strip("`").partition(": ")
            if sep:
                fields[key] = val.strip()
    if fields.get("source_hash") != decode_source_hash():
        return None
    return float(fields["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_70b", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-extras", action="store_true",
                    help="measure only --workload (by default, the default llama3_70b line "
                         "also carries short runs of the other workloads under 'workloads')")
    ap.add_argument("--layers", type=int, default=0, help="0 = the workload's own count")
    ap.add_argument("--split-blocks", type=int, default=0)
    ap.add_argument("--batch", type=int, default=0, help="0 = the workload's own batch")
    ap.add_argument("--prefill-queries", type=int, default=0,
                    help="append this many tokens per sequence per step and attend with "
                         "all of them at once through kvq_prefill_attention (0: one "
                         "decode query per sequence)")
    ap.add_argument("--eager", action="store_true",
                    help="time the eager steps only (default: also one step captured in a "
                         "HIP graph, replayed; its time is the line's value)")
    ap.add_argument("--two-call", action="store_true",
                    help="append with kvq_append, then kvq_decode_attention, even where one "
                         "kvq_append_decode_attention launch could do both")
    ap.add_argument("--identity-pool", action="store_true",
                    help="blocks in order instead of a seeded permutation")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=0,
                    help="sequences of layer 0 the oracle decodes (0: enough for about "
                         "16 s of CPU work, at most the whole batch)")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--flush-mb", type=int, default=-1,
                    help="MiB of scratch read before every timed step so that no KV "
                         "bytes stay in L2 / the Infinity Cache between steps (-1: 1024 "
                         "when a step reads under 2 GB of KV, else 0)")
    ap.add_argument("--flush-write", action="store_true",
                    help="flush by writing the scratch instead of reading it (the "
                         "dirty lines are then written back during the next step)")
    ap.add_argument("--offload-blocks", type=int, default=0,
                    help="only time packing this many blocks of the workload's layout, the "
                         "copy of the pack to pinned host memory and back, and the unpack, "
                         "then exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB device buffer 3 times (reference kernel for "
                         "the FETCH_SIZE / WRITE_SIZE counter scale) and exit")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of exactly 1 GiB, three times: under
    rocprofv3 --pmc its FETCH_SIZE and WRITE_SIZE per dispatch give the factor
    that turns those counters into bytes."""
    dev = torch.device("cuda:0")
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "repeats": 3}))


def read_probe(nbytes=4 << 30, reps=10):
    """The HBM read rate of a kernel that only reads (kvq_read_probe: one pass
    over a 4 GiB buffer with 16-byte non-temporal loads over the whole GPU),
    HIP events around each launch on the current stream: the ceiling the
    decode's KV stream is compared with, measured in the same run."""
    import quantized_paged_kv_append_amd as kq
    dev = torch.device("cuda:0")
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        kq.kvq_read_probe(buf, sink)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        kq.kvq_read_probe(buf, sink)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    del buf
    torch.cuda.empty_cache()
    gbps = nbytes / (ms / 1e3) / 1e9
    return {"GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBS, 4),
            "bytes": nbytes, "launch_ms_median": round(ms, 4), "launches": reps}


def offload_bench(args):
    """Offload of quantized blocks: kvq_pack_blocks into a device buffer,
    that buffer to pinned host memory and back (hipMemcpyAsync through torch),
    kvq_unpack_blocks into other blocks; one JSON line with each rate and the
    packed bytes per block against the 16-bit cache's."""
    import quantized_paged_kv_append_amd as kq
    dev = torch.device("cuda:0")
    w = workloads.get(args.workload)
    LL = kq.make_layout(w.num_kv_heads, w.head_dim, w.block_size, w.k_code, w.v_code,
                        w.k_mode, w.v_mode, w.group_size, w.torch_dtype)
    L16 = kq.make_layout(w.num_kv_heads, w.head_dim, w.block_size, "none16", "none16",
                         "token_sym", "token_sym", 0, w.torch_dtype)
    n = args.offload_blocks
    cache = kq.PagedCache(LL, 2 * n, w.batch if w.k_mode == "channel_block" else 0, device=dev)
    for t in cache.planes.values():
        if t is not None:
            t.random_(0, 256)   # the bytes' values do not matter for the copies
    per = kq.kvq_block_pack_bytes(LL)
    ids = torch.randperm(n, device=dev).to(torch.int32)
    back_ids = (ids + n).to(torch.int32)
    packed = torch.empty(per * n, dtype=torch.uint8, device=dev)
    host = torch.empty(per * n, dtype=torch.uint8, pin_memory=True)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    times = {"pack": [], "d2h": [], "h2d": [], "unpack": []}
    for it in range(args.warmup + args.steps):
        ev[0].record(stream)
        kq.kvq_pack_blocks(LL, cache, ids, packed)
        ev[1].record(stream)
        host.copy_(packed, non_blocking=True)
        ev[2].record(stream)
        packed.copy_(host, non_blocking=True)
        ev[3].record(stream)
        kq.kvq_unpack_blocks(LL, cache, packed, back_ids)
        ev[4].record(stream)
        torch.cuda.synchronize()
        if it >= args.warmup:
            for k, (a, b) in zip(times, zip(ev[:-1], ev[1:])):
                times[k].append(a.elapsed_time(b))
    nbytes = per * n
    rate = {k: round(nbytes / (float(np.median(v)) / 1e3) / 1e9, 2) for k, v in times.items()}
    print(json.dumps({"metric": "quantized block offload GB/s (pack, to host, from host, unpack)",
                      "value": rate["d2h"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "higher_is_better": True,
                      "config": {"workload": w.name, "blocks": n, "k_code": w.k_code,
                                 "k_mode": w.k_mode, "block_size": w.block_size},
                      "rates_GBps": rate, "bytes_per_block": per,
                      "bytes_per_block_16bit": kq.kvq_block_pack_bytes(L16),
                      "link_bytes_ratio_vs_16bit": round(kq.kvq_block_pack_bytes(L16) / per, 3),
                      "ms_median": {k: round(float(np.median(v)), 4) for k, v in times.items()}}))


def kv_bytes_per_token_head(w):
    """Algorithmic bytes decode reads per (token, KV head, layer): key and
    value codes plus their scales (and zero points)."""
    bits = {"int8": 8, "fp8": 8, "int4": 4, "none16": 16}
    d = w.head_dim
    total = 0.0
    for code, mode in ((w.k_code, w.k_mode), (w.v_code, w.v_mode)):
        total += d * bits[code] / 8
        if code == "none16":
            continue
        if mode == "token_sym":
            total += 4
        elif mode == "group_asym":
            total += (d // w.group_size) * 5
        else:  # per-channel scales amortized over a block
            total += d * 4 / w.block_size
    return total


def append_bytes_per_token(w):
    """Algorithmic bytes of a bulk append per layer-token: 16-bit K and V rows
    in, codes and metadata out, plus the 8-byte slot."""
    return w.num_kv_heads * (2 * w.head_dim * 2 + kv_bytes_per_token_head(w)) + 8


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.offload_blocks:
        offload_bench(args)
        return
    torch.cuda.set_device(torch.device("cuda:0"))
    line = run(args, args.workload)
    explicit = any(a == "--workload" or a.startswith("--workload=") for a in sys.argv[1:])
    if not (args.no_extras or explicit or args.prefill_queries or args.batch or args.layers
            or args.split_blocks):
        # the other workloads, each on its own caches (freed in between), with
        # fewer steps: their per-launch decode and append figures
        extras = {}
        for name in EXTRA_WORKLOADS:
            sub = argparse.Namespace(**vars(args))
            sub.steps, sub.warmup, sub.no_cpu_baseline = min(args.steps, 10), 4, True
            torch.cuda.empty_cache()
            r = run(sub, name)
            extras[name] = {k: r[k] for k in ("value", "ms_per_step", "pct_of_hbm_peak",
                                               "decode_launch_ms",
                                               "decode_launch_ms_p10_p50_p90",
                                               "append_tok_s", "append_GBps", "dtype")}
            extras[name]["roofline"] = {k: r["roofline"][k] for k in
                                        ("achieved", "frac", "traffic", "bytes_per_launch")}
            extras[name]["config"] = {k: r["config"][k] for k in
                                      ("layers", "batch", "context", "num_q_heads",
                                       "k_code", "v_code", "k_mode", "v_mode", "block_size")}
        line["workloads"] = extras
        line["hbm_read_probe"] = read_probe()
    print(json.dumps(line))


# measured after the headline workload in a default run
EXTRA_WORKLOADS = ("llama3_70b_int8", "llama3_8b", "int4_long", "int4_batch", "mixed")


def run(args, wname):
    """Populate one workload's caches, time its steps and return the JSON
    line's fields (the caches are freed on return)."""
    import quantized_paged_kv_append_amd as kq

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = workloads.get(wname)
    if args.batch:
        w = workloads.get(wname, batch=args.batch)
    layers = args.layers or w.layers
    nq = args.prefill_queries
    LL = kq.make_layout(w.num_kv_heads, w.head_dim, w.block_size, w.k_code, w.v_code,
                        w.k_mode, w.v_mode, w.group_size, w.torch_dtype)
    lens = workloads.lengths(w)
    B, Hq, H, d, bs = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    new_per_step = nq if nq else w.new_tokens
    # eager steps, then (unless --eager) as many graph replays
    total_steps = (args.warmup + args.steps) * (1 if args.eager else 2)
    headroom = new_per_step * total_steps
    nb = workloads.pool_blocks(lens, bs, headroom_tokens=headroom + bs)
    maxb = (int(lens.max()) + headroom) // bs + 2
    max_ctx = int(lens.max()) + headroom

    # ---- pool and the prompt's placement ----------------------------------
    order = torch.from_numpy(workloads.pool_order(nb, permuted=not args.identity_pool)).to(dev)
    stack = torch.empty(nb, dtype=torch.int32, device=dev)
    top = torch.empty(1, dtype=torch.int32, device=dev)
    kq.kvq_pool_init(stack, top, order)
    tables = torch.full((B, maxb), -1, dtype=torch.int32, device=dev)
    ctx = torch.zeros(B, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    T0 = int(lens.sum())
    slots0 = torch.empty(T0, dtype=torch.int64, device=dev)
    kq.kvq_blocks_reserve(stack, top, tables, ctx, torch.from_numpy(lens).to(dev), bs,
                          slots0, status, ctx)
    stage_rows0 = None
    if w.k_mode == "channel_block":
        stage_rows0 = torch.from_numpy(np.repeat(np.arange(B, dtype=np.int32), lens)).to(dev)

    # ---- populate every layer (bulk append, timed per call) ---------------
    warm = kq.PagedCache(LL, nb, B if w.k_mode == "channel_block" else 0, device=dev)
    wk, wv = workloads.kv_rows(w, 64, layer=0, device=dev, chunk=12345)
    kq.kvq_append(LL, warm, wk, wv, slots0[:64], None if stage_rows0 is None else stage_rows0[:64])
    torch.cuda.synchronize()          # first launch (code object load) is not timed
    del warm, wk, wv
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    append_ms = 0.0
    chunk = 1 << 19
    # every layer's planes first, so that the input generation's temporaries
    # do not fragment the allocator between them (the 16-bit cache of the 70B
    # shape holds 172 GB)
    caches = [kq.PagedCache(LL, nb, B if w.k_mode == "channel_block" else 0, device=dev)
              for _ in range(layers)]
    for layer in range(layers):
        cache = caches[layer]
        for c0 in range(0, T0, chunk):
            n = min(chunk, T0 - c0)
            k, v = workloads.kv_rows(w, n, layer=layer, device=dev, chunk=c0 // chunk)
            ev[0].record(stream)
            kq.kvq_append(LL, cache, k, v, slots0[c0:c0 + n],
                          None if stage_rows0 is None else stage_rows0[c0:c0 + n])
            ev[1].record(stream)
            ev[1].synchronize()
            append_ms += ev[0].elapsed_time(ev[1])
            del k, v
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "pool reservation for the prompt failed"
    append_tok_s = T0 * layers / (append_ms / 1e3)
    append_gbs = append_tok_s * append_bytes_per_token(w) / 1e9

    # ---- per-step inputs: new K/V rows and queries for every layer ---------
    Tn = B * new_per_step
    new_kv = [workloads.kv_rows(w, Tn, layer=layer, device=dev, chunk=999) for layer in range(layers)]
    if nq:
        qs = [workloads.query_rows(w, B * nq, device=dev, layer=layer) for layer in range(layers)]
        qstart = torch.arange(0, B * nq + 1, nq, dtype=torch.int32, device=dev)
    else:
        qs = [workloads.queries(w, device=dev, layer=layer) for layer in range(layers)]
    new_tok = torch.full((B,), new_per_step, dtype=torch.int32, device=dev)
    slots = torch.empty(Tn, dtype=torch.int64, device=dev)
    stage_rows = None
    if w.k_mode == "channel_block":
        stage_rows = torch.from_numpy(np.repeat(np.arange(B, dtype=np.int32), new_per_step)).to(dev)
    if nq:
        out = torch.empty((B * nq, Hq, d), dtype=w.torch_dtype, device=dev)
        ws = torch.empty(kq.kvq_prefill_workspace_bytes(LL, B, Hq, nq, max_ctx, args.split_blocks),
                         dtype=torch.uint8, device=dev)
    else:
        out = torch.empty((B, Hq, d), dtype=w.torch_dtype, device=dev)
        ws = torch.empty(kq.kvq_decode_workspace_bytes(LL, B, Hq, max_ctx, args.split_blocks),
                         dtype=torch.uint8, device=dev)
    dec_ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(layers)] for _ in range(args.steps)]

    # one launch appends and attends for byte codes with per-token scales and
    # for 16-bit rows (the layouts kvq_append_decode_attention takes)
    fused = not nq and not args.two_call and (
        (w.k_code == w.v_code and w.k_code in ("int8", "fp8")
         and w.k_mode == w.v_mode == "token_sym") or w.k_code == w.v_code == "none16")

    def step(evs=None):
        kq.kvq_blocks_reserve(stack, top, tables, ctx, new_tok, bs, slots, status, ctx)
        for layer in range(layers):
            k, v = new_kv[layer]
            if fused:
                if evs is not None:
                    evs[layer][0].record(stream)
                kq.kvq_append_decode_attention(LL, caches[layer], k, v, qs[layer], tables, ctx,
                                               max_ctx, out, ws, split_blocks=args.split_blocks)
                if evs is not None:
                    evs[layer][1].record(stream)
                continue
            kq.kvq_append(LL, caches[layer], k, v, slots, stage_rows)
            if evs is not None:
                evs[layer][0].record(stream)
            if nq:
                kq.kvq_prefill_attention(LL, caches[layer], qs[layer], qstart, nq, tables, ctx,
                                         max_ctx, out, ws, split_blocks=args.split_blocks)
            else:
                kq.kvq_decode_attention(LL, caches[layer], qs[layer], tables, ctx, max_ctx, out,
                                        ws, split_blocks=args.split_blocks)
            if evs is not None:
                evs[layer][1].record(stream)

    # working sets that fit in the caches are flushed between steps
    kv_step_est = float(lens.sum()) * H * kv_bytes_per_token_head(w) * layers
    flush_mb = args.flush_mb if args.flush_mb >= 0 else (1024 if kv_step_est < 2e9 else 0)
    flush_buf = torch.ones(flush_mb << 20, dtype=torch.uint8, device=dev) if flush_mb else None
    flush_sink = torch.zeros(2, dtype=torch.int64, device=dev)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]

    # the last warm-up step runs right before the timed ones, with no idle gap
    # between them (the first launch after the GPU idles for the host's
    # reads runs ~30 us slower); the lengths are read before it, so the timed
    # steps start from them plus one step's tokens
    for _ in range(max(args.warmup - 1, 0)):
        step()
    torch.cuda.synchronize()
    ctx_before = ctx.cpu().numpy().astype(np.int64) + (new_per_step if args.warmup > 0 else 0)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.warmup > 0:
        step()
    t_start.record(stream)
    wall0 = time.perf_counter()
    for s_ in range(args.steps):
        if flush_buf is not None:
            if args.flush_write:
                flush_buf.fill_(s_ & 0xFF)
            else:   # a read leaves clean lines: nothing to write back later
                flush_sink[s_ % 2] = flush_buf.view(torch.int64).sum()
        step_ev[s_][0].record(stream)
        step(dec_ev[s_])
        step_ev[s_][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    # per-launch decode durations (events recorded on the launch stream)
    dec_ms = [a.elapsed_time(b) for evs in dec_ev for a, b in evs]
    wall = time.perf_counter() - wall0
    assert int(status.item()) == 0, "pool reservation during the steps failed"
    bracket_ms = t_start.elapsed_time(t_end) / args.steps
    # with a flush, a step is timed from its own events (the flush between
    # steps is not part of the work); otherwise the whole bracket counts
    step_ms = (float(np.mean([a.elapsed_time(b) for a, b in step_ev])) if flush_buf is not None
               else bracket_ms)

    # context attended at each timed step: before + new tokens of that step
    ctx_tokens = [(ctx_before + new_per_step * (s + 1)).sum() for s in range(args.steps)]
    bpth = kv_bytes_per_token_head(w)
    kv_bytes_step = float(np.mean(ctx_tokens)) * H * bpth * layers
    value = kv_bytes_step / (step_ms / 1e3) / 1e9
    eager_ms, eager_value = step_ms, value

    # ---- the same step captured once in a HIP graph, replayed -------------
    # (the library makes no allocation, memset or host synchronization, so
    # the graph holds its kernels only; per-launch figures stay the eager ones)
    graph_ms = None
    if not args.eager:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        for _ in range(max(args.warmup - 1, 0)):   # the last one as in the eager steps
            g.replay()
        torch.cuda.synchronize()
        ctx_g = ctx.cpu().numpy().astype(np.int64) + (new_per_step if args.warmup > 0 else 0)
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.warmup > 0:
            g.replay()
        g0.record(stream)
        for s_ in range(args.steps):
            if flush_buf is not None:
                flush_sink[s_ % 2] = flush_buf.view(torch.int64).sum()
            gev[s_][0].record(stream)
            g.replay()
            gev[s_][1].record(stream)
        g1.record(stream)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "pool reservation during the graph replays failed"
        graph_ms = (float(np.mean([a.elapsed_time(b) for a, b in gev])) if flush_buf is not None
                    else g0.elapsed_time(g1) / args.steps)
        ctx_tokens_g = [(ctx_g + new_per_step * (s + 1)).sum() for s in range(args.steps)]
        kv_bytes_step = float(np.mean(ctx_tokens_g)) * H * bpth * layers
        step_ms = graph_ms
        value = kv_bytes_step / (step_ms / 1e3) / 1e9
    dec_avg_ms = float(np.mean(dec_ms))
    dec_bytes_launch = float(np.mean(ctx_tokens)) * H * bpth
    achieved = dec_bytes_launch / (dec_avg_ms / 1e3) / 1e9

    cpu = None
    if not args.no_cpu_baseline and not nq:
        cpu = cpu_baseline(w, lens, args)
    roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": committed_traffic(w.name),
            "kernel": ("decode_split_kernel + decode_reduce_kernel (one "
                       + ("kvq_append_decode_attention, which also codes the step's "
                          "new rows)" if fused else "kvq_decode_attention)")),
            "bytes_per_launch": dec_bytes_launch}
    prefill = None
    if nq:
        # MFMA work per launch: every (query, head) pair takes 4 d flops per
        # position it sees (QK and PV, a multiply and an add each)
        vis = [sum(int(c) - nq + i + 1 for c in (ctx_before + nq * (s + 1)) for i in range(nq))
               for s in range(args.steps)]
        flops = float(np.mean(vis)) * Hq * 4 * d
        tflops = flops / (dec_avg_ms / 1e3) / 1e12
        prefill = {"queries_per_sequence": nq, "flops_per_launch": flops,
                   "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_MFMA_F16_TFLOPS, 4),
                   "hbm_frac": roof["frac"]}
        roof = ({"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_F16_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_F16_TFLOPS, 4),
                 "traffic": None, "flops_per_launch": flops}
                if tflops / PEAK_MFMA_F16_TFLOPS > roof["frac"] else dict(roof, traffic=None))
        roof["kernel"] = "prefill_split_kernel + prefill_reduce_kernel (one kvq_prefill_attention)"

    line = {
        "metric": ("prefill-attn KV GB/s (multi-query, causal) + MFMA TFLOP/s" if nq else
                   "decode-attn KV GB/s (% of 8 TB/s HBM) + append tok/s, INT8/FP8/INT4"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8_e4m3", "int8": "int8", "int4": "int4",
                  "none16": w.src_dtype.replace("float", "f").replace("bfloat", "bf")}[w.k_code]
                 + " codes, fp16 MFMA / fp32 accumulate",
        "data": "synthetic (seeded N(0,1) K/V/q with key outlier channels; workloads.py)",
        "config": {
            "workload": w.name, "layers": layers, "batch": B, "context": int(lens.max()),
            "num_q_heads": Hq, "num_kv_heads": H, "head_dim": d, "block_size": bs,
            "k_code": w.k_code, "v_code": w.v_code, "k_mode": w.k_mode, "v_mode": w.v_mode,
            "new_tokens_per_step": new_per_step, "pool": "identity" if args.identity_pool else "permuted",
            "split_blocks": args.split_blocks or "auto",
            "prefill_queries": nq or None,
            "step": "eager" if args.eager else "hip graph replay",
            "step_calls": ("reserve, then per layer kvq_append_decode_attention" if fused
                           else "reserve, then per layer kvq_append and the attention call"),
        },
        "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "kv_bytes_per_step": kv_bytes_step,
        "decode_launch_ms": round(dec_avg_ms, 5),
        "decode_launch_ms_p10_p50_p90": [round(float(x), 5)
                                         for x in np.percentile(dec_ms, [10, 50, 90])],
        "ms_per_step_bracket": round(bracket_ms, 4),
        "ms_per_step_eager": round(eager_ms, 4),
        "value_eager": round(eager_value, 2),
        "cache_flush_mb": flush_mb,
        "cache_flush": ("write" if args.flush_write else "read") if flush_mb else None,
        "append_tok_s": round(append_tok_s, 1),
        "append_GBps": round(append_gbs, 2),
        "append_bytes_per_token": append_bytes_per_token(w),
        "roofline": roof,
        "prefill": prefill,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    return line


def cpu_baseline(w, lens, args):
    """The oracle, as it stands, on a bounded sample of the same workload:
    layer 0, the first few sequences, every query head. Its own append builds
    its cache from host copies of the same seeded inputs (the benchmark's
    device results are never read), then its decode is timed."""
    from oracle import ref
    import ctypes

    cmap = {"none16": ref.CODE_NONE16, "int8": ref.CODE_INT8, "fp8": ref.CODE_FP8,
            "int4": ref.CODE_INT4}
    mmap = {"token_sym": ref.TOKEN_SYM, "group_asym": ref.GROUP_ASYM,
            "channel_block": ref.CHANNEL_BLOCK}
    OL = ref.layout(w.num_kv_heads, w.head_dim, w.block_size, cmap[w.k_code], cmap[w.v_code],
                    mmap[w.k_mode], mmap[w.v_mode], w.group_size,
                    ref.BF16 if w.src_dtype == "bfloat16" else ref.F16)
    nseq = args.cpu_sample_seqs
    if nseq <= 0:
        # about 1.8 us of one core per (cached token, query head), measured
        # with this oracle; aim at 16 core-seconds of decode
        budget = 16.0 / 1.8e-6
        work = np.cumsum(lens.astype(np.float64) * w.num_q_heads)
        nseq = int(np.searchsorted(work, budget)) + 1
    nseq = max(1, min(nseq, w.batch))
    sl = lens[:nseq].astype(np.int32)
    nb = workloads.pool_blocks(sl, w.block_size)
    stack, top = ref.pool_init(nb)
    tables = np.full((nseq, nb), -1, np.int32)
    slots, st = ref.blocks_reserve(stack, top, tables, np.zeros(nseq, np.int32), sl, w.block_size)
    hc = ref.HostCache(OL, nb, nseq)
    T = int(sl.sum())
    T0 = int(lens.sum())
    chunk = 1 << 19
    rows = np.repeat(np.arange(nseq, dtype=np.int32), sl)
    for c0 in range(0, T, chunk):
        # the same draws as the device populate of layer 0 (same chunk sizes)
        n_gen = min(chunk, T0 - c0)
        n = min(chunk, T - c0)
        k, v = workloads.kv_rows(w, n_gen, layer=0, device="cuda:0", chunk=c0 // chunk)
        kb = k[:n].cpu().contiguous().view(torch.int16).numpy().view(np.uint16).reshape(n, -1)
        vb = v[:n].cpu().contiguous().view(torch.int16).numpy().view(np.uint16).reshape(n, -1)
        del k, v
        ref.append(OL, hc, kb, vb, slots[c0:c0 + n], rows[c0:c0 + n])
    q = workloads.queries(w, device="cuda:0", layer=0)[:nseq]
    qb = q.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    threads = args.cpu_threads or len(os.sched_getaffinity(0))
    qdt = ref.BF16 if w.src_dtype == "bfloat16" else ref.F16
    t0 = time.perf_counter()
    ref.decode(OL, hc, qb, qdt, tables, sl, threads=threads)
    dt = time.perf_counter() - t0
    kv_bytes = float(sl.sum()) * w.num_kv_heads * kv_bytes_per_token_head(w)
    # the same oracle on one core, over the first sequences (about 4 s)
    n1 = max(1, min(nseq, int(np.searchsorted(
        np.cumsum(sl.astype(np.float64) * w.num_q_heads), 4.0 / 1.8e-6)) + 1))
    t0 = time.perf_counter()
    ref.decode(OL, hc, qb[:n1], qdt, tables[:n1], sl[:n1], threads=1)
    dt1 = time.perf_counter() - t0
    kv1 = float(sl[:n1].sum()) * w.num_kv_heads * kv_bytes_per_token_head(w)
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "value_1core": round(kv1 / dt1 / 1e9, 4),
            "sample": f"layer 0 of {w.name}: decode of sequences 0..{nseq - 1} "
                      f"({int(sl.sum())} cached tokens x {w.num_kv_heads} KV heads, all "
                      f"{w.num_q_heads} query heads), fp64 attention, {dt:.2f} s on "
                      f"{threads} threads; value_1core: sequences 0..{n1 - 1} on one "
                      f"thread, {dt1:.2f} s"}


if __name__ == "__main__":
    main()
