"""kvq_append_static on the GPU against the oracle: every byte of every plane
equal (codes saturated at the code range, the given scales and zero points in
the metadata planes, untouched bytes)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import OracleSeqs, bits, oracle_layout
from _gpu_util import (DEV, assert_decode_close, decode_gpu, gpu_cache, lib_layout,
                       need_gpu, planes_equal, kq)

pytestmark = pytest.mark.gpu

CASES = [  # k code, v code, mode, src, d, bs
    ("int8", "int8", "token_sym", "bfloat16", 128, 16),
    ("int8", "int8", "token_sym", "float16", 64, 32),
    ("fp8", "fp8", "token_sym", "bfloat16", 128, 16),
    ("fp8", "fp8", "token_sym", "float16", 64, 16),
    ("int4", "int4", "token_sym", "bfloat16", 128, 32),
    ("int4", "int4", "token_sym", "float16", 64, 16),
    ("int4", "int4", "group_asym", "bfloat16", 128, 32),
    ("int4", "int4", "group_asym", "float16", 64, 16),
    ("fp8", "none16", "token_sym", "bfloat16", 128, 16),
    ("int8", "fp8", "token_sym", "float16", 128, 16),
]


def _workload(kc, vc, mode, src, d, bs, H=3, batch=7):
    return workloads.get("tiny", k_code=kc, v_code=vc, k_mode=mode, v_mode=mode,
                         group_size=32 if mode == "group_asym" else 0, src_dtype=src,
                         head_dim=d, block_size=bs, num_kv_heads=H, num_q_heads=H,
                         batch=batch)


def _params(code, mode, H, d, lo, hi, seed):
    """Seeded static parameters: log-uniform scales in [10^lo, 10^hi] (with
    one power of two, so that exact ties occur) and, for asymmetric groups,
    zero points spread over [0, 15]."""
    if code == "none16":
        return None, None
    g = np.random.default_rng(seed)
    shape = (H, d // 32) if mode == "group_asym" else (H,)
    s = (10.0 ** g.uniform(lo, hi, shape)).astype(np.float32)
    s.flat[0] = 0.25
    z = g.integers(0, 16, shape).astype(np.uint8) if mode == "group_asym" else None
    return s, z


def _dev(a):
    return None if a is None else torch.from_numpy(a).to(DEV)


def _edge_rows(n, H, d, dtype, g):
    """Zero and -0 rows, the largest finite input, tiny magnitudes, quarters
    (exact ties at scale 0.25) and mixed signs far beyond the code range."""
    big = 65504.0 if dtype == torch.float16 else 3.0e38
    rows = torch.randn((n, H, d), generator=g) * 3
    rows[0] = 0.0
    rows[1] = -0.0
    rows[2] = big * torch.sign(torch.randn((H, d), generator=g))
    rows[3] = 1e-6 * torch.randn((H, d), generator=g)
    rows[4] = torch.randint(-80, 81, (H, d), generator=g) / 8.0
    rows[5] = torch.randn((H, d), generator=g) * 300.0
    return rows.to(dtype)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_append_static_matches_oracle_bytewise(case):
    need_gpu()
    kc, vc, mode, src, d, bs = case
    w = _workload(*case)
    H = w.num_kv_heads
    L, LL = oracle_layout(w), lib_layout(w)
    lens = np.array([37, 80, 5, 1, 16, 0, 33], np.int32)
    T = int(lens.sum())
    g = torch.Generator().manual_seed(13)
    k, v = workloads.kv_rows(w, T, seed=4)
    k[:6] = _edge_rows(6, H, d, w.torch_dtype, g)
    v[6:12] = _edge_rows(6, H, d, w.torch_dtype, g)
    # scales from well inside to well below the rows' spread: many codes saturate
    ks, kz = _params(kc, mode, H, d, -2.5, -0.5, 1)
    vs, vz = _params(vc, mode, H, d, -2.5, -0.5, 2)
    nb = workloads.pool_blocks(lens, bs) + 5
    seqs = OracleSeqs(L, nb, len(lens), 16, order=workloads.pool_order(nb, seed=1))
    seqs.cache = ref.HostCache(L, nb, fill=0xA5)
    slots, _ = seqs.grow(lens)
    slots[[3, 50, 120]] = -1
    ref.append_static(L, seqs.cache, bits(k).reshape(T, -1), bits(v).reshape(T, -1), slots,
                      ks, vs, kz, vz)
    gc = gpu_cache(LL, nb)
    kq.kvq_append_static(LL, gc, k.to(DEV), v.to(DEV), torch.from_numpy(slots).to(DEV),
                         _dev(ks), _dev(vs), _dev(kz), _dev(vz))
    torch.cuda.synchronize()
    assert planes_equal(gc, seqs.cache) == []


def _all_finite(dt, d):
    vals = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(dt).float()
    vals = vals[torch.isfinite(vals)].numpy()
    n = (len(vals) + d - 1) // d
    pad = np.concatenate([vals, np.zeros(n * d - len(vals), np.float32)])
    return torch.from_numpy(pad.reshape(n, 1, d)).repeat(1, 2, 1).to(dt)


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("fp8", "token_sym"),
                                       ("int4", "token_sym"), ("int4", "group_asym")])
@pytest.mark.parametrize("src", ["float16", "bfloat16"])
@pytest.mark.parametrize("scale", [1.0, 0.75, 1.0 / 3.0, 2.0 ** -20])
def test_append_static_every_16bit_input(code, mode, src, scale):
    """Exhaustive over the source format: every finite 16-bit value quantized
    at a few fixed scales (a power of two, whose quotients tie exactly, and
    two that are not; 2^-20 drives the whole range into saturation)."""
    need_gpu()
    dt = torch.float16 if src == "float16" else torch.bfloat16
    w = _workload(code, code, mode, src, 128, 16, H=2, batch=1)
    L, LL = oracle_layout(w), lib_layout(w)
    k = _all_finite(dt, 128)
    v = -k.flip(0)
    T = k.shape[0]
    nb = (T + 15) // 16
    slots = np.arange(T, dtype=np.int64)
    shape = (2, 4) if mode == "group_asym" else (2,)
    s = np.full(shape, scale, np.float32)
    z = (np.arange(8, dtype=np.uint8).reshape(2, 4) * 2 + 1) if mode == "group_asym" else None
    hc = ref.HostCache(L, nb, fill=0)
    ref.append_static(L, hc, bits(k).reshape(T, -1), bits(v).reshape(T, -1), slots, s, s, z, z)
    gc = gpu_cache(LL, nb, fill=0)
    kq.kvq_append_static(LL, gc, k.to(DEV), v.to(DEV), torch.from_numpy(slots).to(DEV),
                         _dev(s), _dev(s), _dev(z), _dev(z))
    torch.cuda.synchronize()
    assert planes_equal(gc, hc) == []


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("int4", "group_asym")])
def test_append_static_then_decode(code, mode):
    """A statically quantized cache reads back through decode like any
    other: GPU append_static then GPU decode, against the oracle's append and
    fp64 decode."""
    need_gpu()
    bs = 32 if mode == "group_asym" else 16
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode, v_mode=mode,
                      group_size=32 if mode == "group_asym" else 0, src_dtype="bfloat16",
                      head_dim=128, block_size=bs, num_kv_heads=2, num_q_heads=16, batch=4)
    L, LL = oracle_layout(w), lib_layout(w)
    lens = np.array([300, 17, 0, 64], np.int32)
    T = int(lens.sum())
    k, v = workloads.kv_rows(w, T, seed=6)
    ks, kz = _params(code, mode, 2, 128, -1.5, -1.0, 3)
    vs, vz = _params(code, mode, 2, 128, -1.5, -1.0, 4)
    nb = workloads.pool_blocks(lens, bs) + 2
    seqs = OracleSeqs(L, nb, 4, 20, order=workloads.pool_order(nb, seed=2))
    slots, _ = seqs.grow(lens)
    ref.append_static(L, seqs.cache, bits(k).reshape(T, -1), bits(v).reshape(T, -1), slots,
                      ks, vs, kz, vz)
    gc = gpu_cache(LL, nb, fill=0)
    kq.kvq_append_static(LL, gc, k.to(DEV), v.to(DEV), torch.from_numpy(slots).to(DEV),
                         _dev(ks), _dev(vs), _dev(kz), _dev(vz))
    q = workloads.queries(w, seed=6)
    exp = ref.decode(L, seqs.cache, bits(q), ref.BF16, seqs.tables, seqs.lens, threads=8)
    got = decode_gpu(LL, gc, q.to(DEV), torch.from_numpy(seqs.tables).to(DEV),
                     torch.from_numpy(seqs.lens).to(DEV), int(lens.max()))
    assert_decode_close(got, exp, f"static {code}/{mode}")


@pytest.mark.parametrize("src", ["bfloat16", "float16"])
@pytest.mark.parametrize("d,bs", [(128, 16), (64, 32)])
def test_append_static_channel_keys_bytewise_and_decode(src, d, bs):
    """Static per-channel INT8 keys next to static per-token INT8 values,
    appended in chunks: codes, the block scale rows and value planes equal to
    the oracle's, the stage rows of every partial last block too (earlier
    stage contents are never read), then decode against the oracle."""
    need_gpu()
    H, B = 4, 5
    w = workloads.get("mixed", batch=B, src_dtype=src, head_dim=d, block_size=bs,
                      num_kv_heads=H, num_q_heads=4 * H)
    L, LL = oracle_layout(w), lib_layout(w)
    lens_final = np.array([40, 19, 16, 3, 77], np.int32)
    starts = np.concatenate([[0], np.cumsum(lens_final)[:-1]])
    k, v = workloads.kv_rows(w, int(lens_final.sum()), seed=9)
    g = np.random.default_rng(5)
    ks = (10.0 ** g.uniform(-2.5, -1.0, (H, d))).astype(np.float32)
    ks[0, :4] = 0.25
    vs = (10.0 ** g.uniform(-2.0, -1.0, H)).astype(np.float32)
    chunks = [[1, 1, 1, 1, 1], [8, 0, 15, 2, 8], [31, 18, 0, 0, 60], [0, 0, 0, 0, 8]]
    nb = 40
    seqs = OracleSeqs(L, nb, B, 8, order=workloads.pool_order(nb, seed=2), max_seqs=B)
    seqs.cache = ref.HostCache(L, nb, B, fill=0x5A)
    gc = gpu_cache(LL, nb, B, fill=0x5A)
    done = np.zeros(B, np.int64)
    for ch in chunks:
        ch = np.asarray(ch, np.int32)
        idx = np.concatenate([starts[b] + done[b] + np.arange(ch[b]) for b in range(B)]).astype(np.int64)
        slots, rows = seqs.grow(ch)
        kk, vv = k[idx], v[idx]
        ref.append_static(L, seqs.cache, bits(kk).reshape(len(idx), -1),
                          bits(vv).reshape(len(idx), -1), slots, ks, vs, stage_rows=rows)
        kq.kvq_append_static(LL, gc, kk.to(DEV), vv.to(DEV), torch.from_numpy(slots).to(DEV),
                             _dev(ks), _dev(vs), stage_rows=torch.from_numpy(rows).to(DEV))
        done += ch
    torch.cuda.synchronize()
    assert planes_equal(gc, seqs.cache, ["k_codes", "k_scale", "v_codes", "v_scale"]) == []
    # the stage rows that decode reads: each sequence's partial last block
    st_g = gc.planes["k_stage"].cpu().numpy().reshape(B, H, bs, 2 * d)
    st_h = seqs.cache.planes["k_stage"].reshape(B, H, bs, 2 * d)
    for b, Lb in enumerate(lens_final):
        assert np.array_equal(st_g[b, :, :Lb % bs], st_h[b, :, :Lb % bs]), b
    q = workloads.queries(w, seed=9)
    exp = ref.decode(L, seqs.cache, bits(q), DT_[src], seqs.tables, seqs.lens, threads=8)
    got = decode_gpu(LL, gc, q.to(DEV), torch.from_numpy(seqs.tables).to(DEV),
                     torch.from_numpy(seqs.lens).to(DEV), int(lens_final.max()))
    assert_decode_close(got, exp, f"static channel keys {src} d{d} bs{bs}")


DT_ = {"float16": ref.F16, "bfloat16": ref.BF16}
