"""kvq_decode_attention on the GPU against the oracle (fp64 attention): caches
built by the oracle and copied to the device, so decode is tested on its own.
Tolerance |gpu - oracle| <= 2e-3 + 1e-3 |oracle| elementwise."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import DT, OracleSeqs, bits, oracle_layout
from _gpu_util import (DEV, assert_decode_close, decode_gpu, lib_layout, need_gpu,
                       upload)

pytestmark = pytest.mark.gpu

LENS = (37, 80, 5, 1, 16, 0, 17, 300, 15, 33)


def _setup(code="int8", d=128, bs=16, G=4, H=2, src="bfloat16", lens=LENS, seed=0,
           permuted=True, kscale=1.0, name="tiny", mode="token_sym", vmode=None, fill=0):
    w = workloads.get(name, k_code=code, v_code=code, k_mode=mode, v_mode=vmode or mode,
                      group_size=32 if mode == "group_asym" else 0,
                      src_dtype=src, head_dim=d, block_size=bs,
                      num_kv_heads=H, num_q_heads=G * H, batch=len(lens),
                      n_outliers=2, outlier_factor=8.0)
    L, LL = oracle_layout(w), lib_layout(w)
    lens = np.asarray(lens, np.int32)
    nb = workloads.pool_blocks(lens, bs) + 3
    order = workloads.pool_order(nb, seed=seed, permuted=permuted)
    maxb = int(lens.max()) // bs + 2
    s = OracleSeqs(L, nb, len(lens), maxb, order=order)
    if fill:
        s.cache = ref.HostCache(L, nb, len(lens), fill=fill)
    k, v = workloads.kv_rows(w, int(lens.sum()), seed=seed)
    if kscale != 1.0:
        k = (k.float() * kscale).to(w.torch_dtype)
    s.append(k, v, lens)
    q = workloads.queries(w, seed=seed)
    return w, L, LL, s, q


def _run(w, L, LL, s, q, out_dtype=torch.float32, sm_scale=0.0, split_blocks=0,
         max_len=None):
    exp = ref.decode(L, s.cache, bits(q), DT[w.src_dtype], s.tables, s.lens,
                     sm_scale=sm_scale, threads=8)
    gc = upload(s.cache, LL)
    got = decode_gpu(LL, gc, q.to(DEV), torch.from_numpy(s.tables).to(DEV),
                     torch.from_numpy(s.lens).to(DEV),
                     int(s.lens.max()) if max_len is None else max_len, out_dtype,
                     sm_scale, split_blocks)
    return got, exp


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("fp8", "token_sym"),
                                       ("int4", "token_sym"), ("int4", "group_asym"),
                                       ("none16", "token_sym")])
@pytest.mark.parametrize("d,bs", [(128, 16), (64, 16), (128, 32), (64, 32)])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_decode_matches_oracle(code, mode, d, bs, G):
    need_gpu()
    w, L, LL, s, q = _setup(code, d, bs, G, mode=mode)
    got, exp = _run(w, L, LL, s, q)
    assert_decode_close(got, exp, f"{code}/{mode} d{d} bs{bs} G{G}")
    assert (got[5] == 0).all()           # empty context


@pytest.mark.parametrize("src", ["bfloat16", "float16"])
@pytest.mark.parametrize("d,bs", [(128, 16), (64, 32)])
def test_decode_passthrough_16bit(src, d, bs):
    """NONE16: rows read as stored (fp16, or bf16 converted to fp16); every
    byte the appends left unwritten is 0xFF, a NaN pattern in both formats."""
    need_gpu()
    w, L, LL, s, q = _setup("none16", d, bs, 8, src=src, fill=0xFF)
    got, exp = _run(w, L, LL, s, q)
    assert_decode_close(got, exp, f"none16 {src} d{d} bs{bs}")
    assert (got[5] == 0).all()


@pytest.mark.parametrize("src", ["bfloat16", "float16"])
@pytest.mark.parametrize("d,bs", [(128, 16), (64, 16), (128, 32), (64, 32)])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_decode_channel_block_keys(src, d, bs, G):
    """INT8 keys with one scale per channel per block, the partial last block
    read raw from the sequence's stage row, INT8 per-token values. Every byte
    the appends left unwritten is 0xFF (NaN in the float planes and stage),
    which the decode must never let through."""
    need_gpu()
    w, L, LL, s, q = _setup("int8", d, bs, G, src=src, mode="channel_block",
                            vmode="token_sym", fill=0xFF)
    got, exp = _run(w, L, LL, s, q)
    assert_decode_close(got, exp, f"channel keys {src} d{d} bs{bs} G{G}")
    assert (got[5] == 0).all()


@pytest.mark.parametrize("split", [1, 3, 64, 256])
def test_decode_channel_block_split_counts(split):
    need_gpu()
    w, L, LL, s, q = _setup("int8", lens=(7000, 1, 250, 64, 0, 4133), G=8, mode="channel_block",
                            vmode="token_sym", fill=0xFF)
    got, exp = _run(w, L, LL, s, q, split_blocks=split)
    assert_decode_close(got, exp, f"channel keys split {split}")


@pytest.mark.parametrize("split", [1, 2, 3, 5, 64, 65, 130, 256])
@pytest.mark.parametrize("code,mode,bs", [("fp8", "token_sym", 16), ("int4", "group_asym", 32)])
def test_decode_split_counts(split, code, mode, bs):
    need_gpu()
    w, L, LL, s, q = _setup(code, lens=(7000, 1, 250, 64, 0, 4133), G=8, mode=mode, bs=bs)
    got, exp = _run(w, L, LL, s, q, split_blocks=split)
    assert_decode_close(got, exp, f"{code} split {split}")


# Per-token 8-bit codes go two 16-token tiles per softmax update: shares of
# 1, 2, 3 and 5 blocks leave every count of whole blocks after the ring (with
# and without a partial block), and shares of 256 blocks take the ring through
# several 64-block id windows.
@pytest.mark.parametrize("split", [0, 1, 2, 3, 5, 256])
@pytest.mark.parametrize("code", ["int8", "fp8"])
@pytest.mark.parametrize("d,bs", [(128, 16), (64, 16), (128, 32), (64, 32)])
def test_decode_paired_tiles_every_remainder(code, d, bs, split):
    need_gpu()
    lens = tuple(16 * k + r for k in range(9) for r in (0, 7)) + (1100, 2100, 4111)
    w, L, LL, s, q = _setup(code, d, bs, G=4, lens=lens)
    got, exp = _run(w, L, LL, s, q, split_blocks=split)
    assert_decode_close(got, exp, f"{code} d{d} bs{bs} split {split}")
    assert (got[0] == 0).all()           # empty context


@pytest.mark.parametrize("split", [0, 21, 40])
@pytest.mark.parametrize("mode", ["token_sym", "group_asym"])
@pytest.mark.parametrize("d,bs", [(128, 16), (64, 16), (128, 32), (64, 32)])
def test_decode_int4_long_shares(d, bs, mode, split):
    """INT4 with wave shares of many tiles, so that the kernel takes pairs of
    whole 16-token tiles from its ring and the last tiles of a share one at a
    time (whole or ragged), for both scale modes, both head sizes and both
    block sizes."""
    need_gpu()
    w, L, LL, s, q = _setup("int4", d=d, bs=bs, lens=(3001, 700, 93, 1, 0, 1290), G=8,
                            mode=mode)
    got, exp = _run(w, L, LL, s, q, split_blocks=split)
    assert_decode_close(got, exp, f"int4/{mode} d{d} bs{bs} split {split}")
    assert (got[4] == 0).all()


@pytest.mark.parametrize("split", [0, 3, 40])
@pytest.mark.parametrize("code,mode,bs", [("int8", "token_sym", 16), ("int4", "group_asym", 32)])
def test_decode_skewed_batch_over_planning_chunks(split, code, mode, bs):
    """300 sequences (past one 256-sequence chunk of the split planner): most
    short, three long, some empty, and a max_context_len above every length,
    so the launch holds more workgroups than the plan has items."""
    need_gpu()
    rng = np.random.default_rng(7)
    lens = rng.integers(0, 40, 300)
    lens[[3, 150, 299]] = [5000, 2600, 4100]
    lens[[0, 256, 257, 298]] = 0
    w, L, LL, s, q = _setup(code, lens=tuple(int(x) for x in lens), G=4, mode=mode, bs=bs)
    got, exp = _run(w, L, LL, s, q, split_blocks=split, max_len=int(lens.max()) + bs)
    assert_decode_close(got, exp, f"{code} skewed split {split}")
    assert (got[[0, 256, 257, 298]] == 0).all()


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("src", ["float16", "bfloat16"])
def test_decode_output_and_query_dtypes(out_dtype, src):
    need_gpu()
    w, L, LL, s, q = _setup("int8", src=src)
    got, exp = _run(w, L, LL, s, q, out_dtype=out_dtype)
    assert_decode_close(got, exp, f"{src}->{out_dtype}")


def test_decode_custom_scale_and_peaked_softmax():
    need_gpu()
    w, L, LL, s, q = _setup("int8", kscale=4.0)
    got, exp = _run(w, L, LL, s, q, sm_scale=0.4)
    assert_decode_close(got, exp, "sm 0.4, keys x4")


def test_decode_tiny_workload():
    """The tiny workload exactly: 1 sequence x 256 tokens, 4 query / 2 KV heads,
    d = 64, fp16, 2 key outlier channels x10, INT8 per-token scales, block 16."""
    need_gpu()
    w = workloads.get("tiny")
    L, LL = oracle_layout(w), lib_layout(w)
    lens = workloads.lengths(w)
    nb = workloads.pool_blocks(lens, w.block_size)
    s = OracleSeqs(L, nb, 1, nb, order=workloads.pool_order(nb))
    k, v = workloads.kv_rows(w, int(lens.sum()))
    s.append(k, v, lens)
    q = workloads.queries(w)
    got, exp = _run(w, L, LL, s, q)
    assert_decode_close(got, exp, "tiny")


@pytest.mark.parametrize("code,mode", [("fp8", "token_sym"), ("int4", "group_asym")])
def test_decode_paged_is_bit_identical_to_contiguous_and_permuted(code, mode):
    need_gpu()
    outs = []
    for permuted, seed_order in ((False, 0), (True, 1), (True, 2)):
        w, L, LL, s, q = _setup(code, G=8, permuted=permuted, seed=0, mode=mode)
        if permuted:   # same inputs, a different physical placement
            nb = s.cache.num_blocks
            s2 = OracleSeqs(L, nb, len(LENS), s.tables.shape[1],
                            order=workloads.pool_order(nb, seed=seed_order))
            k, v = workloads.kv_rows(w, int(np.sum(LENS)), seed=0)
            s2.append(k, v, np.asarray(LENS, np.int32))
            s = s2
        gc = upload(s.cache, LL)
        got = decode_gpu(LL, gc, q.to(DEV), torch.from_numpy(s.tables).to(DEV),
                         torch.from_numpy(s.lens).to(DEV), int(s.lens.max()))
        outs.append(got.cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_decode_gqa_equals_mha_with_duplicated_heads():
    """Query head h reads KV head h / G: GQA over H = 2 equals MHA over the
    KV heads duplicated G = 4 times. One-block ranges give both launches the
    same partials (the work partition otherwise depends on H, and with it the
    fp16 rounding of the probabilities), so they agree to fp32 rounding; each
    also matches the oracle, whose GQA and MHA outputs agree to fp64
    rounding."""
    need_gpu()
    w, L, LL, s, q = _setup("int8", G=4, H=2, lens=(90, 17, 300))
    got_gqa, exp_gqa = _run(w, L, LL, s, q, split_blocks=1)
    assert_decode_close(got_gqa, exp_gqa, "GQA")
    w8 = workloads.get("tiny", k_code="int8", v_code="int8", src_dtype="bfloat16",
                       head_dim=128, block_size=16, num_kv_heads=8, num_q_heads=8,
                       batch=3)
    L8, LL8 = oracle_layout(w8), lib_layout(w8)
    lens = np.array([90, 17, 300], np.int32)
    nb = workloads.pool_blocks(lens, 16) + 3
    s8 = OracleSeqs(L8, nb, 3, 21)
    k, v = workloads.kv_rows(w, int(lens.sum()), seed=0)
    s8.append(k.repeat_interleave(4, 1), v.repeat_interleave(4, 1), lens)
    gc = upload(s8.cache, LL8)
    got_mha = decode_gpu(LL8, gc, q.to(DEV), torch.from_numpy(s8.tables).to(DEV),
                         torch.from_numpy(s8.lens).to(DEV), 300, split_blocks=1)
    assert torch.allclose(got_gqa, got_mha, atol=1e-6, rtol=1e-6)
    exp_mha = ref.decode(L8, s8.cache, bits(q), DT[w8.src_dtype], s8.tables, s8.lens,
                         threads=8)
    assert np.allclose(exp_gqa, exp_mha, rtol=1e-12, atol=1e-12)
    assert_decode_close(got_mha, exp_mha, "MHA")


def test_decode_llama3_8b_workload_full():
    """The Llama-3-8B layer workload at full size (64 sequences, lengths
    uniform in [1024, 8192], 32 q / 8 KV heads, INT8), every output checked."""
    need_gpu()
    w = workloads.get("llama3_8b")
    L, LL = oracle_layout(w), lib_layout(w)
    lens = workloads.lengths(w)
    nb = workloads.pool_blocks(lens, w.block_size)
    s = OracleSeqs(L, nb, w.batch, int(lens.max()) // 16 + 1, order=workloads.pool_order(nb))
    k, v = workloads.kv_rows(w, int(lens.sum()))
    s.append(k, v, lens)
    q = workloads.queries(w)
    got, exp = _run(w, L, LL, s, q)
    err = assert_decode_close(got, exp, "llama3_8b")
    print(f"llama3_8b max err {err:.2e}")


def test_decode_reuses_one_workspace_across_shapes():
    """One workspace serves calls of growing and shrinking batch and split
    counts, each matching the oracle: no call depends on what an earlier one
    left in the workspace."""
    need_gpu()
    import quantized_paged_kv_append_amd as kq
    shapes = [((37, 80, 5, 1), 3), ((300, 0, 17, 16, 64, 15, 33, 2, 1, 90), 2),
              ((37, 80), 0), ((513, 1, 260), 1), ((0, 3, 0), 0), ((700, 3), 5)]
    ws = None
    for lens, split in shapes:
        w, L, LL, s, q = _setup("fp8", lens=lens)
        need = kq.kvq_decode_workspace_bytes(LL, len(lens), q.shape[1], int(max(lens)), split)
        if ws is None:
            ws = torch.full((1 << 22,), 0xFF, dtype=torch.uint8, device=DEV)
        assert need <= ws.numel()
        exp = ref.decode(L, s.cache, bits(q), DT[w.src_dtype], s.tables, s.lens, threads=8)
        gc = upload(s.cache, LL)
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
        kq.kvq_decode_attention(LL, gc, q.to(DEV), torch.from_numpy(s.tables).to(DEV),
                                torch.from_numpy(s.lens).to(DEV), int(max(lens)), out, ws,
                                split_blocks=split)
        torch.cuda.synchronize()
        assert_decode_close(out, exp, f"lens {lens} split {split}")


@pytest.mark.parametrize("code,mode,bs,split", [("fp8", "token_sym", 16, 0),
                                                ("int4", "group_asym", 32, 3)])
def test_decode_many_merges_grouped(code, mode, bs, split):
    """700 sequences x 6 query heads: 4200 cross-split merges, so the merge
    runs four heads per workgroup and its last workgroup of every sequence
    has two heads past the end; skewed short contexts, empty ones included,
    with several splits each."""
    need_gpu()
    rng = np.random.default_rng(7)
    lens = tuple(int(x) for x in rng.integers(0, 200, size=700))
    w, L, LL, s, q = _setup(code, lens=lens, G=3, H=2, mode=mode, bs=bs, d=64)
    got, exp = _run(w, L, LL, s, q, split_blocks=split)
    assert_decode_close(got, exp, f"{code} grouped merges")
    empty = np.nonzero(np.asarray(lens) == 0)[0]
    assert (got[torch.from_numpy(empty).to(got.device)] == 0).all()
