"""Quantization error of each mode on the synthetic keys and values (N(0,1)
with key outlier channels x8, the 8B layer's distribution), computed with the
oracle: RMS and max |x_hat - x| per mode, and the decode-output error of each
quantized cache against fp64 attention over the unquantized rows. A diagnostic
stand-in for the pages' quality claims, not a dataset evaluation; the
assertions are the orderings the pages state (fewer bits cost more error; per
channel scales keep more of the keys than per token scales when some channels
carry outliers; groups of 32 help 4-bit codes). Run with -s to see the table.
No GPU."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import OracleSeqs, bits, oracle_layout


def _rows(n=1024, seed=0):
    w = workloads.get("llama3_8b")
    k, v = workloads.kv_rows(w, n, seed=seed)
    return w, k.float().numpy(), v.float().numpy()


def _err(x, xh):
    e = (xh.astype(np.float64) - x.astype(np.float64)).ravel()
    return float(np.sqrt(np.mean(e * e))), float(np.abs(e).max())


def _per_token(x, mode):
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        for h in range(x.shape[1]):
            r = x[t, h]
            if mode == "int8":
                q, s = ref.quant_sym(r, 127)
                out[t, h] = q * s
            elif mode == "int4":
                q, s = ref.quant_sym(r, 7)
                out[t, h] = q * s
            elif mode == "fp8":
                q, s = ref.quant_fp8(r)
                out[t, h] = np.array([ref.e4m3_value(c) for c in q.tolist()]) * s
            else:  # int4 g32 asymmetric
                for g in range(0, r.size, 32):
                    q, s, z = ref.quant_asym4(r[g:g + 32])
                    out[t, h, g:g + 32] = (q.astype(np.float32) - z) * s
    return out


def _per_channel_block(x, bs=16):
    out = np.empty_like(x)
    for t0 in range(0, x.shape[0], bs):
        for h in range(x.shape[1]):
            q, s = ref.quant_channel_block(x[t0:t0 + bs, h])
            out[t0:t0 + bs, h] = q * s
    return out


def test_reconstruction_error_orderings():
    w, k, v = _rows()
    res = {}
    for mode in ("int8", "fp8", "int4", "int4_g32"):
        res[("K", mode)] = _err(k, _per_token(k, mode))
        res[("V", mode)] = _err(v, _per_token(v, mode))
    res[("K", "int8_channel_block")] = _err(k, _per_channel_block(k))
    print("\nside  mode                 RMS        max")
    for (side, mode), (rms, mx) in res.items():
        print(f"{side:5s} {mode:20s} {rms:.3e}  {mx:.3e}")
    for side in ("K", "V"):
        assert res[(side, "int8")][0] < res[(side, "int4_g32")][0] < res[(side, "int4")][0]
    # per-channel keys beat per-token keys when channels carry outliers
    assert res[("K", "int8_channel_block")][0] < res[("K", "int8")][0]


@pytest.mark.parametrize("seed", [0])
def test_decode_output_error_against_unquantized_attention(seed):
    base = workloads.get("tiny", head_dim=128, num_kv_heads=2, num_q_heads=8, batch=4,
                         src_dtype="bfloat16", n_outliers=4, outlier_factor=8.0)
    lens = np.array([700, 64, 333, 1024], np.int32)
    T = int(lens.sum())
    k, v = workloads.kv_rows(base, T, seed=seed)
    q = workloads.queries(base, seed=seed)
    outs = {}
    for name, code, mode, vmode, bs in (("none16", "none16", "token_sym", None, 16),
                                        ("int8", "int8", "token_sym", None, 16),
                                        ("fp8", "fp8", "token_sym", None, 16),
                                        ("int4_g32", "int4", "group_asym", None, 32),
                                        ("int4", "int4", "token_sym", None, 16),
                                        ("int8_channel_K", "int8", "channel_block", "token_sym", 16)):
        w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode, v_mode=vmode or mode,
                          group_size=32 if mode == "group_asym" else 0, head_dim=128,
                          num_kv_heads=2, num_q_heads=8, batch=4, src_dtype="bfloat16",
                          block_size=bs)
        L = oracle_layout(w)
        nb = workloads.pool_blocks(lens, bs) + 2
        s = OracleSeqs(L, nb, 4, 1024 // bs + 2, max_seqs=4)
        s.append(k, v, lens)
        outs[name] = ref.decode(L, s.cache, bits(q), ref.BF16, s.tables, s.lens, threads=8)
    exact = outs.pop("none16")
    print("\ndecode output error vs unquantized (fp64 attention over bf16 rows)")
    errs = {}
    for name, o in outs.items():
        errs[name] = _err(exact, o)
        print(f"{name:16s} RMS {errs[name][0]:.3e}  max {errs[name][1]:.3e}")
    assert errs["int8"][0] < errs["int4_g32"][0] < errs["int4"][0]
    assert errs["int8_channel_K"][0] < errs["int8"][0]
