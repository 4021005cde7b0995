"""Seeded synthetic inputs shared by the tests, the smoke check and bench.py.

This module holds shapes, seeds and random draws only -- none of the
quantization or attention arithmetic. Both the GPU path and the CPU oracle are
fed from the tensors made here (the oracle through host copies).

Workloads (KV shapes from the pages: Llama-3-8B and Llama-3-70B with 8 KV heads
and head dimension 128, block size 16 as the paged default; "KV Cache
Optimization" glossary, "Technical Architecture"; "KV Cache Optimization:
Strategies ...", "How vLLM Implements KV Cache Optimization"):

  tiny        1 layer, 1 sequence of 256 tokens, 4 q / 2 KV heads, d 64, fp16,
              2 key outlier channels x10, INT8 per-token scales, bs 16
  llama3_8b   1 layer, 64 sequences, lengths uniform in [1024, 8192], 32 q /
              8 KV heads, d 128, bf16, 4 key outlier channels x8, INT8, bs 16
  llama3_70b  80 layers, 16 sequences x 32768 tokens, 64 q / 8 KV heads, d 128,
              bf16, FP8 E4M3, bs 16
  llama3_70b_int8  the same shape with INT8 per-token-per-head codes
  llama3_70b_bf16  the same shape with the 16-bit passthrough cache (the
              unquantized baseline the quantized codes are measured against)
  int4_long   80 layers, 1 sequence of 131072 tokens, INT4 with per-32 group
              scale and zero point, bs 32
  int4_batch  80 layers, 32 sequences, log-normal lengths (median 4096, cap
              65536), INT4 group-asymmetric, bs 32
  mixed       1 layer, 256 sequences, log-normal lengths (median 2048, cap
              32768), INT8 per-channel-per-block keys, INT8 per-token values,
              8 new tokens per sequence per step

Random recipe: K, V and q are N(0, 1) drawn in fp32 with torch generators
seeded per (seed, role, layer) and rounded to the source dtype; the chosen
outlier channels of K (drawn once per run without replacement) are multiplied
by the outlier factor before rounding. Lengths and block-pool permutations
come from numpy's default_rng([seed, role]). Log-normal lengths are
clamp(round(median * exp(sigma * z)), 1, cap) with sigma = 1.
"""
from dataclasses import dataclass, field, replace

import numpy as np
import torch

ROLE_LENGTHS, ROLE_OUTLIERS, ROLE_K, ROLE_V, ROLE_Q, ROLE_POOL = range(6)


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    src_dtype: str                 # "float16" | "bfloat16"
    k_code: str                    # "int8" | "fp8" | "int4" | "none16"
    v_code: str
    k_mode: str                    # "token_sym" | "group_asym" | "channel_block"
    v_mode: str
    group_size: int = 0
    lengths: tuple = ("fixed", 256)
    n_outliers: int = 0
    outlier_factor: float = 1.0
    new_tokens: int = 1            # tokens appended per sequence per step
    extra: dict = field(default_factory=dict)

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def torch_dtype(self):
        return getattr(torch, self.src_dtype)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 4, 2, 64, 16, "float16", "int8", "int8",
                     "token_sym", "token_sym", lengths=("fixed", 256),
                     n_outliers=2, outlier_factor=10.0),
    "llama3_8b": Workload("llama3_8b", 1, 64, 32, 8, 128, 16, "bfloat16", "int8",
                          "int8", "token_sym", "token_sym",
                          lengths=("uniform", 1024, 8192), n_outliers=4,
                          outlier_factor=8.0),
    "llama3_70b": Workload("llama3_70b", 80, 16, 64, 8, 128, 16, "bfloat16", "fp8",
                           "fp8", "token_sym", "token_sym",
                           lengths=("fixed", 32768), n_outliers=4,
                           outlier_factor=8.0),
    "llama3_70b_int8": Workload("llama3_70b_int8", 80, 16, 64, 8, 128, 16, "bfloat16", "int8",
                                "int8", "token_sym", "token_sym",
                                lengths=("fixed", 32768), n_outliers=4,
                                outlier_factor=8.0),
    "llama3_70b_bf16": Workload("llama3_70b_bf16", 80, 16, 64, 8, 128, 16, "bfloat16",
                                "none16", "none16", "token_sym", "token_sym",
                                lengths=("fixed", 32768), n_outliers=4,
                                outlier_factor=8.0),
    "int4_long": Workload("int4_long", 80, 1, 64, 8, 128, 32, "bfloat16", "int4",
                          "int4", "group_asym", "group_asym", group_size=32,
                          lengths=("fixed", 131072), n_outliers=4,
                          outlier_factor=8.0),
    "int4_batch": Workload("int4_batch", 80, 32, 64, 8, 128, 32, "bfloat16", "int4",
                           "int4", "group_asym", "group_asym", group_size=32,
                           lengths=("lognormal", 4096, 65536, 1.0), n_outliers=4,
                           outlier_factor=8.0),
    "mixed": Workload("mixed", 1, 256, 32, 8, 128, 16, "bfloat16", "int8", "int8",
                      "channel_block", "token_sym",
                      lengths=("lognormal", 2048, 32768, 1.0), n_outliers=4,
                      outlier_factor=8.0, new_tokens=8),
}


def get(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def lengths(w: Workload, seed: int = 0) -> np.ndarray:
    """Context length of every sequence (int32 [batch])."""
    kind = w.lengths[0]
    if kind == "fixed":
        return np.full(w.batch, w.lengths[1], np.int32)
    rng = np.random.default_rng([seed, ROLE_LENGTHS])
    if kind == "uniform":
        lo, hi = w.lengths[1], w.lengths[2]
        return rng.integers(lo, hi + 1, size=w.batch).astype(np.int32)
    if kind == "lognormal":
        median, cap, sigma = w.lengths[1], w.lengths[2], w.lengths[3]
        z = rng.standard_normal(w.batch)
        L = np.rint(median * np.exp(sigma * z))
        return np.clip(L, 1, cap).astype(np.int32)
    raise ValueError(kind)


def outlier_channels(w: Workload, seed: int = 0) -> np.ndarray:
    if w.n_outliers == 0:
        return np.zeros(0, np.int64)
    rng = np.random.default_rng([seed, ROLE_OUTLIERS])
    return np.sort(rng.choice(w.head_dim, size=w.n_outliers, replace=False))


def _gen(device, seed, role, layer, chunk=0):
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1000 + role) * 1000 + layer) * 100003 + chunk)
    return g


def kv_rows(w: Workload, num_tokens: int, layer: int = 0, seed: int = 0,
            device="cpu", chunk: int = 0):
    """New K and V rows [num_tokens][H][d] in the source dtype.

    `chunk` selects an independent draw, so that a long stream of tokens can be
    made in pieces."""
    shape = (num_tokens, w.num_kv_heads, w.head_dim)
    k = torch.randn(shape, generator=_gen(device, seed, ROLE_K, layer, chunk),
                    device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=_gen(device, seed, ROLE_V, layer, chunk),
                    device=device, dtype=torch.float32)
    oc = outlier_channels(w, seed)
    if len(oc):
        k[..., torch.as_tensor(oc, device=device)] *= w.outlier_factor
    return k.to(w.torch_dtype), v.to(w.torch_dtype)


def queries(w: Workload, seed: int = 0, device="cpu", step: int = 0,
            layer: int = 0):
    """Decode queries [batch][Hq][d] in the source dtype."""
    g = _gen(device, seed, ROLE_Q, layer, step)
    q = torch.randn((w.batch, w.num_q_heads, w.head_dim), generator=g,
                    device=device, dtype=torch.float32)
    return q.to(w.torch_dtype)


def query_rows(w: Workload, num_rows: int, seed: int = 0, device="cpu", step: int = 0,
               layer: int = 0):
    """Multi-query rows [num_rows][Hq][d] in the source dtype (a draw of its
    own, independent of the decode queries)."""
    g = _gen(device, seed, ROLE_Q, layer, 50000 + step)
    q = torch.randn((num_rows, w.num_q_heads, w.head_dim), generator=g,
                    device=device, dtype=torch.float32)
    return q.to(w.torch_dtype)


def pool_order(num_blocks: int, seed: int = 0, permuted: bool = True) -> np.ndarray:
    """Initial free-stack order: a seeded permutation (a fragmented pool) or
    the identity."""
    if not permuted:
        return np.arange(num_blocks, dtype=np.int32)
    rng = np.random.default_rng([seed, ROLE_POOL])
    return rng.permutation(num_blocks).astype(np.int32)


def pool_blocks(lens: np.ndarray, block_size: int, headroom_tokens: int = 0) -> int:
    """Pool size for a batch: every sequence's blocks at its length plus
    `headroom_tokens` more tokens (upper bound, for sizing buffers)."""
    L = lens.astype(np.int64) + headroom_tokens
    return int(((L + block_size - 1) // block_size).sum())
