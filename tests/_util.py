"""Helpers for the tests: host copies of inputs and oracle-side cache set-up.

Inputs come from workloads.py (seeded, synthetic); expected values come from
the CPU oracle only.
"""
import numpy as np
import torch

from oracle import ref

CODE = {"none16": ref.CODE_NONE16, "int8": ref.CODE_INT8, "fp8": ref.CODE_FP8,
        "int4": ref.CODE_INT4}
MODE = {"token_sym": ref.TOKEN_SYM, "group_asym": ref.GROUP_ASYM,
        "channel_block": ref.CHANNEL_BLOCK}
DT = {"float16": ref.F16, "bfloat16": ref.BF16}


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a 16-bit float tensor (host copy)."""
    assert t.element_size() == 2
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dtype)


def oracle_layout(w):
    return ref.layout(w.num_kv_heads, w.head_dim, w.block_size, CODE[w.k_code],
                      CODE[w.v_code], MODE[w.k_mode], MODE[w.v_mode],
                      w.group_size, DT[w.src_dtype])


class OracleSeqs:
    """A batch of sequences in an oracle cache, placed through the oracle's
    block pool (tables and slots from orc_blocks_reserve)."""

    def __init__(self, L, num_blocks, batch, max_blocks, order=None,
                 max_seqs=None):
        self.L = L
        self.cache = ref.HostCache(L, num_blocks,
                                   max_seqs if max_seqs is not None else batch)
        self.stack, self.top = ref.pool_init(num_blocks, order)
        self.tables = np.full((batch, max_blocks), -1, np.int32)
        self.lens = np.zeros(batch, np.int32)

    def grow(self, new_tokens):
        """Reserve slots for new_tokens[b] more tokens of every sequence.
        Returns the slot mapping (batch order) and the stage rows."""
        new_tokens = np.asarray(new_tokens, np.int32)
        slots, st = ref.blocks_reserve(self.stack, self.top, self.tables,
                                       self.lens, new_tokens, self.L.block_size)
        assert st == 0, "oracle pool exhausted"
        rows = np.repeat(np.arange(len(new_tokens), dtype=np.int32), new_tokens)
        self.lens = self.lens + new_tokens
        return slots, rows

    def append(self, k, v, new_tokens):
        """k, v: torch [T][H][d] rows in batch order for new_tokens."""
        slots, rows = self.grow(new_tokens)
        ref.append(self.L, self.cache, bits(k).reshape(k.shape[0], -1),
                   bits(v).reshape(v.shape[0], -1), slots, rows)
        return slots, rows
