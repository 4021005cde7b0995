"""The decode's split plan is made on the device from the context lengths; the
grid and the workspace are sized on the host from batch and max_context_len
alone. This checks, for many length mixes, that the plan's item count (its
rule replayed here from the planning constants in the library's internal
header) never exceeds the bound the host sizes the workspace for (read back
from kvq_decode_workspace_bytes), so that no split is left out and no partial
lands outside the workspace. Host-only; no GPU."""
import math
import re
from pathlib import Path

import numpy as np
import pytest
import torch

ROOT = Path(__file__).resolve().parents[1]
kq = pytest.importorskip("quantized_paged_kv_append_amd")


def _constants():
    text = (ROOT / "quantized_paged_kv_append_amd" / "csrc" / "kvq_internal.h").read_text()
    names = ("kDecodeWaves", "kDecodeMaxWaveBlocks", "kDecodeTargetWavesLog2",
             "kDecodeUniformWavesLog2", "kDecodeMinWaveTokens", "kDecodeSkewWaveBlocks",
             "kDecodeSkewWaveBlocksChannel")
    out = {}
    for n in names:
        m = re.search(rf"constexpr int {n} = (\d+);", text)
        assert m, n
        out[n] = int(m.group(1))
    return out


def _plan_items(lens, max_len, bs, H, c):
    """Items of the device plan (the rule the split kernel and the reduce
    derive from the lengths): every non-empty or empty sequence's splits."""
    n = (np.minimum(np.maximum(lens, 0), max_len) + bs - 1) // bs
    tot = int(n.sum())
    nonzero = n[n > 0]
    uniform = len(nonzero) > 0 and int(n.max()) * 8 <= int(nonzero.min()) * 9
    lg = c["kDecodeUniformWavesLog2"] if uniform else c["kDecodeTargetWavesLog2"]
    cap = c["kDecodeMaxWaveBlocks"] if uniform else min(c["kDecodeSkewWaveBlocks"],
                                                        c["kDecodeSkewWaveBlocksChannel"])
    wmin = math.ceil(c["kDecodeMinWaveTokens"] / bs)
    w = min(max(math.ceil(tot * H / 2 ** lg), wmin), cap)
    S = c["kDecodeWaves"] * w
    return int(((n + S - 1) // S).sum())


def _host_bound(L, batch, Hq, max_len, d):
    """Items the workspace holds: kvq_decode_workspace_bytes is
    round_up(items d 4, 256) + round_up(items 2 4, 256) for items = bound Hq."""
    total = kq.kvq_decode_workspace_bytes(L, batch, Hq, max_len)
    lo, hi = 0, 1 << 40
    while lo < hi:   # largest bound whose workspace fits in `total`
        mid = (lo + hi + 1) // 2
        items = mid * Hq
        need = -(-items * d * 4 // 256) * 256 + -(-items * 8 // 256) * 256
        if need <= total:
            lo = mid
        else:
            hi = mid - 1
    return lo


@pytest.mark.parametrize("H,Hq,d,bs", [(8, 64, 128, 16), (8, 32, 128, 32), (2, 4, 64, 16),
                                       (1, 8, 128, 16)])
def test_plan_items_never_exceed_the_host_bound(H, Hq, d, bs):
    c = _constants()
    L = kq.make_layout(H, d, bs, "int8", src_dtype=torch.bfloat16)
    rng = np.random.default_rng(H * 1000 + bs)
    cases = []
    for batch in (1, 2, 3, 16, 64, 255, 256, 257, 1000, 3000):
        for max_len in (1, 15, 16, 17, 1000, 32768, 131072):
            cases.append((batch, max_len, np.full(batch, max_len)))          # equal
            cases.append((batch, max_len, rng.integers(0, max_len + 1, batch)))
            skew = np.zeros(batch, np.int64)
            skew[0] = max_len                                               # one long
            cases.append((batch, max_len, skew))
            ln = np.minimum(np.round(max(max_len // 16, 1) * np.exp(rng.normal(0, 1, batch))),
                            max_len)
            cases.append((batch, max_len, ln.astype(np.int64)))             # log-normal
    for batch, max_len, lens in cases:
        if batch * ((max_len + bs - 1) // bs) > 2 ** 31 - 1:
            continue
        items = _plan_items(lens.astype(np.int64), max_len, bs, H, c)
        bound = _host_bound(L, batch, Hq, max_len, d)
        assert items <= bound, (batch, max_len, items, bound)


def test_prefill_partial_index_stays_in_the_workspace():
    """Multi-query attention: split j of sequence b writes column c's partial
    at ((b J + j) H + g) CT16 + c for c < nq_b G, with CT = ceil(max_query_len
    G / 16) and J from max_context_len; the kernels cut nq_b to
    min(query_start[b+1] - query_start[b], len_b, max_query_len). A sequence
    with more queries than max_query_len (a broken precondition) must not
    reach past the workspace. The rule is replayed here; the kernels' own
    expression is checked for the same cut."""
    src = (ROOT / "quantized_paged_kv_append_amd" / "csrc" / "kvq_prefill.hip").read_text()
    # both split kernels (register-streaming and LDS-staged) cut the count
    assert src.count("min(min(pa.qstart[b + 1] - q0, L), pa.max_q)") == 2
    assert src.count("min(min(a.qstart[b + 1] - q0, L), a.max_q)") == 1
    rng = np.random.default_rng(7)
    for H, Hq, d, bs, code, mode in ((8, 64, 128, 16, "int8", "token_sym"),
                                     (2, 4, 64, 32, "fp8", "token_sym"),
                                     (8, 32, 128, 16, "int8", "token_sym"),
                                     (8, 64, 128, 32, "int4", "group_asym"),
                                     (2, 16, 64, 16, "int8", "channel_block")):
        G = Hq // H
        staged = mode == "token_sym" and code in ("int8", "fp8")
        L = kq.make_layout(H, d, bs, code, k_mode=mode,
                           v_mode="token_sym" if mode == "channel_block" else mode,
                           group_size=32 if mode == "group_asym" else 0,
                           src_dtype=torch.bfloat16)
        for _ in range(200):
            B = int(rng.choice([rng.integers(1, 9), rng.integers(30, 40)]))
            max_q = int(rng.integers(1, 40))
            max_len = int(rng.choice([rng.integers(max_q, 3000), rng.integers(max_q, 40000)]))
            lens = rng.integers(0, max_len + 1, B)
            # query counts up to 3x the bound: the clamp must hold them
            nq_raw = rng.integers(0, 3 * max_q + 1, B)
            total = kq.kvq_prefill_workspace_bytes(L, B, Hq, max_q, max_len)
            maxblk = max(1, -(-max_len // bs))
            CT = -(-max_q * G // 16)
            if staged:   # 8-bit per-token codes: split length from the block visits
                units = 2048 if B >= 32 else 1024
                S = min(512, max(32, -(-B * H * -(-CT // 8) * maxblk // units) // 32 * 32))
                J0 = -(-maxblk // S)
                if J0 > 1 and maxblk - (J0 - 1) * S < S // 4:   # short last split spread
                    per_chunk = max(1, 64 // bs)
                    S2 = -(-(-(-maxblk // (J0 - 1))) // per_chunk) * per_chunk
                    if S2 <= 512:
                        S = S2
            else:
                S = min(64, max(32, -(-maxblk // 16)))
            J = -(-maxblk // S)
            partials = B * J * H * CT * 16
            need = -(-partials * d * 4 // 256) * 256 + -(-partials * 8 // 256) * 256
            assert need == total, (B, max_q, max_len, need, total)   # the rule replayed exactly
            worst = -1
            for b in range(B):
                nq = min(int(nq_raw[b]), int(lens[b]), max_q)
                nblk = -(-int(lens[b]) // bs)
                for j in range(J):
                    if j * S >= nblk or nq == 0:
                        continue
                    worst = max(worst, ((b * J + j) * H + (H - 1)) * CT * 16 + nq * G - 1)
            assert worst < partials, (B, max_q, max_len, worst, partials)


def test_prefill_short_last_split_is_spread():
    """A 32768-token context plus 8 new tokens is 2049 blocks of 16; the
    visit rule asks for 256-block splits, which would leave a one-block
    ninth split. It is spread: 8 splits of 260 blocks (whole 64-token
    chunks). A 512-token chunk on the same context keeps 5 splits (4 x 520
    would pass the 512-block bound)."""
    L = kq.make_layout(8, 128, 16, "fp8", src_dtype=torch.bfloat16)
    for B, max_q, J in ((16, 8, 8), (1, 512, 5)):
        max_len = 32768 + max_q
        CT = -(-max_q * 8 // 16)
        partials = B * J * 8 * CT * 16
        need = -(-partials * 128 * 4 // 256) * 256 + -(-partials * 8 // 256) * 256
        assert kq.kvq_prefill_workspace_bytes(L, B, 64, max_q, max_len) == need, (B, max_q)
