"""GPU-side helpers for the parity tests: device copies of oracle inputs and
the library calls the benchmark makes. Expected values always come from the
oracle, computed from the same seeded inputs."""
import numpy as np
import pytest
import torch

from oracle import ref

kq = pytest.importorskip("quantized_paged_kv_append_amd")
from quantized_paged_kv_append_amd import kvq as kqb  # noqa: E402

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
TORCH_DT = {"float16": torch.float16, "bfloat16": torch.bfloat16}


def need_gpu():
    if DEV is None:
        pytest.skip("no GPU")


def lib_layout(w):
    return kq.make_layout(w.num_kv_heads, w.head_dim, w.block_size, w.k_code, w.v_code,
                          w.k_mode, w.v_mode, w.group_size, TORCH_DT[w.src_dtype])


def gpu_cache(L, num_blocks, max_seqs=0, fill=0xA5):
    c = kq.PagedCache(L, num_blocks, max_seqs, device=DEV)
    for t in c.planes.values():
        if t is not None:
            t.fill_(fill)
    return c


def upload(host_cache, L):
    """Device copy of an oracle-built cache (decode is then tested on its
    own, independent of the GPU append)."""
    c = kq.PagedCache(L, host_cache.num_blocks, host_cache.max_seqs, device=DEV)
    for name, t in c.planes.items():
        if t is not None:
            t.copy_(torch.from_numpy(host_cache.planes[name]))
    return c


def planes_equal(gpu_cache_, host_cache, names=None):
    bad = []
    for name in names or kq.PagedCache.NAMES:
        g = gpu_cache_.planes[name]
        h = host_cache.planes[name]
        if g is None:
            assert h is None
            continue
        gn = g.cpu().numpy()
        if not np.array_equal(gn, h):
            idx = np.nonzero(gn != h)[0]
            bad.append((name, len(idx), int(idx[0]), int(gn[idx[0]]), int(h[idx[0]])))
    return bad


def decode_gpu(L, cache, q, tables, lens, max_len, out_dtype=torch.float32, sm_scale=0.0,
               split_blocks=0):
    B, Hq, d = q.shape
    ws = torch.empty(kq.kvq_decode_workspace_bytes(L, B, Hq, max_len, split_blocks),
                     dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, d), float("nan"), dtype=out_dtype, device=DEV)
    kq.kvq_decode_attention(L, cache, q, tables, lens, max_len, out, ws,
                            sm_scale=sm_scale, split_blocks=split_blocks)
    torch.cuda.synchronize()
    return out


def assert_decode_close(got, exp, what=""):
    """|gpu - oracle| <= 2e-3 + 1e-3 |oracle| elementwise (fp32 output); for a
    16-bit output the oracle is rounded to that dtype first and one unit in
    its last place is added to the bound."""
    g = got.double().cpu().numpy()
    if got.dtype == torch.float32:
        e = exp
        tol = 2e-3 + 1e-3 * np.abs(e)
    else:
        e = torch.from_numpy(exp).to(got.dtype).double().numpy()
        ulp = np.abs(e) * (2.0 ** -7 if got.dtype == torch.bfloat16 else 2.0 ** -10)
        tol = 2e-3 + 1e-3 * np.abs(e) + ulp
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - e)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert (err <= tol).all(), (f"{what}: max err {err.max():.3e} at {worst} "
                                f"got {g[worst]:.6f} exp {e[worst]:.6f}")
    return float(err.max())
