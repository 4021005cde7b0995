"""Quantize-on-append codes at their rounding boundaries, GPU against the
oracle byte for byte.

"Dynamic KV Cache Quantization for Fast LLM Inference", section
"Understanding Dynamic Quantization Techniques for KV Caches": a code is the
value over the scale, rounded. The kernels form the binary32 quotient y =
x / s from a reciprocal, redo it with a true division when y is near a
rounding boundary, and round y to the code (the hardware converter for
E4M3). These tests put y exactly on every binary32 value within 64 ulps of
each boundary:
  * E4M3: every midpoint between neighbouring codes (normal and subnormal)
    and every binade edge;
  * INT8: every half-integer n + 1/2, n < 127;
with caller-given scales (kvq_append_static: the quotient is chosen exactly),
and again with scales computed from each row's own maximum (kvq_append), on
rows whose quotients fall within 64 ulps of a boundary. Expected codes come
from the oracle only."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import bits, oracle_layout
from _gpu_util import DEV, gpu_cache, kq, lib_layout, need_gpu, planes_equal

pytestmark = pytest.mark.gpu

F32 = np.float32
ULPS = np.arange(-64, 65)


def _ulp_window(centres):
    """Every binary32 value within 64 ulps of each centre (positive)."""
    c = np.asarray(centres, F32).view(np.uint32).astype(np.int64)
    return (c[:, None] + ULPS[None, :]).astype(np.uint32).view(F32).ravel()


def _e4m3_boundaries():
    """Positive E4M3 rounding boundaries: midpoints between neighbouring codes
    in the binade [1, 2) (the others are these times 2^k), the subnormal
    midpoints (k + 1/2) 2^-9, and the binade edge 1."""
    mant = [(8 + i + 0.5) / 8 for i in range(8)]          # 1.0625 .. 1.9375
    sub = [(k + 0.5) * 2.0 ** -9 for k in range(8)]        # below 2^-6
    return np.array(mant, F32), np.array(sub, F32), np.array([1.0], F32)


def _pairs_for(targets, xs=tuple(1.0 + k / 64.0 for k in range(64))):
    """For every target quotient y find an fp16-exact x and a binary32 s with
    fl32(x / s) == y exactly (searching s around x / y). Returns x, s."""
    y = np.asarray(targets, F32)
    X = np.zeros_like(y)
    S = np.zeros_like(y)
    todo = np.ones(len(y), bool)
    for x in xs:
        x32 = F32(x)
        s0 = x32 / y
        for d in (0, 1, -1, 2, -2, 3, -3, 4, -4):
            s = (s0.view(np.uint32).astype(np.int64) + d).astype(np.uint32).view(F32)
            ok = todo & (x32 / s == y)
            X[ok], S[ok] = x32, s[ok]
            todo &= ~ok
    assert not todo.any(), f"{todo.sum()} quotients not reached"
    return X, S


def _static_rows(X, S, exps, d):
    """One (head) row per pair: x 2^k for every k in exps (quotients y 2^k,
    exact) and their negatives, zeros after."""
    n = len(X)
    rows = np.zeros((n, d), F32)
    vals = np.concatenate([np.outer(X, 2.0 ** np.asarray(exps, np.float64)),
                           -np.outer(X, 2.0 ** np.asarray(exps, np.float64))], axis=1)
    assert vals.shape[1] <= d
    rows[:, :vals.shape[1]] = vals
    return rows, S


def _run_static(code, rows, scales, d=64, heads=4096):
    """rows[i] with static scale scales[i], packed as heads of one token per
    launch (keys and values sides both used); every plane compared."""
    n = len(rows)
    done = 0
    while done < n:
        H = min(heads, (n - done + 1) // 2) or 1
        kr, ks = rows[done:done + H], scales[done:done + H]
        vr, vs = rows[done + H:done + 2 * H], scales[done + H:done + 2 * H]
        if len(vr) < H:   # pad the value side with a copy of the key side
            vr = np.concatenate([vr, kr[len(vr):]])
            vs = np.concatenate([vs, ks[len(vs):]])
        w = workloads.get("tiny", k_code=code, v_code=code, k_mode="token_sym",
                          v_mode="token_sym", src_dtype="float16", head_dim=d,
                          block_size=16, num_kv_heads=H, num_q_heads=H, batch=1)
        L, LL = oracle_layout(w), lib_layout(w)
        k = torch.from_numpy(kr.reshape(1, H, d)).to(torch.float16)
        v = torch.from_numpy(vr.reshape(1, H, d)).to(torch.float16)
        assert (k.float().numpy().reshape(H, d) == kr).all()   # the inputs are fp16-exact
        slots = np.array([3], np.int64)
        hc = ref.HostCache(L, 1, fill=0)
        ks32, vs32 = np.ascontiguousarray(ks, F32), np.ascontiguousarray(vs, F32)
        ref.append_static(L, hc, bits(k).reshape(1, -1), bits(v).reshape(1, -1), slots,
                          ks32, vs32, None, None)
        gc = gpu_cache(LL, 1, fill=0)
        kq.kvq_append_static(LL, gc, k.to(DEV), v.to(DEV), torch.from_numpy(slots).to(DEV),
                             torch.from_numpy(ks32).to(DEV), torch.from_numpy(vs32).to(DEV))
        torch.cuda.synchronize()
        assert planes_equal(gc, hc) == [], f"{code}: rows {done}..{done + 2 * H}"
        done += 2 * H


def test_e4m3_static_quotients_at_every_boundary_offset():
    need_gpu()
    mant, sub, edge = _e4m3_boundaries()
    # normal midpoints and the edge, scaled into every normal binade 2^-6 .. 2^8
    tn = _ulp_window(np.concatenate([mant, edge]))
    X, S = _pairs_for(tn)
    rows_n, s_n = _static_rows(X, S, range(-6, 9), 64)
    # subnormal midpoints: absolute spacing, no scaling
    ts = _ulp_window(sub)
    X2, S2 = _pairs_for(ts)
    rows_s, s_s = _static_rows(X2, S2, [0], 64)
    rows = np.concatenate([rows_n, rows_s])
    scales = np.concatenate([s_n, s_s])
    print(f"E4M3 static: {len(rows)} rows, {2 * (len(tn) * 15 + len(ts))} boundary quotients")
    _run_static("fp8", rows, scales)


def test_int8_static_quotients_at_every_half_integer_offset():
    need_gpu()
    t = _ulp_window(np.arange(127, dtype=np.float64) + 0.5)
    X, S = _pairs_for(t)
    rows, s = _static_rows(X, S, [0], 64)
    print(f"INT8 static: {len(rows)} rows, {2 * len(t)} boundary quotients")
    _run_static("int8", rows, s)


def _dynamic_pairs(qmax, near, n_amax=3000, seed=0):
    """Rows for the dynamic path: for fp16 row maxima A (scale s = fl32(A /
    qmax)), every fp16 x below A whose quotient fl32(x / s) lies within 64
    ulps of a rounding boundary (`near` decides). Rows are [A, x...], zeros
    after, 64 wide."""
    g = np.random.default_rng(seed)
    allv = np.arange(0, 1 << 16, dtype=np.uint16).view(np.float16).astype(F32)
    allv = allv[np.isfinite(allv) & (allv > 0)]
    A = np.sort(g.choice(allv[allv >= 2.0 ** -8], n_amax, replace=False))
    rows = []
    for a in A:
        s = F32(a) / F32(qmax)
        xs = allv[allv < a]
        y = xs / s
        sel = xs[near(y)]
        for c0 in range(0, len(sel), 31):
            part = sel[c0:c0 + 31]
            r = np.zeros(64, F32)
            r[0] = a
            r[1:1 + len(part)] = part
            r[32:32 + len(part)] = -part
            rows.append(r)
    return np.array(rows, F32)


def _near_e4m3(y):
    u = y.view(np.uint32) & 0xFFFFF
    return (np.abs(u.astype(np.int64) - 0x80000) <= 64) | (np.abs(u.astype(np.int64)) <= 64) | \
        (np.abs(u.astype(np.int64) - 0x100000) <= 64)


def _near_int8(y):
    f = y - np.floor(y)
    ulp = np.spacing(y)
    return np.abs(f - 0.5) <= 64 * ulp


@pytest.mark.parametrize("code", ["fp8", "int8"])
def test_dynamic_scales_quotients_near_boundaries(code):
    """Scales from each row's own maximum (non-unit, from about 3000 fp16
    maxima): every fp16 element whose quotient lands within 64 ulps of a
    rounding boundary."""
    need_gpu()
    qmax = 448.0 if code == "fp8" else 127.0
    rows = _dynamic_pairs(qmax, _near_e4m3 if code == "fp8" else _near_int8)
    H, d = 8, 64
    T = (len(rows) + H - 1) // H
    pad = np.zeros((T * H - len(rows), d), F32)
    rows = np.concatenate([rows, pad]).reshape(T, H, d)
    print(f"{code} dynamic: {len(rows.reshape(-1, d))} rows")
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode="token_sym",
                      v_mode="token_sym", src_dtype="float16", head_dim=d, block_size=16,
                      num_kv_heads=H, num_q_heads=H, batch=1)
    L, LL = oracle_layout(w), lib_layout(w)
    k = torch.from_numpy(rows).to(torch.float16)
    v = -k.flip(0)
    nb = (T + 15) // 16
    slots = np.arange(T, dtype=np.int64)
    hc = ref.HostCache(L, nb, fill=0)
    ref.append(L, hc, bits(k).reshape(T, -1), bits(v).reshape(T, -1), slots)
    gc = gpu_cache(LL, nb, fill=0)
    kq.kvq_append(LL, gc, k.to(DEV), v.to(DEV), torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert planes_equal(gc, hc) == []
