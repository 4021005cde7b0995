"""Pins of the oracle's static-scale quantizers and append (a fixed, caller-given
scale and zero point in place of the ones taken from each vector's or block's
range):
hand-worked values, saturation, the reduction to the dynamic quantizers when
the given scale is the one they would compute, round-trip bounds, and brute
force over a small cache. No GPU."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from _util import OracleSeqs, bits, oracle_layout

rng = np.random.default_rng(4321)


def f32(x):
    return np.asarray(x, np.float32)


def test_sym_static_hand_worked_ties_and_saturation():
    # s = 0.25: x / s = 1.2, -2.96, 8, 2.5, -1.5, 40, -1000 (all exact in fp32
    # except the first two); ties go to even, then the code range clips.
    x = f32([0.3, -0.74, 2.0, 0.625, -0.375, 10.0, -250.0])
    assert ref.quant_sym_static(x, 127, 0.25).tolist() == [1, -3, 8, 2, -2, 40, -127]
    assert ref.quant_sym_static(x, 7, 0.25).tolist() == [1, -3, 7, 2, -2, 7, -7]
    # exactly at the edge: 127.5 s rounds to 128 (even), clipped to 127
    assert ref.quant_sym_static(f32([127.5, -127.5, 126.5]), 127, 1.0).tolist() == [127, -127, 126]
    assert ref.quant_sym_static(f32([7.5, 6.5, -7.49]), 7, 1.0).tolist() == [7, 6, -7]


def test_fp8_static_hand_worked_and_saturation():
    # s = 2: x / s = 448 (max finite), 1e4 (saturates), -0.5, 0, 1.125 (a
    # grid point: exponent 0, mantissa 1/8), -3e38 / 2 (saturates).
    x = f32([896.0, 2e4, -1.0, 0.0, 2.25, -3e38])
    q = ref.quant_fp8_static(x, 2.0)
    assert [ref.e4m3_value(c) for c in q.tolist()] == [448.0, 448.0, -0.5, 0.0, 1.125, -448.0]
    assert q[1] == 0x7E and q[5] == 0xFE


def test_asym4_static_hand_worked():
    # s = 0.5, z = 3: codes rne(x / s) + 3 in [0, 15].
    x = f32([-1.5, 0.0, 1.75, 50.0, -50.0, 0.25, 6.0])
    # x / s = -3, 0, 3.5 -> 4, 100 -> 15, -100 -> -15, 0.5 -> 0, 12
    assert ref.quant_asym4_static(x, 0.5, 3).tolist() == [0, 3, 7, 15, 0, 3, 15]
    assert ref.quant_asym4_static(x, 0.5, 0).tolist() == [0, 0, 4, 15, 0, 0, 12]
    assert ref.quant_asym4_static(x, 0.5, 15).tolist() == [12, 15, 15, 15, 0, 15, 15]
    # quotients beyond the int32 range still saturate on the right side
    big = f32([3e9, -3e9, 1e38, -1e38])
    assert ref.quant_asym4_static(big, 1.0, 3).tolist() == [15, 0, 15, 0]
    assert ref.quant_sym_static(big, 127, 1.0).tolist() == [127, -127, 127, -127]


@pytest.mark.parametrize("qmax", [127, 7])
def test_sym_static_equals_dynamic_at_the_dynamic_scale(qmax):
    for _ in range(200):
        x = f32(rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 3))
        q, s = ref.quant_sym(x, qmax)
        assert (ref.quant_sym_static(x, qmax, float(s)) == q).all()


def test_fp8_and_asym4_static_equal_dynamic_at_the_dynamic_parameters():
    for _ in range(200):
        x = f32(rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 3))
        q, s = ref.quant_fp8(x)
        assert (ref.quant_fp8_static(x, float(s)) == q).all()
        g = f32(rng.standard_normal(32) * 10.0 ** rng.uniform(-3, 3) + rng.choice([0.0, 2.0, -2.0]))
        q, s, z = ref.quant_asym4(g)
        assert (ref.quant_asym4_static(g, float(s), int(z)) == q).all()


@pytest.mark.parametrize("qmax", [127, 7])
def test_sym_static_bound_inside_and_clip_outside(qmax):
    for _ in range(200):
        s = float(np.float32(10.0 ** rng.uniform(-3, 1)))
        x = f32(rng.standard_normal(128) * s * qmax * rng.uniform(0.2, 2.0))
        q = ref.quant_sym_static(x, qmax, s).astype(np.float64)
        inside = np.abs(x) <= (qmax + 0.5) * s * (1 - 2.0 ** -20)
        err = np.abs(x.astype(np.float64) - q * s)
        assert err[inside].max(initial=0) <= s * (0.5 + 2.0 ** -16)
        assert (q[~inside] == np.sign(x[~inside]) * qmax).all()


def test_fp8_static_matches_torch_cast_in_range():
    # Within the format's range the code is the e4m3 cast of x / s (round to
    # nearest even); beyond it the code is +-448.
    for _ in range(50):
        s = float(np.float32(10.0 ** rng.uniform(-3, 1)))
        x = f32(rng.standard_normal(256) * s * 10.0 ** rng.uniform(0, 3))
        y = f32(x / np.float32(s))
        q = ref.quant_fp8_static(x, s)
        vals = np.array([ref.e4m3_value(c) for c in q.tolist()])
        inside = np.abs(y) < 464.0          # halfway to the next binade step rounds down
        want = torch.from_numpy(y[inside]).to(torch.float8_e4m3fn).float().numpy()
        assert (vals[inside] == want).all()
        assert (vals[~inside] == np.sign(y[~inside]) * 448.0).all()


def test_fp8_static_quotient_near_every_midpoint():
    # x placed at, and one float32 step either side of, m * s for every
    # midpoint m between two positive E4M3 values, under scales that are not
    # powers of two: the code is the cast of the correctly rounded quotient
    # x / s, which near a midpoint decides the code (a product with 1 / s can
    # land on the other side of it).
    vals = np.array([ref.e4m3_value(c) for c in range(0x7F)], np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0
    for s in (0.3, 1.0 / 3.0, 0.7, 3.1, 0.05, 17.0):
        s = float(np.float32(s))
        base = f32(mids * s)
        x = np.concatenate([np.nextafter(base, f32(-np.inf)), base, np.nextafter(base, f32(np.inf))])
        x = np.concatenate([x, -x]).astype(np.float32)
        y = f32(x / np.float32(s))
        q = ref.quant_fp8_static(x, s)
        got = np.array([ref.e4m3_value(c) for c in q.tolist()])
        want = torch.from_numpy(y).to(torch.float8_e4m3fn).float().numpy()
        assert (got == want).all(), s


def test_asym4_static_bound_inside_and_clip_outside():
    for _ in range(300):
        s = float(np.float32(10.0 ** rng.uniform(-3, 1)))
        z = int(rng.integers(0, 16))
        x = f32(rng.uniform(-20, 20, 32) * s)
        q = ref.quant_asym4_static(x, s, z).astype(np.float64)
        lo, hi = (-z - 0.5) * s, (15 - z + 0.5) * s
        inside = (x >= lo * (1 - 2.0 ** -20)) & (x <= hi * (1 - 2.0 ** -20))
        xh = (q - z) * s
        assert np.abs(x - xh)[inside].max(initial=0) <= s * (0.5 + 2.0 ** -16)
        assert (q[~inside & (x > 0)] == 15).all() and (q[~inside & (x < 0)] == 0).all()


def _static_params(L, H, d, mode, seed):
    g = np.random.default_rng(seed)
    if mode == ref.GROUP_ASYM:
        ng = d // L.group_size
        return (f32(10.0 ** g.uniform(-1.5, -0.5, (H, ng))),
                g.integers(0, 16, (H, ng)).astype(np.uint8))
    return f32(10.0 ** g.uniform(-2.5, -1.0, H)), None


@pytest.mark.parametrize("code,mode", [("int8", "token_sym"), ("fp8", "token_sym"),
                                       ("int4", "token_sym"), ("int4", "group_asym")])
def test_append_static_places_codes_and_static_metadata(code, mode):
    # Brute force over a small paged cache: every appended (token, head) row
    # holds the static codes of its input, and its metadata the given values.
    w = workloads.get("tiny", k_code=code, v_code=code, k_mode=mode, v_mode=mode,
                      group_size=32 if mode == "group_asym" else 0,
                      src_dtype="bfloat16", head_dim=64, block_size=16,
                      num_kv_heads=2, num_q_heads=8, batch=2)
    L = oracle_layout(w)
    H, d = 2, 64
    lens = np.array([21, 16], np.int32)
    k, v = workloads.kv_rows(w, int(lens.sum()), seed=3)
    ks, kz = _static_params(L, H, d, L.k_mode, 1)
    vs, vz = _static_params(L, H, d, L.v_mode, 2)
    s = OracleSeqs(L, 10, 2, 4, order=rng.permutation(10).astype(np.int32))
    slots, _ = s.grow(lens)
    ref.append_static(L, s.cache, bits(k).reshape(len(slots), -1),
                      bits(v).reshape(len(slots), -1), slots, ks, vs, kz, vz)
    for side, x, sc, zp in ((0, k, ks, kz), (1, v, vs, vz)):
        for t, slot in enumerate(slots):
            b = 0 if t < 21 else 1
            pos = t if b == 0 else t - 21
            for h in range(H):
                row = x[t, h].float().numpy()
                got = ref.dequant_token(L, s.cache, side, s.tables[b], lens[b], b, pos, h)
                if mode == "group_asym":
                    want = np.concatenate([
                        (ref.quant_asym4_static(row[g * 32:(g + 1) * 32], float(sc[h, g]),
                                                int(zp[h, g])).astype(np.float32)
                         - np.float32(zp[h, g])) * sc[h, g] for g in range(2)])
                elif code == "fp8":
                    want = f32([ref.e4m3_value(c) for c in ref.quant_fp8_static(row, float(sc[h]))]) * sc[h]
                else:
                    qm = 127 if code == "int8" else 7
                    want = ref.quant_sym_static(row, qm, float(sc[h])).astype(np.float32) * sc[h]
                assert (got == want).all(), (side, t, h)
    # metadata planes hold the static values
    scale = s.cache.scale(0)
    if mode == "group_asym":
        scale = scale.reshape(10, H, 16, 2)
        zero = s.cache.planes["k_zero"].reshape(10, H, 16, 2)
        for t, slot in enumerate(slots):
            assert (scale[slot // 16, :, slot % 16] == ks).all()
            assert (zero[slot // 16, :, slot % 16] == kz).all()
    else:
        scale = scale.reshape(10, H, 16)
        for slot in slots:
            assert (scale[slot // 16, :, slot % 16] == ks).all()


def test_append_static_channel_keys_equal_dynamic_at_the_block_scales():
    # One full block per sequence: static per-channel scales equal to the
    # block's own dynamic scales give the dynamic codes and scale row; the
    # stage row holds the raw rows either way.
    w = workloads.get("mixed", batch=2)
    L = oracle_layout(w)
    H, d, bs = w.num_kv_heads, w.head_dim, w.block_size
    k, v = workloads.kv_rows(w, 2 * bs, seed=8)
    dyn = OracleSeqs(L, 6, 2, 2, order=np.arange(6, dtype=np.int32), max_seqs=2)
    dyn.append(k, v, [bs, bs])
    blocks = dyn.tables[:, 0]
    sc = dyn.cache.scale(0).reshape(6, H, d)
    for b in range(2):
        st = OracleSeqs(L, 6, 2, 2, order=np.arange(6, dtype=np.int32), max_seqs=2)
        slots, rows = st.grow([bs, bs])
        ref.append_static(L, st.cache, bits(k).reshape(2 * bs, -1), bits(v).reshape(2 * bs, -1),
                          slots, np.ascontiguousarray(sc[blocks[b]]),
                          f32(np.full(H, 0.05)), stage_rows=rows)
        kc_d = dyn.cache.planes["k_codes"].reshape(6, H, bs, d)
        kc_s = st.cache.planes["k_codes"].reshape(6, H, bs, d)
        assert (kc_s[blocks[b]] == kc_d[blocks[b]]).all()
        assert (st.cache.scale(0).reshape(6, H, d)[blocks[b]] == sc[blocks[b]]).all()
        assert (st.cache.planes["k_stage"] == dyn.cache.planes["k_stage"]).all()


def test_append_static_channel_keys_brute_force_and_tail():
    # Every key element is rne(x / s_c) clipped to [-127, 127]; a block's scale
    # row is the given one from its first slot on; the partial tail reads back
    # raw from the stage row.
    w = workloads.get("mixed", batch=2)
    L = oracle_layout(w)
    H, d, bs = w.num_kv_heads, w.head_dim, w.block_size
    lens = np.array([21, 9], np.int32)
    k, v = workloads.kv_rows(w, 30, seed=2)
    ks = f32(10.0 ** rng.uniform(-2.5, -1.0, (H, d)))
    s = OracleSeqs(L, 6, 2, 2, order=rng.permutation(6).astype(np.int32), max_seqs=2)
    slots, rows = s.grow(lens)
    ref.append_static(L, s.cache, bits(k).reshape(30, -1), bits(v).reshape(30, -1), slots,
                      ks, f32(np.full(H, 0.05)), stage_rows=rows)
    codes = s.cache.planes["k_codes"].view(np.int8).reshape(6, H, bs, d)
    for t, slot in enumerate(slots):
        for h in range(H):
            want = [ref.quant_sym_static(f32([xe]), 127, float(se))[0]
                    for xe, se in zip(k[t, h].float().numpy(), ks[h])]
            assert (codes[slot // bs, h, slot % bs] == want).all()
    scale = s.cache.scale(0).reshape(6, H, d)
    for b in range(2):
        for j in range((lens[b] + bs - 1) // bs):
            assert (scale[s.tables[b, j]] == ks).all()
    # sequence 0: positions 16..20 are the partial tail, read raw
    for pos in (16, 20):
        got = ref.dequant_token(L, s.cache, 0, s.tables[0], 21, 0, pos, 1)
        assert (got == k[pos, 1].float().numpy()).all()
    got = ref.dequant_token(L, s.cache, 0, s.tables[0], 21, 0, 3, 1)
    assert (got == codes[slots[3] // bs, 1, slots[3] % bs].astype(np.float32) * ks[1]).all()


def test_append_static_passthrough_side_and_rejections():
    # INT8 keys with static scales next to 16-bit values: the value rows are
    # stored as given. Per-channel keys need their stage rows.
    w = workloads.get("tiny", k_code="int8", v_code="none16", src_dtype="float16",
                      head_dim=64, block_size=16, num_kv_heads=2, num_q_heads=2, batch=1)
    L = oracle_layout(w)
    k, v = workloads.kv_rows(w, 5, seed=0)
    s = OracleSeqs(L, 2, 1, 2, order=np.arange(2, dtype=np.int32))
    slots, _ = s.grow([5])
    ref.append_static(L, s.cache, bits(k).reshape(5, -1), bits(v).reshape(5, -1), slots,
                      f32([0.05, 0.02]), None)
    vcodes = s.cache.planes["v_codes"].view(np.uint16).reshape(2, 2, 16, 64)
    for t, slot in enumerate(slots):
        assert (vcodes[slot // 16, :, slot % 16] == bits(v[t])).all()
    wc = workloads.get("mixed")
    Lc = oracle_layout(wc)
    sc = OracleSeqs(Lc, 4, 1, 4)
    slots, _ = sc.grow([3])
    kc, vc = workloads.kv_rows(wc, 3, seed=0)
    with pytest.raises(ValueError):
        ref.append_static(Lc, sc.cache, bits(kc).reshape(3, -1), bits(vc).reshape(3, -1),
                          slots, f32(np.ones((wc.num_kv_heads, wc.head_dim))),
                          f32(np.ones(wc.num_kv_heads)))
