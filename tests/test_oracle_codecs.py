"""Pins of the oracle's codecs and closed forms against what the pages and
the mathematics fix (closed forms the pages print, format definitions, exact
special cases, invariants, library routines). No GPU."""
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

from oracle import ref

GOLD = Path(__file__).parent / "golden"
rng = np.random.default_rng(1234)


def f32(x):
    return np.asarray(x, np.float32)


# ---------------------------------------------------------------------------
# Closed forms printed on the pages.
# ---------------------------------------------------------------------------

def test_bytes_per_token_matches_printed_values():
    g = json.loads((GOLD / "bytes_per_token.json").read_text())
    H, d, layers = g["kv_heads"], g["head_dim"], g["layers"]
    for bits, code in (("16", ref.CODE_NONE16), ("8", ref.CODE_INT8),
                       ("8", ref.CODE_FP8), ("4", ref.CODE_INT4)):
        for src in (ref.F16, ref.BF16):
            L = ref.layout(H, d, 16, code, src_dtype=src)
            assert ref.bytes_per_token(L, layers) == g["bytes_per_token"][bits]


def test_cache_size_closed_forms():
    g = json.loads((GOLD / "cache_size.json").read_text())["facts"]
    one, many, ratio = g
    L16 = ref.layout(one["kv_heads"], one["head_dim"], 16, ref.CODE_NONE16)
    per_tok = ref.bytes_per_token(L16, one["layers"])
    assert per_tok * one["tokens"] == one["bytes"] == 40 * 2 ** 30
    assert many["requests"] * per_tok * one["tokens"] == many["bytes"]
    L8 = ref.layout(8, 128, 16, ref.CODE_INT8)
    L4 = ref.layout(8, 128, 16, ref.CODE_INT4)
    assert ref.bytes_per_token(L8, 80) / per_tok == ratio["ratio_int8"]
    assert ref.bytes_per_token(L4, 80) / per_tok == ratio["ratio_int4"]


def test_bytes_per_token_metadata_terms():
    # 80 layers x 8 KV heads x d 128. Per layer, per side: TOKEN_SYM adds one
    # fp32 per head (8*4 = 32 B); GROUP_ASYM g32 adds (4 groups)*(4+1) per
    # head (160 B); CHANNEL_BLOCK bs16 adds 8*128*4/16 = 256 B.
    L = ref.layout(8, 128, 16, ref.CODE_FP8)
    assert ref.bytes_per_token(L, 80, 1) == 163840 + 80 * 2 * 32
    L = ref.layout(8, 128, 32, ref.CODE_INT4, k_mode=ref.GROUP_ASYM, group_size=32)
    assert ref.bytes_per_token(L, 80, 1) == 81920 + 80 * 2 * 160
    L = ref.layout(8, 128, 16, ref.CODE_INT8, k_mode=ref.CHANNEL_BLOCK)
    assert ref.bytes_per_token(L, 1, 1) == 2048 + 256 + 32
    assert ref.bytes_per_token(ref.layout(8, 128, 16, ref.CODE_NONE16), 1, 1) == 4096


def test_bytes_per_token_rejects_bad_input():
    assert ref.bytes_per_token(ref.layout(8, 96, 16, ref.CODE_INT8), 1) == ref.ERR_INVALID
    assert ref.bytes_per_token(ref.layout(8, 128, 16, ref.CODE_INT8), 0) == ref.ERR_INVALID
    bad = ref.layout(8, 128, 16, ref.CODE_FP8, k_mode=ref.GROUP_ASYM, group_size=32)
    assert ref.bytes_per_token(bad, 1) == ref.ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# Symmetric absmax INT8 / INT4.
# ---------------------------------------------------------------------------

def test_int8_hand_worked_ties_to_even():
    # max|x| = 127 gives scale exactly 1, so codes are rne(x): ties go to even.
    x = f32([127.0, 63.5, -1.5, 0.5, 2.5, -2.5, -127.0, 0.25, 1.4999999, 3.5])
    q, s = ref.quant_sym(x, 127)
    assert s == 1.0
    assert q.tolist() == [127, 64, -2, 0, 2, -2, -127, 0, 1, 4]
    # max|x| = 254 gives scale 2: x / 2 = 127, 0.5, 1.5, -2.5, -0.5.
    q, s = ref.quant_sym(f32([254.0, 1.0, 3.0, -5.0, -1.0]), 127)
    assert s == 2.0 and q.tolist() == [127, 0, 2, -2, 0]


@pytest.mark.parametrize("qmax", [127, 7])
def test_sym_round_trip_bound(qmax):
    for _ in range(300):
        d = int(rng.choice([64, 128]))
        x = f32(rng.standard_normal(d) * 10.0 ** rng.uniform(-3, 3))
        q, s = ref.quant_sym(x, qmax)
        assert np.abs(q).max() <= qmax
        err = np.abs(x.astype(np.float64) - q.astype(np.float64) * float(s))
        assert err.max() <= float(s) * (0.5 + 2.0 ** -16)
        a = np.abs(x).max()
        assert abs(float(s) - a / qmax) <= a / qmax * 2.0 ** -23


@pytest.mark.parametrize("qmax", [127, 7])
def test_sym_exact_recovery_on_grid(qmax):
    for _ in range(200):
        k = rng.integers(-qmax, qmax + 1, size=128)
        k[rng.integers(128)] = qmax * rng.choice([-1, 1])
        e = int(rng.integers(-20, 12))
        x = f32(k * 2.0 ** e)
        q, s = ref.quant_sym(x, qmax)
        assert s == 2.0 ** e
        assert (q == k).all()


def test_sym_zero_row_and_sign_and_power_of_two():
    q, s = ref.quant_sym(np.zeros(64, np.float32), 127)
    assert s == 1.0 and not q.any()
    for _ in range(100):
        x = f32(rng.standard_normal(128) * 3)
        q, s = ref.quant_sym(x, 127)
        qn, sn = ref.quant_sym(-x, 127)
        assert sn == s and (qn == -q).all()
        k = int(rng.integers(-8, 9))
        qk, sk = ref.quant_sym(f32(x * 2.0 ** k), 127)
        assert sk == np.float32(s * 2.0 ** k) and (qk == q).all()


@pytest.mark.parametrize("bits", [8, 4])
def test_absmax_rule_hand_worked(bits):
    # "Dynamic KV Cache Quantization for Fast LLM Inference", section
    # "Understanding Dynamic Quantization Techniques for KV Caches": the scale
    # is the row's largest magnitude over 2^(bits-1) - 1 and a code is the
    # value over the scale, rounded. Rows chosen so that the scale is a power
    # of two (exact), with the expected codes worked out by hand; halves go
    # to the even neighbour.
    qmax = 2 ** (bits - 1) - 1
    if bits == 8:
        # max 15.875 = 127 / 8 -> scale 1/8; x * 8 = 0.5, 1.5, 2.5, -3.5, 127, 8, 40.48
        x = [0.0625, 0.1875, 0.3125, -0.4375, 15.875, 1.0, 5.06]
        want = [0, 2, 2, -4, 127, 8, 40]
        scale = 0.125
    else:
        # max 1.75 = 7 / 4 -> scale 1/4; x * 4 = 0.5, 1.5, -2.5, 7, -4, 1.2, -6.5
        x = [0.125, 0.375, -0.625, 1.75, -1.0, 0.3, -1.625]
        want = [0, 2, -2, 7, -4, 1, -6]
        scale = 0.25
    q, s = ref.quant_sym(f32(x), qmax)
    assert float(s) == scale
    assert q.tolist() == want


@pytest.mark.parametrize("bits", [8, 4])
def test_absmax_rule_against_exact_rationals(bits):
    # The same rule checked with exact rational arithmetic on heavy-tailed
    # (Laplace) rows of 48 elements: the fp32 scale is the correctly rounded
    # quotient max|x| / (2^(bits-1) - 1), and each code is the integer nearest
    # to the exact ratio x / scale (halves to even). Elements whose exact
    # ratio lies within 2^-18 of a rounding boundary are skipped: there the
    # fp32 rounding of the quotient itself decides, which the hand-worked
    # ties above cover.
    from fractions import Fraction
    qmax = 2 ** (bits - 1) - 1
    r = np.random.default_rng(77 + bits)
    for _ in range(40):
        x = f32(r.laplace(0.0, 10.0 ** r.uniform(-2, 2), 48))
        q, s = ref.quant_sym(x, qmax)
        a = max(abs(Fraction(float(v))) for v in x)
        s_exact = a / qmax
        # a correctly rounded fp32 scale lies within half an ulp (2^-24
        # relative) of the exact quotient
        s32 = Fraction(float(s))
        assert abs(s32 - s_exact) <= s_exact * Fraction(1, 2 ** 24)
        for xi, qi in zip(x, q):
            y = Fraction(float(xi)) / s32
            fl = y.numerator // y.denominator
            frac = y - fl
            if abs(frac - Fraction(1, 2)) < Fraction(1, 2 ** 18):
                continue
            nearest = fl + 1 if frac > Fraction(1, 2) else fl
            nearest = max(-qmax, min(qmax, nearest))
            assert int(qi) == nearest, (float(xi), float(s), int(qi), nearest)


# ---------------------------------------------------------------------------
# FP8 E4M3.
# ---------------------------------------------------------------------------

def test_e4m3_format_points():
    g = json.loads((GOLD / "e4m3.json").read_text())
    for code, val in g["values"].items():
        assert ref.e4m3_value(int(code, 16)) == val
    for code in g["nan"]:
        assert math.isnan(ref.e4m3_value(int(code, 16)))
    z = ref.e4m3_value(int(g["negative_zero"], 16))
    assert z == 0.0 and math.copysign(1.0, z) < 0


def test_e4m3_value_table_is_monotone_and_symmetric():
    vals = [ref.e4m3_value(c) for c in range(127)]
    assert all(a < b for a, b in zip(vals, vals[1:]))
    for c in range(127):
        assert ref.e4m3_value(c | 0x80) == -vals[c]


def test_e4m3_encode_matches_torch_cast():
    # torch's float32 -> float8_e4m3fn cast is the library routine for the
    # same format (round to nearest even); compare on every fp32 value whose
    # magnitude stays within the format's range.
    grid = np.concatenate([
        np.linspace(-448, 448, 200001, dtype=np.float32),
        f32(rng.standard_normal(200000) * 50),
        f32(np.sign(rng.standard_normal(100000)) * 2.0 ** rng.uniform(-12, 8.8, 100000)),
    ])
    grid = grid[np.abs(grid) <= 448]
    t = torch.from_numpy(grid).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([ref.e4m3_encode(y) for y in grid.tolist()], np.uint8)
    assert (ours == t).all()


def test_e4m3_encode_round_trip_midpoints_saturation():
    for c in list(range(127)) + [c | 0x80 for c in range(127)]:
        assert ref.e4m3_encode(ref.e4m3_value(c)) == c
    for c in range(126):
        lo, hi = ref.e4m3_value(c), ref.e4m3_value(c + 1)
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2
        assert ref.e4m3_encode(mid) == (c if c % 2 == 0 else c + 1)
        assert ref.e4m3_encode(np.nextafter(mid, np.float32(0))) == c
        assert ref.e4m3_encode(np.nextafter(mid, np.float32(1000))) == c + 1
    assert ref.e4m3_encode(448.0 * (1 + 2 ** -23)) == 0x7E
    assert ref.e4m3_encode(1e30) == 0x7E
    assert ref.e4m3_encode(-500.0) == 0xFE
    assert ref.e4m3_encode(-0.0) == 0x80
    assert ref.e4m3_encode(-1e-30) == 0x80


def _e4m3_half_spacing(y):
    a = abs(y)
    e = max(math.floor(math.log2(a)), -6) if a > 0 else -6
    return 2.0 ** (e - 3) / 2


def test_fp8_round_trip_bound_and_exact_recovery():
    for _ in range(200):
        x = f32(rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 3))
        q, s = ref.quant_fp8(x)
        for xi, qi in zip(x.tolist(), q.tolist()):
            y = xi / float(s)
            xh = ref.e4m3_value(qi) * float(s)
            assert abs(xi - xh) <= float(s) * _e4m3_half_spacing(y) * (1 + 2 ** -16) \
                + abs(xi) * 2 ** -23
    on_grid = np.array([ref.e4m3_value(c) for c in range(127)], np.float64)
    for _ in range(100):
        v = rng.choice(on_grid, size=128) * rng.choice([-1, 1], size=128)
        v[rng.integers(128)] = 448.0
        e = int(rng.integers(-10, 6))
        x = f32(v * 2.0 ** e)
        q, s = ref.quant_fp8(x)
        assert s == 2.0 ** e
        assert all(ref.e4m3_value(c) == vi for c, vi in zip(q.tolist(), v.tolist()))


def test_fp8_zero_row():
    q, s = ref.quant_fp8(np.zeros(128, np.float32))
    assert s == 1.0 and not q.any()


# ---------------------------------------------------------------------------
# INT4 asymmetric per group, and the nibble layout.
# ---------------------------------------------------------------------------

def test_asym4_exact_recovery_on_grid():
    for _ in range(300):
        z0 = int(rng.integers(0, 16))
        k = rng.integers(0, 16, size=32)
        k[0], k[1] = 0, 15
        rng.shuffle(k)
        e = int(rng.integers(-16, 8))
        x = f32((k - z0) * 2.0 ** e)
        q, s, z = ref.quant_asym4(x)
        assert s == 2.0 ** e and z == z0 and (q == k).all()


def test_asym4_round_trip_bound_and_range():
    for _ in range(500):
        x = f32(rng.standard_normal(32) * 10.0 ** rng.uniform(-3, 3)
                + rng.choice([0.0, 3.0, -3.0]))
        q, s, z = ref.quant_asym4(x)
        assert q.max() <= 15 and 0 <= z <= 15
        xh = (q.astype(np.float64) - z) * float(s)
        assert np.abs(x - xh).max() <= float(s) * (0.5 + 2.0 ** -10)


def test_asym4_special_groups():
    q, s, z = ref.quant_asym4(np.zeros(32, np.float32))
    assert s == 1.0 and z == 0 and not q.any()
    # all positive: range widened to [0, max], zero point 0
    q, s, z = ref.quant_asym4(f32(np.linspace(1, 15, 32)))
    assert z == 0 and s == 1.0 and q.max() == 15
    # all negative: zero point 15
    q, s, z = ref.quant_asym4(f32(-np.linspace(1, 15, 32)))
    assert z == 15 and s == 1.0 and q.min() == 0


def test_int4_nibble_layout():
    d = 128
    nib = (np.arange(d) * 7 % 16).astype(np.uint8)
    packed = ref.int4_pack(nib)
    assert (ref.int4_unpack(packed, d) == nib).all()
    # element e = 32 i + 2 r + t sits in byte 4 r + i (n = d/32 = 4)
    def at(e):
        i, r, t = e // 32, (e % 32) // 2, e % 2
        return (packed[4 * r + i] >> (4 * t)) & 0xF
    for e in (0, 1, 2, 31, 32, 33, 64, 100, 127):
        assert at(e) == nib[e]
    one = np.zeros(d, np.uint8)
    one[127] = 9  # i = 3, r = 15, t = 1 -> byte 63, high nibble
    assert ref.int4_pack(one)[63] == 0x90 and ref.int4_pack(one)[:63].sum() == 0
    one = np.zeros(64, np.uint8)
    one[33] = 5   # d = 64: n = 2, i = 1, r = 0, t = 1 -> byte 1, high nibble
    assert ref.int4_pack(one).tolist()[1] == 0x50


# ---------------------------------------------------------------------------
# Per-channel-per-block keys.
# ---------------------------------------------------------------------------

def test_channel_block_exact_recovery_and_bound():
    for bs in (16, 32):
        for _ in range(30):
            k = rng.integers(-127, 128, size=(bs, 128))
            rows = rng.integers(0, bs, size=128)
            k[rows, np.arange(128)] = 127 * rng.choice([-1, 1], size=128)
            e = rng.integers(-12, 8, size=128)
            x = f32(k * 2.0 ** e[None, :])
            q, s = ref.quant_channel_block(x)
            assert (s == 2.0 ** e).all() and (q == k).all()
            y = f32(rng.standard_normal((bs, 128)) * (1 + 8 * (rng.random(128) < 0.05)))
            q, s = ref.quant_channel_block(y)
            err = np.abs(y - q.astype(np.float64) * s.astype(np.float64)[None, :])
            assert (err <= s[None, :].astype(np.float64) * (0.5 + 2.0 ** -16)).all()
