"""Pins of the oracle's FP8 window (the window KV kept in FP8: "DeepSeek-V4.1-Flash,
expliqué pas à pas", FP4 KV cache section).  The format is a reading: E4M3FN codes,
one E8M0 scale per 512-channel row, the smallest power of two X with amax <= 448 X,
codes nearest to x / X with ties to the even byte.  Checked against torch's float8
conversion, numpy's log2, exact rationals and the bf16 attention path it reduces to."""
import math
from fractions import Fraction

import numpy as np
import torch

import oracle
from sparse_attention_fp4_cache_amd.workloads import bf16_bits_to_f32, to_bf16_bits


def _rows(rng, n, spread=6.0):
    x = rng.standard_normal((n, 512)) * np.exp(rng.uniform(-spread, spread, (n, 1)))
    x[:, 7] *= 8.0  # an outlier channel
    return to_bf16_bits(x.astype(np.float32))


def test_scale_is_smallest_power_of_two_covering_amax():
    x = _rows(np.random.default_rng(20), 3000)
    _, sc = oracle.swa_fp8_quant(x)
    amax = np.abs(bf16_bits_to_f32(x).astype(np.float64)).max(axis=1)
    e = sc.astype(np.int64) - 127
    assert np.all(amax <= 448.0 * np.exp2(e)) and np.all(amax > 448.0 * np.exp2(e - 1))
    assert np.array_equal(e, np.ceil(np.log2(amax / 448.0)).astype(np.int64))


def test_codes_match_torch_float8_rne():
    x = _rows(np.random.default_rng(21), 2000)
    codes, sc = oracle.swa_fp8_quant(x)
    xs = bf16_bits_to_f32(x).astype(np.float64) * np.exp2(-(sc.astype(np.float64) - 127))[:, None]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_ties_go_to_even_codes_and_zero_rows():
    # row scale 2^0 (amax 448): x = midpoints between neighbouring E4M3 values
    mids, want = [], []
    for b in range(0x08, 0x7E):  # normal codes, pairs (b, b+1)
        lo, hi = oracle.e4m3_value(b), oracle.e4m3_value(b + 1)
        m = (Fraction(lo) + Fraction(hi)) / 2
        if m.denominator & (m.denominator - 1) or float(m) != m:
            continue
        mids.append(float(m))
        want.append(b if b % 2 == 0 else b + 1)
    xb = np.zeros((1, 512), np.uint16)
    xb[0, 0] = to_bf16_bits(np.array([448.0], np.float32))[0]
    n = 0
    for v, w in zip(mids, want):
        bits = to_bf16_bits(np.array([v], np.float32))[0]
        if bf16_bits_to_f32(bits) != v or n >= 511:
            continue  # only midpoints that bf16 holds exactly
        xb[0, 1 + n] = bits
        want[n] = w
        n += 1
    assert n > 20
    codes, sc = oracle.swa_fp8_quant(xb)
    assert sc[0] == 127
    assert list(codes[0, 1:1 + n]) == want[:n]
    z = np.zeros((2, 512), np.uint16)
    z[1] = 0x8000  # -0.0
    codes, sc = oracle.swa_fp8_quant(z)
    assert list(sc) == [0, 0] and np.all(codes[0] == 0) and np.all(codes[1] == 0x80)


def test_dequant_is_exact_and_within_half_a_step():
    x = _rows(np.random.default_rng(22), 1000)
    codes, sc = oracle.swa_fp8_quant(x)
    d = oracle.swa_fp8_dequant(codes, sc)
    xv = bf16_bits_to_f32(x).astype(np.float64)
    dv = bf16_bits_to_f32(d).astype(np.float64)
    X = np.exp2(sc.astype(np.float64) - 127)[:, None]
    # E4M3: 3 mantissa bits; a normal value's half-step is |v| / 16 at most, the
    # subnormal half-step 2^-10 X
    assert np.all(np.abs(dv - xv) <= np.maximum(np.abs(xv) / 16.0, 2.0 ** -10 * X))
    # quantising the dequantised rows gives back the same values (the scale may halve
    # when the largest value rounded down onto 224 X)
    c2, s2 = oracle.swa_fp8_quant(d)
    assert np.array_equal(oracle.swa_fp8_dequant(c2, s2), d)
    assert np.all((s2 == sc) | (s2 == sc - 1))


def test_exact_rational_brute_force_on_small_rows():
    rng = np.random.default_rng(23)
    x = _rows(rng, 6, spread=3.0)
    codes, sc = oracle.swa_fp8_quant(x)
    grid = [(b, Fraction(oracle.e4m3_value(b))) for b in range(0x7F)]
    for r in range(x.shape[0]):
        vals = [Fraction(float(v)) for v in bf16_bits_to_f32(x[r])]
        amax = max(abs(v) for v in vals)
        e = -127
        while Fraction(448) * Fraction(2) ** e < amax:
            e += 1
        assert sc[r] == e + 127
        for c in range(0, 512, 7):
            a = abs(vals[c]) / Fraction(2) ** e
            best = min(grid, key=lambda g: (abs(g[1] - a), g[0] & 1))
            assert codes[r, c] & 0x7F == best[0]
            assert (codes[r, c] >> 7) == (1 if math.copysign(1.0, float(vals[c])) < 0 else 0)


def test_fp8_window_attention_equals_bf16_when_rows_are_fp8_values():
    # window rows whose values are already E4M3 values times a power of two quantise
    # losslessly, so the FP8-window attention equals the bf16-window attention
    rng = np.random.default_rng(24)
    lat = to_bf16_bits(rng.standard_normal((128, 512)).astype(np.float32))
    key = to_bf16_bits(rng.standard_normal((128, 128)).astype(np.float32))
    c = oracle.Cache(128)
    oracle.fp4_cache_write(c, lat, key, np.arange(128))
    H, W = 16, 8
    q = to_bf16_bits(rng.standard_normal((1, H, 512)).astype(np.float32))
    e4 = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    vals = rng.choice(e4, (1, W, 512)) * np.where(rng.random((1, W, 512)) < 0.5, -1, 1)
    vals[0, :, 0] = 448.0
    vals = vals * np.exp2(rng.integers(-6, 3, (1, W, 1)))
    win = to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(win).astype(np.float64), vals)
    codes, sc = oracle.swa_fp8_quant(win)
    assert np.array_equal(oracle.swa_fp8_dequant(codes, sc), win)
    idx = np.sort(rng.choice(128, (1, 16), replace=False), axis=1).astype(np.int32)
    bt = np.zeros((1, 2), np.int32)
    bt[0] = [0, 1]
    swa_len = np.array([W - 2], np.int32)
    o8, l8 = oracle.sparse_attn_decode_fp8win(c, q, idx, bt, codes, sc, swa_len, 0.05)
    o16, l16 = oracle.sparse_attn_decode(c, q, idx, bt, win, swa_len, 0.05)
    assert np.array_equal(o8, o16) and np.array_equal(l8, l16)
