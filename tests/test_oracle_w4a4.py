"""Pins for the oracle's W4A4 variant (CPU only): the MXFP4 activation
quantizer against hand-worked blocks of the OCP MX conversion, the scalar
E2M1 encoder, and closed-form properties; the W4A4 product against the
weight-only product on activations that are exactly MXFP4 (where quantizing
changes nothing) and against a correctly rounded brute force."""

import math

import numpy as np
import pytest

import oracle

MX = oracle.FMT_MXFP4
MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _bf16(a):
    return oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(np.asarray(a, dtype=np.float32)))


def _block(values):
    row = np.zeros(32, np.float32)
    row[:len(values)] = values
    return row[None, :]


def test_worked_block_amax_one():
    # amax 1 -> floor(log2 1) - 2 = -2: scale 2^-2 (byte 125), v = 4 x.
    x = _block([1.0, 0.375, 0.3125, 0.4375, -0.0625, 0.1875, 0.625, 0.875, -0.5, 0.0, -0.0])
    codes, scales = oracle.quantize_act_mxfp4(x)
    assert scales.tolist() == [[125]]
    # v:    4 -> 4.0 (6); 1.5 -> 1.5 (3); 1.25 tie 1 / 1.5 -> 1 (2); 1.75 tie
    # 1.5 / 2 -> 2 (4); -0.25 tie 0 / 0.5 -> -0 (8); 0.75 tie 0.5 / 1 -> 1 (2);
    # 2.5 tie 2 / 3 -> 2 (4); 3.5 tie 3 / 4 -> 4 (6); -2 (12); 0 (0); -0 (8).
    assert codes[0, :11].tolist() == [6, 3, 2, 4, 8, 2, 4, 6, 12, 0, 8]
    assert not codes[0, 11:].any()


def test_worked_block_saturation_and_tie_at_five():
    # amax 1.75 -> floor(log2 1.75) = 0 -> scale 2^-2; v = 7 saturates to 6.
    x = _block([1.75, 1.25, 1.5, -1.0, 1.125])
    codes, scales = oracle.quantize_act_mxfp4(x)
    assert scales.tolist() == [[125]]
    # v: 7 -> 6 (7); 5 tie 4 / 6 -> 4 (6); 6 (7); -4 (14); 4.5 -> 4 (6).
    assert codes[0, :5].tolist() == [7, 6, 7, 14, 6]


def test_scale_exponent_closed_form():
    rng = np.random.default_rng(11)
    for _ in range(200):
        e = int(rng.integers(-120, 120))
        blk = _bf16(rng.standard_normal(32) * 2.0 ** e)
        codes, scales = oracle.quantize_act_mxfp4(blk[None, :])
        amax = float(np.max(np.abs(blk)))
        x_scale = 2.0 ** (int(scales[0, 0]) - 127)
        # The largest element lands in [4, 8) after the scaling: 2^e <= amax < 2^(e+1)
        # with e = floor(log2 amax), and X = 2^(e-2).
        assert 4.0 <= amax / x_scale < 8.0


def test_scale_edge_cases():
    # All zeros: byte 0, codes 0.
    c, s = oracle.quantize_act_mxfp4(_block([0.0] * 32))
    assert s.tolist() == [[0]] and not c.any()
    # Smallest bf16 subnormal 2^-133: e = -135 clamps to -127; v = 2^-6 -> code 0.
    c, s = oracle.quantize_act_mxfp4(_block([2.0 ** -133]))
    assert s.tolist() == [[0]] and not c.any()
    # amax 2^-125: floor(log2) - 2 = -127 exactly, v = 4 -> code 6.
    c, s = oracle.quantize_act_mxfp4(_block([2.0 ** -125]))
    assert s.tolist() == [[0]] and c[0, 0] == 6
    # Largest finite bf16 (1.9921875 * 2^127): e = 125, byte 252, v = 7.97 -> 6.
    big = float(_bf16([3.3895313892515355e38])[0])
    c, s = oracle.quantize_act_mxfp4(_block([big, -big / 2]))
    assert s.tolist() == [[252]] and c[0, :2].tolist() == [7, 14]
    # A non-finite element marks its block NaN (0xFF) with zero codes; the
    # other block of the row is unaffected.
    row = np.zeros((1, 64), np.float32)
    row[0, 3] = np.inf
    row[0, 40] = 1.0
    c, s = oracle.quantize_act_mxfp4(row)
    assert s.tolist() == [[255, 125]] and not c[0, :32].any() and c[0, 40] == 6
    row[0, 3] = np.nan
    c, s = oracle.quantize_act_mxfp4(row)
    assert s[0, 0] == 255


def test_vectorized_encoder_matches_scalar_encoder():
    # Every midpoint of the E2M1 grid, both signs, the grid itself, values
    # past 6, and random bf16 values against the Fraction-based encoder.
    mids = [(a + b) / 2 for a, b in zip(MAGS, MAGS[1:])]
    vals = MAGS + mids + [6.5, 7.0, 7.999, 1e-30, 0.2499, 0.2501]
    rng = np.random.default_rng(3)
    vals += [float(v) for v in _bf16(rng.uniform(-8, 8, 2000))]
    vals += [-v for v in vals] + [-0.0]
    got = oracle.e2m1_nearest_even(np.array(vals))
    want = [oracle.e2m1_encode(v) for v in vals]
    assert got.tolist() == want


def test_nearest_by_brute_force():
    # Each code is a nearest point of the E2M1 grid (both signs) to x / X.
    rng = np.random.default_rng(4)
    x = _bf16(rng.standard_normal((6, 128)) * np.exp(rng.uniform(-8, 8, (6, 1))))
    codes, scales = oracle.quantize_act_mxfp4(x)
    grid = np.array([oracle.E2M1_TABLE[c] for c in range(16)], np.float64)
    for i in range(6):
        for t in range(128):
            v = float(x[i, t]) * 2.0 ** (127 - int(scales[i, t // 32]))
            best = np.min(np.abs(grid - v))
            assert abs(float(grid[codes[i, t]]) - v) == best


def _exact_mxfp4_rows(rng, m, k):
    # Rows that are exactly MXFP4: per block a random exponent, random E2M1
    # codes, and one element forced to magnitude 4 or 6 so that the block's
    # scale is the chosen exponent.
    codes = rng.integers(0, 16, size=(m, k)).astype(np.uint8)
    exps = rng.integers(-30, 30, size=(m, k // 32))
    for i in range(m):
        for b in range(k // 32):
            codes[i, 32 * b + int(rng.integers(0, 32))] = int(rng.choice([6, 7, 14, 15]))
    vals = oracle.E2M1_TABLE[codes].astype(np.float64) * np.repeat(2.0 ** exps, 32, axis=1)
    return vals.astype(np.float32), codes, (exps + 127).astype(np.uint8)


def test_exact_mxfp4_activations_quantize_to_themselves():
    rng = np.random.default_rng(5)
    x, codes, scales = _exact_mxfp4_rows(rng, 5, 256)
    assert np.array_equal(_bf16(x), x)
    got_c, got_s = oracle.quantize_act_mxfp4(x)
    assert np.array_equal(got_s, scales)
    assert np.array_equal(got_c, codes)
    assert np.array_equal(oracle.dequantize_act_mxfp4(got_c, got_s), x.astype(np.float64))


def test_w4a4_equals_w4a16_on_exact_activations():
    # Where Q(x) = x the W4A4 product is the weight-only product.
    rng = np.random.default_rng(6)
    n, k, m = 40, 256, 4
    x, _, _ = _exact_mxfp4_rows(rng, m, k)
    w = rng.standard_normal((n, k)).astype(np.float32)
    packed, scales = oracle.quantize_mxfp4(w)
    y4 = oracle.w4a4_linear(x, packed, scales, k)
    y16 = oracle.linear(x, packed, scales, k, MX)
    assert np.allclose(y4, y16, rtol=1e-14, atol=0)


def test_w4a4_one_hot_activation():
    # x = 1 at column c of row i (quantized exactly: amax 1 -> code 4.0 x 2^-2)
    # picks column c of the dequantized weight.
    rng = np.random.default_rng(7)
    n, k = 24, 128
    w = rng.standard_normal((n, k)).astype(np.float32)
    packed, scales = oracle.quantize_mxfp4(w)
    wd = oracle.dequantize(packed, scales, k, MX)
    x = np.zeros((3, k), np.float32)
    cols = [0, 77, 127]
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = oracle.w4a4_linear(x, packed, scales, k)
    for i, c in enumerate(cols):
        assert np.array_equal(y[i], wd[:, c].astype(np.float64))


def test_w4a4_against_fsum_bruteforce():
    # Tiny case: correctly rounded sums of the dequantized operands' products.
    rng = np.random.default_rng(8)
    n, k, m = 5, 64, 3
    x = _bf16(rng.standard_normal((m, k)))
    w = rng.standard_normal((n, k)).astype(np.float32)
    packed, scales = oracle.quantize_mxfp4(w)
    wd = oracle.dequantize(packed, scales, k, MX)
    xc, xs = oracle.quantize_act_mxfp4(x)
    y = oracle.w4a4_linear(x, packed, scales, k)
    for i in range(m):
        for j in range(n):
            terms = []
            for t in range(k):
                xv = oracle.e2m1_value(int(xc[i, t])) * 2.0 ** (int(xs[i, t // 32]) - 127)
                terms.append(float(xv) * float(wd[j, t]))
            assert math.isclose(y[i, j], math.fsum(terms), rel_tol=1e-13, abs_tol=1e-300)
