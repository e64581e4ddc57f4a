"""Pins for the oracle's NVFP4 W4A4 variant (CPU only): the vectorized E4M3FN
rounding against the exact scalar encoder and against torch's float8_e4m3fn
conversion; the NVFP4 activation quantizer against hand-worked blocks, a
pure-Python brute force built on the exact scalar encoders, and closed-form
properties; the W4A4 product against the weight-only product on activations
that are exactly NVFP4 and against a correctly rounded brute force."""

import math
import struct

import numpy as np
import pytest
import torch

import oracle
import synth

NV = oracle.FMT_NVFP4


def _bf16(a):
    return oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(np.asarray(a, dtype=np.float32)))


def _block(values, k=16):
    row = np.zeros(k, np.float32)
    row[:len(values)] = values
    return row[None, :]


def _f32(v):
    """Round a Python float to float32 (a double from one correctly rounded
    double operation on float32 operands rounds to the float32 result of the
    same operation: 53 >= 2 * 24 + 2)."""
    return struct.unpack("f", struct.pack("f", v))[0]


# ------------------------------------------------------------------ E4M3FN rounding

def test_e4m3_vectorized_matches_scalar_encoder():
    mags = sorted({float(v) for v in oracle.E4M3FN_TABLE[:0x7F]})
    mids = [(a + b) / 2 for a, b in zip(mags, mags[1:])]
    rng = np.random.default_rng(5)
    rand = list(np.exp(rng.uniform(math.log(1e-5), math.log(1e3), 2000)))
    vals = mags + mids + [m * (1 + 1e-9) for m in mids] + [m * (1 - 1e-9) for m in mids] + rand + \
        [0.0, 448.0, 463.99, 464.0, 464.01, 500.0, 1e30, math.inf, 2.0 ** -10, 2.0 ** -10 * 1.0001, 2.0 ** -11]
    got = oracle.e4m3fn_nearest_even(np.array(vals))
    want = [oracle.e4m3fn_encode(v) for v in vals]
    assert got.tolist() == want


def test_e4m3_matches_torch_float8_within_range():
    # torch's float8_e4m3fn conversion rounds to nearest even; inside the
    # finite range it must agree with the oracle byte for byte.
    rng = np.random.default_rng(6)
    v = np.concatenate([np.exp(rng.uniform(math.log(2.0 ** -12), math.log(448.0), 20000)),
                        [(a + b) / 2 for a, b in zip(oracle.E4M3FN_TABLE[:0x7E], oracle.E4M3FN_TABLE[1:0x7F])]])
    v = v.astype(np.float32)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3fn_nearest_even(v.astype(np.float64)), want)


# ------------------------------------------------------------------ activation quantizer

def test_worked_block_exact_scale():
    # G_x = 1/64, amax 6: s = (6 / 6) / (1/64) = 64 = 2^6, byte 0x68 (exponent
    # field 13); q = 64 / 64 = 1, so codes are E2M1(x): 6 (7), 3 (5), -1.5
    # (11), 0.75 tie 0.5 / 1 -> 1 (2), 0.25 tie 0 / 0.5 -> 0 (0), -0.25 -> -0
    # (8), 5 tie 4 / 6 -> 4 (6), 2.5 tie 2 / 3 -> 2 (4), 0 (0), -0 (8).
    x = _block([6.0, 3.0, -1.5, 0.75, 0.25, -0.25, 5.0, 2.5, 0.0, -0.0])
    codes, scales = oracle.quantize_act_nvfp4(x, 1 / 64)
    assert scales.tolist() == [[0x68]]
    assert codes[0, :10].tolist() == [7, 5, 11, 2, 0, 8, 6, 4, 0, 8]


def test_worked_block_rounded_scale():
    # G_x = 1/64, amax 7: s = fl32(7/6) * 64 = 74.67, between the E4M3 values
    # 72 (0x69) and 80 (0x6A): S = 72, q = 1.125.  x / q: 7 -> 6.22 -> 6 (7);
    # 2.5 -> 2.22 -> 2 (4); -1.6875 -> -1.5 (11); 0.5625 -> 0.5 (1); 2.8125
    # -> 2.5 tie 2 / 3 -> 2 (4); 3.9375 -> 3.5 tie 3 / 4 -> 4 (6).
    x = _block([7.0, 2.5, -1.6875, 0.5625, 2.8125, 3.9375])
    codes, scales = oracle.quantize_act_nvfp4(x, 1 / 64)
    assert scales.tolist() == [[0x69]]
    assert codes[0, :6].tolist() == [7, 4, 11, 1, 4, 6]


def test_worked_block_subnormal_scale():
    # G_x = 1, amax 2^-5: s = 2^-5 / 6 = 2.67 * 2^-9 -> subnormal S = 3 * 2^-9
    # (byte 0x03); x / q: 2^-5 -> 5.33 -> 6 (7); 2^-7 -> 1.33 -> 1.5 (3);
    # -2^-8 -> -0.67 -> -0.5 (9).
    x = _block([2.0 ** -5, 2.0 ** -7, -(2.0 ** -8)])
    codes, scales = oracle.quantize_act_nvfp4(x, 1.0)
    assert scales.tolist() == [[0x03]]
    assert codes[0, :3].tolist() == [7, 3, 9]


def test_scale_underflow_saturation_and_nonfinite():
    # Scale rounding to zero: s = 2^-14 / 6 is under half of 2^-9, S = 0 and
    # every code is 0 with the sign kept.
    c, s = oracle.quantize_act_nvfp4(_block([-(2.0 ** -14), 2.0 ** -15]), 1.0)
    assert s.tolist() == [[0]] and c[0, :3].tolist() == [8, 0, 0]
    # Saturation at 448: G_x = 2^-10, amax 9984 -> s = 9984 / 6 * 1024 > 448,
    # S = 448 (0x7E), q = 0.4375, 9984 / q saturates to 6; 0.75 / q = 1.71,
    # nearer 1.5 than 2 (3).
    c, s = oracle.quantize_act_nvfp4(_block([9984.0, 0.75]), 2.0 ** -10)
    assert s.tolist() == [[0x7E]] and c[0, :2].tolist() == [7, 3]
    # A non-finite element marks its block NaN (0x7F) with zero codes (signs
    # kept); the other block of the row is unaffected.
    row = np.zeros((1, 32), np.float32)
    row[0, 3] = np.inf
    row[0, 5] = -1.0
    row[0, 20] = 6.0
    c, s = oracle.quantize_act_nvfp4(row, 1 / 64)
    assert s.tolist() == [[0x7F, 0x68]]
    assert c[0, :16].tolist() == [0] * 5 + [8] + [0] * 10 and c[0, 20] == 7
    row[0, 3] = np.nan
    assert oracle.quantize_act_nvfp4(row, 1 / 64)[1].tolist() == [[0x7F, 0x68]]


def _bruteforce(x, gx):
    """One block at a time in scalar Python: the exact scalar encoders of the
    formats module and explicit float32 rounding of every step."""
    m, k = x.shape
    codes = np.zeros((m, k), np.uint8)
    scales = np.zeros((m, k // 16), np.uint8)
    gx = _f32(float(gx))
    for i in range(m):
        for b in range(k // 16):
            blk = [float(v) for v in x[i, 16 * b:16 * b + 16]]
            signs = [8 if math.copysign(1.0, v) < 0 else 0 for v in blk]
            if not all(math.isfinite(v) for v in blk):
                scales[i, b] = 0x7F
                codes[i, 16 * b:16 * b + 16] = signs
                continue
            amax = max(abs(v) for v in blk)
            sv = _f32(_f32(amax / 6.0) / gx) if gx != 0 else math.inf
            sb = oracle.e4m3fn_encode(sv if math.isfinite(sv) else math.inf)
            scales[i, b] = sb
            q = _f32(float(oracle.E4M3FN_TABLE[sb]) * gx)
            for j, v in enumerate(blk):
                if q == 0.0:
                    codes[i, 16 * b + j] = signs[j]
                else:
                    r = _f32(v / q) if math.isfinite(q) else math.copysign(0.0, v)
                    codes[i, 16 * b + j] = oracle.e2m1_encode(r) | signs[j]
    return codes, scales


@pytest.mark.parametrize("seed", range(6))
def test_quantizer_matches_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    e = int(rng.integers(-30, 30))
    x = _bf16(rng.standard_normal((3, 64)) * 2.0 ** e)
    x[0, :16] = 0.0                                     # an all-zero block
    x[1, 16] *= 64.0                                    # one outlier
    gx = np.float32(float(np.max(np.abs(x))) / (6 * 448) * rng.uniform(0.3, 3.0))
    got = oracle.quantize_act_nvfp4(x, gx)
    want = _bruteforce(x, gx)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_quantizer_on_the_workload_activations():
    # A slice of the prefill workload's activations with the calibrated G_x.
    x = oracle.bf16_bits_to_f32(synth.activations(synth.PREFILL, 4, 5120))[:, :512]
    gx = np.float32(np.float32(np.max(np.abs(x))) / np.float32(6 * 448))
    got = oracle.quantize_act_nvfp4(x, gx)
    want = _bruteforce(x, gx)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_power_of_two_rescaling_and_sign_symmetry():
    rng = np.random.default_rng(7)
    x = _bf16(rng.standard_normal((4, 64)))
    gx = np.float32(0.00123)
    c0, s0 = oracle.quantize_act_nvfp4(x, gx)
    for j in (-8, -1, 3, 10):
        c, s = oracle.quantize_act_nvfp4((x * np.float32(2.0 ** j)).astype(np.float32), np.float32(gx * 2.0 ** j))
        assert np.array_equal(c, c0) and np.array_equal(s, s0), j
    c, s = oracle.quantize_act_nvfp4(-x, gx)
    assert np.array_equal(s, s0) and np.array_equal(c, c0 ^ 8)


def test_grid_activations_round_trip():
    # x = E2M1(c) * S * G_x with a 6 in every block and G_x a power of two:
    # s = S exactly, q = S * G_x, and the codes come back unchanged.
    rng = np.random.default_rng(8)
    gx = 2.0 ** -9
    codes = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    codes[:, ::16] = 7
    sb = rng.integers(0x08, 0x70, (5, 4)).astype(np.uint8)      # normal scales, no overflow
    x = (oracle.dequantize_act_nvfp4(codes, sb) * gx).astype(np.float32)
    assert np.array_equal(_bf16(x), x)
    c, s = oracle.quantize_act_nvfp4(x, gx)
    assert np.array_equal(s, sb)
    # Codes of zero magnitude may differ only in sign where x is +-0.
    assert np.array_equal(c, codes)


# ------------------------------------------------------------------ W4A4 product

def test_product_equals_weight_only_on_grid_activations():
    # With G_x and G_w powers of two and x exactly NVFP4 at G_x, quantizing
    # changes nothing and alpha * (x_hat @ w.T) is the weight-only product.
    rng = np.random.default_rng(9)
    n, k = 24, 64
    w = rng.standard_normal((n, k)).astype(np.float32)
    packed, scales, _ = oracle.quantize_nvfp4(w, global_scale=np.float32(2.0 ** -8))
    gw, gx = np.float32(2.0 ** -8), 2.0 ** -9
    codes = rng.integers(0, 16, (3, k)).astype(np.uint8)
    codes[:, ::16] = 15
    sb = rng.integers(0x20, 0x60, (3, k // 16)).astype(np.uint8)
    x = (oracle.dequantize_act_nvfp4(codes, sb) * gx).astype(np.float32)
    got = oracle.w4a4_nvfp4_linear(x, packed, scales, k, gw, gx)
    want = oracle.linear(x, packed, scales, k, NV, gw)
    assert np.array_equal(got, want)


def test_product_matches_correctly_rounded_bruteforce():
    rng = np.random.default_rng(10)
    n, k = 6, 48
    packed, scales, gw = oracle.quantize_nvfp4(rng.standard_normal((n, k)).astype(np.float32))
    x = _bf16(rng.standard_normal((2, k)))
    gx = np.float32(float(np.max(np.abs(x))) / (6 * 448))
    xc, xs = _bruteforce(x, gx)
    xq = [[float(oracle.E2M1_TABLE[xc[i, t]]) * float(oracle.E4M3FN_TABLE[xs[i, t // 16]]) for t in range(k)]
          for i in range(2)]
    wq = oracle.dequantize(packed, scales, k, NV, 1.0)
    alpha = _f32(float(gx) * float(gw))
    want = np.array([[alpha * math.fsum(xq[i][t] * float(wq[j, t]) for t in range(k)) for j in range(n)]
                     for i in range(2)])
    got = oracle.w4a4_nvfp4_linear(x, packed, scales, k, gw, gx)
    assert np.allclose(got, want, rtol=1e-12, atol=0)
    # The global scales enter once, as a product after the sum.
    assert np.allclose(oracle.w4a4_nvfp4_linear(x, packed, scales, k, gw * 2, gx), 2 * got, rtol=1e-6)


def test_product_nan_row():
    rng = np.random.default_rng(12)
    packed, scales, gw = oracle.quantize_nvfp4(rng.standard_normal((4, 32)).astype(np.float32))
    x = _bf16(rng.standard_normal((2, 32)))
    x[1, 20] = np.inf
    y = oracle.w4a4_nvfp4_linear(x, packed, scales, 32, gw, 0.01)
    assert np.isfinite(y[0]).all() and np.isnan(y[1]).all()
