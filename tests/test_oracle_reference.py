"""Pins for the oracle's dequantization, linear layer and quantizers (CPU only).

The oracle is checked against things that do not come from itself: exact
rational products, closed-form special cases, fp64 brute force with a
rounding-error bound, hand-built layouts, the byte counts printed on the pages
and, for the quantizers, an independent vectorized implementation (synth).
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import quantize as oq
from conftest import read_golden

NV, MX = oracle.FMT_NVFP4, oracle.FMT_MXFP4


def _f32_of_fraction(v):
    # v has at most ~30 significant bits here, so float(v) is exact in float64
    # and the float32 conversion rounds once (nearest even, IEEE overflow).
    d = float(v)
    assert Fraction(d) == v
    with np.errstate(over="ignore"):
        return np.float32(d)


def test_unpack_low_nibble_first():
    # Byte 0x21 holds element 0 = code 1 (low nibble) and element 1 = code 2.
    packed = np.array([[0x21, 0xF0]], dtype=np.uint8)
    assert oracle.unpack_codes(packed, 4).tolist() == [[1, 2, 0, 15]]


@pytest.mark.parametrize("g", [1.0, 2.0 ** -7, 0.02 * 3.1 / 2688, 1.7e-5])
def test_dequant_product_exhaustive_nvfp4(g):
    # Every (code, scale byte) pair: fl32(fl32(E2M1 * E4M3) * G) must equal the
    # exact rational product rounded once (the inner product is exact).
    g = np.float32(g)
    codes = np.arange(16, dtype=np.uint8)
    for sb in range(256):
        packed = (codes[0::2] | (codes[1::2] << 4)).reshape(1, 8)
        scales = np.full((1, 1), sb, dtype=np.uint8)
        w = oracle.dequantize(packed, scales, 16, NV, g)[0]
        s = oracle.E4M3FN_TABLE[sb]
        for c in range(16):
            t = oracle.E2M1_TABLE[c]
            if math.isnan(s):
                assert math.isnan(w[c])
                continue
            exact = Fraction(float(t)) * Fraction(float(s)) * Fraction(float(g))
            want = _f32_of_fraction(exact)
            if exact == 0:
                assert w[c] == 0
            else:
                assert w[c] == want, (c, sb)


def test_dequant_product_exhaustive_mxfp4():
    codes = np.arange(32, dtype=np.uint8) % 16
    packed = (codes[0::2] | (codes[1::2] << 4)).reshape(1, 16).astype(np.uint8)
    for sb in range(256):
        w = oracle.dequantize(packed, np.full((1, 1), sb, dtype=np.uint8), 32, MX, 123.0)[0]
        s = oracle.E8M0_TABLE[sb]
        for c in range(16):
            t = oracle.E2M1_TABLE[c]
            if math.isnan(s):
                assert math.isnan(w[c])
                continue
            exact = Fraction(float(t)) * Fraction(2) ** (sb - 127)   # MXFP4 ignores any global scale
            if exact == 0:
                assert w[c] == 0
            elif abs(exact) > Fraction(float(np.finfo(np.float32).max)):
                assert np.isinf(w[c]) and (w[c] > 0) == (exact > 0)
            else:
                assert w[c] == _f32_of_fraction(exact), (c, sb)


def test_scale_indexing_hand_built():
    # Two rows, K = 64, NVFP4 (4 groups of 16).  Every code is 0x2 (= 1.0), and
    # the scale of group j in row r is 2^(r+j) (E4M3 bytes 0x38 + 8(r+j)).
    k = 64
    packed = np.full((2, k // 2), 0x22, dtype=np.uint8)
    scales = np.array([[0x38 + 8 * (r + j) for j in range(4)] for r in range(2)], dtype=np.uint8)
    w = oracle.dequantize(packed, scales, k, NV, 0.5)
    for r in range(2):
        for kk in range(k):
            assert w[r, kk] == 0.5 * 2.0 ** (r + kk // 16)
    # MXFP4: group 32, scale byte 127 + j.
    scales = np.array([[127 + j + r for j in range(2)] for r in range(2)], dtype=np.uint8)
    w = oracle.dequantize(packed, scales, k, MX, 99.0)
    for r in range(2):
        for kk in range(k):
            assert w[r, kk] == 2.0 ** (r + kk // 32)


def test_unit_scale_reduces_to_plain_sum():
    # All codes 1.0, unit scales, G = 1  =>  y[m, n] = sum_k x[m, k].
    rng = np.random.default_rng(5)
    x = oracle.bf16_bits_to_f32(synth.round_bf16_bits(rng.standard_normal((3, 96), dtype=np.float32)))
    packed = np.full((5, 48), 0x22, dtype=np.uint8)
    y = oracle.linear(x, packed, np.full((5, 6), 0x38, dtype=np.uint8), 96, NV, 1.0)
    want = np.array([math.fsum(map(float, row)) for row in x])
    assert np.allclose(y, want[:, None], rtol=0, atol=1e-12)
    y = oracle.linear(x, packed, np.full((5, 3), 0x7F, dtype=np.uint8), 96, MX)
    assert np.allclose(y, want[:, None], rtol=0, atol=1e-12)


def test_unit_scale_matches_integer_matrix_product():
    # Unit scales: W is a plain matrix over {+-0, .5, 1, 1.5, 2, 3, 4, 6}; compare
    # with an fp64 matmul of that matrix written out from the code table.
    rng = np.random.default_rng(6)
    k, n = 64, 7
    codes = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    mags = [0, .5, 1, 1.5, 2, 3, 4, 6]
    wmat = np.array([[(-1.0 if c & 8 else 1.0) * mags[c & 7] for c in row] for row in codes])
    x = rng.standard_normal((2, k))
    x = oracle.bf16_bits_to_f32(synth.round_bf16_bits(x.astype(np.float32)))
    y = oracle.linear(x, packed, np.full((n, k // 16), 0x38, np.uint8), k, NV, 1.0)
    assert np.allclose(y, x.astype(np.float64) @ wmat.T, rtol=1e-14, atol=1e-14)


def test_one_hot_selects_a_weight_column():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((24, 64)) * 0.02).astype(np.float32)
    packed, scales, g = oracle.quantize_nvfp4(w)
    deq = oracle.dequantize(packed, scales, 64, NV, g)
    for kk in (0, 1, 15, 16, 33, 63):
        x = np.zeros((1, 64), dtype=np.float32)
        x[0, kk] = 1.0
        y = oracle.linear(x, packed, scales, 64, NV, g)
        assert np.array_equal(y[0], deq[:, kk].astype(np.float64))


def test_linear_against_fp64_bruteforce_tiny():
    # BLAS fp64 against correctly rounded sums: |y - y_exact| <= gamma_K * sum|x w|
    # with gamma_K = K u / (1 - K u), u = 2^-53 (Higham, dot-product bound).
    rng = np.random.default_rng(8)
    for fmt, k, n, m in [(NV, 64, 9, 2), (MX, 96, 5, 3)]:
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        if fmt == NV:
            packed, scales, g = oracle.quantize_nvfp4(w)
        else:
            (packed, scales), g = oracle.quantize_mxfp4(w), 1.0
        x = oracle.bf16_bits_to_f32(synth.round_bf16_bits(rng.standard_normal((m, k)).astype(np.float32)))
        y = oracle.linear(x, packed, scales, k, fmt, g)
        ye = oracle.linear_f64_bruteforce(x, packed, scales, k, fmt, g)
        deq = oracle.dequantize(packed, scales, k, fmt, g).astype(np.float64)
        u = 2.0 ** -53
        gamma = k * u / (1 - k * u)
        bound = gamma * (np.abs(x.astype(np.float64)) @ np.abs(deq).T)
        assert np.all(np.abs(y - ye) <= bound + 1e-300)


def test_fp32_accumulation_within_bound():
    # The pages' own reference accumulates in f32; that result stays within
    # gamma_K (u = 2^-24) of the fp64 one, which the tolerance is built around.
    rng = np.random.default_rng(9)
    k, n = 256, 512
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    packed, scales, g = synth.quantize_nvfp4_block(w, oq.nvfp4_global_scale(w)) + (oq.nvfp4_global_scale(w),)
    x = oracle.bf16_bits_to_f32(synth.round_bf16_bits(rng.standard_normal((1, k)).astype(np.float32)))
    deq = oracle.dequantize(packed, scales, k, NV, g)
    y32 = (x @ deq.T).astype(np.float64)
    y64 = oracle.linear(x, packed, scales, k, NV, g)
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    bound = gamma * (np.abs(x.astype(np.float64)) @ np.abs(deq.astype(np.float64)).T)
    assert np.all(np.abs(y32 - y64) <= bound)


def test_gate_up_is_concatenation_of_halves():
    rng = np.random.default_rng(10)
    k = 64
    wg = (rng.standard_normal((6, k)) * 0.02).astype(np.float32)
    wu = (rng.standard_normal((6, k)) * 0.03).astype(np.float32)
    pg, sg_, gg = oracle.quantize_nvfp4(wg)
    pu, su, gu = oracle.quantize_nvfp4(wu)
    x = oracle.bf16_bits_to_f32(synth.round_bf16_bits(rng.standard_normal((2, k)).astype(np.float32)))
    y = oracle.gate_up(x, pg, sg_, pu, su, k, NV, gg, gu)
    assert np.array_equal(y[:, :6], oracle.linear_f64_bruteforce(x, pg, sg_, k, NV, gg))
    assert np.array_equal(y[:, 6:], oracle.linear_f64_bruteforce(x, pu, su, k, NV, gu))


def test_quantizer_round_trip_representable_nvfp4():
    # Weights built as E2M1 * S * G with each block's largest magnitude 6 * S * G
    # quantize back to the same codes and scales.
    rng = np.random.default_rng(11)
    n, k = 4, 64
    g = np.float32(2.0 ** -9)
    sbytes = rng.integers(0x30, 0x50, size=(n, k // 16)).astype(np.uint8)
    codes = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    codes[:, ::16] = 0x7       # each block holds a +6 so amax/6 = S*G exactly
    codes[codes == 0x8] = 0x0  # -0.0 would come back as +0.0 only through sign; keep it simple
    s = oracle.E4M3FN_TABLE[sbytes]
    w = (oracle.E2M1_TABLE[codes] * np.repeat(s, 16, axis=1) * g).astype(np.float32)
    packed, scales, g2 = oracle.quantize_nvfp4(w, global_scale=g)
    assert np.array_equal(scales, sbytes)
    assert np.array_equal(oracle.unpack_codes(packed, k), codes)


def test_quantizer_round_trip_representable_mxfp4():
    rng = np.random.default_rng(12)
    n, k = 3, 96
    ebytes = rng.integers(100, 140, size=(n, k // 32)).astype(np.uint8)
    codes = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    codes[codes == 0x8] = 0x0
    # floor(log2(amax/6)) = e requires amax in [6 * 2^e, 12 * 2^e): put a 6 in each block
    codes[:, ::32] = 0x7
    s = oracle.E8M0_TABLE[ebytes]
    w = (oracle.E2M1_TABLE[codes] * np.repeat(s, 32, axis=1)).astype(np.float32)
    packed, scales = oracle.quantize_mxfp4(w)
    assert np.array_equal(scales, ebytes)
    assert np.array_equal(oracle.unpack_codes(packed, k), codes)


def test_mxfp4_exponent_hand_worked():
    # floor(log2(amax / 6)): amax 6 -> 0; just below 6 -> -1; 12 -> 1;
    # 0.06 -> log2(0.01) = -6.64 -> -7; 0 -> -127 (all-zero block).
    assert oq.mxfp4_exponent(6.0) == 0
    assert oq.mxfp4_exponent(np.nextafter(np.float32(6.0), np.float32(0))) == -1
    assert oq.mxfp4_exponent(12.0) == 1
    assert oq.mxfp4_exponent(0.06) == -7
    assert oq.mxfp4_exponent(0.0) == -127
    assert oq.mxfp4_exponent(1e-45) == -127


def test_nvfp4_degenerate_blocks():
    w = np.zeros((2, 32), dtype=np.float32)
    w[1, 16:] = 0.5
    packed, scales, g = oracle.quantize_nvfp4(w)
    assert scales[0].tolist() == [0, 0] and scales[1, 0] == 0
    assert oracle.unpack_codes(packed, 32)[0].tolist() == [0] * 32
    # G = amax/2688, block scale = (0.5/6)/G = 448 exactly -> 0x7E, codes 6 * 0.5/0.5... = 0x7
    assert scales[1, 1] == 0x7E
    assert oracle.unpack_codes(packed, 32)[1, 16:].tolist() == [0x7] * 16


@pytest.mark.parametrize("fmt,n,k", [(NV, 64, 256), (MX, 48, 256), (NV, 8, 1024), (MX, 8, 512)])
def test_synth_quantizer_matches_oracle(fmt, n, k):
    w = synth.weight(synth.TINY, 7 + fmt, n, k)
    w[0, :16] *= 1e-9          # a block whose scale underflows
    w[1, 32:64] = 0.0          # an all-zero block
    w[2, 5] = -1e-30           # a tiny negative: encodes to -0
    if fmt == NV:
        g = oq.nvfp4_global_scale(w)
        p1, s1, g1 = oracle.quantize_nvfp4(w)
        p2, s2 = synth.quantize_nvfp4_block(w, g)
        assert g1 == g
    else:
        p1, s1 = oracle.quantize_mxfp4(w)
        p2, s2 = synth.quantize_mxfp4_block(w)
    assert np.array_equal(s1, s2)
    assert np.array_equal(p1, p2)


def test_synth_streaming_matches_whole_tensor():
    # Two-pass block streaming gives the same bytes as quantizing the whole tensor.
    n, k = 4096 + 40, 64
    p, s, g = synth.packed_weight(synth.TINY, 9, n, k, synth.FMT_NVFP4)
    w = synth.weight(synth.TINY, 9, n, k)
    g2 = oq.nvfp4_global_scale(w)
    p2, s2 = synth.quantize_nvfp4_block(w, g2)
    assert g == g2 and np.array_equal(p, p2) and np.array_equal(s, s2)


def test_page_byte_counts():
    # The packed lm_head is K*N/2 code bytes plus K*N/16 E4M3 bytes.
    vals = {k: v for k, v in read_golden("page_sizes.txt")}
    n, k = int(vals["lm_head_n"]), int(vals["lm_head_k"])
    assert k // 2 == int(vals["lm_head_packed_u8_cols"])
    # Shape arithmetic of the oracle's quantizer on a slice of the head's rows.
    w = synth.weight(synth.LM_HEAD, 0, 16, k)
    packed, scales, _ = oracle.quantize_nvfp4(w)
    per_row = packed.shape[1] + scales.shape[1]
    total = per_row * n
    assert total == k * n // 2 + k * n // 16
    assert round(total / 2 ** 30, 4) == float(vals["lm_head_packed_gib"])
    # The dequantized bf16 head: 2 bytes per weight.  The page prints 2.3683
    # GiB; the shape gives 2.36816..., i.e. 2.3682 to four places.
    assert abs(2 * k * n / 2 ** 30 - float(vals["lm_head_bf16_gib"])) < 2e-4
