"""Pins for the oracle's format decoders and encoders (CPU only).

Each decoder is checked against values written out by hand from the OCP
specifications (tests/golden) and, exhaustively, against torch's own float8
conversions, an implementation that shares nothing with the oracle.
"""

import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats
from conftest import read_golden


def _same(a, b):
    a, b = float(a), float(b)
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


def test_e2m1_table_matches_hand_values():
    rows = read_golden("e2m1_values.txt")
    assert len(rows) == 16
    for code, value in rows:
        assert _same(oracle.E2M1_TABLE[int(code, 16)], float(value)), code


@pytest.mark.parametrize("name,table", [("e4m3fn_points.txt", "E4M3FN_TABLE"),
                                        ("e8m0_points.txt", "E8M0_TABLE")])
def test_scale_tables_match_hand_values(name, table):
    tab = getattr(oracle, table)
    for byte, value in read_golden(name):
        assert _same(tab[int(byte, 16)], float(value)), (name, byte)


def test_e4m3fn_exhaustive_against_torch():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for b in range(256):
        assert _same(oracle.E4M3FN_TABLE[b], ref[b]), hex(b)


def test_e8m0_exhaustive_against_torch():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).float().numpy()
    for b in range(256):
        assert _same(oracle.E8M0_TABLE[b], ref[b]), hex(b)


def test_e2m1_against_torch_fp4_definition():
    # torch ships the packed fp4 dtype without a cast, so build the values from
    # float8_e4m3fn: E2M1 code (s, e1 e0, m) is the E4M3 byte (s, 0 e1 e0 ?, m 0 0)
    # rebased by the bias difference 7 - 1 = 6 for normals.  Subnormal codes
    # 0x1 / 0x9 are 0.5 and the zeros are +-0.
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0:
            expect = (-1) ** s * 0.5 * m
            if m == 0:
                expect = -0.0 if s else 0.0
        else:
            byte = (s << 7) | ((e + 6) << 3) | (m << 2)
            expect = float(torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).float())
        assert _same(oracle.E2M1_TABLE[c], expect), c


def test_e4m3_encode_matches_torch_in_range():
    rng = random.Random(1)
    vals = [0.0, 2.0 ** -10, 1.5 * 2 ** -9, 2.5 * 2 ** -9, 3.5 * 2 ** -9, 449.0, 464.0, 463.99,
            0.96875, 1.0625, 1.1875, 240.0, 248.0, 2.0 ** -6, 0.0146484375]
    vals += [rng.uniform(0, 464) for _ in range(300)]
    vals += [2.0 ** rng.uniform(-12, 8) for _ in range(600)]
    x = torch.tensor(vals, dtype=torch.float32)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v, r, f in zip(vals, ref, x.numpy()):
        assert formats.e4m3fn_encode(float(f)) == r, v


def test_e4m3_encode_saturates():
    # Reading taken: overflow saturates to the largest finite value.
    for v in (464.0, 465.0, 480.0, 1e6, float("inf")):
        assert formats.e4m3fn_encode(v) == 0x7E
        assert formats.e4m3fn_encode(-v) == 0xFE
    assert formats.e4m3fn_encode(float("nan")) == 0x7F


def test_e2m1_encode_midpoints_go_to_even_code():
    # Nearest-even rounding between the magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
    cases = {0.25: 0x0, 0.75: 0x2, 1.25: 0x2, 1.75: 0x4, 2.5: 0x4, 3.5: 0x6, 5.0: 0x6,
             0.2499: 0x0, 0.2501: 0x1, 5.0001: 0x7, 6.0: 0x7, 7.0: 0x7, 100.0: 0x7,
             -0.0: 0x8, -0.1: 0x8, -0.3: 0x9, -6.0: 0xF, -1e9: 0xF}
    for v, c in cases.items():
        assert formats.e2m1_encode(v) == c, v


def test_e2m1_encode_is_nearest_by_brute_force():
    rng = random.Random(2)
    for _ in range(2000):
        v = rng.uniform(-7, 7)
        c = formats.e2m1_encode(v)
        got = Fraction(float(oracle.E2M1_TABLE[c]))
        best = min(abs(Fraction(v) - Fraction(float(oracle.E2M1_TABLE[d]))) for d in range(16))
        if abs(v) <= 6:
            assert abs(Fraction(v) - got) == best, v


def test_e4m3_encode_is_nearest_by_brute_force():
    rng = random.Random(3)
    finite = [Fraction(float(oracle.E4M3FN_TABLE[b])) for b in range(0x7F)]
    for _ in range(500):
        v = 2.0 ** rng.uniform(-11, 9)
        b = formats.e4m3fn_encode(v)
        if v <= 448:
            best = min(abs(Fraction(v) - f) for f in finite)
            assert abs(Fraction(v) - Fraction(float(oracle.E4M3FN_TABLE[b]))) == best, v


def test_encoders_round_trip_every_value():
    for c in range(16):
        v = float(oracle.E2M1_TABLE[c])
        assert formats.e2m1_encode(v) == c
    for b in range(256):
        v = float(oracle.E4M3FN_TABLE[b])
        if not math.isnan(v):
            assert formats.e4m3fn_encode(v) == b


def test_bf16_rounding_against_torch():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.3895314e38,
                                  1e-40, -0.0], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(x), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_bits_to_f32(ref).view(np.uint32), back.view(np.uint32))


def test_synth_bf16_rounding_against_torch():
    import synth
    rng = np.random.default_rng(14)
    x = rng.standard_normal(50000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.round_bf16_bits(x), ref)
