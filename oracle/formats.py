"""Element and scale formats of NVFP4 and MXFP4, from their bit-field definitions.

Oracle code (test infrastructure only).

The pages name the formats but never print their value tables:
* "keep the ModelOpt NVFP4 lm_head packed" (vllm.cpp PR #263), section
  "Why this row matters": NVFP4 weights are packed 4-bit codes with FP8 scales.
* "re-verify 27B NVFP4 on the nvidia ModelOpt checkpoint" (vllm.cpp PR #178),
  section "Layer 3 - ModelOpt NVFP4 naming": F8 block scale + F32 global.
* "native MXFP4 keep-quant" (vllm.cpp PR #38), commit list: MXFP4 block scales
  are E8M0 (the launcher's kFE8M0fnu scale type), with no global scale.

The value of each bit pattern therefore comes from the OCP definitions:
* E2M1 (OCP Microscaling Formats (MX) v1.0, FP4 element): 1 sign bit, 2
  exponent bits with bias 1, 1 mantissa bit; exponent field 0 is subnormal
  (0 or 0.5); no inf, no NaN; largest magnitude 6.
* E4M3FN (OCP 8-bit Floating Point Specification, E4M3): 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal
  (m/8 * 2^-6); S.1111.111 is NaN; no inf; largest magnitude 448.
* E8M0 (OCP MX v1.0, scale): an unsigned 8-bit biased exponent, value
  2^(b-127); 0xFF is NaN.

Each decoder below evaluates those formulas with exact rationals and rounds
once to float32 (every finite value of the three formats is exactly a float32,
E8M0's 2^-127 as a subnormal).
"""

from fractions import Fraction
import math

import numpy as np


def _fraction_to_f32(v):
    # Every finite value of these formats has at most 4 significant bits and an
    # exponent inside float32's range, so this conversion is exact.
    f = np.float32(float(v))
    assert Fraction(float(f)) == v
    return f


def e2m1_value(code):
    """Value of a 4-bit E2M1 code (sign bit 3, exponent bits 2..1, mantissa bit 0)."""
    code = int(code)
    if not 0 <= code <= 15:
        raise ValueError("E2M1 code out of range")
    sign = -1 if (code >> 3) & 1 else 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = Fraction(m, 2)                      # subnormal: 2^(1-1) * (0 + m/2)
    else:
        mag = Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    if mag == 0:
        return np.float32(-0.0) if sign < 0 else np.float32(0.0)
    return _fraction_to_f32(sign * mag)


def e4m3fn_value(byte):
    """Value of an FP8 E4M3FN byte (bias 7, no inf, S.1111.111 = NaN)."""
    byte = int(byte)
    if not 0 <= byte <= 255:
        raise ValueError("E4M3 byte out of range")
    sign = -1 if byte & 0x80 else 1
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return np.float32(np.nan)
    if e == 0:
        mag = Fraction(m, 8) * Fraction(1, 2 ** 6)
    else:
        mag = (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    if mag == 0:
        return np.float32(-0.0) if sign < 0 else np.float32(0.0)
    return _fraction_to_f32(sign * mag)


def e8m0_value(byte):
    """Value of an E8M0 scale byte: 2^(byte-127); 0xFF is NaN."""
    byte = int(byte)
    if not 0 <= byte <= 255:
        raise ValueError("E8M0 byte out of range")
    if byte == 0xFF:
        return np.float32(np.nan)
    return _fraction_to_f32(Fraction(2) ** (byte - 127))


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float32)
E4M3FN_TABLE = np.array([e4m3fn_value(b) for b in range(256)], dtype=np.float32)
E8M0_TABLE = np.array([e8m0_value(b) for b in range(256)], dtype=np.float32)

# Positive finite magnitudes with their codes, in increasing order (both
# formats are sign-magnitude and monotonic in the magnitude bits).
_E2M1_POS = [(Fraction(float(E2M1_TABLE[c])), c) for c in range(8)]
_E4M3_POS = [(Fraction(float(E4M3FN_TABLE[b])), b) for b in range(0x7F)]
E4M3_MAX = Fraction(448)
E2M1_MAX = Fraction(6)


def _nearest_even(mag, table):
    """Round a non-negative rational to the nearest table entry.

    Ties go to the entry whose code has a zero least-significant bit (round
    half to even); magnitudes beyond the last entry saturate to it.
    """
    if mag >= table[-1][0]:
        return table[-1][1]
    for (lo, clo), (hi, chi) in zip(table, table[1:]):
        if lo <= mag <= hi:
            dlo, dhi = mag - lo, hi - mag
            if dlo < dhi:
                return clo
            if dhi < dlo:
                return chi
            return clo if clo % 2 == 0 else chi
    raise AssertionError("unreachable")


def _is_negative(x):
    return math.copysign(1.0, x) < 0


def e4m3fn_encode(x):
    """Encode a real number to E4M3FN: round to nearest, ties to even, saturate at 448.

    Reading taken: the pages only say the block scale is "rounded to FP8-E4M3";
    round-half-to-even with saturation to the largest finite value (no NaN
    from overflow) is the plain reading of rounding to a format whose largest
    value (448) the workload recipe itself uses.  The sign of the input is kept.
    """
    x = float(x)
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if _is_negative(x) else 0
    mag = Fraction(abs(x)) if not math.isinf(x) else E4M3_MAX
    return sign | _nearest_even(mag, _E4M3_POS)


def e2m1_encode(x):
    """Encode a real number to an E2M1 code: round to nearest, ties to even code, saturate at 6.

    The sign bit follows the sign of the input, so a small negative number
    encodes to 0x8 (negative zero).
    """
    x = float(x)
    if math.isnan(x):
        raise ValueError("E2M1 has no NaN")
    sign = 0x8 if _is_negative(x) else 0
    mag = Fraction(abs(x)) if not math.isinf(x) else E2M1_MAX
    return sign | _nearest_even(mag, _E2M1_POS)
