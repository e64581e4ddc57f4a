"""Bit-exact parity of every W4A16 kernel on inputs whose sums are exact.

With activations that are small integers (|x| <= 3, exact in bf16), block
scales that are powers of two (2^-2 .. 2^2) and a power-of-two NVFP4 global
scale, every product x * E2M1(code) * S is a multiple of 2^-3 of magnitude at
most 72, so every partial sum over k <= 9216 terms -- in whatever order and
grouping a kernel adds them -- is a multiple of 2^-3 below 2^20 and exactly
representable in float32.  Each output is then bf16(exact sum * G), one
rounding, whatever the kernel: the oracle's float64 result rounded once to
bf16 must equal the kernel's bits, on every kernel route (VALU GEMV, MFMA
decode split and unsplit on 64- and 96-row tiles, wave-split MFMA decode with idle waves and ragged
last stages, tile GEMM whole and with K-split tail tiles)."""

import numpy as np
import pytest

import fp4_weight_only_e2m1_amd as fp4
import oracle
from gpu_util import decode_kernel, u8, x_dev, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4
GS = {NV: 16, MX: 32}
# Power-of-two scale bytes: E4M3 0x28..0x48 = 2^-2..2^2; E8M0 125..129 = 2^-2..2^2.
SCALE_BYTES = {NV: np.array([0x28, 0x30, 0x38, 0x40, 0x48], np.uint8), MX: np.arange(125, 130, dtype=np.uint8)}

# (fmt, n, k, m, kernel)
CASES = [
    (NV, 300, 800, 5, 6),      # wave-split, 1 stage per wave, ragged last stage
    (MX, 1000, 800, 3, 6),
    (NV, 17, 8160, 3, 6),      # wave-split, 8 stages per wave, ragged last stage
    (MX, 2048, 544, 2, 6),     # wave-split, wave 0 without a stage
    (NV, 5120, 6144, 8, 6),    # o_proj shape
    (MX, 12288, 1056, 1, 6),   # wave-split for MXFP4 m = 1, 2 on 12288 rows
    (NV, 16384, 1056, 1, 0),   # VALU GEMV
    (MX, 640, 9216, 2, 0),     # VALU GEMV, K split
    (NV, 640, 9216, 4, 2),     # MFMA decode, K split
    (MX, 8192, 1056, 8, 2),    # MFMA decode, unsplit
    (NV, 16896, 1056, 8, 2),   # MFMA decode, 96-row tiles
    (MX, 18432, 800, 4, 2),    # MFMA decode, 96-row tiles, ragged last stage
    (NV, 300, 1056, 16, 2),    # MFMA decode, 16 x rows
    (MX, 300, 1056, 24, 2),    # MFMA decode, two activation groups
    (NV, 512, 5120, 100, 1),   # tile GEMM, K-split tail tile
    (MX, 1024, 1056, 200, 1),  # tile GEMM, ragged last K step
]


@pytest.mark.parametrize("fmt,n,k,m,kernel", CASES)
def test_exact_sums_bitwise(fmt, n, k, m, kernel):
    rng = np.random.default_rng(1000 + n + k + m)
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = SCALE_BYTES[fmt][rng.integers(0, 5, (n, k // GS[fmt]))]
    g = np.float32(2.0 ** -3) if fmt == NV else np.float32(1.0)
    x = rng.integers(-3, 4, (m, k)).astype(np.float32)
    xbits = oracle.f32_to_bf16_bits(x)
    assert np.array_equal(oracle.bf16_bits_to_f32(xbits), x)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    info = fp4.fp4_dispatch_info()
    got = y_host_bits(fp4.fp4_w4a16_linear(x_dev(xbits), pc, ps, n, float(g), fmt, info=info))
    assert info.kernel == kernel, info.as_dict()
    if m <= 32:
        assert kernel == decode_kernel(fmt, n, k, m)
    ref = oracle.linear(x, packed, scales, k, fmt, g)
    sums = ref / np.float64(g)                                    # exact: G is a power of two
    assert np.all(np.abs(sums) < 2.0 ** 20) and np.all(sums * 8 == np.round(sums * 8))
    want = oracle.f32_to_bf16_bits(ref.astype(np.float32))
    got = np.where((got & 0x7FFF) == 0, np.uint16(0), got)      # a zero sum may carry either sign
    want = np.where((want & 0x7FFF) == 0, np.uint16(0), want)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%d of %d outputs differ; first %s: got %#06x want %#06x" % (
        len(bad), got.size, tuple(bad[0]), got[tuple(bad[0])], want[tuple(bad[0])])
