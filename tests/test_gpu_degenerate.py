"""Degenerate scale bytes and global scales through every compute kernel
(VALU GEMV m = 1, MFMA decode m = 4, 12 and 24, tile GEMM m = 40) against the
oracle: zero, smallest, largest, negative and NaN block scales, blocks of
the largest code, and G = 0.  The oracle defines these as the formats do (a
NaN scale makes its block's weights NaN, and that output column NaN); the
kernels must give NaN in exactly those places and the layer's tolerance
elsewhere."""

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import assert_close, decode_kernel, u8, x_dev, y_host

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4


def _degenerate_weight(fmt, n, k):
    packed, scales, g = synth.packed_weight(synth.TINY, 90 + fmt, n, k, fmt)
    packed, scales = packed.copy(), scales.copy()
    if fmt == NV:
        scales[3, 2] = 0x00                 # zero scale: the block's weights are 0
        scales[5, 0] = 0xB8                 # -1.0: a negative E4M3 scale
        scales[7, 1] = 0x7E                 # 448, the largest E4M3 value ...
        packed[7, 8:16] = 0x77              # ... times code 6 in every position of the block
        scales[9, 3] = 0x7F                 # NaN
        scales[11, :] = 0x01                # 2^-9, the smallest subnormal, in every block
        scales[13, 4] = 0xFF                # -NaN
    else:
        scales[3, 0] = 0x00                 # 2^-127
        scales[5, 1] = 0xFF                 # NaN
        scales[7, 0] = 0x86                 # 2^7 ...
        packed[7, 0:16] = 0x77              # ... times code 6
        scales[9, :] = 0x7F                 # 1.0 everywhere in the row
    return packed, scales, g


def _compare(y, y_ref, what, extreme=(7,)):
    nan_ref = np.isnan(y_ref)
    assert np.array_equal(np.isnan(y), nan_ref), what
    fin = ~nan_ref.any(axis=0)              # columns without NaN
    assert np.isfinite(y[:, fin]).all(), what
    # The column of the largest scale x code is checked on its own, so its
    # magnitude does not set the rms term of the others' tolerance.
    big = np.zeros_like(fin)
    big[list(extreme)] = True
    assert_close(y[:, fin & ~big], y_ref[:, fin & ~big], what)
    assert_close(y[:, big], y_ref[:, big], what + " (largest-scale column)")


@pytest.mark.parametrize("fmt,g_mode", [(NV, "workload"), (NV, "zero"), (MX, "workload")])  # MXFP4 has no G
@pytest.mark.parametrize("m", [1, 4, 12, 24, 40])
@pytest.mark.parametrize("k", [1056, 8448])   # m <= 8: the wave-split kernel; past 32 K stages, the 64-row kernels
def test_degenerate_scales(fmt, m, g_mode, k):
    n = 300
    packed, scales, g = _degenerate_weight(fmt, n, k)
    if g_mode == "zero":
        g = np.float32(0.0)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    info = fp4.fp4_dispatch_info()
    y = y_host(fp4.fp4_w4a16_linear(x_dev(xbits), pc, ps, n, float(g), fmt, info=info))
    assert info.kernel == (decode_kernel(fmt, n, k, m) if m <= 32 else 1)
    y_ref = oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g)
    nan_rows = {NV: (9, 13), MX: (5,)}[fmt]
    assert all(np.isnan(y_ref[:, r]).all() for r in nan_rows)
    _compare(y, y_ref, "degenerate fmt=%d m=%d G=%s" % (fmt, m, g_mode))
    if g_mode == "zero":
        others = [c for c in range(n) if c not in nan_rows]
        assert (y[:, others] == 0).all()
