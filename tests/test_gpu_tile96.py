"""The MFMA decode kernel on 96-row tiles (six waves of one 16-row block),
which unsplit calls of m = 3..8 take where 64-row tiles would give CUs
unequal workgroup counts: parity with the oracle (ragged k included), the
exhaustive code x scale table bit for bit, the SwiGLU epilogue, and bitwise
equality with the 64-row tiles of the same rows -- the tile size never
changes an output's summation order."""

import numpy as np
import pytest

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import assert_close, u8, x_dev, y_host, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4


def _linear(pc, ps, n, g, fmt, xbits, info=None):
    return fp4.fp4_w4a16_linear(x_dev(xbits), pc, ps, n, float(g), fmt, info=info)


@pytest.mark.parametrize("fmt,n,k,m", [(NV, 16896, 544, 5), (MX, 16896, 1056, 8), (MX, 18432, 320, 3),
                                       (NV, 18432, 992, 7)])
def test_tile96_matches_oracle(fmt, n, k, m):
    packed, scales, g = synth.packed_weight(synth.TINY, 90, n, k, fmt)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    info = fp4.fp4_dispatch_info()
    y = _linear(pc, ps, n, g, fmt, xbits, info)
    assert (info.kernel, info.splits, info.grid_x, info.grid_y, info.block) == (2, 1, n // 96, 1, 384), info.as_dict()
    assert fp4.fp4_workspace_bytes(m, n, k, fmt) == 0
    y_ref = oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g)
    assert_close(y_host(y), y_ref, "tile96 fmt=%d n=%d k=%d m=%d" % (fmt, n, k, m))


@pytest.mark.parametrize("fmt,k", [(NV, 1056), (MX, 2048)])
def test_tile96_equals_tile64_bitwise(fmt, k):
    # Rows 0..7 of an m = 9 call (64-row tiles) equal the m = 8 call (96-row
    # tiles) bit for bit, and the fused 2 x 8448-row launch (96-row tiles)
    # equals the two separate 8448-row launches (64-row tiles).
    nh = 8448
    pg, sg, gg = synth.packed_weight(synth.TINY, 91, nh, k, fmt)
    pu, su, gu = synth.packed_weight(synth.TINY, 92, nh, k, fmt)
    xbits = synth.activations(synth.TINY, 9, k)
    pc, ps = fp4.fp4_prepare_gate_up(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
    info = fp4.fp4_dispatch_info()
    y8 = y_host_bits(fp4.fp4_w4a16_gate_up(x_dev(xbits[:8]), pc, ps, nh, float(gg), float(gu), fmt, info=info))
    assert (info.kernel, info.grid_x, info.block) == (2, 2 * nh // 96, 384), info.as_dict()
    y9 = y_host_bits(fp4.fp4_w4a16_gate_up(x_dev(xbits), pc, ps, nh, float(gg), float(gu), fmt, info=info))
    assert (info.kernel, info.grid_x, info.block) == (2, 2 * nh // 64, 256), info.as_dict()
    assert np.array_equal(y8, y9[:8])
    for half, (p, s, g) in enumerate(((pg, sg, gg), (pu, su, gu))):
        qc, qs = fp4.fp4_prepare(u8(p), u8(s), nh, k, fmt)
        yh = y_host_bits(_linear(qc, qs, nh, g, fmt, xbits[:8], info))
        assert (info.kernel, info.grid_x, info.block) == (2, nh // 64, 256), info.as_dict()
        assert np.array_equal(y8[:, half * nh:(half + 1) * nh], yh), half
    y_ref = oracle.gate_up(oracle.bf16_bits_to_f32(xbits[:8]), pg, sg, pu, su, k, fmt, gg, gu)
    assert_close(oracle.bf16_bits_to_f32(y8).astype(np.float64), y_ref, "tile96 gate_up")


@pytest.mark.parametrize("fmt", [NV, MX])
def test_tile96_exhaustive_table(fmt):
    # Every (code, scale byte) pair, 16896 rows = 66 repeats of the 256-row
    # table (k = 32): each output of a one-hot call is one decoded weight
    # times G, bit for bit, through the 96-row tiles.
    from test_gpu_exhaustive import G_VALUES, check, expected_bits, run, table_weight
    n, k = 16896, 32
    packed, scales = table_weight(fmt, n, k)
    for g in G_VALUES[fmt][:2]:
        for cols in (list(range(8)), list(range(8, 16))):
            got = run(packed, scales, n, k, fmt, g, cols, 2, splits=False, grid_x=n // 96)
            want = expected_bits(packed[:256], scales[:256], k, fmt, g, cols)
            check(got, np.tile(want, (1, n // 256)), "tile96 table fmt=%d G=%r" % (fmt, g))


@pytest.mark.parametrize("fmt,m", [(MX, 4), (NV, 8)])
def test_tile96_swiglu(fmt, m):
    # The SwiGLU epilogue on 96-row tiles (three 32-row gate/up blocks each).
    nh, k = 8448, 1024
    pg, sg, gg = synth.packed_weight(synth.TINY, 93, nh, k, fmt)
    pu, su, gu = synth.packed_weight(synth.TINY, 94, nh, k, fmt)
    pc, ps = fp4.fp4_prepare_gate_up_interleaved(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    info = fp4.fp4_dispatch_info()
    y = fp4.fp4_w4a16_gate_up_swiglu(x_dev(xbits), pc, ps, nh, float(gg), float(gu), fmt, info=info)
    assert (info.kernel, info.grid_x, info.block) == (2, 2 * nh // 96, 384), info.as_dict()
    ref = oracle.gate_up_swiglu(oracle.bf16_bits_to_f32(xbits), pg, sg, pu, su, k, fmt, gg, gu)
    assert_close(y_host(y), ref, "tile96 swiglu fmt=%d m=%d" % (fmt, m))
