"""GPU parity of the wave-split MFMA decode kernel (K split over the four
waves of a 16-row workgroup, partial sums added in LDS in wave order) against
the oracle, at the edges of the shapes it serves: one stage (three waves
idle), a wave with no stage of its own, ragged last stages, a ragged last
row tile, the largest layer (124 64-row tiles) and the longest K (32 stages,
8 per wave) it takes, every m = 1..8; and bit for bit: a call equals the
same rows of a call with more rows, and the fused gate_up equals the two
separate launches, where all of them run this kernel."""

import numpy as np
import pytest

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import assert_close, sample_rows, u8, x_dev, y_host, y_host_bits

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4

# (fmt, n, k): K stages of 256 codes -> the stages each wave streams.
SHAPES = [
    (NV, 300, 256),     # 1 stage: waves 1..3 have none
    (MX, 64, 32),       # the smallest k
    (NV, 2048, 544),    # 3 stages: wave 0 has none (stage ranges 0, 0..1, 1..2, 2..3)
    (MX, 1000, 800),    # 4 stages, the last one ragged (32 of 256 codes)
    (NV, 17, 8160),     # 32 stages (8 per wave), ragged last stage; one full tile and one row
    (NV, 5120, 6144),   # o_proj
]


@pytest.mark.parametrize("fmt,n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
def test_wave_split_matches_oracle(fmt, n, k, m):
    packed, scales, g = synth.packed_weight(synth.TINY, 140, n, k, fmt)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    info = fp4.fp4_dispatch_info()
    y = y_host(fp4.fp4_w4a16_linear(x_dev(xbits), pc, ps, n, float(g), fmt, info=info))
    assert (info.kernel, info.splits, info.grid_x, info.grid_y) == (6, 1, -(-n // 256) * 256 // 16, 1), info.as_dict()
    y_ref = oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g)
    assert np.isfinite(y).all()
    assert_close(y, y_ref, "wave-split fmt=%d n=%d k=%d m=%d" % (fmt, n, k, m))


@pytest.mark.parametrize("fmt", [NV, MX])
def test_wave_split_largest_layer(fmt):
    # 7936 rows (124 64-row tiles, the most the kernel takes) x 8192 codes
    # (32 stages): sampled rows against the oracle, all of m = 1..8 on one x.
    n, k = 7936, 8192
    packed, scales, g = synth.packed_weight(synth.TINY, 141, n, k, fmt)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    x8 = synth.activations(synth.TINY, 8, k)
    rows = sample_rows(n, 256, seed=141)
    ref = oracle.linear_rows(oracle.bf16_bits_to_f32(x8), packed, scales, k, fmt, g, rows)
    y8 = None
    for m in range(8, 0, -1):
        info = fp4.fp4_dispatch_info()
        y = fp4.fp4_w4a16_linear(x_dev(x8[:m]), pc, ps, n, float(g), fmt, info=info)
        assert info.kernel == 6 and info.grid_x == n // 16, info.as_dict()
        bits = y_host_bits(y)
        if y8 is None:
            y8 = bits
            assert_close(oracle.bf16_bits_to_f32(bits)[:, rows].astype(np.float64), ref, "largest layer")
        assert np.array_equal(bits, y8[:m]), m


@pytest.mark.parametrize("fmt,nh,k,m", [(MX, 5120, 6144, 8), (NV, 300, 800, 1), (NV, 7936, 2048, 5)])
def test_wave_split_fused_gate_up_equals_split(fmt, nh, k, m):
    pg, sg, gg = synth.packed_weight(synth.TINY, 142, nh, k, fmt)
    pu, su, gu = synth.packed_weight(synth.TINY, 143, nh, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    xd = x_dev(xbits)
    pc, ps = fp4.fp4_prepare_gate_up(u8(pg), u8(sg), u8(pu), u8(su), nh, k, fmt)
    info = fp4.fp4_dispatch_info()
    y = y_host_bits(fp4.fp4_w4a16_gate_up(xd, pc, ps, nh, float(gg), float(gu), fmt, info=info))
    assert info.kernel == 6 and info.grid_x == 2 * (-(-nh // 256) * 256) // 16, info.as_dict()
    cg, cs = fp4.fp4_prepare(u8(pg), u8(sg), nh, k, fmt)
    cu, cus = fp4.fp4_prepare(u8(pu), u8(su), nh, k, fmt)
    yg = y_host_bits(fp4.fp4_w4a16_linear(xd, cg, cs, nh, float(gg), fmt))
    yu = y_host_bits(fp4.fp4_w4a16_linear(xd, cu, cus, nh, float(gu), fmt))
    assert np.array_equal(y[:, :nh], yg) and np.array_equal(y[:, nh:], yu)
