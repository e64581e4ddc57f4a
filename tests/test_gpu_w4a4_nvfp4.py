"""GPU parity of the NVFP4 W4A4 variant against the oracle: the activation
quantizer bit for bit (random rows at several per-tensor scales, every E4M3
scale value and every midpoint between two of them, every E2M1 midpoint at
each of those scales, degenerate blocks), the product within the layer's
tolerance on each W4A16 kernel it runs (GEMV, MFMA decode, wave-split MFMA
decode, tile GEMM with and without split tail tiles), bit for bit equal to
the weight-only product where the activations are exactly NVFP4, the fused gate_up equal to two calls, RED
checks, and sampled outputs at the prefill shape."""

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import (DEV, assert_close, prepared, sample_rows, tolerance_violations, u8, weight, x_dev, y_host,
                      y_host_bits)

pytestmark = pytest.mark.gpu

NV = fp4.FMT_NVFP4
RED_SHARE = 0.25


def _calibrated(x):
    """The per-tensor scale a calibration over x gives: amax / (6 * 448), float32."""
    return np.float32(np.float32(np.max(np.abs(x))) / np.float32(6 * 448))


def _quant(xbits, gx):
    m, k = xbits.shape
    codes, scales = fp4.fp4_quantize_act_nvfp4(x_dev(xbits), float(gx))
    torch.cuda.synchronize()
    cb = codes.cpu().numpy()
    c = np.empty((m, k), np.uint8)
    c[:, 0::2] = cb & 0x0F
    c[:, 1::2] = cb >> 4
    return c, scales.cpu().numpy()


def _check_quant(xbits, gx, what):
    got_c, got_s = _quant(xbits, gx)
    want_c, want_s = oracle.quantize_act_nvfp4(oracle.bf16_bits_to_f32(xbits), gx)
    bad = np.argwhere(got_s != want_s)
    assert not bad.size, "%s: scales differ at %s: got %s want %s" % (what, bad[:3].tolist(), got_s[tuple(bad[0])],
                                                                   want_s[tuple(bad[0])])
    bad = np.argwhere(got_c != want_c)
    assert not bad.size, "%s: codes differ at %s: got %s want %s" % (what, bad[:3].tolist(), got_c[tuple(bad[0])],
                                                                  want_c[tuple(bad[0])])


@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (17, 1056), (130, 4096), (64, 5120)])
def test_quantizer_bitwise(m, k):
    rng = np.random.default_rng(m * 13 + k)
    x = rng.standard_normal((m, k)).astype(np.float32) * np.exp2(rng.uniform(-6, 6, (m, 1))).astype(np.float32)
    xbits = oracle.f32_to_bf16_bits(x)
    xf = oracle.bf16_bits_to_f32(xbits)
    g = _calibrated(xf)
    for gx in (g, np.float32(g * 0.37), np.float32(g * 5.5), np.float32(2.0 ** -9)):
        _check_quant(xbits, gx, "m=%d k=%d gx=%r" % (m, k, gx))


def test_quantizer_every_scale_and_tie():
    # G_x = 1/64 and a block maximum of 6 t / 64 make s = t exactly (6 t / 64
    # has at most 7 significant bits, so it is a bf16 value).  t runs over
    # every positive E4M3 value, every midpoint between two of them, and the
    # bf16 neighbours of those block maxima; each block also holds every E2M1
    # midpoint and grid value times q = S / 64 (S the oracle's scale for the
    # block), so each tie of the element rounding is taken at every scale.
    gx = np.float32(1 / 64)
    vals = oracle.E4M3FN_TABLE[1:0x7F].astype(np.float64)
    mids = (np.concatenate([[0.0], vals[:-1]]) + vals) / 2
    ts = np.concatenate([vals, mids, [464.0, 512.0]])
    amax = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits((6 * ts / 64).astype(np.float32)))
    assert np.array_equal(amax.astype(np.float64), 6 * ts / 64)
    bits = oracle.f32_to_bf16_bits(amax)
    amaxes = np.concatenate([amax, oracle.bf16_bits_to_f32(bits + 1), oracle.bf16_bits_to_f32(bits - 1)])
    rows = []
    for a in amaxes:
        _, sb = oracle.quantize_act_nvfp4(np.array([[a] + [0.0] * 15], np.float32), gx)
        q = float(oracle.E4M3FN_TABLE[sb[0, 0]]) / 64
        elems = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 0.125]
        blk = [a] + [e * q * (-1 if j % 2 else 1) for j, e in enumerate(elems)]
        rows.append(blk)
    x = np.array(rows, np.float32)
    x = np.concatenate([x, -x], axis=1)                                     # k = 32: the block and its negation
    xbits = oracle.f32_to_bf16_bits(x)
    assert np.array_equal(oracle.bf16_bits_to_f32(xbits), x)               # every value is a bf16
    _check_quant(xbits, gx, "every scale and tie")


def test_quantizer_degenerate_blocks():
    rows = np.zeros((6, 64), np.float32)
    rows[0, 3] = np.inf                        # non-finite blocks: byte 0x7F, codes 0 with signs
    rows[0, 5] = -2.0
    rows[1, 20] = np.nan
    rows[1, 40] = -np.inf
    rows[2, :16] = -0.0                         # all-zero blocks, both zero signs
    rows[3, :3] = [2.0 ** -20, -(2.0 ** -21), 0.0]   # scale rounds to 0: codes 0
    rows[4, :2] = [3.0e38, -1.0]               # saturating scale, saturating code
    rows[5, 16:32] = np.linspace(-1, 1, 16)
    xbits = oracle.f32_to_bf16_bits(rows)
    for gx in (np.float32(1e-3), np.float32(1.0), np.float32(2.0 ** -30)):
        _check_quant(xbits, gx, "degenerate gx=%r" % gx)


def _weights(n, k, seed):
    return synth.packed_weight(synth.TINY, 130 + seed, n, k, NV)


# (n, k, m, kernel, tail split): one case per W4A16 kernel the product runs.
LINEAR = [
    (8192, 1024, 1, 0, False),     # VALU GEMV
    (384, 8448, 2, 0, False),      # VALU GEMV, K split in three
    (512, 2048, 1, 6, False),      # wave-split MFMA decode
    (300, 1056, 8, 6, False),      # wave-split MFMA decode, ragged n and k
    (8192, 1024, 4, 2, False),     # MFMA decode, unsplit
    (256, 17408, 4, 2, False),     # MFMA decode, K split
    (640, 2048, 24, 2, False),     # MFMA decode, two activation groups
    (1024, 1024, 200, 1, False),   # tile GEMM
    (512, 5120, 100, 1, True),     # tile GEMM, split tail tiles
    (700, 2080, 300, 1, False),    # tile GEMM, ragged
]


@pytest.mark.parametrize("n,k,m,kernel,split", LINEAR)
def test_linear_matches_oracle(n, k, m, kernel, split):
    packed, scales, gw = _weights(n, k, 0)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, NV)
    xbits = synth.activations(synth.TINY, m, k)
    x = oracle.bf16_bits_to_f32(xbits)
    gx = _calibrated(x)
    info = fp4.fp4_dispatch_info()
    y = y_host(fp4.fp4_w4a4_nvfp4_linear(x_dev(xbits), pc, ps, n, float(gw), float(gx), info=info))
    assert info.kernel == kernel, info.as_dict()
    if kernel == 1:
        assert (info.splits > 1) == split, info.as_dict()
    ref = oracle.w4a4_nvfp4_linear(x, packed, scales, k, gw, gx)
    assert np.isfinite(y).all()
    assert_close(y, ref, "w4a4 nvfp4 n=%d k=%d m=%d" % (n, k, m))
    # RED: the same comparison against the oracle with input_scale left out of
    # alpha, with the weight's global scale dropped, and against the
    # weight-only product (no activation quantization) must flag outputs.
    reds = [("input scale dropped", ref / float(np.float32(gx))),
            ("weight global scale dropped", oracle.w4a4_nvfp4_linear(x, packed, scales, k, 1.0, gx)),
            ("nibbles swapped", oracle.w4a4_nvfp4_linear(x, ((packed & 0x0F) << 4 | packed >> 4).astype(np.uint8),
                                                          scales, k, gw, gx))]
    for name, mref in reds:
        share = float(tolerance_violations(y, mref)[0].mean())
        assert share >= RED_SHARE, "comparison did not catch '%s' (%.1f%%)" % (name, 100 * share)
    # The activation quantization is visible: the weight-only product differs
    # from the W4A4 one by more than the tolerance somewhere.
    assert tolerance_violations(y, oracle.linear(x, packed, scales, k, NV, gw))[0].any()


@pytest.mark.parametrize("m", [1, 8, 100])
def test_equals_weight_only_on_nvfp4_activations(m):
    # x exactly NVFP4 at a power-of-two G_x with a power-of-two G_w: the
    # quantizer returns x / G_x, and every partial sum is the weight-only
    # call's times G_x, so the outputs are the same bits.
    n, k = 512, 2048
    rng = np.random.default_rng(m)
    w = rng.standard_normal((n, k)).astype(np.float32)
    gw = np.float32(2.0 ** -9)
    packed, scales, _ = oracle.quantize_nvfp4(w, global_scale=gw)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, NV)
    gx = 2.0 ** -7
    codes = rng.integers(0, 16, (m, k)).astype(np.uint8)
    codes[:, ::16] = 7
    sb = rng.integers(0x20, 0x60, (m, k // 16)).astype(np.uint8)
    x = (oracle.dequantize_act_nvfp4(codes, sb) * gx).astype(np.float32)
    xbits = oracle.f32_to_bf16_bits(x)
    assert np.array_equal(oracle.bf16_bits_to_f32(xbits), x)
    xd = x_dev(xbits)
    a = y_host_bits(fp4.fp4_w4a4_nvfp4_linear(xd, pc, ps, n, float(gw), gx))
    b = y_host_bits(fp4.fp4_w4a16_linear(xd, pc, ps, n, float(gw), NV))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("m", [1, 4, 64])
def test_gate_up_equals_two_calls(m):
    nh, k = 512, 2048
    pg, sg, gg = _weights(nh, k, 1)
    pu, su, gu = _weights(nh, k, 2)
    pc, ps = fp4.fp4_prepare_gate_up(u8(pg), u8(sg), u8(pu), u8(su), nh, k, NV)
    cg, cs = fp4.fp4_prepare(u8(pg), u8(sg), nh, k, NV)
    cu, cu_s = fp4.fp4_prepare(u8(pu), u8(su), nh, k, NV)
    xbits = synth.activations(synth.TINY, m, k)
    gx = _calibrated(oracle.bf16_bits_to_f32(xbits))
    xd = x_dev(xbits)
    y = y_host_bits(fp4.fp4_w4a4_nvfp4_gate_up(xd, pc, ps, nh, float(gg), float(gu), float(gx)))
    yg = y_host_bits(fp4.fp4_w4a4_nvfp4_linear(xd, cg, cs, nh, float(gg), float(gx)))
    yu = y_host_bits(fp4.fp4_w4a4_nvfp4_linear(xd, cu, cu_s, nh, float(gu), float(gx)))
    assert np.array_equal(y[:, :nh], yg) and np.array_equal(y[:, nh:], yu)


def test_nan_block_poisons_its_row_only():
    n, k, m = 256, 1024, 4
    packed, scales, gw = _weights(n, k, 3)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, NV)
    x = oracle.bf16_bits_to_f32(synth.activations(synth.TINY, m, k)).copy()
    x[2, 77] = np.inf
    xbits = oracle.f32_to_bf16_bits(x)
    y = y_host(fp4.fp4_w4a4_nvfp4_linear(x_dev(xbits), pc, ps, n, float(gw), 0.01))
    assert np.isnan(y[2]).all()
    assert np.isfinite(np.delete(y, 2, axis=0)).all()


@pytest.mark.parametrize("m", [8, 1024])
def test_prefill_shape_sampled(m):
    # The prefill workload's NVFP4 weight (17408 x 5120) with its activations
    # and their calibrated G_x, through the launch the benchmark times.
    n, k = 17408, 5120
    packed, scales, gw = weight(synth.PREFILL, 0, n, k, NV)
    pc, ps, _ = prepared(synth.PREFILL, 0, n, k, NV)
    xbits = synth.activations(synth.PREFILL, m, k)
    x = oracle.bf16_bits_to_f32(xbits)
    gx = _calibrated(x)
    y = y_host(fp4.fp4_w4a4_nvfp4_linear(x_dev(xbits), pc, ps, n, float(gw), float(gx)))
    rows = sample_rows(n, 256, seed=m)
    ref = oracle.w4a4_nvfp4_linear(x, packed[rows], scales[rows], k, gw, gx)
    assert np.isfinite(y).all()
    assert_close(y[:, rows], ref, "w4a4 nvfp4 prefill m=%d" % m)


@pytest.mark.parametrize("n,k,m", [(5120, 6144, 8), (512, 5120, 100), (300, 1056, 1)])
def test_deterministic_on_poisoned_workspace(n, k, m):
    packed, scales, gw = _weights(n, k, 4)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, NV)
    xd = x_dev(synth.activations(synth.TINY, m, k))
    need = fp4.fp4_w4a4_nvfp4_workspace_bytes(m, n, k)
    outs = []
    for fill in (0x00, 0xFF, 0x7F, 0x5A):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        outs.append(y_host_bits(fp4.fp4_w4a4_nvfp4_linear(xd, pc, ps, n, float(gw), 0.003, workspace=ws)))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
