"""GPU parity at the documented size limits: n = FP4_MAX_N weight rows,
k = FP4_MAX_K codes, m = FP4_MAX_M activation rows -- each kernel that such
a call selects, against the oracle on sampled outputs (every activation row
for the largest n and k; sampled activation rows for the largest m).

Weights at the largest n are random code bytes with scale bytes drawn from
a normal range (synth's quantizer would need the weight as float32 first:
2^24 x 32 floats); everything is seeded."""

import numpy as np
import pytest
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth
from gpu_util import DEV, assert_close, sample_rows, u8, x_dev, y_host

pytestmark = pytest.mark.gpu

NV, MX = fp4.FMT_NVFP4, fp4.FMT_MXFP4
MAX_N, MAX_K, MAX_M = 1 << 24, 1 << 20, 1 << 20


def _random_weight(seed, n, k, fmt):
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    g = 16 if fmt == NV else 32
    lo, hi = (0x28, 0x40) if fmt == NV else (0x78, 0x80)   # E4M3 2^-2 .. 2^1; E8M0 2^-7 .. 2^0
    scales = rng.integers(lo, hi, (n, k // g), dtype=np.uint8)
    return packed, scales, np.float32(0.01 if fmt == NV else 1.0)


@pytest.mark.parametrize("m,kernel", [(1, 0), (8, 2), (64, 1)])
def test_max_n(m, kernel):
    # 2^24 rows x 32 codes (prepared: k padded to 1024, 8 GiB of codes).
    n, k, fmt = MAX_N, 32, NV
    packed, scales, g = _random_weight(1, n, k, fmt)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    info = fp4.fp4_dispatch_info()
    y = fp4.fp4_w4a16_linear(x_dev(xbits), pc, ps, n, float(g), fmt, info=info)
    assert info.kernel == kernel, info.as_dict()
    rows = sample_rows(n, 1024, seed=m)
    got = y[:, torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    del y, pc, ps
    torch.cuda.empty_cache()
    ref = oracle.linear_rows(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g, rows)
    assert np.isfinite(got).all()
    assert_close(got, ref, "max n m=%d" % m)


@pytest.mark.parametrize("m,kernel", [(1, 0), (3, 2), (33, 1)])
def test_max_k(m, kernel):
    # 256 rows x 2^20 codes: the K splits reach 256 (GEMV), 128 (MFMA decode)
    # and 512 (the tile GEMM's single tail tile).
    n, k, fmt = 256, MAX_K, MX
    packed, scales, g = _random_weight(2, n, k, fmt)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    info = fp4.fp4_dispatch_info()
    y = y_host(fp4.fp4_w4a16_linear(x_dev(xbits), pc, ps, n, float(g), fmt, info=info))
    assert info.kernel == kernel and info.splits > 1, info.as_dict()
    ref = oracle.linear(oracle.bf16_bits_to_f32(xbits), packed, scales, k, fmt, g)
    assert np.isfinite(y).all()
    assert_close(y, ref, "max k m=%d" % m)


@pytest.mark.parametrize("route", ["w4a16_nvfp4", "w4a16_mxfp4", "w4a4_mxfp4", "w4a4_nvfp4"])
def test_max_m(route):
    # 2^20 activation rows x 32 codes against 300 weight rows (8192 x 2 tiles).
    m, n, k = MAX_M, 300, 32
    fmt = NV if route.endswith("nvfp4") else MX
    packed, scales, g = synth.packed_weight(synth.TINY, 3, n, k, fmt)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    xbits = synth.activations(synth.TINY, m, k)
    xd = x_dev(xbits)
    x = oracle.bf16_bits_to_f32(xbits)
    rows = sample_rows(m, 2048, seed=4)
    gx = np.float32(np.float32(np.max(np.abs(x))) / np.float32(6 * 448))
    if route.startswith("w4a16"):
        y = fp4.fp4_w4a16_linear(xd, pc, ps, n, float(g), fmt)
        ref = oracle.linear(x[rows], packed, scales, k, fmt, g)
    elif route == "w4a4_mxfp4":
        y = fp4.fp4_w4a4_linear(xd, pc, ps, n)
        ref = oracle.w4a4_linear(x[rows], packed, scales, k)
    else:
        y = fp4.fp4_w4a4_nvfp4_linear(xd, pc, ps, n, float(g), float(gx))
        ref = oracle.w4a4_nvfp4_linear(x[rows], packed, scales, k, g, gx)
    got = y[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    assert np.isfinite(got).all()
    assert_close(got, ref, "max m %s" % route)
