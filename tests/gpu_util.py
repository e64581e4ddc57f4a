"""Helpers shared by the GPU tests: device transfer, the layer's tolerance,
and cached synthetic weights.  Inputs come from synth; expected values come
from the oracle; the HIP path is only ever the thing under test."""

import functools

import numpy as np
import torch

import fp4_weight_only_e2m1_amd as fp4
import oracle
import synth

DEV = torch.device("cuda:0")


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def x_dev(xbits):
    xbits = np.ascontiguousarray(xbits, dtype=np.uint16)
    return torch.from_numpy(xbits.view(np.int16)).to(DEV).view(torch.bfloat16)


def y_host_bits(y):
    torch.cuda.synchronize()
    return y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def y_host(y):
    return oracle.bf16_bits_to_f32(y_host_bits(y)).astype(np.float64)


def tolerance_violations(y, y_ref):
    """Elements outside |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref), rms over the whole call."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    bound = 2.0 ** -7 * np.abs(y_ref) + 1e-3 * rms
    return np.abs(y - y_ref) > bound, rms


def assert_close(y, y_ref, what=""):
    bad, rms = tolerance_violations(y, y_ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join("%s: got %.6g want %.6g" % (tuple(i), y[tuple(i)], y_ref[tuple(i)]) for i in idx)
        raise AssertionError("%s: %d of %d outside tolerance (rms %.4g); %s" %
                             (what, int(bad.sum()), bad.size, rms, detail))


@functools.lru_cache(maxsize=8)
def weight(workload, tensor, n, k, fmt):
    """Canonical packed weight (codes, scales, G) from synth, cached per test session."""
    return synth.packed_weight(workload, tensor, n, k, fmt)


@functools.lru_cache(maxsize=16)
def prepared(workload, tensor, n, k, fmt):
    packed, scales, g = weight(workload, tensor, n, k, fmt)
    pc, ps = fp4.fp4_prepare(u8(packed), u8(scales), n, k, fmt)
    torch.cuda.synchronize()
    return pc, ps, g


def sample_rows(n, count, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, size=min(count, n), replace=False).tolist())
    rows.update([0, 1, n - 1, n - 2] if n > 2 else range(n))
    return np.array(sorted(rows), dtype=np.int64)


def decode_kernel(fmt, n, k, m, act=False):
    """Dispatch-info kernel of a decode call (m = 1..32) on a layer of n rows
    per projection: 6, the wave-split MFMA decode, for at most 32 K stages of
    256 codes and either m <= 8 on layers of fewer than 128 64-row tiles or,
    for MXFP4, m <= 2 on fewer than 256 (never for the SwiGLU epilogue);
    else 0, the VALU GEMV, at m = 1, 2 and 2, the 64-row MFMA decode, at
    m = 3..32."""
    tiles = -(-n // 256) * 256 // 64
    small = m <= 8 and tiles < 128
    mx_rows = fmt == fp4.FMT_MXFP4 and m <= 2 and tiles < 256
    if not act and m >= 1 and -(-k // 256) <= 32 and (small or mx_rows):
        return 6
    return 0 if m < 3 else 2


def decode_splits(n, k):
    """K splits of the MFMA decode (kernel 2) on a layer of n rows per
    projection: none for at least 128 64-row tiles, else about 512 workgroups
    per projection with at least 4 stages of 256 codes per split."""
    tiles = -(-n // 256) * 256 // 64
    if tiles >= 128:
        return 1
    return max(1, min(512 // tiles, -(-k // 256) // 4))


def decode_tile_rows(n, k, m, proj):
    """Rows per workgroup of the MFMA decode (kernel 2): 128 for launches of at
    least 2048 64-row tiles, 96 (six waves) for unsplit launches whose rows are
    a multiple of 96 and whose busiest of 256 CUs holds fewer rows on 96-row
    tiles than on 64-row ones (both at m <= 8 only), else 64."""
    rows = proj * (-(-n // 256) * 256)
    if m > 8:
        return 64
    if rows // 64 >= 2048:
        return 128
    if decode_splits(n, k) == 1 and rows % 96 == 0:
        busiest64 = -(-(rows // 64) // 256) * 64
        busiest96 = -(-(rows // 96) // 256) * 96
        if busiest96 < busiest64:
            return 96
    return 64
