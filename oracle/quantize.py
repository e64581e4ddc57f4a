"""Plain quantizers from fp32 weights to packed NVFP4 / MXFP4 (oracle; test infrastructure only).

The pages give the packed layout but not the quantizer; the workload recipe
fixes it, and these functions follow it step by step, one block at a time:

NVFP4 (group 16, E4M3FN block scale, FP32 global scale that multiplies):
  G = amax(W) / (448 * 6)                       float32, left to right
  s = amax(block) / 6 / G                       float32, left to right
  scale byte = E4M3FN(s)                        round to nearest even, saturate
  code = E2M1(w / (S * G))                      S = decoded scale byte, the
                                                ratio taken in float64
MXFP4 (group 32, E8M0 block scale, no global scale):
  e = floor(log2(amax(block) / 6))              clamped to [-127, 127]
  scale byte = e + 127
  code = E2M1(w / 2^e)

Codes are packed two per byte, the even element in the low nibble: byte j of a
row holds elements 2j (bits 3..0) and 2j+1 (bits 7..4).  Scales are one byte
per group, row-major [N, K/group].  This is the layout described in
"keep the ModelOpt NVFP4 lm_head packed" (vllm.cpp PR #263), section
"Why this row matters" (U8 [248320, 2560] plus one FP8 scale per 16 weights),
and in "native MXFP4 keep-quant" (vllm.cpp PR #38), commit list (E8M0 scale
[N, K/32], no global).

Readings taken where the recipe is silent:
* A block whose decoded scale is zero (all-zero block, or a scale that rounds
  to zero) gets code 0 for every element.
* A block of all zeros in MXFP4 gets e = -127 (scale byte 0) and codes 0.
* The MXFP4 exponent is the recipe's floor(log2(amax/6)) taken literally; the
  largest element of a block then lands in [6, 12) and saturates to 6.
"""

import math

import numpy as np

from .formats import E4M3FN_TABLE, e2m1_encode, e4m3fn_encode


def _pack_codes(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    assert k % 2 == 0
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def nvfp4_global_scale(w):
    """G = amax(W) / (448 * 6), evaluated in float32."""
    amax = np.float32(np.max(np.abs(np.asarray(w, dtype=np.float32))))
    return np.float32(amax / np.float32(448 * 6))


def quantize_nvfp4(w, global_scale=None):
    """Quantize fp32 weights [N, K] to NVFP4.

    Returns (packed uint8 [N, K/2], scale bytes uint8 [N, K/16], G float32).
    ``global_scale`` may be given to quantize a slice of a larger tensor with
    the tensor's own G.
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % 16:
        raise ValueError("K must be a multiple of 16")
    g = nvfp4_global_scale(w) if global_scale is None else np.float32(global_scale)
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((n, k // 16), dtype=np.uint8)
    for r in range(n):
        for b in range(k // 16):
            blk = w[r, 16 * b:16 * b + 16]
            amax_b = np.float32(np.max(np.abs(blk)))
            if g == 0:
                s = np.float32(0.0)
            else:
                s = np.float32(np.float32(amax_b / np.float32(6.0)) / g)
            sb = e4m3fn_encode(float(s))
            scales[r, b] = sb
            sg = float(E4M3FN_TABLE[sb]) * float(g)   # exact in float64
            for j in range(16):
                if sg == 0.0:
                    codes[r, 16 * b + j] = 0
                else:
                    codes[r, 16 * b + j] = e2m1_encode(float(blk[j]) / sg)
    return _pack_codes(codes), scales, g


def mxfp4_exponent(amax_block):
    """floor(log2(amax / 6)) for amax > 0, clamped to [-127, 127]; -127 for amax == 0."""
    amax_block = float(amax_block)
    if amax_block == 0.0:
        return -127
    _, e2 = math.frexp(amax_block / 6.0)    # amax/6 = f * 2^e2 with f in [0.5, 1)
    return max(-127, min(127, e2 - 1))


def quantize_mxfp4(w):
    """Quantize fp32 weights [N, K] to MXFP4: (packed uint8 [N, K/2], scale bytes uint8 [N, K/32])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((n, k // 32), dtype=np.uint8)
    for r in range(n):
        for b in range(k // 32):
            blk = w[r, 32 * b:32 * b + 32]
            amax_b = float(np.max(np.abs(blk)))
            e = mxfp4_exponent(amax_b)
            scales[r, b] = e + 127
            if amax_b == 0.0:
                continue
            for j in range(32):
                codes[r, 32 * b + j] = e2m1_encode(math.ldexp(float(blk[j]), -e))
    return _pack_codes(codes), scales
