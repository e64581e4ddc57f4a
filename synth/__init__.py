"""Seeded synthetic inputs for the W4A16 FP4 linear layer.

Both the oracle-based tests and the benchmark draw their inputs from here.  The
module holds the random draws and the workload recipe that turns fp32 weights
into packed FP4 bytes; it holds no part of the dequantization or of the
contraction that the layer computes.

Recipe (the pages measure real NVFP4 / MXFP4 checkpoints, which are not
available; these draws stand in for them, at the same shapes):
* weights  W = standard_normal(float32) * 0.02, drawn in blocks of 4096 rows;
* activations x = bf16(standard_normal(float32)), rounded to nearest even;
* generator: numpy PCG64 seeded with SeedSequence([workload, tensor, block]).

Quantization to packed bytes follows the workload recipe:
* NVFP4: G = amax(W)/(448*6); block scale = amax(block)/6/G rounded to
  FP8-E4M3 (nearest even, saturated at 448); code = nearest-even E2M1 of
  w/(S*G) in float64.
* MXFP4: block scale 2^floor(log2(amax(block)/6)) stored as E8M0; code =
  nearest-even E2M1 of w/2^e.
Codes are packed two per byte, the even element in the low nibble.

The fast quantizer here uses torch's float8_e4m3fn conversion for the scale
and threshold comparisons for the codes.  The oracle holds an independent,
element-by-element implementation of the same recipe, and the tests require
the two to agree byte for byte.
"""

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

CHUNK_ROWS = 4096

# Workload identifiers used in the seeds.
TINY, GATE_UP, LM_HEAD, DECODE_27B, PREFILL = 0, 1, 2, 3, 4
FMT_NVFP4, FMT_MXFP4 = 0, 1

# E2M1 rounding boundaries on the magnitude axis.  A boundary is the midpoint
# between two neighbouring magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; at an exact
# midpoint the even code wins, so the comparison is strict ('>') where the
# lower code is even and inclusive ('>=') where the upper code is even.
_E2M1_UP = ((0.25, False), (0.75, True), (1.25, False), (1.75, True),
            (2.5, False), (3.5, True), (5.0, False))


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(workload, tensor, block):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload, tensor, block])))


def weight_block(workload, tensor, block, rows, k):
    """Rows [4096*block, 4096*block + rows) of the fp32 weight of (workload, tensor)."""
    w = _rng(workload, tensor, block).standard_normal((rows, k), dtype=np.float32)
    w *= np.float32(0.02)
    return w


def _blocks(n):
    return [(b, min(CHUNK_ROWS, n - b * CHUNK_ROWS)) for b in range((n + CHUNK_ROWS - 1) // CHUNK_ROWS)]


def weight(workload, tensor, n, k):
    """The full fp32 weight [n, k] (for small shapes)."""
    return np.concatenate([weight_block(workload, tensor, b, r, k) for b, r in _blocks(n)], axis=0)


def round_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def activations(workload, m, k):
    """bf16 activations [m, k] as uint16 bit patterns."""
    x = _rng(workload, 100 + m, 0).standard_normal((m, k), dtype=np.float32)
    return round_bf16_bits(x)


def _e2m1_codes(v):
    """Nearest-even E2M1 codes of float64 values (sign from the sign bit, saturating)."""
    mag = np.abs(v)
    code = np.zeros(v.shape, dtype=np.uint8)
    for bound, inclusive in _E2M1_UP:
        code += (mag >= bound) if inclusive else (mag > bound)
    code |= np.signbit(v).astype(np.uint8) << 3
    return code


def _pack(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _e4m3_bytes_and_values(s):
    """float32 -> (E4M3FN bytes, decoded float32), nearest even, saturated at 448."""
    import torch
    t = torch.from_numpy(np.minimum(s, np.float32(448.0)).astype(np.float32))
    f8 = t.to(torch.float8_e4m3fn)
    return f8.view(torch.uint8).numpy().copy(), f8.to(torch.float32).numpy().copy()


def quantize_nvfp4_block(w, g):
    """NVFP4-quantize fp32 rows w [r, k] with global scale g: (packed [r, k/2], scales [r, k/16])."""
    r, k = w.shape
    wb = w.reshape(r, k // 16, 16)
    amax = np.abs(wb).max(axis=2)
    g = np.float32(g)
    if g == 0:
        s = np.zeros_like(amax)
    else:
        s = (amax / np.float32(6.0)) / g
    sbytes, svals = _e4m3_bytes_and_values(s.astype(np.float32))
    sg = svals.astype(np.float64) * np.float64(g)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = wb.astype(np.float64) / sg[:, :, None]
    codes = _e2m1_codes(v)
    codes[np.broadcast_to((sg == 0)[:, :, None], codes.shape)] = 0
    return _pack(codes.reshape(r, k)), sbytes


def quantize_mxfp4_block(w):
    """MXFP4-quantize fp32 rows w [r, k]: (packed [r, k/2], scales [r, k/32])."""
    r, k = w.shape
    wb = w.reshape(r, k // 32, 32)
    amax = np.abs(wb).max(axis=2).astype(np.float64)
    _, e2 = np.frexp(amax / 6.0)
    e = np.clip(e2.astype(np.int32) - 1, -127, 127)
    e = np.where(amax == 0, -127, e)
    v = np.ldexp(wb.astype(np.float64), -e[:, :, None])
    codes = _e2m1_codes(v)
    codes[np.broadcast_to((amax == 0)[:, :, None], codes.shape)] = 0
    return _pack(codes.reshape(r, k)), (e + 127).astype(np.uint8)


def packed_weight(workload, tensor, n, k, fmt):
    """Quantized weight of (workload, tensor) at shape [n, k], streamed in 4096-row blocks.

    Returns (packed uint8 [n, k/2], scales uint8 [n, k/g], G float32 or 1.0).
    NVFP4 takes two passes (amax, then quantize) so the fp32 weight is never
    held whole.
    """
    blocks = _blocks(n)
    gsz = 16 if fmt == FMT_NVFP4 else 32
    packed = np.empty((n, k // 2), dtype=np.uint8)
    scales = np.empty((n, k // gsz), dtype=np.uint8)
    with ThreadPoolExecutor(_threads()) as pool:
        if fmt == FMT_NVFP4:
            amaxes = list(pool.map(
                lambda br: np.float32(np.abs(weight_block(workload, tensor, br[0], br[1], k)).max()),
                blocks))
            g = np.float32(np.float32(max(amaxes)) / np.float32(448 * 6))
        else:
            g = np.float32(1.0)

        def work(br):
            b, rows = br
            w = weight_block(workload, tensor, b, rows, k)
            if fmt == FMT_NVFP4:
                p, s = quantize_nvfp4_block(w, g)
            else:
                p, s = quantize_mxfp4_block(w)
            packed[b * CHUNK_ROWS:b * CHUNK_ROWS + rows] = p
            scales[b * CHUNK_ROWS:b * CHUNK_ROWS + rows] = s

        list(pool.map(work, blocks))
    return packed, scales, g
