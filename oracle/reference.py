"""Reference dequantization and W4A16 linear (oracle; test infrastructure only).

What the method computes ("native MXFP4 keep-quant", vllm.cpp PR #38, commit
list: the device W4A16 GEMM is checked against an independent CPU dequant to
f32 followed by an f32 matmul; "keep the ModelOpt NVFP4 lm_head packed",
vllm.cpp PR #263, section "Why this row matters": the packed weight is
consumed directly by a W4A16 GEMM):

  w[n, k] = fl32( fl32( E2M1(code[n, k]) * S(n, k // g) ) * G )
  y[m, n] = sum_k x[m, k] * w[n, k]

with code[n, k] the nibble (k & 1) of byte W[n, k >> 1] (low nibble first),
S the decoded block scale (E4M3FN for NVFP4, g = 16; E8M0 for MXFP4, g = 32),
G the float32 global scale for NVFP4 (a multiplier, as in "re-verify 27B NVFP4
on the nvidia ModelOpt checkpoint", vllm.cpp PR #178, section "Layer 3 -
ModelOpt NVFP4 naming") and 1 for MXFP4 (no global scale, "native MXFP4
keep-quant", commit list).  x is bf16, widened exactly to float.

Readings taken where the pages are silent:
* The multiplication order is (E2M1 * S) * G: the first product is exact, the
  second rounds once to float32.
* The sum over k is taken in float64 here (each product of two float32 values
  is exact in float64); the GPU result is compared against it with the
  tolerance |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref).
* The fused gate_up output is [gate(x) | up(x)] along the output dimension
  ("MXFP4 decode-graph + gate_up FUSION default-ON", vllm.cpp PR #54, step 2),
  each half with its own global scale for NVFP4.
"""

import math

import numpy as np

from .formats import E2M1_TABLE, E4M3FN_TABLE, E8M0_TABLE

FMT_NVFP4 = 0
FMT_MXFP4 = 1
GROUP = {FMT_NVFP4: 16, FMT_MXFP4: 32}


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32: the bf16 bits are the top half."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x):
    """Round float32 to bf16 (round to nearest, ties to even), returning uint16 bits.

    bf16 keeps float32's sign and exponent and the top 7 mantissa bits; the
    dropped 16 bits decide the rounding.  NaN stays a (quiet) NaN.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    upper = u >> np.uint64(16)
    lower = u & np.uint64(0xFFFF)
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & np.uint64(1)) == 1))
    out = upper + round_up.astype(np.uint64)
    nan = np.isnan(x)
    out = np.where(nan, (upper | np.uint64(0x40)), out)
    return out.astype(np.uint16)


def unpack_codes(packed, k):
    """Packed bytes [N, K/2] -> codes [N, K]; element 2j is the low nibble of byte j."""
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    codes = np.empty((n, k), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    return codes


def _scale_values(scales, fmt):
    table = E4M3FN_TABLE if fmt == FMT_NVFP4 else E8M0_TABLE
    return table[np.asarray(scales, dtype=np.uint8)]


def dequantize(packed, scales, k, fmt, global_scale=1.0):
    """Dequantized float32 weights [N, K]: fl32(fl32(E2M1 * S) * G)."""
    if fmt not in GROUP:
        raise ValueError("unknown format")
    g = GROUP[fmt]
    codes = unpack_codes(packed, k)
    elem = E2M1_TABLE[codes]                                    # float32
    s = np.repeat(_scale_values(scales, fmt), g, axis=1)[:, :k]  # scale of element k is S[k // g]
    gs = np.float32(global_scale) if fmt == FMT_NVFP4 else np.float32(1.0)
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        prod = (elem * s).astype(np.float32)
        return (prod * gs).astype(np.float32)


def linear(x, packed, scales, k, fmt, global_scale=1.0):
    """y = x @ w.T with x float32 [M, K] (bf16 values), w from ``dequantize``; float64 result."""
    x = np.asarray(x, dtype=np.float32)
    w = dequantize(packed, scales, k, fmt, global_scale)
    return x.astype(np.float64) @ w.astype(np.float64).T


def linear_rows(x, packed, scales, k, fmt, global_scale, rows):
    """y[:, rows] only: dequantizes just the selected output rows of W (for sampled checks)."""
    rows = np.asarray(rows, dtype=np.int64)
    return linear(x, np.asarray(packed)[rows], np.asarray(scales)[rows], k, fmt, global_scale)


def gate_up(x, packed_gate, scales_gate, packed_up, scales_up, k, fmt,
            global_gate=1.0, global_up=1.0):
    """Fused gate_up reference: [linear(x, gate) | linear(x, up)] along the output axis."""
    yg = linear(x, packed_gate, scales_gate, k, fmt, global_gate)
    yu = linear(x, packed_up, scales_up, k, fmt, global_up)
    return np.concatenate([yg, yu], axis=1)


def linear_f64_bruteforce(x, packed, scales, k, fmt, global_scale=1.0):
    """Sequential, correctly rounded dot products (math.fsum of exact products); tiny inputs only."""
    x = np.asarray(x, dtype=np.float32)
    w = dequantize(packed, scales, k, fmt, global_scale)
    m, n = x.shape[0], w.shape[0]
    y = np.zeros((m, n), dtype=np.float64)
    for i in range(m):
        for j in range(n):
            y[i, j] = math.fsum(float(x[i, t]) * float(w[j, t]) for t in range(k))
    return y


def greedy_argmax(logits):
    """Greedy token per row: the index of the row's largest value, the lowest
    such index when several are equal.

    The lowest-index rule for exact ties is the one the reference engine's
    sampler applies ("re-verify 27B NVFP4 on the nvidia ModelOpt checkpoint",
    vllm.cpp PR #178, section on the 35B correctness result: at the divergence
    position two logits were the same float and the lower token id won).
    Values compare as numbers (-0 equals +0); a NaN counts as larger than every
    number, so the first NaN of a row wins.  A plain loop over each row.
    """
    a = np.asarray(logits, dtype=np.float64)
    if a.ndim == 1:
        a = a[None, :]
    out = np.empty(a.shape[0], dtype=np.int64)
    for i in range(a.shape[0]):
        best = 0
        for j in range(1, a.shape[1]):
            v, b = a[i, j], a[i, best]
            if math.isnan(b):
                break
            if math.isnan(v) or v > b:
                best = j
        out[i] = best
    return out


def moe_decode(x, experts, k, fmt, expert_offsets, pair_tokens):
    """Grouped MoE W4A16 reference: for every routed (token, expert) pair p,
    y[p] = linear(x[pair_tokens[p]], W_e) with e the expert whose range
    [expert_offsets[e], expert_offsets[e + 1]) holds p.

    The grouped route computes, per expert, the same W4A16 product as the
    dense layer ("MXFP4 decode-graph + gate_up FUSION default-ON", vllm.cpp
    PR #54, the later commit on the dense-template marlin port: the dense
    projections had run as the single-expert case of the grouped MoE route).
    experts: list of (packed, scales, global_scale) per expert.  Plain loops.
    """
    x = np.asarray(x, dtype=np.float32)
    offsets = [int(v) for v in expert_offsets]
    tokens = [int(v) for v in pair_tokens]
    n = np.asarray(experts[0][0]).shape[0]
    y = np.zeros((len(tokens), n), dtype=np.float64)
    for e, (packed, scales, g) in enumerate(experts):
        for p in range(offsets[e], offsets[e + 1]):
            y[p] = linear(x[tokens[p]:tokens[p] + 1], packed, scales, k, fmt, g)[0]
    return y


def silu(v):
    """silu(v) = v / (1 + e^-v) = v * sigmoid(v), float64."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def gate_up_swiglu(x, packed_gate, scales_gate, packed_up, scales_up, k, fmt, global_gate=1.0, global_up=1.0):
    """The MLP step after the fused gate_up: silu(x W_gate^T) * (x W_up^T), with
    each product the layer's exact result (float64 sums).

    Reading taken: the pages feed the fused gate_up into the MLP of the model
    family they run ("MXFP4 decode-graph + gate_up FUSION default-ON",
    vllm.cpp PR #54, step 2) without naming its activation; the gated silu
    MLP of that family is used.
    """
    g = linear(x, packed_gate, scales_gate, k, fmt, global_gate)
    u = linear(x, packed_up, scales_up, k, fmt, global_up)
    return silu(g) * u


# --- W4A4 variant: MXFP4 activations against MXFP4 weights ------------------
#
# The pages describe a second numerics contract next to the weight-only one:
# the compressed-tensors MXFP4 scheme with its activations also quantized
# (W4A4), run by a GEMM that takes both operands as 4-bit codes with
# block-32 E8M0 scales ("native MXFP4 keep-quant", vllm.cpp PR #38, commit
# list: the W0 vehicle's scheme and the W1 kernel, block 32 with non-NVFP4
# scales).  The pages keep it off the default path; here it is a separate,
# opt-in entry point.
#
# Readings taken where the pages are silent (they name the scheme, not its
# activation quantizer):
# * Activations are quantized per row, per block of 32 consecutive k, at call
#   time, by the OCP MX v1.0 conversion: shared scale X = 2^e with
#   e = floor(log2(amax)) - 2 (2 = the largest exponent of E2M1), clamped to
#   at least -127; amax = 0 gives e = -127.  Elements become E2M1(x / X):
#   nearest magnitude, ties to the even code, saturating at 6; the sign bit
#   follows the input, so a small negative value becomes code 0x8.
# * A block holding an Inf or NaN gets scale byte 0xFF (E8M0 NaN) and codes 0.
# * The product is the exact sum of (E2M1 * X)(x) * w over k, w the MXFP4
#   weight as the weight-only oracle dequantizes it (float64 here).

# E2M1 magnitudes by code 0..7 (sign-magnitude, increasing).
_E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_nearest_even(v):
    """E2M1 codes of float64 values: nearest magnitude, ties to the even code,
    saturating at 6, sign bit from the input's sign bit.  Vectorized form of
    ``e2m1_encode`` (the two are checked against each other)."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.abs(v)
    lo = np.clip(np.searchsorted(_E2M1_MAGS, mag, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    d_lo = mag - _E2M1_MAGS[lo]
    d_hi = _E2M1_MAGS[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 3)


def quantize_act_mxfp4(x):
    """Dynamic MXFP4 quantization of activation rows.

    x: float32 [M, K] holding bf16 values, K a multiple of 32.  Returns
    (codes uint8 [M, K], one E2M1 code per element; scales uint8 [M, K/32],
    E8M0 bytes), block by block as the readings above state.
    """
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    codes = np.zeros((m, k), dtype=np.uint8)
    scales = np.zeros((m, k // 32), dtype=np.uint8)
    for b in range(k // 32):
        blk = x[:, 32 * b:32 * b + 32].astype(np.float64)
        finite = np.all(np.isfinite(blk), axis=1)
        amax = np.max(np.abs(np.where(np.isfinite(blk), blk, 0.0)), axis=1)
        _, ex = np.frexp(amax)                        # amax = f 2^ex, f in [0.5, 1)
        e = np.where(amax > 0, ex - 1 - 2, -127)      # floor(log2 amax) - 2
        e = np.maximum(e, -127)
        scales[:, b] = np.where(finite, e + 127, 0xFF).astype(np.uint8)
        v = np.ldexp(blk, -e[:, None])                # exact: a power-of-two scaling
        c = e2m1_nearest_even(np.where(finite[:, None], v, 0.0))
        codes[:, 32 * b:32 * b + 32] = np.where(finite[:, None], c, 0)
    return codes, scales


def dequantize_act_mxfp4(codes, scales):
    """float64 [M, K]: E2M1(code) * 2^(scale byte - 127); NaN where the byte is 0xFF."""
    codes = np.asarray(codes, dtype=np.uint8)
    sv = E8M0_TABLE[np.asarray(scales, dtype=np.uint8)].astype(np.float64)
    return E2M1_TABLE[codes].astype(np.float64) * np.repeat(sv, 32, axis=1)


def w4a4_linear(x, packed, scales, k):
    """W4A4 MXFP4 product: y = Q(x) @ w.T in float64, Q = ``quantize_act_mxfp4``
    and w the MXFP4 weight [N, K] (``dequantize``, group 32, no global scale)."""
    xc, xs = quantize_act_mxfp4(x)
    xq = dequantize_act_mxfp4(xc, xs)
    w = dequantize(packed, scales, k, FMT_MXFP4).astype(np.float64)
    return xq @ w.T


# --- W4A4 variant: NVFP4 activations against NVFP4 weights ------------------
#
# The pages' other W4A4 arm is ModelOpt's: an NVFP4 checkpoint carries a
# per-tensor activation scale (input_scale); consuming it sets the GEMM's
# alpha (0.0078125 on the pages' checkpoint) and routes the layer to a GEMM
# over 4-bit activations instead of the weight-only one ("keep the ModelOpt
# NVFP4 lm_head packed", vllm.cpp PR #263, section "Round-1 findings
# resolved", item 1; "re-verify 27B NVFP4 on the nvidia ModelOpt checkpoint",
# vllm.cpp PR #178, section "W4A16 is the default for ModelOpt").  The pages
# keep it behind an opt-in switch for A/B runs; here it is a separate, opt-in
# entry point.
#
# Readings taken where the pages are silent (they name the scale and alpha,
# not the activation quantizer):
# * The activations are quantized per row, per block of 16 consecutive k, by
#   the same two-level NVFP4 rule as the weights, with G_x = input_scale (a
#   float32 per-tensor scale that multiplies, like the weights' G):
#     s = fl32(fl32(amax / 6) / G_x)        amax = max |x| over the block
#     S = E4M3FN(s)                          nearest, ties to even, saturating at 448
#     q = fl32(S * G_x)
#     code = E2M1(fl32(x / q))               nearest, ties to the even code,
#                                            saturating at 6, sign bit of x
#   every step in float32 (each division and product correctly rounded), so
#   each decision is taken on the float32 value.  A block with q == 0 gets
#   code 0 (sign kept) for every element.
# * A block holding an Inf or NaN gets scale byte 0x7F (E4M3FN NaN) and codes
#   0 (sign kept), so its products are NaN.
# * alpha = fl32(G_x * G_w) multiplies the sum, as G_w alone does in the
#   weight-only product: y = alpha * sum_k (E2M1(cx) S_x)(E2M1(cw) S_w),
#   the sum exact (float64 here).

# Positive finite E4M3FN magnitudes, increasing (bytes 0x00..0x7E).
_E4M3_MAGS = E4M3FN_TABLE[:0x7F].astype(np.float64)


def e4m3fn_nearest_even(v):
    """E4M3FN bytes of non-negative float64 values: nearest magnitude, ties to
    the even byte, saturating at 448 (+Inf included).  Vectorized form of
    ``e4m3fn_encode`` for non-negative inputs (the two are checked against
    each other)."""
    mag = np.asarray(v, dtype=np.float64)
    lo = np.clip(np.searchsorted(_E4M3_MAGS, mag, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = mag - _E4M3_MAGS[lo]
    d_hi = _E4M3_MAGS[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(take_hi, hi, lo).astype(np.uint8)


def quantize_act_nvfp4(x, input_scale):
    """NVFP4 quantization of activation rows with a per-tensor scale.

    x: float32 [M, K] holding bf16 values, K a multiple of 16; input_scale:
    the float32 G_x.  Returns (codes uint8 [M, K], one E2M1 code per element;
    scales uint8 [M, K/16], E4M3FN bytes), block by block as the readings
    above state.
    """
    x = np.asarray(x, dtype=np.float32)
    gx = np.float32(input_scale)
    m, k = x.shape
    if k % 16:
        raise ValueError("K must be a multiple of 16")
    codes = np.zeros((m, k), dtype=np.uint8)
    scales = np.zeros((m, k // 16), dtype=np.uint8)
    sign = (np.signbit(x).astype(np.uint8) << 3)
    with np.errstate(over="ignore", under="ignore", divide="ignore", invalid="ignore"):
        for b in range(k // 16):
            blk = x[:, 16 * b:16 * b + 16]
            finite = np.all(np.isfinite(blk), axis=1)
            amax = np.max(np.abs(np.where(np.isfinite(blk), blk, np.float32(0))), axis=1).astype(np.float32)
            s = ((amax / np.float32(6)).astype(np.float32) / gx).astype(np.float32)
            sb = e4m3fn_nearest_even(s.astype(np.float64))
            q = (E4M3FN_TABLE[sb] * gx).astype(np.float32)
            r = (blk / q[:, None]).astype(np.float32)
            c = e2m1_nearest_even(np.where((q > 0)[:, None], r, np.float32(0)).astype(np.float64)) & 0x7
            c = np.where((finite & (q > 0))[:, None], c, 0).astype(np.uint8)
            codes[:, 16 * b:16 * b + 16] = c | sign[:, 16 * b:16 * b + 16]
            scales[:, b] = np.where(finite, sb, 0x7F)
    return codes, scales


def dequantize_act_nvfp4(codes, scales):
    """float64 [M, K]: E2M1(code) * S, S the E4M3FN block scale (NaN for byte 0x7F / 0xFF), no G_x."""
    codes = np.asarray(codes, dtype=np.uint8)
    sv = E4M3FN_TABLE[np.asarray(scales, dtype=np.uint8)].astype(np.float64)
    return E2M1_TABLE[codes].astype(np.float64) * np.repeat(sv, 16, axis=1)


def w4a4_nvfp4_linear(x, packed, scales, k, global_scale, input_scale):
    """W4A4 NVFP4 product: alpha * (Q(x) @ w.T) in float64, Q = ``quantize_act_nvfp4``
    without G_x, w the NVFP4 weight [N, K] without G_w, alpha = fl32(G_x * G_w)."""
    xc, xs = quantize_act_nvfp4(x, input_scale)
    xq = dequantize_act_nvfp4(xc, xs)
    w = dequantize(packed, scales, k, FMT_NVFP4, 1.0).astype(np.float64)
    alpha = float(np.float32(np.float32(input_scale) * np.float32(global_scale)))
    with np.errstate(invalid="ignore", over="ignore"):
        return (xq @ w.T) * alpha
