"""Oracle for the W4A16 FP4 weight-only linear layer (test infrastructure only).

This package is a plain, slow, CPU implementation of what the FP4 weight-only
linear layer computes, written from the format definitions and from the pages
that describe the method:

* "keep the ModelOpt NVFP4 lm_head packed" (vllm.cpp PR #263), section
  "Why this row matters": the packed weight is U8 [N, K/2] plus one FP8 scale
  byte per 16 weights; the head is run as a W4A16 GEMM instead of being
  dequantized to bf16.
* "re-verify 27B NVFP4 on the nvidia ModelOpt checkpoint" (vllm.cpp PR #178),
  section "Layer 3 - ModelOpt NVFP4 naming": an NVFP4 weight is the U8 codes, an
  F8 block scale and an F32 global scale that multiplies.
* "native MXFP4 keep-quant" (vllm.cpp PR #38), commit list: MXFP4 is group 32
  with E8M0 scales of shape [N, K/32] and no global scale; the device GEMM is
  checked against an independent CPU dequant followed by an f32 matmul.
* "MXFP4 decode-graph + gate_up FUSION default-ON" (vllm.cpp PR #54), step 2:
  the fused gate_up GEMM over concatenated [gate; up] rows equals the two
  separate GEMMs.

The value tables of E2M1, E4M3FN and E8M0 are not printed on those pages; they
are taken from the OCP specifications ("OCP Microscaling Formats (MX) v1.0" for
E2M1 and E8M0, "OCP 8-bit Floating Point Specification (OFP8)" for E4M3FN).

Only the tests, the smoke entry point and the CPU-baseline leg of the
benchmark may import this package.  The product path (the HIP library and its
Python binding) never does, and the two share no code.
"""

from .formats import (
    E2M1_TABLE,
    E4M3FN_TABLE,
    E8M0_TABLE,
    e2m1_value,
    e4m3fn_value,
    e8m0_value,
    e2m1_encode,
    e4m3fn_encode,
)
from .quantize import quantize_nvfp4, quantize_mxfp4
from .reference import (
    FMT_NVFP4,
    FMT_MXFP4,
    GROUP,
    unpack_codes,
    dequantize,
    linear,
    linear_rows,
    gate_up,
    linear_f64_bruteforce,
    greedy_argmax,
    moe_decode,
    silu,
    gate_up_swiglu,
    e2m1_nearest_even,
    quantize_act_mxfp4,
    dequantize_act_mxfp4,
    w4a4_linear,
    e4m3fn_nearest_even,
    quantize_act_nvfp4,
    dequantize_act_nvfp4,
    w4a4_nvfp4_linear,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
)

__all__ = [
    "E2M1_TABLE", "E4M3FN_TABLE", "E8M0_TABLE",
    "e2m1_value", "e4m3fn_value", "e8m0_value", "e2m1_encode", "e4m3fn_encode",
    "quantize_nvfp4", "quantize_mxfp4",
    "FMT_NVFP4", "FMT_MXFP4", "GROUP",
    "unpack_codes", "dequantize", "linear", "linear_rows", "gate_up", "greedy_argmax", "moe_decode", "silu", "gate_up_swiglu",
    "e2m1_nearest_even", "quantize_act_mxfp4", "dequantize_act_mxfp4", "w4a4_linear",
    "e4m3fn_nearest_even", "quantize_act_nvfp4", "dequantize_act_nvfp4", "w4a4_nvfp4_linear",
    "linear_f64_bruteforce", "bf16_bits_to_f32", "f32_to_bf16_bits",
]
