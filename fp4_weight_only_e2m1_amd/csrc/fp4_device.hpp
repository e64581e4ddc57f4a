// Device-side decoders for E2M1 codes and their block scales on gfx950.
//
// Formats (the pages name them but do not print their tables; the bit-level
// definitions are the OCP MX v1.0 E2M1 / E8M0 types and the OCP FP8 E4M3FN
// type):
//   E2M1 code: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
//              magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
//   NVFP4 scale: E4M3FN byte, one per 16 codes ("re-verify 27B NVFP4 on the
//              nvidia ModelOpt checkpoint", section "Layer 3 - ModelOpt NVFP4
//              naming").
//   MXFP4 scale: E8M0 byte b = 2^(b-127), one per 32 codes ("native MXFP4
//              keep-quant", commit list).
//
// gfx950 conversion instructions used here:
//   v_cvt_scalef32_pk_{bf16,f32}_fp4 turns one byte (two codes, low nibble
//   first) into two values multiplied by 2^(E - 127), where E is the biased
//   exponent field of the f32 scale operand; the operand's mantissa is not
//   used.  An E8M0 byte therefore is its scale operand exactly (its bits
//   shifted into the exponent field), while an E4M3 scale, which has a
//   mantissa, is applied with an ordinary f32 multiply.
//   v_cvt_f32_fp8 decodes an OCP E4M3FN byte to f32 exactly (NaN included).
#pragma once

#include <cstdint>
#include <hip/hip_runtime.h>

namespace fp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two codes of byte `sel` of `word` -> two bf16, scaled by 2^(E-127) of `scale`.
template <int SEL>
__device__ __forceinline__ bf16x2_t cvt_fp4x2_bf16(uint32_t word, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, SEL);
}

// Two codes of byte `sel` of `word` -> two f32, scaled by 2^(E-127) of `scale`.
template <int SEL>
__device__ __forceinline__ f32x2_t cvt_fp4x2_f32(uint32_t word, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, SEL);
}

// The f32 whose exponent field is the E8M0 byte: the scale operand that makes
// v_cvt_scalef32_pk_* multiply by 2^(b-127).
__device__ __forceinline__ float e8m0_as_scale_operand(uint32_t b) {
  return __uint_as_float((b & 0xFFu) << 23);
}

// E4M3FN byte `SEL` of `word` -> f32 (exact).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), SEL);
}

__device__ __forceinline__ uint32_t bf16x2_bits(bf16x2_t v) {
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

__device__ __forceinline__ bf16x2_t bits_bf16x2(uint32_t u) {
  bf16x2_t v;
  __builtin_memcpy(&v, &u, 4);
  return v;
}

// a.x*b.x + a.y*b.y + c, bf16 inputs, f32 accumulate (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(bf16x2_t a, uint32_t b_bits, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, bits_bf16x2(b_bits), c, false);
}

// f32 pair -> bf16 pair, round to nearest even (lowers to v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return bf16x2_bits(__builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return static_cast<uint16_t>(f32x2_to_bf16x2_rne(f, 0.0f) & 0xFFFFu);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load that bypasses cache retention (the weight stream is read once).
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace fp4
