// NVFP4 quantization of activation rows with a per-tensor scale, for the
// NVFP4 W4A4 arm: the pages' ModelOpt checkpoints carry a per-tensor
// input_scale whose use sets the GEMM's alpha and routes the layer to a GEMM
// over 4-bit activations ("keep the ModelOpt NVFP4 lm_head packed", vllm.cpp
// PR #263, section "Round-1 findings resolved", item 1; "re-verify 27B NVFP4
// on the nvidia ModelOpt checkpoint", vllm.cpp PR #178, section "W4A16 is the
// default for ModelOpt").
//
// Quantizer (the two-level NVFP4 rule of the weights, G_x = input_scale; the
// pages name the scale, not the rule): per row and 16-element block,
//   s = fl32(fl32(amax / 6) / G_x),  S = E4M3FN(s) nearest-even, saturating at 448,
//   q = fl32(S * G_x),  code = E2M1(fl32(|x| / q)) nearest-even, saturating at 6,
// with the sign bit of x; codes are 0 (sign kept) where q == 0; a block
// holding an Inf or NaN gets scale byte 0x7F and codes 0.  Every division is
// the correctly rounded float32 one, so every decision is taken on the same
// float32 value as the definition's.
//
// gfx950's block-scaled MFMA takes E8M0 scales per 32 elements only, so the
// NVFP4 activations (E4M3 scales per 16) cannot feed it.  Instead the GEMM
// side stays the W4A16 one: the quantized activations are written back as
// bf16 x_hat = E2M1(code) * S, which is exact (at most 2 x 4 significant bits,
// magnitudes 2^-10 .. 2688), and G_x joins G_w in the scale applied after
// the sum.  The products and their float32 sum are then those of a GEMM over
// the 4-bit operands.
//
// Two lanes per (row, block), each taking 8 consecutive values (one 16-byte
// load); consecutive lanes read consecutive bytes of a row.
#include "fp4_common.hpp"

namespace fp4 {
namespace {

constexpr int kThreads = 256;

// E4M3FN value nearest to s >= 0 (ties to even), saturating at 448.
__device__ __forceinline__ float e4m3_nearest_even(float s) {
  if (s >= 448.0f) return 448.0f;            // also +Inf; 464 and above would round past 448
  if (s < 0.015625f) return rintf(s * 512.0f) * 0.001953125f;   // subnormals: multiples of 2^-9
  uint32_t b = __float_as_uint(s);
  b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;         // 3 mantissa bits, ties to even
  return __uint_as_float(b);
}

// E4M3FN byte of an E4M3FN value v >= 0.
__device__ __forceinline__ uint32_t e4m3_byte(float v) {
  if (v < 0.015625f) return static_cast<uint32_t>(v * 512.0f);
  const uint32_t b = __float_as_uint(v);
  return ((((b >> 23) & 0xFFu) - 120u) << 3) | ((b >> 20) & 7u);
}

// E2M1 magnitude of code c (0..7) as float.
__device__ __forceinline__ float e2m1_mag(uint32_t c) {
  const uint32_t e = c >> 1, mbit = c & 1u;
  return e == 0 ? 0.5f * mbit : __uint_as_float((126u + e) << 23) * (1.0f + 0.5f * mbit);
}

template <bool QDQ>
__global__ __launch_bounds__(kThreads) void act_nvfp4_kernel(const uint16_t* __restrict__ x, int64_t total,
                                                             float gx, uint16_t* __restrict__ xhat,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;   // total is even: both lanes of a pair leave together
  const int h = static_cast<int>(i & 1);
  const int64_t e0 = i * 8;                 // first element: row * k + 16 * block + 8 * h
  const uint4 v = *reinterpret_cast<const uint4*>(x + e0);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t amax = 0, nonfinite = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t b = (w[j / 2] >> (16 * (j & 1))) & 0xFFFFu;
    const uint32_t mag = b & 0x7FFFu;       // bf16 magnitudes order as integers
    amax = mag > amax ? mag : amax;
    nonfinite |= (b & 0x7F80u) == 0x7F80u;
  }
  const uint32_t oa = static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 1, 2));
  amax = oa > amax ? oa : amax;
  nonfinite |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(nonfinite), 1, 2));

  uint32_t sbyte = 0x7Fu, cword = 0;
  uint32_t out[4] = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};   // NaN block
  if (!nonfinite) {
    const float a = __uint_as_float(amax << 16);
    const float s = (a / 6.0f) / gx;
    const float sv = e4m3_nearest_even(s);
    sbyte = e4m3_byte(sv);
    const float q = sv * gx;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = (w[j / 2] >> (16 * (j & 1))) & 0xFFFFu;
      uint32_t c = 0;
      if (q > 0.0f) {
        const float r = __uint_as_float((b & 0x7FFFu) << 16) / q;
        // Nearest E2M1 magnitude: each threshold is a midpoint of the grid;
        // at a midpoint the even code wins (> keeps the lower, >= takes the upper).
        c = (r > 0.25f) + (r >= 0.75f) + (r > 1.25f) + (r >= 1.75f) + (r > 2.5f) + (r >= 3.5f) + (r > 5.0f);
      }
      const uint32_t sign = b & 0x8000u;
      cword |= (c | (sign >> 12)) << (4 * j);
      // E2M1(c) * S is exact in bf16: its float32 bits end in 16 zeros.
      const uint32_t hb = (__float_as_uint(e2m1_mag(c) * sv) >> 16) | sign;
      if (j & 1)
        out[j / 2] |= hb << 16;
      else
        out[j / 2] = hb;
    }
  }
  if constexpr (QDQ) {
    *reinterpret_cast<uint4*>(xhat + e0) = make_uint4(out[0], out[1], out[2], out[3]);
  } else {
    if (nonfinite) {
      // Codes 0 with each element's sign.
#pragma unroll
      for (int j = 0; j < 8; ++j) cword |= (((w[j / 2] >> (16 * (j & 1))) >> 12) & 8u) << (4 * j);
    }
    *reinterpret_cast<uint32_t*>(codes + e0 / 2) = cword;
    if (h == 0) scales[e0 / 16] = static_cast<uint8_t>(sbyte);
  }
}

}  // namespace

hipError_t launch_act_nvfp4(const uint16_t* x, int m, int k, float gx, uint16_t* xhat, uint8_t* codes,
                            uint8_t* scales, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(m) * k / 8;   // k % 32 == 0: an even count of lanes
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks <= 0 || blocks >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  if (xhat)
    hipLaunchKernelGGL(act_nvfp4_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, x,
                       total, gx, xhat, nullptr, nullptr);
  else
    hipLaunchKernelGGL(act_nvfp4_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, x,
                       total, gx, nullptr, codes, scales);
  return hipGetLastError();
}

}  // namespace fp4
