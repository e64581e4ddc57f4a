// Repack a canonical packed FP4 weight into the prepared layout, and the
// dequantize export that tests compare bit for bit against the oracle.
//
// Canonical input ("keep the ModelOpt NVFP4 lm_head packed", vllm.cpp PR #263,
// section "Why this row matters": U8 [N, K/2] codes plus one scale byte per
// group; "native MXFP4 keep-quant", vllm.cpp PR #38, commit list: E8M0 scales
// [N, K/32]):
//   codes [n][k/2], scales [n][k/g], both row-major.
// Prepared output (one layout read by both the decode GEMV and the MFMA GEMM,
// so a weight is stored once):
//   codes  [n_pad][k_pad/2]: the same bytes, rows padded to a multiple of 256
//          and each row padded to a multiple of 1024 codes, padding zero;
//   scales [n_pad/16][k_pad/32][16][P]: for each group of 16 rows and each
//          32-code segment, the 16 rows' P scale bytes are adjacent (P = 2 for
//          NVFP4, 1 for MXFP4), so a decode lane fetches the scales of its rows
//          with one 8- or 16-byte load and a wave's loads are contiguous;
//          padding zero.
// Zero padding decodes to zero weights (code 0 is +0), so padded rows and
// columns add nothing to any sum.
#include "fp4_common.hpp"
#include "fp4_device.hpp"

namespace fp4 {
namespace {

// One thread per 16-byte chunk of the prepared codes.
__global__ __launch_bounds__(256) void prepare_codes_kernel(const uint8_t* __restrict__ in, int n, int k,
                                                            int64_t n_pad, int64_t k_pad,
                                                            uint8_t* __restrict__ out) {
  const int64_t chunks_per_row = k_pad / 32;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_pad * chunks_per_row) return;
  const int64_t row = i / chunks_per_row;
  const int64_t c = i - row * chunks_per_row;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < n && c < k / 32)
    v = *reinterpret_cast<const uint4*>(in + row * (k / 2) + c * 16);
  *reinterpret_cast<uint4*>(out + row * (k_pad / 2) + c * 16) = v;
}

// One thread per (16-row group, 32-code segment): gathers the 16 rows' P
// scale bytes of the segment (P = 2 for NVFP4, 1 for MXFP4).
template <int P>
__global__ __launch_bounds__(256) void prepare_scales_kernel(const uint8_t* __restrict__ in, int n,
                                                             int64_t kg_real, int64_t n_pad, int64_t ksegs,
                                                             uint8_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= (n_pad / kRowGroup) * ksegs) return;
  const int64_t rg = i / ksegs;
  const int64_t seg = i - rg * ksegs;
  uint32_t w[4 * P] = {};
#pragma unroll
  for (int r = 0; r < kRowGroup; ++r) {
    const int64_t row = rg * kRowGroup + r;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int64_t kg = seg * P + j;
      uint32_t b = 0;
      if (row < n && kg < kg_real) b = in[row * kg_real + kg];
      const int byte = r * P + j;
      w[byte >> 2] |= b << (8 * (byte & 3));
    }
  }
  uint4* o = reinterpret_cast<uint4*>(out + i * kRowGroup * P);
#pragma unroll
  for (int q = 0; q < P; ++q) o[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
}

// One thread per 8 consecutive weights (one 32-bit code word), decoded with
// the instruction sequences of the compute kernels:
//   NVFP4: E2M1 -> f32 (v_cvt_scalef32_pk_f32_fp4, unit scale), times the
//          E4M3 scale (v_cvt_f32_fp8), then times G: fl32(fl32(E2M1 * S) * G);
//   MXFP4: E2M1 * 2^(b-127) -> bf16 in one v_cvt_scalef32_pk_bf16_fp4 with
//          the E8M0 byte as the scale operand, widened exactly to f32.
// (The compute kernels round the NVFP4 product to bf16, which is exact: it
// has at most 6 significant bits; they apply G after the sum over k.)
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, int n, int k,
                                                      int64_t k_pad, int64_t ksegs, float gscale,
                                                      float* __restrict__ out) {
  constexpr int G = group_size(FMT);
  const int64_t words_per_row = k / 8;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(n) * words_per_row) return;
  const int64_t row = i / words_per_row;
  const int64_t wi = i - row * words_per_row;
  const uint32_t word = *reinterpret_cast<const uint32_t*>(codes + row * (k_pad / 2) + wi * 4);
  const int64_t kg = (wi * 8) / G;
  const uint32_t sb = scales[scale_offset(row, kg, ksegs, scales_per_seg(FMT))];
  f32x2_t p[4];
  if constexpr (FMT == kFmtMxfp4) {
    const float sop = e8m0_as_scale_operand(sb);
    const uint32_t b[4] = {bf16x2_bits(cvt_fp4x2_bf16<0>(word, sop)), bf16x2_bits(cvt_fp4x2_bf16<1>(word, sop)),
                           bf16x2_bits(cvt_fp4x2_bf16<2>(word, sop)), bf16x2_bits(cvt_fp4x2_bf16<3>(word, sop))};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j].x = __uint_as_float(b[j] << 16);
      p[j].y = __uint_as_float(b[j] & 0xFFFF0000u);
    }
  } else {
    const float s = e4m3_to_f32<0>(sb);
    p[0] = cvt_fp4x2_f32<0>(word, 1.0f);
    p[1] = cvt_fp4x2_f32<1>(word, 1.0f);
    p[2] = cvt_fp4x2_f32<2>(word, 1.0f);
    p[3] = cvt_fp4x2_f32<3>(word, 1.0f);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j].x = (p[j].x * s) * gscale;
      p[j].y = (p[j].y * s) * gscale;
    }
  }
  float4* o = reinterpret_cast<float4*>(out + row * k + wi * 8);
  o[0] = make_float4(p[0].x, p[0].y, p[1].x, p[1].y);
  o[1] = make_float4(p[2].x, p[2].y, p[3].x, p[3].y);
}

// Interleaved gate_up layout: prepared row R holds gate row 16 (R / 32) +
// R % 16 when R % 32 < 16, else the up row with that index, so each 32-row
// block pairs 16 gate rows with the same 16 up rows.  Per-projection row
// padding to n_pad as in the plain layout (2 n_pad prepared rows).
__device__ __forceinline__ int64_t il_source_row(int64_t R, int& h) {
  h = static_cast<int>((R >> 4) & 1);
  return (R >> 5) * 16 + (R & 15);
}

__global__ __launch_bounds__(256) void prepare_codes_il_kernel(const uint8_t* __restrict__ gate,
                                                               const uint8_t* __restrict__ up, int n, int k,
                                                               int64_t n_pad, int64_t k_pad,
                                                               uint8_t* __restrict__ out) {
  const int64_t chunks_per_row = k_pad / 32;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= 2 * n_pad * chunks_per_row) return;
  const int64_t R = i / chunks_per_row;
  const int64_t c = i - R * chunks_per_row;
  int h;
  const int64_t row = il_source_row(R, h);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < n && c < k / 32) v = *reinterpret_cast<const uint4*>((h ? up : gate) + row * (k / 2) + c * 16);
  *reinterpret_cast<uint4*>(out + R * (k_pad / 2) + c * 16) = v;
}

template <int P>
__global__ __launch_bounds__(256) void prepare_scales_il_kernel(const uint8_t* __restrict__ gate,
                                                                const uint8_t* __restrict__ up, int n,
                                                                int64_t kg_real, int64_t n_pad, int64_t ksegs,
                                                                uint8_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= (2 * n_pad / kRowGroup) * ksegs) return;
  const int64_t rg = i / ksegs;  // prepared 16-row group: all gate or all up rows
  const int64_t seg = i - rg * ksegs;
  const uint8_t* in = (rg & 1) ? up : gate;
  const int64_t row0 = (rg >> 1) * kRowGroup;
  uint32_t w[4 * P] = {};
#pragma unroll
  for (int r = 0; r < kRowGroup; ++r) {
    const int64_t row = row0 + r;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int64_t kg = seg * P + j;
      uint32_t b = 0;
      if (row < n && kg < kg_real) b = in[row * kg_real + kg];
      const int byte = r * P + j;
      w[byte >> 2] |= b << (8 * (byte & 3));
    }
  }
  uint4* o = reinterpret_cast<uint4*>(out + i * kRowGroup * P);
#pragma unroll
  for (int q = 0; q < P; ++q) o[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
}

}  // namespace

// Workgroups of a one-dimensional launch of `items` threads in groups of 256,
// or 0 when that exceeds the grid's x limit (sizes no device could hold).
inline unsigned blocks_for(int64_t items) {
  const int64_t b = (items + 255) / 256;
  return b > 0x7FFFFFFF ? 0u : static_cast<unsigned>(b);
}

hipError_t launch_prepare_interleaved(const uint8_t* gate_codes, const uint8_t* gate_scales, const uint8_t* up_codes,
                                      const uint8_t* up_scales, int n, int k, int fmt, uint8_t* prep_codes,
                                      uint8_t* prep_scales, hipStream_t stream) {
  const PreparedShape s = prepared_shape(n, k, fmt);
  const int64_t code_chunks = 2 * s.n_pad * (s.k_pad / 32);
  if (blocks_for(code_chunks) == 0 || blocks_for((2 * s.n_pad / kRowGroup) * s.ksegs) == 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prepare_codes_il_kernel, dim3(static_cast<unsigned>((code_chunks + 255) / 256)), dim3(256), 0,
                     stream, gate_codes, up_codes, n, k, s.n_pad, s.k_pad, prep_codes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items = (2 * s.n_pad / kRowGroup) * s.ksegs;
  const dim3 grid(static_cast<unsigned>((items + 255) / 256));
  const int64_t kg_real = k / group_size(fmt);
  if (fmt == kFmtNvfp4)
    hipLaunchKernelGGL(prepare_scales_il_kernel<2>, grid, dim3(256), 0, stream, gate_scales, up_scales, n, kg_real,
                       s.n_pad, s.ksegs, prep_scales);
  else
    hipLaunchKernelGGL(prepare_scales_il_kernel<1>, grid, dim3(256), 0, stream, gate_scales, up_scales, n, kg_real,
                       s.n_pad, s.ksegs, prep_scales);
  return hipGetLastError();
}

hipError_t launch_prepare(const uint8_t* codes, const uint8_t* scales, int n, int k, int fmt,
                          uint8_t* prep_codes, uint8_t* prep_scales, hipStream_t stream) {
  const PreparedShape s = prepared_shape(n, k, fmt);
  const int64_t code_chunks = s.n_pad * (s.k_pad / 32);
  if (blocks_for(code_chunks) == 0 || blocks_for((s.n_pad / kRowGroup) * s.ksegs) == 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prepare_codes_kernel, dim3(static_cast<unsigned>((code_chunks + 255) / 256)), dim3(256), 0,
                     stream, codes, n, k, s.n_pad, s.k_pad, prep_codes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items = (s.n_pad / kRowGroup) * s.ksegs;
  const dim3 grid(static_cast<unsigned>((items + 255) / 256));
  const int64_t kg_real = k / group_size(fmt);
  if (fmt == kFmtNvfp4)
    hipLaunchKernelGGL(prepare_scales_kernel<2>, grid, dim3(256), 0, stream, scales, n, kg_real, s.n_pad, s.ksegs,
                       prep_scales);
  else
    hipLaunchKernelGGL(prepare_scales_kernel<1>, grid, dim3(256), 0, stream, scales, n, kg_real, s.n_pad, s.ksegs,
                       prep_scales);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int n, int k, int fmt, float gscale,
                          float* out, hipStream_t stream) {
  const PreparedShape s = prepared_shape(n, k, fmt);
  const int64_t items = static_cast<int64_t>(n) * (k / 8);
  if (blocks_for(items) == 0) return hipErrorInvalidValue;
  const dim3 grid(blocks_for(items));
  if (fmt == kFmtNvfp4)
    hipLaunchKernelGGL(dequant_kernel<kFmtNvfp4>, grid, dim3(256), 0, stream, codes, scales, n, k, s.k_pad,
                       s.ksegs, gscale, out);
  else
    hipLaunchKernelGGL(dequant_kernel<kFmtMxfp4>, grid, dim3(256), 0, stream, codes, scales, n, k, s.k_pad,
                       s.ksegs, 1.0f, out);
  return hipGetLastError();
}

}  // namespace fp4
