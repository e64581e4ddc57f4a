// Prefill-shaped W4A16 FP4 GEMM (m > 8 activation rows) on gfx950 bf16 MFMA.
//
// At large m the layer is a dense contraction (2*m*n*k flops over n*k/2 code
// bytes), so it runs on the matrix cores: each weight fragment is decoded to
// bf16 in registers -- E2M1 * S is exact in bf16 (at most 6 significant bits)
// -- and fed to v_mfma_f32_16x16x32_bf16 with f32 accumulation; the NVFP4
// global scale multiplies in the epilogue.  (The pages run prefill on a
// dequantized bf16 GEMM: "MXFP4 decode-graph + gate_up FUSION default-ON",
// vllm.cpp PR #54, step 3: prefill untouched; here the packed weight is used
// directly at every m.)
//
// Operand layout of v_mfma_f32_16x16x32_bf16 used below: lane l supplies row
// (l % 16) of A and column (l % 16) of B, each with 8 consecutive k values
// (8 * (l / 16) .. +7); the 4 results of lane l are C[4 * (l / 16) + r][l % 16].
// Both operands use the same k assignment, so the sum over k is the same for
// any internal k order of the instruction.
#include "fp4_common.hpp"
#include "fp4_device.hpp"

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTileM = 128;
constexpr int kTileN = 128;
constexpr int kWaveTiles = 4;  // 4 x 4 MFMA tiles of 16 x 16 per wave

union Frag {
  bf16x8_t v;
  uint32_t u[4];
  uint4 q;
};

template <int FMT>
__device__ __forceinline__ void decode_b(uint32_t word, uint32_t sbyte, Frag& f) {
  if constexpr (FMT == kFmtMxfp4) {
    const float sop = e8m0_as_scale_operand(sbyte);
    f.u[0] = bf16x2_bits(cvt_fp4x2_bf16<0>(word, sop));
    f.u[1] = bf16x2_bits(cvt_fp4x2_bf16<1>(word, sop));
    f.u[2] = bf16x2_bits(cvt_fp4x2_bf16<2>(word, sop));
    f.u[3] = bf16x2_bits(cvt_fp4x2_bf16<3>(word, sop));
  } else {
    const float s = e4m3_to_f32<0>(sbyte);
    const f32x2_t p0 = cvt_fp4x2_f32<0>(word, 1.0f);
    const f32x2_t p1 = cvt_fp4x2_f32<1>(word, 1.0f);
    const f32x2_t p2 = cvt_fp4x2_f32<2>(word, 1.0f);
    const f32x2_t p3 = cvt_fp4x2_f32<3>(word, 1.0f);
    f.u[0] = f32x2_to_bf16x2_rne(p0.x * s, p0.y * s);
    f.u[1] = f32x2_to_bf16x2_rne(p1.x * s, p1.y * s);
    f.u[2] = f32x2_to_bf16x2_rne(p2.x * s, p2.y * s);
    f.u[3] = f32x2_to_bf16x2_rne(p3.x * s, p3.y * s);
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void mfma_kernel(const MfmaArgs a) {
  constexpr int G = group_size(FMT);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int lk = lane >> 4;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kTileM + (wave >> 1) * 64;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTileN + (wave & 1) * 64;
  const int64_t row_bytes = a.k_pad / 2;

  f32x4_t acc[kWaveTiles][kWaveTiles];
#pragma unroll
  for (int i = 0; i < kWaveTiles; ++i)
#pragma unroll
    for (int j = 0; j < kWaveTiles; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < a.k_pad; k0 += 32) {
    const int64_t kk = k0 + 8 * lk;
    Frag af[kWaveTiles], bf[kWaveTiles];
#pragma unroll
    for (int i = 0; i < kWaveTiles; ++i) {
      const int64_t m = m0 + 16 * i + li;
      af[i].q = make_uint4(0u, 0u, 0u, 0u);
      if (m < a.m && kk < a.k) af[i].q = *reinterpret_cast<const uint4*>(a.x + m * a.k + kk);
    }
#pragma unroll
    for (int j = 0; j < kWaveTiles; ++j) {
      const int64_t row = n0 + 16 * j + li;
      const uint32_t word = *reinterpret_cast<const uint32_t*>(a.codes + row * row_bytes + kk / 2);
      const uint32_t sb = a.scales[scale_offset(row, kk / G, a.ksegs, scales_per_seg(FMT))];
      decode_b<FMT>(word, sb, bf[j]);
    }
#pragma unroll
    for (int i = 0; i < kWaveTiles; ++i)
#pragma unroll
      for (int j = 0; j < kWaveTiles; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i].v, bf[j].v, acc[i][j], 0, 0, 0);
  }

#pragma unroll
  for (int j = 0; j < kWaveTiles; ++j) {
    const int64_t row = n0 + 16 * j + li;
    const int h = static_cast<int>(row / a.n_proj_pad);
    const int64_t lr = row - static_cast<int64_t>(h) * a.n_proj_pad;
    if (lr >= a.n_proj) continue;
    const float g = a.gscale[h];
    const int64_t col = static_cast<int64_t>(h) * a.n_proj + lr;
#pragma unroll
    for (int i = 0; i < kWaveTiles; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + 16 * i + 4 * lk + r;
        if (m < a.m) a.y[m * a.ldy + col] = f32_to_bf16_rne(acc[i][j][r] * g);
      }
    }
  }
}

}  // namespace

hipError_t launch_mfma(const MfmaArgs& a, int fmt, hipStream_t stream, dim3* grid_out, dim3* block_out) {
  const dim3 grid(static_cast<unsigned>(a.rows_total / kTileN), static_cast<unsigned>((a.m + kTileM - 1) / kTileM));
  const dim3 block(256);
  if (grid_out) *grid_out = grid;
  if (block_out) *block_out = block;
  if (fmt == kFmtNvfp4)
    hipLaunchKernelGGL(mfma_kernel<kFmtNvfp4>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(mfma_kernel<kFmtMxfp4>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace fp4
