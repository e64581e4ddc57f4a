// Tile order and result stores shared by the prefill tile GEMMs (the W4A16
// GEMM in mfma_gemm.hip and the W4A4 GEMM in w4a4.hip).  Both compute
// kGemmBM x kGemmBN tiles of y with kGemmWavesM x 4 waves, wave (wm, wn)
// holding activation rows [128 wm, +128) and weight rows [64 wn, +64) as
// acc[i][j] (i: 32-row activation block, j: 32-row weight block) in the
// 32 x 32 MFMA result layout with the weights as the A operand: result e of
// lane l is weight row 8 (e / 4) + 4 (l / 32) + e % 4, activation row l % 32.
#pragma once

#include "fp4_common.hpp"
#include "fp4_device.hpp"

namespace fp4 {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// Buffer descriptor word 3 for raw (unformatted) 32-bit accesses.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kGroupM = 8;  // activation-row tiles per tile-order group

// Output column of prepared weight row `row`, or -1 for a padding row.
__device__ __forceinline__ int64_t out_col(const MfmaArgs& a, int64_t row, int& h) {
  h = static_cast<int>(row / a.n_proj_pad);
  const int64_t lr = row - static_cast<int64_t>(h) * a.n_proj_pad;
  return lr < a.n_proj ? static_cast<int64_t>(h) * a.n_proj + lr : -1;
}

// (m_tile, n_tile) of tile t.  Tiles are ordered in groups of kGroupM
// activation-row tiles, weight-tile-major inside a group, so the 64 tiles an
// XCD holds at once form an 8 x 8 block that shares 8 x tiles and 8 weight
// tiles in its L2 (x is re-read from outside the XCD once per 8 weight tiles).
__device__ __forceinline__ void tile_coords(const GemmPlan& pl, int t, int64_t& m0, int64_t& n0) {
  const int group = t / (kGroupM * pl.n_tiles);
  const int in_group = t - group * kGroupM * pl.n_tiles;
  const int rows = pl.m_tiles - group * kGroupM < kGroupM ? pl.m_tiles - group * kGroupM : kGroupM;
  const int n_tile = in_group / rows;
  const int m_tile = group * kGroupM + (in_group - n_tile * rows);
  m0 = static_cast<int64_t>(m_tile) * kGemmBM;
  n0 = static_cast<int64_t>(n_tile) * kGemmBN;
}

// Data-parallel tile `t` of workgroup `bid` < dp_tiles.  Workgroup b runs on
// XCD b % 8, so XCD x gets the ids x, x + 8, ...; it is given the contiguous
// run of tiles starting at x * q + min(x, r) (q = tiles / 8, r = tiles % 8).
__device__ __forceinline__ int dp_tile_of(const GemmPlan& pl, int bid) {
  const int xcd = bid % 8;
  const int q = pl.dp_tiles / 8;
  const int rr = pl.dp_tiles % 8;
  return xcd * q + (xcd < rr ? xcd : rr) + bid / 8;
}

// Scale by the projection's global scale and store bf16 y, four consecutive
// output columns (weight rows) of one activation row per lane and (i, j, e4).
// (The W4A16 GEMM keeps this store and the partial store below written out in
// its kernel body: formed through these helpers, its K loop's registers spill.)
__device__ __forceinline__ void store_tile_bf16(const MfmaArgs& a, int64_t m0, int64_t n0, int wave,
                                                const f32x16_t (&acc)[4][2]) {
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int lh = lane >> 5;
  const int wm = wave / 4;
  const int wn = wave % 4;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      int h;
      const int64_t col = out_col(a, n0 + wn * 64 + 32 * j + 8 * e4 + 4 * lh, h);
      if (col < 0) continue;
      const float g = a.gscale[h];
      const int64_t lr = col - static_cast<int64_t>(h) * a.n_proj;
      const bool vec = lr + 4 <= a.n_proj && ((col | a.ldy) & 3) == 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 128 + 32 * i + l32;
        if (m >= a.m) continue;
        uint16_t* dst = a.y + m * a.ldy + col;
        const float v0 = acc[i][j][4 * e4] * g, v1 = acc[i][j][4 * e4 + 1] * g;
        const float v2 = acc[i][j][4 * e4 + 2] * g, v3 = acc[i][j][4 * e4 + 3] * g;
        if (vec) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(f32x2_to_bf16x2_rne(v0, v1), f32x2_to_bf16x2_rne(v2, v3));
        } else {
          const float w[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2)
            if (lr + q2 < a.n_proj) dst[q2] = f32_to_bf16_rne(w[q2]);
        }
      }
    }
}

// Store tail unit u's fp32 partial tile [x row][weight row].  Buffer stores:
// with plain stores the compiler's register allocation of the K loop spills.
__device__ __forceinline__ void store_tile_partial(const MfmaArgs& a, int u, int wave, const f32x16_t (&acc)[4][2]) {
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int lh = lane >> 5;
  const int wm = wave / 4;
  const int wn = wave % 4;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      a.partial + static_cast<int64_t>(u) * kGemmBM * kGemmBN, 0, kGemmBM * kGemmBN * 4, kBufferRsrcWord3);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int mr = wm * 128 + 32 * i + l32;
        const int nr = wn * 64 + 32 * j + 8 * e4 + 4 * lh;
        const f32x4_t v = {acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2], acc[i][j][4 * e4 + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rsrc, (mr * kGemmBN + nr) * 4, 0, 0);
      }
}

}  // namespace fp4
