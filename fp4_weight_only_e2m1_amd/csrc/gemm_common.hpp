// Tile order and result stores shared by the prefill tile GEMMs (the W4A16
// GEMM in mfma_gemm.hip: 128 x 256 tiles, 4 waves; the W4A4 GEMM in w4a4.hip:
// 256 x 256 tiles, 8 waves).  Wave w = 4 wm + wn holds FI 32-row activation
// blocks, rows [32 FI wm, +32 FI) (FI = 4 for whole tiles), and weight rows
// [64 wn, +64) of its tile as acc[i][j] (i: activation block, j: 32-row
// weight block) in the 32 x 32 MFMA result layout with the weights as the A
// operand: result e of lane l is weight row 8 (e / 4) + 4 (l / 32) + e % 4,
// activation row l % 32.
#pragma once

#include "fp4_common.hpp"
#include "fp4_device.hpp"

namespace fp4 {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
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
template <int BM = kGemmBM>
__device__ __forceinline__ void tile_coords(const GemmPlan& pl, int t, int64_t& m0, int64_t& n0) {
  const int group = t / (kGroupM * pl.n_tiles);
  const int in_group = t - group * kGroupM * pl.n_tiles;
  const int rows = pl.m_tiles - group * kGroupM < kGroupM ? pl.m_tiles - group * kGroupM : kGroupM;
  const int n_tile = in_group / rows;
  const int m_tile = group * kGroupM + (in_group - n_tile * rows);
  m0 = static_cast<int64_t>(m_tile) * BM;
  n0 = static_cast<int64_t>(n_tile) * kGemmBN;
}

// Data-parallel tile `t` of workgroup `bid` < dp_tiles.  Workgroup b runs on
// XCD b % X (X = pl.xcds), so XCD x gets the ids x, x + X, ...; it is given
// the contiguous run of tiles starting at x * q + min(x, r) (q = tiles / X,
// r = tiles % X).
__device__ __forceinline__ int dp_tile_of(const GemmPlan& pl, int bid) {
  const int nx = pl.xcds;
  const int xcd = bid % nx;
  const int q = pl.dp_tiles / nx;
  const int rr = pl.dp_tiles % nx;
  return xcd * q + (xcd < rr ? xcd : rr) + bid / nx;
}

// Position of workgroup `bid` among the workgroups [first, end) of a launch
// when those are numbered XCD by XCD (all of XCD 0's in launch order, then
// XCD 1's, ...; workgroup b runs on XCD b % nx), so that consecutive work
// items given to consecutive positions share an XCD and its L2.  A bijection
// of [first, end) onto [0, end - first).
__device__ __forceinline__ int xcd_major_index(int bid, int first, int end, int nx) {
  const int x = bid % nx;
  int idx = 0;
  for (int x2 = 0; x2 < x; ++x2) {
    const int f = first + ((x2 - first % nx) + nx) % nx;  // first workgroup >= first on XCD x2
    if (f < end) idx += (end - f + nx - 1) / nx;
  }
  const int fx = first + ((x - first % nx) + nx) % nx;
  return idx + (bid - fx) / nx;
}

// Result stores through LDS.  In the MFMA result layout a lane holds 4
// consecutive output columns of one activation row, and the 32 lanes of a
// half-wave hold 32 different rows, so direct stores write 8-byte (bf16) or
// 16-byte (fp32) pieces a row apart.  Instead each wave first writes its
// fragments into a row-major tile in LDS (rows padded by 16 bytes, so the 32
// rows a store instruction touches start in different banks), and the
// workgroup then writes whole rows, 16 contiguous bytes per lane (measured
// on MI355X for the W4A4 GEMM at m = 1024: the direct stores cost about a
// third of the kernel's time; the W4A16 GEMM at m = 1024 likewise).  `lds` is
// the workgroup's stage memory, free
// once the K loop is done; every wave's K loop must have finished reading it
// and no copy into it may be in flight.
constexpr int kStageYRow = kGemmBN * 2 + 16;  // bytes per staged bf16 row
constexpr int kStagePRow = kGemmBN * 4 + 16;  // bytes per staged fp32 row

// bf16 y of a whole tile: BM x 256 outputs, scaled by the projection's global
// scale (a tile never spans two projections: n_proj_pad is a multiple of 256),
// staged PASS rows at a time (PASS a multiple of 32 dividing 128, or 128).
// FI: 32-row activation fragments per wave (wave w = 4 wm + wn holds tile rows
// [32 FI wm, +32 FI)).  Rows of the tile no wave holds are staged with stale
// LDS bytes; callers choose FI so that they lie at or past m and are never
// stored.
template <int BM, int THREADS, int PASS = BM, int FI = 4>
__device__ __forceinline__ void store_tile_bf16_staged(const MfmaArgs& a, int64_t m0, int64_t n0, int wave,
                                                       const f32x16_t (&acc)[FI][2], char* lds) {
  static_assert(PASS % 32 == 0 && (128 % PASS == 0 || PASS % 128 == 0) && BM % PASS == 0, "pass rows");
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int l32 = lane & 31;
  const int lh = lane >> 5;
  const int wm = wave / 4;
  const int wn = wave % 4;
  const int h = static_cast<int>(n0 / a.n_proj_pad);
  const float g = h == 0 ? a.gscale[0] : a.gscale[1];
  // Row r, 8-column chunk c: thread t takes chunk t % 32 of rows t / 32 + (THREADS / 32) q.
  const int c8 = t & 31;
  const int64_t lr = n0 - static_cast<int64_t>(h) * a.n_proj_pad + 8 * c8;  // column within the projection
  const int64_t col = static_cast<int64_t>(h) * a.n_proj + lr;
  const bool vec = lr + 8 <= a.n_proj && ((col | a.ldy) & 7) == 0;
  for (int pass = 0; pass < BM / PASS; ++pass) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int row0 = wm * 32 * FI + 32 * i;  // first tile row of fragment row i (wave-uniform)
      if (row0 / PASS != pass) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int row = row0 - pass * PASS + l32;
          const int cc = wn * 64 + 32 * j + 8 * e4 + 4 * lh;
          *reinterpret_cast<uint2*>(lds + row * kStageYRow + 2 * cc) =
              make_uint2(f32x2_to_bf16x2_rne(acc[i][j][4 * e4] * g, acc[i][j][4 * e4 + 1] * g),
                         f32x2_to_bf16x2_rne(acc[i][j][4 * e4 + 2] * g, acc[i][j][4 * e4 + 3] * g));
        }
    }
    __syncthreads();
    if (lr >= a.n_proj) continue;
    for (int row = t >> 5; row < PASS; row += THREADS / 32) {
      const int64_t m = m0 + pass * PASS + row;
      if (m >= a.m) break;
      const uint4 v = *reinterpret_cast<const uint4*>(lds + row * kStageYRow + 16 * c8);
      uint16_t* dst = a.y + m * a.ldy + col;
      if (vec) {
        *reinterpret_cast<uint4*>(dst) = v;
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        for (int e = 0; e < 8 && lr + e < a.n_proj; ++e) dst[e] = static_cast<uint16_t>(w[e / 2] >> (16 * (e & 1)));
      }
    }
  }
}

// SwiGLU gate_up on the interleaved weight (prepared row R is gate row
// 16 (R / 32) + R % 16 when R % 32 < 16, else the up row with that index):
// y[m][16 (R / 32) + R % 16] = bf16(silu(g) * u) with g, u the float32 sums
// times their projections' global scales, for the tile's BM x 128 outputs.
// The scaled sums are staged PASS rows at a time as float32 rows; each thread
// then forms 8 consecutive outputs of one row (8 gate and the matching 8 up
// values) and writes them as 16 bytes.  silu(v) = v / (1 + e^-v), computed as
// the reduce launch computes it for split tiles.
template <int BM, int THREADS, int PASS, int FI = 4>
__device__ __forceinline__ void store_tile_swiglu_staged(const MfmaArgs& a, int64_t m0, int64_t n0, int wave,
                                                         const f32x16_t (&acc)[FI][2], char* lds) {
  static_assert(PASS % 32 == 0 && (128 % PASS == 0 || PASS % 128 == 0) && BM % PASS == 0, "pass rows");
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int l32 = lane & 31;
  const int lh = lane >> 5;
  const int wm = wave / 4;
  const int wn = wave % 4;
  // Output chunk of a thread: columns 8 c8 .. 8 c8 + 7 of the tile's 128.
  const int c8 = t & 15;
  const int g0 = 32 * (c8 >> 1) + 8 * (c8 & 1);  // staged column of its first gate value; up is 16 further
  const int64_t col = n0 / 2 + 8 * c8;
  const bool vec = col + 8 <= a.n_proj && ((col | a.ldy) & 7) == 0;
  for (int pass = 0; pass < BM / PASS; ++pass) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int row0 = wm * 32 * FI + 32 * i;  // first tile row of fragment row i (wave-uniform)
      if (row0 / PASS != pass) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int row = row0 - pass * PASS + l32;
          const int cc = wn * 64 + 32 * j + 8 * e4 + 4 * lh;  // 4 rows of one 16-row gate or up group
          const float g = (cc & 31) < 16 ? a.gscale[0] : a.gscale[1];
          const f32x4_t v = {acc[i][j][4 * e4] * g, acc[i][j][4 * e4 + 1] * g, acc[i][j][4 * e4 + 2] * g,
                             acc[i][j][4 * e4 + 3] * g};
          *reinterpret_cast<f32x4_t*>(lds + row * kStagePRow + 4 * cc) = v;
        }
    }
    __syncthreads();
    if (col >= a.n_proj) continue;
    for (int row = t >> 4; row < PASS; row += THREADS / 16) {
      const int64_t m = m0 + pass * PASS + row;
      if (m >= a.m) break;
      const char* src = lds + row * kStagePRow + 4 * g0;
      const f32x4_t ga = *reinterpret_cast<const f32x4_t*>(src);
      const f32x4_t gb = *reinterpret_cast<const f32x4_t*>(src + 16);
      const f32x4_t ua = *reinterpret_cast<const f32x4_t*>(src + 64);
      const f32x4_t ub = *reinterpret_cast<const f32x4_t*>(src + 80);
      const float gv[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
      const float uv[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float y0 = gv[2 * q] * __builtin_amdgcn_rcpf(1.0f + __expf(-gv[2 * q])) * uv[2 * q];
        const float y1 = gv[2 * q + 1] * __builtin_amdgcn_rcpf(1.0f + __expf(-gv[2 * q + 1])) * uv[2 * q + 1];
        w[q] = f32x2_to_bf16x2_rne(y0, y1);
      }
      uint16_t* dst = a.y + m * a.ldy + col;
      if (vec) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        for (int e = 0; e < 8 && col + e < a.n_proj; ++e) dst[e] = static_cast<uint16_t>(w[e / 2] >> (16 * (e & 1)));
      }
    }
  }
}

// fp32 partial tile of tail unit u, row-major [BM][256], staged PASS rows at
// a time (PASS a multiple of 32 dividing 128, or 128).  Only the rows below m
// are written (the reduce launch reads no others): at small m the partials
// would otherwise outweigh the weights.
template <int BM, int THREADS, int PASS, int FI = 4>
__device__ __forceinline__ void store_tile_partial_staged(const MfmaArgs& a, int u, int64_t m0, int wave,
                                                          const f32x16_t (&acc)[FI][2], char* lds) {
  static_assert(PASS % 32 == 0 && (128 % PASS == 0 || PASS % 128 == 0) && BM % PASS == 0, "pass rows");
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int l32 = lane & 31;
  const int lh = lane >> 5;
  const int wm = wave / 4;
  const int wn = wave % 4;
  float* dst = a.partial + static_cast<int64_t>(u) * BM * kGemmBN;
  const int64_t valid = a.m - m0;  // tile rows below m
  for (int pass = 0; pass < BM / PASS; ++pass) {
    if (pass * PASS >= valid) break;  // uniform: no barrier is skipped by part of the workgroup
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int row0 = wm * 32 * FI + 32 * i;  // first tile row of fragment row i (wave-uniform)
      if (row0 / PASS != pass) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int row = row0 - pass * PASS + l32;
          const int col = wn * 64 + 32 * j + 8 * e4 + 4 * lh;
          const f32x4_t v = {acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2], acc[i][j][4 * e4 + 3]};
          *reinterpret_cast<f32x4_t*>(lds + row * kStagePRow + 4 * col) = v;
        }
    }
    __syncthreads();
    // PASS rows x 64 chunks of 4 floats: thread t takes chunk t % 64 of rows t / 64 + (THREADS / 64) q.
    for (int row = t >> 6; row < PASS && pass * PASS + row < valid; row += THREADS / 64)
      *reinterpret_cast<f32x4_t*>(dst + (pass * PASS + row) * kGemmBN + 4 * (t & 63)) =
          *reinterpret_cast<const f32x4_t*>(lds + row * kStagePRow + 16 * (t & 63));
  }
}

}  // namespace fp4
