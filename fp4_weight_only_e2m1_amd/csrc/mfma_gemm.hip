// Prefill-shaped W4A16 FP4 GEMM (m > 8 activation rows) on gfx950 bf16 MFMA.
//
// At large m the layer is a dense contraction (2*m*n*k flops over n*k/2 code
// bytes), so it runs on the matrix cores.  The pages run prefill through a
// dequantized bf16 GEMM ("MXFP4 decode-graph + gate_up FUSION default-ON",
// vllm.cpp PR #54, step 3: prefill untouched; "keep the ModelOpt NVFP4 lm_head
// packed", section "Why this row matters": the bf16 head cost 2.37 GiB/step);
// here the packed weight is used directly.
//
// Tiling: a 256-thread workgroup computes a 128 (m) x 256 (n) tile of y over
// K in steps of 64.  Each step is staged in LDS, double buffered:
//   x  tile 128 x 64 bf16  (16 KiB),
//   W  tile 256 x 64 codes (8 KiB, still packed 4-bit),
//   scales of the W tile   (1 KiB NVFP4 / 512 B MXFP4).
// Wave w owns output columns [64w, 64w + 64) and all 128 rows: it decodes
// only its own 64 weight rows, so every code is decoded once per workgroup,
// and issues 4 x 2 v_mfma_f32_32x32x16_bf16 per 16-code step with f32
// accumulators.  E2M1 * S is exact in bf16 (at most 6 significant bits), so
// decoding before the MFMA loses nothing; the NVFP4 global scale multiplies in
// the epilogue.
//
// v_mfma_f32_32x32x16_bf16 operands: lane l supplies row (l % 32) of A and
// column (l % 32) of B, each with 8 consecutive k (8 * (l / 32) .. +7); result
// j (0..15) of lane l is C[8 * (j / 4) + 4 * (l / 32) + j % 4][l % 32].
#include "fp4_common.hpp"
#include "fp4_device.hpp"

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kMT = kBM / 32;          // 32-row MFMA tiles per wave
constexpr int kNT = kBN / 4 / 32;      // 32-column MFMA tiles per wave
constexpr int kAChunks = kBM * kBK * 2 / 16;  // 16-byte chunks of the x tile
constexpr int kBChunks = kBN * kBK / 2 / 16;  // 16-byte chunks of the code tile

union Frag {
  bf16x8_t v;
  uint32_t u[4];
  uint4 q;
};

// x tile: row r holds 8 chunks of 16 bytes; chunk c sits at c ^ (r & 7), so a
// fragment read (32 rows, one chunk) touches 8 distinct chunk slots per 8 rows.
__device__ __forceinline__ int a_slot(int r, int c) { return r * 8 + (c ^ (r & 7)); }

// Code tile: row r holds 32 bytes = 8 dwords.  Dword d of row r sits at
// d ^ (2 * ((r >> 3) & 3)) so that the 32 rows x 2 dwords of a fragment read
// fall in distinct banks.  The XOR moves whole 16-byte halves (bit 2) and
// swaps dword pairs inside a half (bit 1).
__device__ __forceinline__ int b_dword(int r, int d) { return r * 8 + (d ^ (2 * ((r >> 3) & 3))); }

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

// Global -> register staging of one K step (what one thread moves).
template <int FMT>
struct Stage {
  static constexpr int P = scales_per_seg(FMT);
  static constexpr int kSChunks = kBN / kRowGroup * (kBK / 32) * kRowGroup * P / 16;  // 64 NVFP4, 32 MXFP4
  uint4 a[kAChunks / kThreads];
  uint4 b[kBChunks / kThreads];
  uint4 s;
};

template <int FMT>
__device__ __forceinline__ void load_stage(const MfmaArgs& a, int64_t m0, int64_t n0, int64_t k0, Stage<FMT>& st) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kAChunks / kThreads; ++i) {
    const int c = t + i * kThreads;
    const int r = c >> 3;
    const int64_t m = m0 + r;
    const int64_t kk = k0 + (c & 7) * 8;
    st.a[i] = make_uint4(0u, 0u, 0u, 0u);
    if (m < a.m && kk < a.k) st.a[i] = *reinterpret_cast<const uint4*>(a.x + m * a.k + kk);
  }
  const int64_t row_bytes = a.k_pad / 2;
#pragma unroll
  for (int i = 0; i < kBChunks / kThreads; ++i) {
    const int c = t + i * kThreads;
    st.b[i] = *reinterpret_cast<const uint4*>(a.codes + (n0 + (c >> 1)) * row_bytes + k0 / 2 + (c & 1) * 16);
  }
  // Scales of the tile: 16 row groups x 2 segments x (16 * P) contiguous bytes.
  constexpr int P = Stage<FMT>::P;
  if (t < Stage<FMT>::kSChunks) {
    constexpr int per_group = 2 * 16 * P / 16;  // 16-byte chunks per row group
    const int rg = t / per_group;
    const int within = t % per_group;
    const uint8_t* src = a.scales + ((n0 / kRowGroup + rg) * a.ksegs + k0 / 32) * kRowGroup * P + within * 16;
    st.s = *reinterpret_cast<const uint4*>(src);
  }
}

template <int FMT>
__device__ __forceinline__ void store_stage(const Stage<FMT>& st, uint4* As, uint32_t* Bs, uint4* Ss) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kAChunks / kThreads; ++i) {
    const int c = t + i * kThreads;
    As[a_slot(c >> 3, c & 7)] = st.a[i];
  }
#pragma unroll
  for (int i = 0; i < kBChunks / kThreads; ++i) {
    const int c = t + i * kThreads;
    const int r = c >> 1;
    const int h = c & 1;
    // Dwords 4h..4h+3 of row r, each to its swizzled slot.
    const uint32_t w[4] = {st.b[i].x, st.b[i].y, st.b[i].z, st.b[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) Bs[b_dword(r, 4 * h + j)] = w[j];
  }
  if (t < Stage<FMT>::kSChunks) Ss[t] = st.s;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void mfma_kernel(const MfmaArgs a, int m_tiles, int n_tiles) {
  constexpr int P = scales_per_seg(FMT);
  constexpr int kSBytes = kBN * kBK / group_size(FMT);
  __shared__ uint4 As[2][kAChunks];
  __shared__ uint32_t Bs[2][kBChunks * 4];
  __shared__ uint4 Ss[2][kSBytes / 16];

  // XCD-aware tile order: workgroup b runs on XCD b % 8, so XCD x holds the
  // ids x, x + 8, x + 16, ...; give it the contiguous tile run starting at
  // x * q + min(x, r) (q = tiles / 8, r = tiles % 8).  Tiles are numbered
  // n-major, so a run shares weight tiles (and x tiles) in that XCD's L2.
  const int tiles = m_tiles * n_tiles;
  const int bid = blockIdx.x;
  const int xcd = bid % 8;
  const int q = tiles / 8;
  const int r = tiles % 8;
  const int t = xcd * q + (xcd < r ? xcd : r) + bid / 8;
  const int n_tile = t / m_tiles;
  const int m_tile = t - n_tile * m_tiles;
  const int64_t m0 = static_cast<int64_t>(m_tile) * kBM;
  const int64_t n0 = static_cast<int64_t>(n_tile) * kBN;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int lh = lane >> 5;

  f32x16_t acc[kMT][kNT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int j = 0; j < kNT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int ksteps = static_cast<int>(a.k_pad / kBK);
  Stage<FMT> st;
  load_stage<FMT>(a, m0, n0, 0, st);
  store_stage<FMT>(st, As[0], Bs[0], Ss[0]);
  __syncthreads();

  for (int ks = 0; ks < ksteps; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < ksteps) load_stage<FMT>(a, m0, n0, static_cast<int64_t>(ks + 1) * kBK, st);
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(Ss[buf]);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      Frag af[kMT], bfr[kNT];
#pragma unroll
      for (int i = 0; i < kMT; ++i) af[i].q = As[buf][a_slot(32 * i + l32, 2 * kk + lh)];
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int r = wave * (kBN / 4) + 32 * j + l32;
        const uint32_t word = Bs[buf][b_dword(r, 2 * kk + lh)];
        // Scale of (row r, group of this 16-code step): segment kk / 2.
        const int kg_in_seg = (kk & 1) * 16 / group_size(FMT);
        const uint32_t sbyte = sb[(((r >> 4) * 2 + (kk >> 1)) * kRowGroup + (r & 15)) * P + kg_in_seg];
        decode_b<FMT>(word, sbyte, bfr[j]);
      }
#pragma unroll
      for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i].v, bfr[j].v, acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < ksteps) store_stage<FMT>(st, As[buf ^ 1], Bs[buf ^ 1], Ss[buf ^ 1]);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    const int64_t row = n0 + wave * (kBN / 4) + 32 * j + l32;
    const int h = static_cast<int>(row / a.n_proj_pad);
    const int64_t lr = row - static_cast<int64_t>(h) * a.n_proj_pad;
    if (lr >= a.n_proj) continue;
    const float g = a.gscale[h];
    const int64_t col = static_cast<int64_t>(h) * a.n_proj + lr;
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + 32 * i + 8 * (e >> 2) + 4 * lh + (e & 3);
        if (m < a.m) a.y[m * a.ldy + col] = f32_to_bf16_rne(acc[i][j][e] * g);
      }
    }
  }
}

}  // namespace

hipError_t launch_mfma(const MfmaArgs& a, int fmt, hipStream_t stream, dim3* grid_out, dim3* block_out) {
  const int m_tiles = static_cast<int>((a.m + kBM - 1) / kBM);
  const int n_tiles = static_cast<int>(a.rows_total / kBN);
  const dim3 grid(static_cast<unsigned>(m_tiles * n_tiles));
  const dim3 block(kThreads);
  if (grid_out) *grid_out = grid;
  if (block_out) *block_out = block;
  if (fmt == kFmtNvfp4)
    hipLaunchKernelGGL(mfma_kernel<kFmtNvfp4>, grid, block, 0, stream, a, m_tiles, n_tiles);
  else
    hipLaunchKernelGGL(mfma_kernel<kFmtMxfp4>, grid, block, 0, stream, a, m_tiles, n_tiles);
  return hipGetLastError();
}

}  // namespace fp4
