// Decode-shaped W4A16 FP4 GEMM on the matrix cores (m = 3..8 activation rows).
//
// At m rows a VALU GEMV spends m/2 v_dot2 per weight on top of the decode, so
// from m = 3 on it is bound by VALU issue before HBM.  Here the VALU only
// decodes (E2M1 -> bf16) and v_mfma_f32_16x16x32_bf16 does the contraction,
// with the m activation rows zero-padded to 16 in registers: no extra HBM
// bytes.  (Why decode is memory-bound: "MXFP4 decode-graph + gate_up FUSION
// default-ON", vllm.cpp PR #54, step 2.)
//
// Work split.  A 512-thread workgroup (8 waves) owns 16 * NB weight rows and
// all of K.  K is cut into 128-code blocks dealt round-robin to the 8 waves.
// For each of its k-blocks a wave loads the x fragments once (global memory;
// x is small and stays in L2) and reuses them for its NB row blocks of 16
// rows: per row block one 16-byte code load per lane, one scale load, 16
// conversions and 4 MFMAs.  Each wave keeps a ring of 2 k-blocks in flight:
// a block's slot is refilled as soon as the block is consumed.  At the end
// the 8 waves' partial tiles are added in LDS in wave order 0..7.
//
// Lane l handles row r = l % 16 of a row block and the 32-code segment
// g = l / 16 of a k-block, so a wave-wide code load covers 16 rows x 64
// contiguous bytes.  Word c (8 codes) of the load is the MFMA's B fragment for
// k index 8g..8g+7; the A fragment is x[r][same 8 codes] (zero for r >= m).
// Both operands use that k assignment, so each MFMA sums exactly the 32 codes
// of words c of the 4 segments.
//
// Summation order of an output: per wave, its k-blocks in order (MFMA
// accumulation); then waves 0..7.  It depends only on k -- not on m, not on
// which rows a workgroup holds (NB), not on fusion -- so results are
// deterministic, batch invariant for every m this kernel serves, and the
// fused gate_up launch equals the two separate ones bit for bit.
//
// Scales: MXFP4 is folded into v_cvt_scalef32_pk_bf16_fp4 (the E8M0 byte is
// the exponent operand).  NVFP4's E4M3 scale has a mantissa the conversion
// ignores, so each code pair is converted to f32, multiplied by the scale
// (exact: at most 6 significant bits) and packed to bf16.
#include "fp4_common.hpp"
#include "fp4_device.hpp"

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = kDecodeMfmaWaves;
constexpr int kThreads = 64 * kWaves;

union Frag {
  bf16x8_t v;
  uint32_t u[4];
  uint4 q;
};

__device__ __forceinline__ uint32_t u4_word(const uint4& v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

template <int FMT>
__device__ __forceinline__ void decode_word(uint32_t word, float s, Frag& f) {
  if constexpr (FMT == kFmtMxfp4) {
    f.u[0] = bf16x2_bits(cvt_fp4x2_bf16<0>(word, s));
    f.u[1] = bf16x2_bits(cvt_fp4x2_bf16<1>(word, s));
    f.u[2] = bf16x2_bits(cvt_fp4x2_bf16<2>(word, s));
    f.u[3] = bf16x2_bits(cvt_fp4x2_bf16<3>(word, s));
  } else {
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

// Everything one lane loads for one k-block.
template <int NB>
struct Block {
  uint4 x[4];       // x[r][kb*128 + 32g + 8c .. +8], c = 0..3
  uint4 code[NB];   // row block b: codes of (row r, segment g)
  uint32_t sb[NB];  // the segment's scale byte(s)
};

// Loads are branch-free (rows >= m and codes past k read a valid address and
// are zeroed afterwards), so every k-block issues the same number of memory
// instructions and the wait for the oldest block of the ring can be exact.
template <int M, int FMT, int NB>
__device__ __forceinline__ void load_block(const GemvArgs& a, int64_t row0, int kb, int r, int g, Block<NB>& blk) {
  constexpr int P = scales_per_seg(FMT);
  const int64_t kx = static_cast<int64_t>(kb) * 128 + 32 * g;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bool ok = r < M && kx + 8 * c < a.k;
    const int64_t off = ok ? static_cast<int64_t>(r) * a.k + kx + 8 * c : 0;
    const uint4 v = *reinterpret_cast<const uint4*>(a.x + off);
    const uint32_t keep = ok ? ~0u : 0u;  // an AND, not a select: keeps the load unconditional
    blk.x[c] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
  }
  const int64_t row_bytes = a.k_pad / 2;
  const int64_t seg = static_cast<int64_t>(kb) * 4 + g;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t row = row0 + 16 * b + r;
    blk.code[b] = load_stream16(a.codes + row * row_bytes + seg * 16);
    const uint8_t* sp = a.scales + (((row0 / kRowGroup + b) * a.ksegs + seg) * kRowGroup + r) * P;
    if constexpr (P == 1) blk.sb[b] = *sp;
    else blk.sb[b] = *reinterpret_cast<const uint16_t*>(sp);
  }
}

template <int FMT, int NB>
__device__ __forceinline__ void compute_block(const Block<NB>& blk, f32x4_t (&acc)[NB]) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float s0, s1;
    if constexpr (FMT == kFmtMxfp4) {
      s0 = s1 = e8m0_as_scale_operand(blk.sb[b]);
    } else {
      s0 = e4m3_to_f32<0>(blk.sb[b]);
      s1 = e4m3_to_f32<1>(blk.sb[b]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      Frag af, bfr;
      af.q = blk.x[c];
      decode_word<FMT>(u4_word(blk.code[b], c), c < 2 ? s0 : s1, bfr);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af.v, bfr.v, acc[b], 0, 0, 0);
    }
  }
}

template <int M, int FMT, int NB>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(const GemvArgs a) {
  constexpr int D = kDecodeMfmaDepth;
  __shared__ f32x4_t red[kWaves][NB][64];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16 * NB;
  // This wave's k-blocks are wave, wave + 8, wave + 16, ...
  const int kblocks = static_cast<int>(a.k_pad / 128);
  const int nk = (kblocks - wave + kWaves - 1) / kWaves;

  f32x4_t acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Ring of D k-blocks in flight: block i lives in slot i % D.  The steady
  // state is straight-line code (consume slot j, refill it with block i + D),
  // so the wait before each use counts exactly the younger blocks' loads.
  Block<NB> ring[D];
  auto kblock = [&](int i) { return wave + i * kWaves; };
  if (nk >= D) {
#pragma unroll
    for (int j = 0; j < D; ++j) load_block<M, FMT, NB>(a, row0, kblock(j), r, g, ring[j]);
    int i0 = 0;
    for (; i0 + 2 * D <= nk; i0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        compute_block<FMT, NB>(ring[j], acc);
        load_block<M, FMT, NB>(a, row0, kblock(i0 + j + D), r, g, ring[j]);
      }
    }
    // D .. 2D-1 blocks remain: the first D are in the ring.
#pragma unroll
    for (int j = 0; j < D; ++j) {
      compute_block<FMT, NB>(ring[j], acc);
      if (i0 + j + D < nk) load_block<M, FMT, NB>(a, row0, kblock(i0 + j + D), r, g, ring[j]);
    }
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (i0 + D + j < nk) compute_block<FMT, NB>(ring[j], acc);
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < nk) load_block<M, FMT, NB>(a, row0, kblock(j), r, g, ring[j]);
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < nk) compute_block<FMT, NB>(ring[j], acc);
  }

  // Lane l holds C[m = 4g + i][n = r] of each row block; add the waves' tiles
  // in wave order.
#pragma unroll
  for (int b = 0; b < NB; ++b) red[wave][b][lane] = acc[b];
  __syncthreads();
  for (int o = threadIdx.x; o < NB * 16 * M; o += kThreads) {
    const int b = o / (16 * M);
    const int rem = o - b * 16 * M;
    const int m = rem / 16;
    const int n = rem - m * 16;
    const int src_lane = n + 16 * (m >> 2);
    float s = red[0][b][src_lane][m & 3];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += red[w][b][src_lane][m & 3];
    const int64_t row = row0 + 16 * b + n;
    const int h = static_cast<int>(row / a.n_proj_pad);
    const int64_t lr = row - static_cast<int64_t>(h) * a.n_proj_pad;
    if (lr < a.n_proj)
      a.y[static_cast<int64_t>(m) * a.ldy + static_cast<int64_t>(h) * a.n_proj + lr] =
          f32_to_bf16_rne(s * a.gscale[h]);
  }
}

template <int M, int FMT>
hipError_t launch_nb(const GemvArgs& a, int nb, hipStream_t stream, dim3* grid_out) {
  const dim3 grid(static_cast<unsigned>(a.rows_total / (16 * nb)));
  if (grid_out) *grid_out = grid;
  const dim3 block(kThreads);
  if (nb == 4) hipLaunchKernelGGL((decode_mfma_kernel<M, FMT, 4>), grid, block, 0, stream, a);
  else if (nb == 2) hipLaunchKernelGGL((decode_mfma_kernel<M, FMT, 2>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((decode_mfma_kernel<M, FMT, 1>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const GemvArgs& a, int nb, hipStream_t stream, dim3* grid_out) {
  switch (a.m) {
    case 3: return launch_nb<3, FMT>(a, nb, stream, grid_out);
    case 4: return launch_nb<4, FMT>(a, nb, stream, grid_out);
    case 5: return launch_nb<5, FMT>(a, nb, stream, grid_out);
    case 6: return launch_nb<6, FMT>(a, nb, stream, grid_out);
    case 7: return launch_nb<7, FMT>(a, nb, stream, grid_out);
    case 8: return launch_nb<8, FMT>(a, nb, stream, grid_out);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const GemvArgs& a, int fmt, hipStream_t stream, dim3* grid_out, dim3* block_out) {
  const int nb = decode_mfma_row_blocks(a.rows_total);
  if (block_out) *block_out = dim3(kThreads);
  return fmt == kFmtNvfp4 ? launch_fmt<kFmtNvfp4>(a, nb, stream, grid_out)
                          : launch_fmt<kFmtMxfp4>(a, nb, stream, grid_out);
}

}  // namespace fp4
