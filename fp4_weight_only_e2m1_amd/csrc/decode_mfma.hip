// Decode-shaped W4A16 FP4 GEMM on the matrix cores (m = 3..8 activation rows).
//
// The weight stream is the same as the VALU GEMV's (same prepared layout, same
// 64-row x split tiles, 16-byte coalesced code loads, same K splits and
// in-order split-K finish), but the contraction runs on v_mfma_f32_16x16x32_bf16 with
// the activation rows zero-padded to 16.  Reason: at m rows the VALU GEMV
// spends m/2 v_dot2 per weight on top of the decode, so from m = 3 on it is
// bound by VALU issue before HBM; here the VALU only decodes (E2M1 -> bf16)
// and one MFMA consumes 16 x 32 weights per lane-quad, with no cross-lane
// reduction at all.  No extra HBM bytes are read: the padding lives in
// registers.  (Why decode is memory-bound: "MXFP4 decode-graph + gate_up
// FUSION default-ON", vllm.cpp PR #54, step 2.)
//
// Wave w of a 256-thread workgroup owns rows [row0 + 16w, +16).  Lane l
// handles row r = l % 16 and, in every 128-code block of the K range, the
// 32-code segment g = l / 16: one 16-byte load per block, so one wave-wide
// load covers 16 rows x 64 contiguous bytes.  Each 8-code word c of the load is
// one MFMA's B fragment (k index 8g..8g+7 of the instruction); the A fragment
// is x[r][same 8 k], read from LDS (zero for r >= m).  Both operands use that
// same k assignment, so the MFMA's sum runs over exactly the 32 codes of
// words c of the 4 segments.
//
// Scales: MXFP4 is folded into v_cvt_scalef32_pk_bf16_fp4 (E8M0 = exponent
// operand).  NVFP4's E4M3 scale has a mantissa the conversion ignores, so each
// code pair is converted to f32, multiplied by the scale (exact: at most 6
// significant bits) and packed to bf16 with v_cvt_pk_bf16_f32.
#include "decode_common.hpp"

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = kDecodeThreads;
constexpr int kBlocksPerSlab = kSlabK / 128;

union Frag {
  bf16x8_t v;
  uint32_t u[4];
  uint4 q;
};

__device__ __forceinline__ uint32_t u4_word(const uint4& v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// x chunk q of activation row m lives at LDS index q ^ (m & 7): the 16-byte
// reads of the 8 rows in one instruction land in 8 different bank groups.
__device__ __forceinline__ int xsw(int m, int q) { return q ^ (m & 7); }

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

template <int M, int FMT>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(const GemvArgs a) {
  constexpr int P = scales_per_seg(FMT);
  __shared__ uint4 xs[M][kGemvMaxSlabsPerSplit * kChunksPerSlab];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int split = blockIdx.y;
  const SlabRange sr = split_slabs(a, split);
  const int slab0 = sr.first;
  const int nsl = sr.count;

  const int64_t roww = static_cast<int64_t>(blockIdx.x) * kGemvTileRows + wave * 16;
  const int64_t row = roww + r;
  const int64_t row_bytes = a.k_pad / 2;
  const uint8_t* cptr = a.codes + row * row_bytes + 16 * g;
  // Scale bytes of (row, segment): this wave's 16 rows are one scale group.
  const uint8_t* sptr = a.scales + ((roww / kRowGroup) * a.ksegs * kRowGroup + r) * P;

  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc1 = {0.f, 0.f, 0.f, 0.f};
  const bool live = r < M;

  uint4 q[kBlocksPerSlab];
  uint32_t sb[kBlocksPerSlab];
  auto load_slab = [&](int slab, uint4* qq, uint32_t* ss) {
#pragma unroll
    for (int b = 0; b < kBlocksPerSlab; ++b)
      qq[b] = load_stream16(cptr + static_cast<int64_t>(slab) * (kSlabK / 2) + 64 * b);
#pragma unroll
    for (int b = 0; b < kBlocksPerSlab; ++b) {
      const int64_t seg = static_cast<int64_t>(slab) * 32 + 4 * b + g;
      const uint8_t* sp = sptr + seg * kRowGroup * P;
      if constexpr (P == 1) ss[b] = *sp;
      else ss[b] = *reinterpret_cast<const uint16_t*>(sp);
    }
  };

  // Start the weight stream first, then stage x while those loads fly.
  load_slab(slab0, q, sb);
  stage_x<M>(a, slab0, nsl, xs, [](int m, int cc) { return xsw(m, cc); });
  for (int j = 0; j < nsl; ++j) {
    uint4 qn[kBlocksPerSlab];
    uint32_t sbn[kBlocksPerSlab];
    if (j + 1 < nsl) load_slab(slab0 + j + 1, qn, sbn);
#pragma unroll
    for (int b = 0; b < kBlocksPerSlab; ++b) {
      float s0, s1;
      if constexpr (FMT == kFmtMxfp4) {
        s0 = s1 = e8m0_as_scale_operand(sb[b]);
      } else {
        s0 = e4m3_to_f32<0>(sb[b]);
        s1 = e4m3_to_f32<1>(sb[b]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        Frag af, bfr;
        af.q = make_uint4(0u, 0u, 0u, 0u);
        if (live) af.q = xs[r][xsw(r, j * kChunksPerSlab + 16 * b + 4 * g + c)];
        decode_word<FMT>(u4_word(q[b], c), c < 2 ? s0 : s1, bfr);
        if (b & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af.v, bfr.v, acc1, 0, 0, 0);
        else acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af.v, bfr.v, acc0, 0, 0, 0);
      }
    }
    if (j + 1 < nsl) {
#pragma unroll
      for (int b = 0; b < kBlocksPerSlab; ++b) {
        q[b] = qn[b];
        sb[b] = sbn[b];
      }
    }
  }

  // Lane l holds C[m = 4g + i][n = r], i = 0..3.
  const int h = static_cast<int>(row / a.n_proj_pad);
  const int64_t lr = row - static_cast<int64_t>(h) * a.n_proj_pad;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * g + i;
    if (m >= M) continue;
    const float v = acc0[i] + acc1[i];
    if (a.splits == 1) {
      if (lr < a.n_proj)
        a.y[static_cast<int64_t>(m) * a.ldy + static_cast<int64_t>(h) * a.n_proj + lr] =
            f32_to_bf16_rne(v * a.gscale[h]);
    } else {
      store_partial(a.partial + (static_cast<int64_t>(split) * M + m) * a.rows_total + row, v);
    }
  }
  if (a.splits > 1) splitk_finish<M>(a, blockIdx.x, split);
}

template <int FMT>
hipError_t launch_fmt(const GemvArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(kThreads);
  switch (a.m) {
    case 3: hipLaunchKernelGGL((decode_mfma_kernel<3, FMT>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<4, FMT>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((decode_mfma_kernel<5, FMT>), grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL((decode_mfma_kernel<6, FMT>), grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL((decode_mfma_kernel<7, FMT>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_mfma_kernel<8, FMT>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const GemvArgs& a, int fmt, hipStream_t stream, dim3* grid_out, dim3* block_out) {
  const dim3 grid(static_cast<unsigned>(a.rows_total / kGemvTileRows), static_cast<unsigned>(a.splits));
  if (grid_out) *grid_out = grid;
  if (block_out) *block_out = dim3(kThreads);
  return fmt == kFmtNvfp4 ? launch_fmt<kFmtNvfp4>(a, grid, stream) : launch_fmt<kFmtMxfp4>(a, grid, stream);
}

}  // namespace fp4
