// Decode-shaped W4A16 FP4 GEMV on the VALU (m = 1, 2 activation rows) for
// gfx950, with a deterministic split-K reduction in the same launch.
//
// What it computes: y[m, n] = G * sum_k x[m, k] * E2M1(code[n, k]) * S(n, k/g)
// ("native MXFP4 keep-quant", vllm.cpp PR #38, commit list: W4A16 GEMM at
// decode, M=1 and M=8; "keep the ModelOpt NVFP4 lm_head packed", vllm.cpp
// PR #263, section "Why this row matters": the packed head is a W4A16 GEMM).
//
// The weight stream is the whole cost at decode ("MXFP4 decode-graph +
// gate_up FUSION default-ON", vllm.cpp PR #54: W4A16 is memory-bound), so the
// kernel is built around it:
//   * A 256-thread workgroup owns 8 ROWS weight rows and one K split.  It is 8
//     teams of 32 lanes; a team owns ROWS rows (8 for the largest layers, 4
//     otherwise: gemv_rows_per_team).  Lane l of a team covers codes
//     [32l, 32l + 32) of each 1024-code slab, so each row's slab is one 16-byte
//     load per lane and 512 contiguous bytes per team (coalesced).
//   * The scale bytes of the team's rows for one k-group are contiguous in
//     the prepared layout: one ROWS-byte (MXFP4) or 2 ROWS-byte (NVFP4, two
//     groups) load per lane per slab.
//   * x for the split is staged once into LDS (at most 8 x 4096 bf16 = 64 KiB)
//     and read back 16 bytes at a time; each read serves ROWS rows.  The 16-byte
//     chunks of a lane are rotated by (lane >> 1) so that 8 consecutive lanes
//     hit 8 distinct 16-byte bank groups.
//   * Decode: v_cvt_scalef32_pk_bf16_fp4 turns each code byte into a bf16
//     pair.  For MXFP4 the E8M0 scale is folded into that conversion (the
//     products are powers-of-two multiples of E2M1 values, exact in bf16).
//     For NVFP4 the conversion is unscaled; the group partial (16 codes) is
//     multiplied by its E4M3 scale with one f32 FMA per row and activation
//     row, because the conversion ignores a scale's mantissa.
//   * Contraction: v_dot2c_f32_bf16, f32 accumulation.
//   * Reduction over the 32 lanes of a team: a transposing butterfly.  At each
//     step a lane keeps half of its partial sums and trades the other half
//     with its partner, so 8*M sums take about 2*8*M shuffles instead of
//     5*8*M.
//   * K split: each (tile, split) workgroup stores its partial sums in a
//     caller workspace [splits][m][rows]; the last workgroup of a tile to
//     arrive adds them in split order and writes y, in the same launch (see
//     splitk_finish).  The split count depends on (k, fmt, rows per
//     projection) only, so summation order -- and hence every output bit -- is
//     the same for any m handled by this kernel and for the fused gate_up
//     launch as for the two separate ones.  There are no locks and nothing
//     waits, so the workspace never needs zeroing (unlike the spin-lock
//     workspace whose missing memset hung the pages' engine: "re-verify 27B
//     NVFP4 on the nvidia ModelOpt checkpoint", section "Rewrite/binding
//     grid").
#include "decode_common.hpp"

namespace fp4 {
namespace {

constexpr int kThreads = kDecodeThreads;
constexpr int kTeamLanes = 32;

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// Rotated position of 16-byte chunk `sub` (0..3) of lane block `lb` in LDS.
__device__ __forceinline__ int xs_index(int lb, int sub) {
  return (lb << 2) | ((sub + (lb >> 1)) & 3);
}

// Value of `v` held by lane (lane ^ o) of the same 32-lane team.  o = 1, 2:
// DPP quad permutes; o = 4, 8: DPP half-row / row mirrors, which pair lane i
// with 7 - i / 15 - i -- not lane ^ o, but the same partition into a lower
// (bit o clear) and an upper half, which is all the butterfly needs;
// o = 16: ds_swizzle-free bpermute across the two 16-lane rows.
template <int O>
__device__ __forceinline__ float partner(float v) {
  const int iv = __float_as_int(v);
  int r;
  if constexpr (O == 1) r = __builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false);       // quad_perm [1,0,3,2]
  else if constexpr (O == 2) r = __builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  else if constexpr (O == 4) r = __builtin_amdgcn_update_dpp(0, iv, 0x141, 0xF, 0xF, false); // row_half_mirror
  else if constexpr (O == 8) r = __builtin_amdgcn_update_dpp(0, iv, 0x140, 0xF, 0xF, false); // row_mirror
  else return __shfl_xor(v, O, kTeamLanes);
  return __int_as_float(r);
}

// One butterfly step per lane bit o = 16, 8, 4, 2, 1.  While a lane holds
// more than one partial sum it keeps one half (the upper half if bit o of its
// lane is set) and adds the partner's copy of that half; with one sum left it
// adds the partner's sum.  COUNT is the number of sums held before the step.
template <int COUNT, int VP, int STEP>
struct Butterfly {
  __device__ __forceinline__ static void run(float (&v)[VP], int lane, int& base, int& plain_mask) {
    if constexpr (STEP < 5) {
      constexpr int O = 16 >> STEP;
      const bool upper = (lane & O) != 0;
      if constexpr (COUNT > 1) {
        constexpr int HALF = COUNT / 2;
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
          const float send = upper ? v[i] : v[i + HALF];
          const float keep = upper ? v[i + HALF] : v[i];
          v[i] = keep + partner<O>(send);
        }
        if (upper) base += HALF;
        Butterfly<HALF, VP, STEP + 1>::run(v, lane, base, plain_mask);
      } else {
        v[0] += partner<O>(v[0]);
        plain_mask |= O;
        Butterfly<1, VP, STEP + 1>::run(v, lane, base, plain_mask);
      }
    }
  }
};

template <int M, int FMT, int ROWS>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const GemvArgs a) {
  static_assert(ROWS == 4 || ROWS == 8, "a team's rows are a half or a quarter of a 16-row scale group");
  __shared__ uint4 xs[M][kGemvMaxSlabsPerSplit * kChunksPerSlab];

  const int tid = threadIdx.x;
  const int team = tid >> 5;
  const int lane = tid & (kTeamLanes - 1);
  const int split = blockIdx.y;
  const SlabRange sr = split_slabs(a, split);
  const int slab0 = sr.first;
  const int nsl = sr.count;
  // ---- this team's ROWS rows ----
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * (kGemvTeams * ROWS) + team * ROWS;
  const int64_t row_bytes = a.k_pad / 2;
  const uint8_t* cptr = a.codes + row0 * row_bytes + lane * 16;
  // Scales: this team's rows are a half (ROWS = 8) or a quarter (ROWS = 4) of
  // a 16-row scale group, starting at row0 & 15.
  const uint8_t* sptr = a.scales + ((row0 / kRowGroup) * a.ksegs * kRowGroup + (row0 & 15)) * scales_per_seg(FMT);

  float acc[ROWS][M];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  uint4 q[ROWS];
  uint4 sc;
  auto load_slab = [&](int slab, uint4* qq, uint4& s) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
      qq[r] = load_stream16(cptr + r * row_bytes + static_cast<int64_t>(slab) * (kSlabK / 2));
    // Segment (slab * 32 + lane): MXFP4 ROWS bytes (row r at byte r), NVFP4
    // 2 ROWS bytes (row r, group j at byte 2r + j).
    const uint8_t* sp = sptr + (static_cast<int64_t>(slab) * kTeamLanes + lane) * kRowGroup * scales_per_seg(FMT);
    if constexpr (FMT == kFmtMxfp4 && ROWS == 4) {
      s = make_uint4(*reinterpret_cast<const uint32_t*>(sp), 0u, 0u, 0u);
    } else if constexpr (FMT == kFmtMxfp4 || ROWS == 4) {
      const uint2 t = *reinterpret_cast<const uint2*>(sp);
      s = make_uint4(t.x, t.y, 0u, 0u);
    } else {
      s = *reinterpret_cast<const uint4*>(sp);
    }
  };

  // Start the weight stream first, then stage x while those loads fly.
  load_slab(slab0, q, sc);
  stage_x<M>(a, slab0, nsl, xs, [](int, int cc) { return xs_index(cc >> 2, cc & 3); });
  for (int j = 0; j < nsl; ++j) {
    uint4 qn[ROWS];
    uint4 scn = sc;
    if (j + 1 < nsl) load_slab(slab0 + j + 1, qn, scn);
    const int lb = j * kTeamLanes + lane;  // lane block within the staged x

    if constexpr (FMT == kFmtMxfp4) {
      float sop[ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
        sop[r] = e8m0_as_scale_operand((r < 4 ? sc.x : sc.y) >> (8 * (r & 3)));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint4 xv[M];
#pragma unroll
        for (int m = 0; m < M; ++m) xv[m] = xs[m][xs_index(lb, c)];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const uint32_t word = u4_get(q[r], c);
          const bf16x2_t w0 = cvt_fp4x2_bf16<0>(word, sop[r]);
          const bf16x2_t w1 = cvt_fp4x2_bf16<1>(word, sop[r]);
          const bf16x2_t w2 = cvt_fp4x2_bf16<2>(word, sop[r]);
          const bf16x2_t w3 = cvt_fp4x2_bf16<3>(word, sop[r]);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float t = acc[r][m];
            t = dot2_bf16(w0, xv[m].x, t);
            t = dot2_bf16(w1, xv[m].y, t);
            t = dot2_bf16(w2, xv[m].z, t);
            t = dot2_bf16(w3, xv[m].w, t);
            acc[r][m] = t;
          }
        }
      }
    } else {
      // Two NVFP4 groups of 16 codes per lane per slab: chunks {0,1} and {2,3}.
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        uint4 xv[2][M];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int m = 0; m < M; ++m) xv[h][m] = xs[m][xs_index(lb, 2 * grp + h)];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const uint32_t sw = u4_get(sc, r >> 1);
          float s;
          switch (2 * (r & 1) + grp) {
            case 0: s = e4m3_to_f32<0>(sw); break;
            case 1: s = e4m3_to_f32<1>(sw); break;
            case 2: s = e4m3_to_f32<2>(sw); break;
            default: s = e4m3_to_f32<3>(sw); break;
          }
          bf16x2_t w[8];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t word = u4_get(q[r], 2 * grp + h);
            w[4 * h + 0] = cvt_fp4x2_bf16<0>(word, 1.0f);
            w[4 * h + 1] = cvt_fp4x2_bf16<1>(word, 1.0f);
            w[4 * h + 2] = cvt_fp4x2_bf16<2>(word, 1.0f);
            w[4 * h + 3] = cvt_fp4x2_bf16<3>(word, 1.0f);
          }
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float p = 0.0f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              p = dot2_bf16(w[4 * h + 0], xv[h][m].x, p);
              p = dot2_bf16(w[4 * h + 1], xv[h][m].y, p);
              p = dot2_bf16(w[4 * h + 2], xv[h][m].z, p);
              p = dot2_bf16(w[4 * h + 3], xv[h][m].w, p);
            }
            acc[r][m] = __builtin_fmaf(p, s, acc[r][m]);
          }
        }
      }
    }
    if (j + 1 < nsl) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) q[r] = qn[r];
      sc = scn;
    }
  }

  // ---- transposing butterfly over the team's 32 lanes ----
  // V partial sums per lane (index r*M + m), padded with zeros to a power of
  // two so that every halving step splits evenly.
  constexpr int V = ROWS * M;
  constexpr int VP = V <= 8 ? 8 : V <= 16 ? 16 : V <= 32 ? 32 : 64;
  float v[VP];
#pragma unroll
  for (int i = 0; i < VP; ++i) v[i] = 0.0f;
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) v[r * M + m] = acc[r][m];

  int base = 0;        // index of v[0] in the original numbering
  int plain_mask = 0;  // lane bits summed over without halving
  constexpr int kFinal = VP > 32 ? VP / 32 : 1;
  Butterfly<VP, VP, 0>::run(v, lane, base, plain_mask);

  __shared__ TileArgmax ta;
  __shared__ ActTile<M> at;
  ArgmaxLocal<M> al;
  const bool argmax_here = a.keys != nullptr && a.splits == 1;
  const bool act_here = a.act != 0 && a.splits == 1;
  if (argmax_here) tile_argmax_begin(ta, al);
  if ((lane & plain_mask) == 0) {
#pragma unroll
    for (int i = 0; i < kFinal; ++i) {
      const int idx = base + i;
      if (idx < V) {
        const int r = idx / M;
        const int m = idx - r * M;
        const int64_t row = row0 + r;
        const int h = static_cast<int>(row / a.n_proj_pad);
        const int64_t lr = row - static_cast<int64_t>(h) * a.n_proj_pad;
        if (act_here) {
          at.v[m][team * ROWS + r] = v[i] * (il_proj(row) == 0 ? a.gscale[0] : a.gscale[1]);
        } else if (a.splits == 1) {
          if (lr < a.n_proj) {
            const int64_t col = static_cast<int64_t>(h) * a.n_proj + lr;
            const uint16_t yb = f32_to_bf16_rne(v[i] * a.gscale[h]);
            if (a.y) a.y[static_cast<int64_t>(m) * a.ldy + col] = yb;
            if (argmax_here) tile_argmax_offer(al, m, argmax_key(yb, col));
          }
        } else {
          store_partial(a.partial + (static_cast<int64_t>(split) * M + m) * a.rows_total + row, v[i]);
        }
      }
    }
  }
  if (argmax_here) tile_argmax_end(ta, al, a.keys, blockIdx.x);
  if (act_here) act_store(at, a, static_cast<int64_t>(blockIdx.x) * (kGemvTeams * ROWS), kGemvTeams * ROWS, M);
  if (a.splits > 1) splitk_finish<M>(a, blockIdx.x, split);
}

template <int FMT, int ROWS>
hipError_t launch_gemv_rows(const GemvArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(kThreads);
  switch (a.m) {
    case 1: hipLaunchKernelGGL((gemv_kernel<1, FMT, ROWS>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<2, FMT, ROWS>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_gemv_fmt(const GemvArgs& a, dim3 grid, hipStream_t stream) {
  return a.tile_rows == kGemvTeams * 8 ? launch_gemv_rows<FMT, 8>(a, grid, stream)
                                       : launch_gemv_rows<FMT, 4>(a, grid, stream);
}

}  // namespace

hipError_t launch_gemv(const GemvArgs& a, int fmt, hipStream_t stream, dim3* grid_out, dim3* block_out) {
  if (a.tile_rows != kGemvTeams * 8 && a.tile_rows != kGemvTeams * 4) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(a.rows_total / a.tile_rows), static_cast<unsigned>(a.splits));
  if (grid_out) *grid_out = grid;
  if (block_out) *block_out = dim3(kThreads);
  return fmt == kFmtNvfp4 ? launch_gemv_fmt<kFmtNvfp4>(a, grid, stream)
                          : launch_gemv_fmt<kFmtMxfp4>(a, grid, stream);
}

}  // namespace fp4
