// Decode-shaped W4A16 FP4 GEMM on the matrix cores (m = 3..8 activation rows).
//
// At m rows a VALU GEMV spends m/2 v_dot2 per weight on top of the decode, so
// from m = 3 on it is bound by VALU issue before HBM.  Here the VALU only
// decodes (E2M1 -> bf16) and v_mfma_f32_16x16x32_bf16 does the contraction,
// with the m activation rows zero-padded to 16 in registers: no extra HBM
// bytes.  (Why decode is memory-bound: "MXFP4 decode-graph + gate_up FUSION
// default-ON", vllm.cpp PR #54, step 2.)
//
// Work split.  A 256-thread workgroup (4 waves) owns a 64-row tile and one K
// split; wave w owns rows 16w .. 16w + 15.  K advances 256 codes per stage.
// Each stage is copied global -> LDS by the load-to-LDS path, so the weight
// stream needs no registers; of kDecodeBuffers stage buffers all but the one
// being consumed are in flight (3 buffers measured best on MI355X: 4
// workgroups fit a CU, and more workgroups beat deeper per-workgroup
// pipelines):
//   codes   64 rows x 128 bytes  (8 KiB: one full 128-byte line per row)
//   x       8 rows x 256 bf16    (4 KiB; rows >= m are never read back)
//   scales  of those codes       (1 KiB)
// A wave then reads, per 128-code block, one 16-byte code chunk per lane,
// decodes its 4 words and issues 4 MFMAs against x fragments read from LDS.
//
// Lane l handles row r = l % 16 of the wave's rows and the 32-code segment
// g = l / 16 of a 128-code block.  Word c (8 codes) of the lane's chunk is the
// MFMA's B fragment for k index 8g..8g+7; the A fragment is x[r][same 8 codes]
// (zero for r >= m).  Both operands use that k assignment, so each MFMA sums
// exactly the 32 codes of words c of the 4 segments.
//
// K is split over workgroups when one K range per 64-row tile would leave the
// chip underfilled; the split count depends on (k, rows per projection) only
// (decode_mfma_splits).  Splits meet in the lock-free split-K finish of the
// decode kernels (decode_common.hpp).  Summation order of an output: its
// split's stages in order (MFMA accumulation), then splits in order.  It does
// not depend on m or on fusion, so results are deterministic, batch invariant
// for every m this kernel serves, and the fused gate_up launch equals the two
// separate ones bit for bit.
//
// Scales: MXFP4 is folded into v_cvt_scalef32_pk_bf16_fp4 (the E8M0 byte is
// the exponent operand).  NVFP4's E4M3 scale has a mantissa the conversion
// ignores, so each code pair is converted to f32, multiplied by the scale
// (exact: at most 6 significant bits) and packed to bf16.
#include "decode_common.hpp"
#include "lds_copy.hpp"

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = kDecodeThreads;  // 4 waves
constexpr int kRows = kDecodeTileRows;     // 64
constexpr int kStageK = kDecodeStageK;     // 256 codes
constexpr int kWChunks = kRows * kStageK / 2 / 16;  // 512 code chunks per stage
constexpr int kXChunks = 8 * kStageK * 2 / 16;      // 256 x chunks per stage (8 rows)
constexpr int kSChunks = 64;                        // scale chunks per stage (1 KiB)
constexpr int kWPer = kWChunks / kThreads;          // 2 copies per lane
static_assert(kXChunks == kThreads, "one x copy per lane");
static_assert(kRows == 64 && kStageK == 256, "layout below assumes 64 x 256 stages");

struct alignas(16) Stage {
  uint4 w[kWChunks];
  uint4 x[kXChunks];
  uint4 s[kSChunks];
};

union Frag {
  bf16x8_t v;
  uint32_t u[4];
};

// LDS bank layout on gfx950: 64 banks of 4 bytes; a 16-byte-per-lane read is
// served 16 lanes at a time and is conflict-free when those 16 lanes touch 16
// different 16-byte bank groups (address / 16 mod 16).
//
// Codes: row rr holds 8 chunks of 16 bytes at rr * 128, chunk c in slot
// c ^ ((rr >> 1) & 7); the 16 lanes reading one chunk index of 16 consecutive
// rows hit bank groups 8 (rr & 1) + slot, all distinct.
__device__ __forceinline__ int w_slot(int rr, int c) { return rr * 8 + (c ^ ((rr >> 1) & 7)); }
// x: row xr (0..7) holds 32 chunks of 8 bf16 at xr * 512, chunk ch in slot
// ch ^ xr: the m <= 8 rows read together hit distinct bank groups.
__device__ __forceinline__ int x_slot(int xr, int ch) { return xr * 32 + (ch ^ xr); }

// Load-to-LDS copies a wave issues per stage: 2 code chunks and 1 x chunk
// per lane, plus one scale chunk per lane in wave 0.
constexpr int kLoadsPerStage = kWPer + 1;

template <int STAGES>
__device__ __forceinline__ void wait_stages_barrier(int wave) {
  if (wave == 0)
    wait_vm_barrier<STAGES * (kLoadsPerStage + 1)>();
  else
    wait_vm_barrier<STAGES * kLoadsPerStage>();
}

// The stage copies of one workgroup: 32-bit lane offsets from wave-uniform
// bases that advance with k.  x rows >= m all fetch the first 16 bytes of x
// (never read back).  In a stage that straddles k (k not a multiple of 256),
// x chunks at or past k are fetched from the zero padding of the prepared
// code rows: every code row then holds at least 32 zero codes from code k on.
template <int M, int FMT>
struct Copier {
  static constexpr int P = scales_per_seg(FMT);
  const uint16_t* x;
  const uint8_t* ct;     // code row row0
  const uint8_t* st;     // scale row group row0 / 16
  const uint8_t* zeros;  // 16 zero bytes
  uint32_t woff[kWPer], xoff, soff;
  int xk;                // first code of this lane's x chunk within a stage
  bool xrow_ok;
  int k;
  uint32_t lds_wave;     // this wave's 1 KiB slice of a stage area

  __device__ __forceinline__ Copier(const GemvArgs& a, int64_t row0, int t, int wave) {
    const int64_t row_bytes = a.k_pad / 2;
    k = a.k;
    x = a.x;
    ct = a.codes + row0 * row_bytes;
    st = a.scales + (row0 / kRowGroup) * a.ksegs * kRowGroup * P;
    zeros = ct + a.k / 2;
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int p = i * kThreads + t;
      const int rr = p >> 3;
      const int c = (p & 7) ^ ((rr >> 1) & 7);
      woff[i] = static_cast<uint32_t>(rr * row_bytes + 16 * c);
    }
    const int xr = t >> 5;
    const int ch = (t & 31) ^ xr;
    xrow_ok = xr < M;
    xoff = xrow_ok ? static_cast<uint32_t>((static_cast<int64_t>(xr) * a.k + 8 * ch) * 2) : 0u;
    xk = 8 * ch;
    // Scales: 4 row groups x 8 segments x 16 rows x P bytes, 128 P contiguous
    // bytes per row group.  MXFP4 fills 32 chunks; lanes 32..63 repeat them.
    const int lane = t & 63;
    const int cpg = 8 * P;  // chunks per row group
    const int ps = lane % (4 * cpg);
    soff = static_cast<uint32_t>((ps / cpg) * a.ksegs * kRowGroup * P + 16 * (ps % cpg));
    lds_wave = 64 * 16 * wave;
  }

  __device__ __forceinline__ void issue(int64_t k0, Stage& sb, int wave) const {
    const uint32_t lw = lds_addr(sb.w) + lds_wave;
    const uint8_t* cb = ct + k0 / 2;
#pragma unroll
    for (int i = 0; i < kWPer; ++i) copy16_sbase(cb, woff[i], lw + i * kThreads * 16);
    const bool in_k = k0 + xk < k;
    const void* xs = !xrow_ok ? static_cast<const void*>(x)
                     : in_k   ? static_cast<const void*>(reinterpret_cast<const uint8_t*>(x + k0) + xoff)
                              : static_cast<const void*>(zeros);
    copy16_vaddr(xs, lds_addr(sb.x) + lds_wave);
    if (wave == 0) copy16_sbase(st + (k0 / 32) * kRowGroup * P, soff, lds_addr(sb.s));
  }
};

template <int FMT>
__device__ __forceinline__ void decode_word(uint32_t word, uint32_t sbyte, Frag& f) {
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

// A fragments of the padding rows r >= m come from a 512-byte zero row in
// LDS instead of the stage (no per-read masking).  All such lanes read the
// same chunk address; the row sits at 128 mod 256 bytes, so its bank group
// (ch + 8 mod 16) differs from those of the real rows (ch ^ r, r < 8).
struct alignas(256) ZeroRow {
  uint4 pad[8];
  uint4 z[32];
};

// One stage for this wave: 2 blocks of 128 codes x 4 MFMA steps.  xrow: this
// lane's x row (r < m: its slots in the stage; else the zero row).
template <int M, int FMT>
__device__ __forceinline__ void compute_stage(const Stage& sb, const uint4* zrow, int wave, int r, int g,
                                              f32x4_t& acc) {
  constexpr int P = scales_per_seg(FMT);
  const int rr = 16 * wave + r;
  const uint8_t* sbytes = reinterpret_cast<const uint8_t*>(sb.s);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint4 code = sb.w[w_slot(rr, 4 * q + g)];
    const int so = ((wave * 8 + 4 * q + g) * kRowGroup + r) * P;
    uint32_t s0, s1;
    if constexpr (P == 2) {
      const uint32_t s2 = *reinterpret_cast<const uint16_t*>(sbytes + so);
      s0 = s2 & 0xFFu;
      s1 = s2 >> 8;
    } else {
      s0 = s1 = sbytes[so];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ch = 16 * q + 4 * g + c;
      const uint4 xv = r < M ? sb.x[x_slot(r, ch)] : zrow[ch];
      Frag af, wf;
      af.u[0] = xv.x;
      af.u[1] = xv.y;
      af.u[2] = xv.z;
      af.u[3] = xv.w;
      const uint32_t word = c == 0 ? code.x : c == 1 ? code.y : c == 2 ? code.z : code.w;
      decode_word<FMT>(word, c < 2 ? s0 : s1, wf);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af.v, wf.v, acc, 0, 0, 0);
    }
  }
}

// Wait until stage s has landed -- with NB buffers, up to NB - 2 younger
// stages stay in flight -- and join the workgroup barrier.
template <int NB>
__device__ __forceinline__ void wait_for_stage(int s, int s1, int wave) {
  if constexpr (NB > 2) {
    if (s + NB - 2 < s1) {
      wait_stages_barrier<NB - 2>(wave);
      return;
    }
    wait_for_stage<NB - 1>(s, s1, wave);
  } else {
    wait_stages_barrier<0>(wave);
  }
}

// Step for stage s in buffer `cur`: wait for it at the workgroup barrier,
// refill the buffer consumed one step ago (`prev`; every wave is past it)
// with stage s + NB - 1, consume `cur`.
template <int M, int FMT, int NB>
__device__ __forceinline__ void pipeline_step(const Copier<M, FMT>& cp, int s, int s1, const Stage& cur, Stage& prev,
                                              const uint4* zrow, int wave, int r, int g, f32x4_t& acc) {
  wait_for_stage<NB>(s, s1, wave);
  if (s + NB - 1 < s1) cp.issue(static_cast<int64_t>(s + NB - 1) * kStageK, prev, wave);
  compute_stage<M, FMT>(cur, zrow, wave, r, g, acc);
}

template <int M, int FMT, int NB>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(const GemvArgs a) {
  __shared__ Stage st[NB];
  __shared__ ZeroRow zero_row;

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int64_t row0 = static_cast<int64_t>(tile) * kRows;
  const int ksteps = (a.k + kStageK - 1) / kStageK;
  const int s0 = static_cast<int>(static_cast<int64_t>(split) * ksteps / a.splits);
  const int s1 = static_cast<int>(static_cast<int64_t>(split + 1) * ksteps / a.splits);

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (t < 32) zero_row.z[t] = make_uint4(0u, 0u, 0u, 0u);  // visible after the first stage barrier
  const Copier<M, FMT> cp(a, row0, t, wave);
#pragma unroll
  for (int j = 0; j < NB - 1; ++j)
    if (s0 + j < s1) cp.issue(static_cast<int64_t>(s0 + j) * kStageK, st[j], wave);
  for (int s = s0; s < s1; s += NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (s + j >= s1) break;
      pipeline_step<M, FMT, NB>(cp, s + j, s1, st[j], st[(j + NB - 1) % NB], zero_row.z, wave, r, g, acc);
    }
  }

  // Lane (r, g) holds C[m = 4g + i][row 16 wave + r].
  const int64_t row = row0 + 16 * wave + r;
  if (a.splits == 1) {
    int h;
    const int64_t col = out_col(a, row, h);
    if (col >= 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < M) a.y[static_cast<int64_t>(m) * a.ldy + col] = f32_to_bf16_rne(acc[i] * a.gscale[h]);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * g + i;
    if (m < M) store_partial(a.partial + (static_cast<int64_t>(split) * M + m) * a.rows_total + row, acc[i]);
  }
  splitk_finish<M>(a, tile, split);
}

template <int FMT>
hipError_t launch_fmt(const GemvArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(kThreads);
  switch (a.m) {
    case 3: hipLaunchKernelGGL((decode_mfma_kernel<3, FMT, kDecodeBuffers>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<4, FMT, kDecodeBuffers>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((decode_mfma_kernel<5, FMT, kDecodeBuffers>), grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL((decode_mfma_kernel<6, FMT, kDecodeBuffers>), grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL((decode_mfma_kernel<7, FMT, kDecodeBuffers>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_mfma_kernel<8, FMT, kDecodeBuffers>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const GemvArgs& a, int fmt, hipStream_t stream, dim3* grid_out, dim3* block_out) {
  const dim3 grid(static_cast<unsigned>(a.rows_total / kRows), static_cast<unsigned>(a.splits));
  if (grid_out) *grid_out = grid;
  if (block_out) *block_out = dim3(kThreads);
  return fmt == kFmtNvfp4 ? launch_fmt<kFmtNvfp4>(a, grid, stream) : launch_fmt<kFmtMxfp4>(a, grid, stream);
}

}  // namespace fp4
