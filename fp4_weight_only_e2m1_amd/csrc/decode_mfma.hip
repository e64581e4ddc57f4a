// Decode-shaped W4A16 FP4 GEMM on the matrix cores (m = 3..32 activation rows).
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
//   x       XR rows x 256 bf16   (XR = 4, 8, 16 or 32 for m <= 4, 8, 16, 32:
//                                 2 to 16 KiB; rows >= m are never read back)
//   scales  of those codes       (1 KiB)
// A wave then reads, per 128-code block, one 16-byte code chunk per lane,
// decodes its 4 words and issues 4 MFMAs against x fragments read from LDS.
// The same code serves two other tile shapes (decode_mfma_tile_rows):
// 128-row tiles, whose waves own two 16-row blocks each (every x fragment
// read from LDS feeds two MFMAs), and 96-row tiles of six waves, launched
// where 64-row tiles would give CUs unequal workgroup counts (the 24576-row
// fused gate_up: 256 workgroups, one per CU, instead of 384); there waves
// 0..3 copy x and the others the scales, and MXFP4 keeps 4 stage buffers.
//
// Lane l handles row r = l % 16 of the wave's rows and the 32-code segment
// g = l / 16 of a 128-code block.  Word c (8 codes) of the lane's chunk is the
// MFMA's B fragment for k index 8g..8g+7; the A fragment is x[r][same 8 codes]
// (zero for r >= m).  Both operands use that k assignment, so each MFMA sums
// exactly the 32 codes of words c of the 4 segments.  Calls of more than 16
// rows run a second MFMA per decoded fragment on activation rows 16 + r, into
// a second accumulator (the same sums, in the same order, for those rows).
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
constexpr int kStageK = kDecodeStageK;     // 256 codes
static_assert(kStageK == 256, "layout below assumes stages of 256 codes");

// x rows staged per stage for calls of up to M activation rows: the next
// power of two from 4 (staging 4 rows instead of 8 at m = 3, 4 halves the x
// copies; measured on MI355X, us: MXFP4 24576 x 4096 m = 4 12.1 -> 11.9,
// the NVFP4 248320 x 5120 head m = 4 128.9 -> 127.0, NVFP4 5120 x 17408
// m = 4 15.6 -> 15.0).
template <int M>
constexpr int kXRows = M > 16 ? 32 : M > 8 ? 16 : M > 4 ? 8 : 4;
// 16-row activation groups of an instance: one MFMA per group per fragment.
template <int M>
constexpr int kGroups = M > 16 ? 2 : 1;

// Tile geometry for W waves of RB row blocks of 16 (a 16 RB W-row tile) and
// XR staged x rows.  Every lane copies 2 RB code chunks per stage; the x
// chunks are copied kXPer per lane by the first kXWaves waves (all of them
// when there are at least as many chunks as lanes), and the scale chunks by
// kSWaves waves from kSWave0 on -- waves without x copies where there are
// enough of those, so that the copies per wave stay even.
template <int RB, int FMT, int XR, int W>
struct Geo {
  static constexpr int kThr = 64 * W;
  static constexpr int kXChunks = XR * kStageK * 2 / 16;  // 256, 512 or 1024 x chunks per stage
  static constexpr int kXWaves = kXChunks >= kThr ? W : kXChunks / 64;
  static constexpr int kXPer = kXChunks / (64 * kXWaves);  // x copies per lane of those waves
  static constexpr int kRows = 16 * RB * W;
  static constexpr int kWChunks = kRows * kStageK / 2 / 16;  // code chunks per stage
  static constexpr int kWPer = kWChunks / kThr;               // 2 RB copies per lane
  static constexpr int P = scales_per_seg(FMT);
  static constexpr int kSReal = 8 * P * RB * W;               // scale chunks of a stage
  static constexpr int kSWaves = (kSReal + 63) / 64;          // waves that copy them
  static constexpr int kSWave0 = W - kXWaves >= kSWaves ? W - kSWaves : 0;
  static constexpr int kSChunks = 64 * kSWaves;               // incl. unused duplicates
  static_assert(kXChunks % (64 * kXWaves) == 0 && kWChunks % kThr == 0, "copy split");
  __device__ static constexpr bool has_x(int wave) { return kXWaves == W || wave < kXWaves; }
  __device__ static constexpr bool has_s(int wave) { return wave >= kSWave0 && wave < kSWave0 + kSWaves; }
};

template <int RB, int FMT, int XR, int W>
struct alignas(16) Stage {
  uint4 w[Geo<RB, FMT, XR, W>::kWChunks];
  uint4 x[Geo<RB, FMT, XR, W>::kXChunks];
  uint4 s[Geo<RB, FMT, XR, W>::kSChunks];
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
// x: row xr (0..XR-1) holds 32 chunks of 8 bf16 at xr * 512, chunk ch in
// slot ch ^ xr: the rows read together hit distinct bank groups.
__device__ __forceinline__ int x_slot(int xr, int ch) { return xr * 32 + (ch ^ xr); }

// Wait until this wave's copies of all but the STAGES youngest stages have
// landed, then join the workgroup barrier.
template <int RB, int FMT, int XR, int W, int STAGES>
__device__ __forceinline__ void wait_stages_barrier(int wave) {
  using G = Geo<RB, FMT, XR, W>;
  if (G::has_x(wave)) {
    if (G::has_s(wave))
      wait_vm_barrier<STAGES * (G::kWPer + G::kXPer + 1)>();
    else
      wait_vm_barrier<STAGES * (G::kWPer + G::kXPer)>();
  } else {
    if (G::has_s(wave))
      wait_vm_barrier<STAGES * (G::kWPer + 1)>();
    else
      wait_vm_barrier<STAGES * G::kWPer>();
  }
}

// x row that activation row xr of a call (or of a grouped MoE pass) reads:
// xr itself, or the pass's token id for it.  Rows past m (ok false) and
// token ids outside [0, tokens_total) read row 0: the former are never
// stored, the latter have their sums zeroed (bad_token_rows).
__device__ __forceinline__ int x_row_of(const GemvArgs& a, int xr, bool ok) {
  if (!ok) return 0;
  if (!a.row_tokens) return xr;
  const int tok = a.row_tokens[xr];
  return tok < 0 || tok >= a.tokens_total ? 0 : tok;
}

// Bit r set: activation row r (< mrows <= 32) of a grouped MoE pass has a
// token id outside [0, tokens_total), so its outputs are zero (the sums of a
// zero x row).  0 outside the grouped MoE decode.  Workgroup-uniform.
__device__ __forceinline__ uint32_t bad_token_rows(const GemvArgs& a, int mrows) {
  uint32_t bad = 0;
  if (a.row_tokens) {
    for (int r = 0; r < mrows; ++r) {
      const int tok = a.row_tokens[r];
      if (tok < 0 || tok >= a.tokens_total) bad |= 1u << r;
    }
  }
  return bad;
}

// The stage copies of one workgroup: 32-bit lane offsets from wave-uniform
// bases that advance with k.  x rows >= m all fetch the first 16 bytes of x
// (never read back).  In a stage that straddles k (k not a multiple of 256),
// x chunks at or past k are fetched from the zero padding of the prepared
// code rows: every code row then holds at least 32 zero codes from code k on.
// Code chunks are fetched with the non-temporal hint (read once); x and the
// scales with the default policy.
template <int M, int FMT, int RB, int W, bool GATHER = false>
struct Copier {
  static constexpr int XR = kXRows<M>;
  using G = Geo<RB, FMT, XR, W>;
  static constexpr int P = G::P;
  const uint16_t* x;
  const uint8_t* ct;     // code row row0
  const uint8_t* st;     // scale row group row0 / 16
  const uint8_t* zeros;  // 16 zero bytes
  uint32_t woff[G::kWPer], xoff[G::kXPer], soff;
  const uint8_t* xrp[GATHER ? G::kXPer : 1];  // GATHER: this lane's x chunk at k = 0
  int xk[G::kXPer];      // first code of this lane's x chunks within a stage
  bool xrow_ok[G::kXPer];
  int k;
  uint32_t lds_wave;     // this wave's 1 KiB slice of the code and x areas
  uint32_t lds_swave;    // this wave's 1 KiB slice of the scale area

  __device__ __forceinline__ Copier(const GemvArgs& a, int64_t row0, int t, int wave, int mrows) {
    const int64_t row_bytes = a.k_pad / 2;
    k = a.k;
    x = a.x;
    ct = a.codes + row0 * row_bytes;
    st = a.scales + (row0 / kRowGroup) * a.ksegs * kRowGroup * P;
    zeros = ct + a.k / 2;
#pragma unroll
    for (int i = 0; i < G::kWPer; ++i) {
      const int p = i * G::kThr + t;
      const int rr = p >> 3;
      const int c = (p & 7) ^ ((rr >> 1) & 7);
      woff[i] = static_cast<uint32_t>(rr * row_bytes + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < G::kXPer; ++i) {
      const int p = i * 64 * G::kXWaves + t;
      const int xr = p >> 5;
      const int ch = (p & 31) ^ xr;
      xrow_ok[i] = xr < mrows;
      if constexpr (GATHER) {
        xrp[i] = reinterpret_cast<const uint8_t*>(a.x + static_cast<int64_t>(x_row_of(a, xr, xrow_ok[i])) * a.k) +
                 16 * ch;
        xoff[i] = 0;
      } else {
        xoff[i] = xrow_ok[i] ? static_cast<uint32_t>((static_cast<int64_t>(xr) * a.k + 8 * ch) * 2) : 0u;
      }
      xk[i] = 8 * ch;
    }
    // Scales of a stage: RB W row groups x 8 segments x 16 rows x P bytes,
    // 128 P contiguous bytes per row group (cpg chunks).  Lane l of scale
    // wave kSWave0 + v lands at chunk 64 v + l of the stage's scale area and
    // fetches chunk (64 v + l) mod kSReal; where kSReal is not a multiple of
    // 64 the upper lanes fetch duplicates into unused chunks.
    const int lane = t & 63;
    const int cpg = 8 * P;
    const int sv = G::has_s(wave) ? wave - G::kSWave0 : 0;
    const int q = (64 * sv + lane) % G::kSReal;
    soff = static_cast<uint32_t>((q / cpg) * a.ksegs * kRowGroup * P + 16 * (q % cpg));
    lds_wave = 64 * 16 * wave;
    lds_swave = 64 * 16 * sv;
  }

  __device__ __forceinline__ const void* x_src(int i, int64_t k0) const {
    if constexpr (GATHER)
      return xrp[i] + 2 * k0;
    else
      return reinterpret_cast<const uint8_t*>(x + k0) + xoff[i];
  }

  __device__ __forceinline__ void issue(int64_t k0, Stage<RB, FMT, XR, W>& sb, int wave) const {
    const uint32_t lw = lds_addr(sb.w) + lds_wave;
    const uint8_t* cb = ct + k0 / 2;
#pragma unroll
    for (int i = 0; i < G::kWPer; ++i) copy16_sbase_nt(cb, woff[i], lw + i * G::kThr * 16);
    if (G::has_x(wave)) {
#pragma unroll
      for (int i = 0; i < G::kXPer; ++i) {
        const bool in_k = k0 + xk[i] < k;
        const void* xs = !xrow_ok[i] ? static_cast<const void*>(x)
                         : in_k      ? x_src(i, k0)
                                     : static_cast<const void*>(zeros);
        copy16_vaddr(xs, lds_addr(sb.x) + lds_wave + i * 64 * G::kXWaves * 16);
      }
    }
    if (G::has_s(wave)) copy16_sbase(st + (k0 / 32) * kRowGroup * P, soff, lds_addr(sb.s) + lds_swave);
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

// One stage for this wave: 2 blocks of 128 codes x 4 MFMA steps for each of
// its RB row blocks and J activation groups; each x fragment read from LDS
// feeds RB MFMAs, each decoded weight fragment J.  zrow: the zero row the
// lanes of rows >= m read instead of x.  XW > 0 (the wave-split kernel, whose
// stages hold XW x rows and no zero row): the lanes of activation row r read
// staged row r mod XW instead; rows past m then hold other rows' or stale
// values, which only reach outputs of rows past m (row r of the product
// depends on row r of x alone), and those are never stored.
template <int M, int FMT, int RB, typename StageT, int XW = 0>
__device__ __forceinline__ void compute_stage(const StageT& sb, const uint4* zrow, int wave, int r, int g,
                                              int mrows, f32x4_t (&acc)[RB][kGroups<M>]) {
  constexpr int J = kGroups<M>;
  constexpr int P = scales_per_seg(FMT);
  const uint8_t* sbytes = reinterpret_cast<const uint8_t*>(sb.s);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    uint4 code[RB];
    uint32_t s0[RB], s1[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int blk = RB * wave + b;  // row group of this block
      code[b] = sb.w[w_slot(16 * blk + r, 4 * q + g)];
      const int so = ((blk * 8 + 4 * q + g) * kRowGroup + r) * P;
      if constexpr (P == 2) {
        const uint32_t s2 = *reinterpret_cast<const uint16_t*>(sbytes + so);
        s0[b] = s2 & 0xFFu;
        s1[b] = s2 >> 8;
      } else {
        s0[b] = s1[b] = sbytes[so];
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ch = 16 * q + 4 * g + c;
      Frag af[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int xr = 16 * j + r;
        uint4 xv;
        if constexpr (XW > 0)
          xv = sb.x[x_slot(xr & (XW - 1), ch)];
        else
          xv = xr < mrows ? sb.x[x_slot(xr, ch)] : zrow[ch];
        af[j].u[0] = xv.x;
        af[j].u[1] = xv.y;
        af[j].u[2] = xv.z;
        af[j].u[3] = xv.w;
      }
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        Frag wf;
        const uint32_t word = c == 0 ? code[b].x : c == 1 ? code[b].y : c == 2 ? code[b].z : code[b].w;
        decode_word<FMT>(word, c < 2 ? s0[b] : s1[b], wf);
#pragma unroll
        for (int j = 0; j < J; ++j)
          acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j].v, wf.v, acc[b][j], 0, 0, 0);
      }
    }
  }
}

// Wait until stage s has landed -- with NB buffers, up to NB - 2 younger
// stages stay in flight -- and join the workgroup barrier.
template <int RB, int FMT, int XR, int W, int NB>
__device__ __forceinline__ void wait_for_stage(int s, int s1, int wave) {
  if constexpr (NB > 2) {
    if (s + NB - 2 < s1) {
      wait_stages_barrier<RB, FMT, XR, W, NB - 2>(wave);
      return;
    }
    wait_for_stage<RB, FMT, XR, W, NB - 1>(s, s1, wave);
  } else {
    wait_stages_barrier<RB, FMT, XR, W, 0>(wave);
  }
}

// Step for stage s in buffer `cur`: wait for it at the workgroup barrier,
// refill the buffer consumed one step ago (`prev`; every wave is past it)
// with stage s + NB - 1, consume `cur`.
template <int M, int FMT, int RB, int NB, int W, bool GATHER>
__device__ __forceinline__ void pipeline_step(const Copier<M, FMT, RB, W, GATHER>& cp, int s, int s1,
                                              const Stage<RB, FMT, kXRows<M>, W>& cur,
                                              Stage<RB, FMT, kXRows<M>, W>& prev, const uint4* zrow, int wave, int r,
                                              int g, int mrows, f32x4_t (&acc)[RB][kGroups<M>]) {
  wait_for_stage<RB, FMT, kXRows<M>, W, NB>(s, s1, wave);
  if (s + NB - 1 < s1) cp.issue(static_cast<int64_t>(s + NB - 1) * kStageK, prev, wave);
  compute_stage<M, FMT, RB>(cur, zrow, wave, r, g, mrows, acc);
}

// One (tile, split) of a decode call with mrows <= M activation rows (M when
// launched per call; the rows of one expert in the grouped MoE launch), on a
// workgroup of W waves; GATHER: the grouped MoE decode, activation row r
// being x row a.row_tokens[r].
template <int M, int FMT, int RB, int NB, int W, bool GATHER = false>
__device__ __forceinline__ void decode_tile(const GemvArgs& a, int tile, int split, int mrows) {
  __shared__ Stage<RB, FMT, kXRows<M>, W> st[NB];
  __shared__ ZeroRow zero_row;
  constexpr int kRows = Geo<RB, FMT, kXRows<M>, W>::kRows;

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(tile) * kRows;
  const int ksteps = (a.k + kStageK - 1) / kStageK;
  const int s0 = static_cast<int>(static_cast<int64_t>(split) * ksteps / a.splits);
  const int s1 = static_cast<int>(static_cast<int64_t>(split + 1) * ksteps / a.splits);

  constexpr int J = kGroups<M>;
  f32x4_t acc[RB][J];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int j = 0; j < J; ++j) acc[b][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (t < 32) zero_row.z[t] = make_uint4(0u, 0u, 0u, 0u);  // visible after the first stage barrier
  const uint32_t bad = GATHER ? bad_token_rows(a, mrows) : 0u;
  const Copier<M, FMT, RB, W, GATHER> cp(a, row0, t, wave, mrows);
#pragma unroll
  for (int j = 0; j < NB - 1; ++j)
    if (s0 + j < s1) cp.issue(static_cast<int64_t>(s0 + j) * kStageK, st[j], wave);
  for (int s = s0; s < s1; s += NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (s + j >= s1) break;
      pipeline_step<M, FMT, RB, NB, W, GATHER>(cp, s + j, s1, st[j], st[(j + NB - 1) % NB], zero_row.z, wave, r, g,
                                       mrows, acc);
    }
  }

  // Lane (r, g) holds C[m = 16j + 4g + i][row 16 (RB wave + b) + r] in
  // acc[b][j][i].
  if (GATHER && bad) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((bad >> (16 * j + 4 * g + i)) & 1u) acc[b][j][i] = 0.0f;
  }
  if (a.splits == 1) {
    // Greedy-argmax keys: lane (r, g) only ever holds activation rows
    // 16j + 4g .. 16j + 4g + 3, so each row's maximum is taken over the 16
    // lanes of group g (lane exchanges within the group), then across the
    // waves.
    __shared__ TileArgmax ta;
    uint64_t best[J][4];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) best[j][i] = 0;
    if constexpr (M <= kDecodeActMaxM) {
      __shared__ ActTile<M> at;
      if (a.act) {
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const int rl = 16 * (RB * wave + b) + r;
          const float gs = il_proj(row0 + rl) == 0 ? a.gscale[0] : a.gscale[1];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * g + i < mrows) at.v[4 * g + i][rl] = acc[b][0][i] * gs;
        }
        act_store(at, a, row0, kRows, mrows);
        return;
      }
    }
    if (a.keys) {
      if (t < kDecodeMaxM) ta.best[t] = 0ull;
      __syncthreads();
    }
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int64_t row = row0 + 16 * (RB * wave + b) + r;
      int h;
      const int64_t col = out_col(a, row, h);
      if (col >= 0) {
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 16 * j + 4 * g + i;
            if (m < mrows) {
              const uint16_t yb = f32_to_bf16_rne(acc[b][j][i] * (h == 0 ? a.gscale[0] : a.gscale[1]));
              if (a.y) a.y[static_cast<int64_t>(m) * a.ldy + col] = yb;
              const uint64_t key = argmax_key(yb, col);
              if (key > best[j][i]) best[j][i] = key;
            }
          }
      }
    }
    if (a.keys) {
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) {
            const uint64_t w = shfl_xor_u64(best[j][i], o);
            if (w > best[j][i]) best[j][i] = w;
          }
          const int m = 16 * j + 4 * g + i;
          if (r == 0 && m < M) atomicMax(&ta.best[m], static_cast<unsigned long long>(best[j][i]));
        }
      __syncthreads();
      if (t < M) a.keys[static_cast<int64_t>(tile) * M + t] = ta.best[t];
    }
    return;
  }
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int64_t row = row0 + 16 * (RB * wave + b) + r;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * j + 4 * g + i;
        if (m < M)
          store_partial(a.partial + (static_cast<int64_t>(split) * M + m) * a.rows_total + row, acc[b][j][i]);
      }
  }
  splitk_finish<M>(a, tile, split);
}

template <int M, int FMT, int RB, int NB, int W>
__global__ __launch_bounds__(64 * W) void decode_mfma_kernel(const GemvArgs a) {
  decode_tile<M, FMT, RB, NB, W>(a, blockIdx.x, blockIdx.y, M);
}

// ---------------------------------------------------------------------------
// Wave-split decode: K split over the waves of one workgroup, for the layers
// decode_kw_used selects (too few rows to fill the chip with whole-K tiles,
// m <= kKwMaxM).
//
// A workgroup owns 16 rows.  Wave w streams stages [w S / 4, (w + 1) S / 4)
// of the S = ceil(k / 256) stages through NB stage buffers of its own --
//   codes   16 rows x 128 bytes   (2 KiB: one full 128-byte line per row)
//   x       XR rows x 256 bf16    (XR = 2, 4, 8 for m <= 2, 4, 8)
//   scales  16 rows x 8 segments x P bytes (256 B NVFP4, 128 B MXFP4)
// -- and waits only for its own copies: no workgroup barrier in the loop.
// The lanes, fragments and MFMAs of a stage are those of the 64-row kernel
// for one row block.  At the end the four waves' sums of each output are
// added in LDS in wave order, so an output's summation order is: its wave's
// stages in order (MFMA accumulation), then the waves 0, 1, 2, 3 in order.
// That order depends on k alone: the same at every m this kernel serves and
// in the fused gate_up launch as in the separate ones.  No partials leave
// the workgroup, so the call needs no workspace and no cross-workgroup
// finish.
template <int M>
constexpr int kKwXRows = M <= 2 ? 2 : M <= 4 ? 4 : 8;

template <int FMT, int XR>
struct alignas(16) KwStage {
  uint4 w[16 * 8];
  uint4 x[XR * 32];
  uint4 s[8 * scales_per_seg(FMT)];
};

template <int M, int FMT, bool GATHER = false>
struct KwCopier {
  static constexpr int XR = kKwXRows<M>;
  static constexpr int P = scales_per_seg(FMT);
  static constexpr int kXPer = XR / 2;      // x copies per lane per stage (2 rows per copy)
  static constexpr int kSLanes = 8 * P;     // lanes that copy a stage's scales
  static constexpr int kLoads = 2 + kXPer + 1;
  const uint16_t* x;
  const uint8_t* ct;     // code row row0
  const uint8_t* st;     // scale row group row0 / 16
  const uint8_t* zeros;  // 16 zero bytes
  uint32_t woff[2], xoff[kXPer];
  const uint8_t* xrp[GATHER ? kXPer : 1];  // GATHER: this lane's x chunk at k = 0
  int xk[kXPer];
  bool xrow_ok[kXPer];
  int k, lane;

  __device__ __forceinline__ KwCopier(const GemvArgs& a, int64_t row0, int lane_, int mrows) {
    const int64_t row_bytes = a.k_pad / 2;
    k = a.k;
    lane = lane_;
    x = a.x;
    ct = a.codes + row0 * row_bytes;
    st = a.scales + (row0 / kRowGroup) * a.ksegs * kRowGroup * P;
    zeros = ct + a.k / 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = i * 64 + lane;
      const int rr = p >> 3;
      const int c = (p & 7) ^ ((rr >> 1) & 7);
      woff[i] = static_cast<uint32_t>(rr * row_bytes + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int p = i * 64 + lane;
      const int xr = p >> 5;
      const int ch = (p & 31) ^ xr;
      xrow_ok[i] = xr < mrows;
      if constexpr (GATHER) {
        xrp[i] = reinterpret_cast<const uint8_t*>(a.x + static_cast<int64_t>(x_row_of(a, xr, xrow_ok[i])) * a.k) +
                 16 * ch;
        xoff[i] = 0;
      } else {
        xoff[i] = xrow_ok[i] ? static_cast<uint32_t>((static_cast<int64_t>(xr) * a.k + 8 * ch) * 2) : 0u;
      }
      xk[i] = 8 * ch;
    }
  }

  __device__ __forceinline__ const void* x_src(int i, int64_t k0) const {
    if constexpr (GATHER)
      return xrp[i] + 2 * k0;
    else
      return reinterpret_cast<const uint8_t*>(x + k0) + xoff[i];
  }

  // Copies of the stage at code k0 into sb: codes (non-temporal), x (chunks
  // at or past k from the codes' zero padding; rows >= m fetch the first
  // chunk of x, never read back into a stored output), and the scales by the
  // first kSLanes lanes.
  __device__ __forceinline__ void issue(int64_t k0, KwStage<FMT, XR>& sb) const {
    const uint8_t* cb = ct + k0 / 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) copy16_sbase_nt(cb, woff[i], lds_addr(sb.w) + i * 64 * 16);
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const bool in_k = k0 + xk[i] < k;
      const void* xs = !xrow_ok[i] ? static_cast<const void*>(x)
                       : in_k      ? x_src(i, k0)
                                   : static_cast<const void*>(zeros);
      copy16_vaddr(xs, lds_addr(sb.x) + i * 64 * 16);
    }
    if (lane < kSLanes) copy16_sbase(st + (k0 / 32) * kRowGroup * P, static_cast<uint32_t>(16 * lane), lds_addr(sb.s));
  }
};

// Wait until at most N of this wave's vector-memory operations are in flight
// and its LDS operations are done (no barrier: the wave-split kernel's waves
// consume only the copies they issued).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// Wait for stage s of a wave's range ending at s1: up to NB - 2 younger
// stages stay in flight.
template <int LOADS, int NB>
__device__ __forceinline__ void kw_wait(int s, int s1) {
  if constexpr (NB > 2) {
    if (s + NB - 2 < s1) {
      wait_vm<(NB - 2) * LOADS>();
      return;
    }
    kw_wait<LOADS, NB - 1>(s, s1);
  } else {
    wait_vm<0>();
  }
}

// One 16-row tile of a wave-split call with mrows <= M activation rows (M when
// launched per call; the rows of one expert's pass in the grouped MoE
// launch).  All threads of the workgroup call it; it reuses its stage buffers
// on the next call only after a workgroup barrier.
template <int M, int FMT, int NB, bool GATHER = false>
__device__ __forceinline__ void kw_tile(const GemvArgs& a, int64_t tile, int mrows) {
  using C = KwCopier<M, FMT, GATHER>;
  using S = KwStage<FMT, C::XR>;
  __shared__ S st[kKwWaves][NB];
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t row0 = tile * kKwRows;
  const int ksteps = (a.k + kDecodeStageK - 1) / kDecodeStageK;
  const int s0 = wave * ksteps / kKwWaves;
  const int s1 = (wave + 1) * ksteps / kKwWaves;

  f32x4_t acc[1][1];
  acc[0][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  S* mine = st[wave];
  const uint32_t bad = GATHER ? bad_token_rows(a, mrows) : 0u;
  const C cp(a, row0, lane, mrows);
#pragma unroll
  for (int j = 0; j < NB - 1; ++j)
    if (s0 + j < s1) cp.issue(static_cast<int64_t>(s0 + j) * kDecodeStageK, mine[j]);
  for (int s = s0; s < s1; s += NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int ss = s + j;
      if (ss >= s1) break;
      kw_wait<C::kLoads, NB>(ss, s1);
      if (ss + NB - 1 < s1) cp.issue(static_cast<int64_t>(ss + NB - 1) * kDecodeStageK, mine[(j + NB - 1) % NB]);
      compute_stage<M, FMT, 1, S, C::XR>(mine[j], nullptr, 0, r, g, mrows, acc);
    }
  }

  // Every copy of this wave has landed (the last wait was for all of them),
  // so its first stage buffer takes its sums: lane (r, g) holds
  // C[m = 4 g + i][row r] in acc[0][0][i].
  if (GATHER && bad) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if ((bad >> (4 * g + i)) & 1u) acc[0][0][i] = 0.0f;
  }
  float* red = reinterpret_cast<float*>(&mine[0]);
  *reinterpret_cast<f32x4_t*>(red + 4 * lane) = acc[0][0];
  __syncthreads();
  if (wave == 0) {
    f32x4_t sum = acc[0][0];
#pragma unroll
    for (int w = 1; w < kKwWaves; ++w) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(&st[w][0]) + 4 * lane);
      sum[0] += v[0];
      sum[1] += v[1];
      sum[2] += v[2];
      sum[3] += v[3];
    }
    // Lane (r, g) now holds y[4 g + i][row r] (before the global scale).
    // Greedy-argmax keys: each activation row's maximum over the tile's 16
    // rows is taken over the 16 lanes of its group g (a maximum: any order).
    const int64_t row = row0 + r;
    int h;
    const int64_t col = out_col(a, row, h);
    const float gs = h == 0 ? a.gscale[0] : a.gscale[1];
    uint64_t best[4] = {0, 0, 0, 0};
    if (col >= 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < mrows) {
          const uint16_t yb = f32_to_bf16_rne(sum[i] * gs);
          if (a.y) a.y[static_cast<int64_t>(m) * a.ldy + col] = yb;
          best[i] = argmax_key(yb, col);
        }
      }
    }
    if (a.keys) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const uint64_t w = shfl_xor_u64(best[i], o);
          if (w > best[i]) best[i] = w;
        }
        const int m = 4 * g + i;
        if (r == 0 && m < M) a.keys[tile * M + m] = best[i];
      }
    }
  }
}

template <int M, int FMT, int NB>
__global__ __launch_bounds__(kThreads) void decode_kw_kernel(const GemvArgs a) {
  kw_tile<M, FMT, NB>(a, blockIdx.x, M);
}

template <int FMT>
hipError_t launch_kw_fmt(const GemvArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(kThreads);
  switch (a.m) {
    case 1: hipLaunchKernelGGL((decode_kw_kernel<1, FMT, kKwBuffers>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_kw_kernel<2, FMT, kKwBuffers>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((decode_kw_kernel<3, FMT, kKwBuffers>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_kw_kernel<4, FMT, kKwBuffers>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((decode_kw_kernel<5, FMT, kKwBuffers>), grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL((decode_kw_kernel<6, FMT, kKwBuffers>), grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL((decode_kw_kernel<7, FMT, kKwBuffers>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_kw_kernel<8, FMT, kKwBuffers>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Grouped MoE decode: workgroup (tile, s) computes 64-row tile `tile` of
// the s-th expert that has routed pairs (in expert order) for its pairs
// [offsets[e], offsets[e + 1]) -- the stage copies fetch each pair's x row by
// its token id (GemvArgs::row_tokens), and the outputs go to the same pair
// rows of y -- 8 pairs per pass.
// The grid has min(experts, pairs) slots, at least as many as experts with
// pairs in any non-decreasing offset table, so idle experts cost no
// workgroups; a slot past the last such expert exits.  Expert e's prepared
// weight sits at e times the prepared size in the stacked buffers.  The
// offsets are clamped to [0, pairs] and a token id outside [0, tokens_total)
// reads zeros, so no routing table can make a workgroup read or write outside
// x and y.
__device__ __forceinline__ void moe_clamped_range(const MoeArgs& moe, int e, int& p0, int& p1) {
  p0 = moe.offsets[e];
  p1 = moe.offsets[e + 1];
  p0 = p0 < 0 ? 0 : p0 > moe.pairs ? moe.pairs : p0;
  p1 = p1 < p0 ? p0 : p1 > moe.pairs ? moe.pairs : p1;
}

// The expert of grid slot `slot`: the slot-th expert (in expert order) that
// has routed pairs, and its clamped pair range, or e = -1 past the last such
// expert.  Wave 0 reads the offsets of 256 experts at a time (4 per lane,
// loads issued together) and counts those with pairs until it reaches the
// slot's; that expert's lane leaves its pair range in LDS.  All threads call
// it; the results are workgroup-uniform.
__device__ __forceinline__ void moe_slot_expert(const MoeArgs& moe, int slot, int& e_out, int& p0_out, int& p1_out) {
  __shared__ int s_expert, s_p0, s_p1;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int seen = 0, found = -1;
    if (lane == 0) s_expert = -1;
    for (int b = 0; b < moe.experts && found < 0; b += 256) {
      int q0[4], q1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        q0[j] = q1[j] = 0;
        const int e = b + 64 * j + lane;
        if (e < moe.experts) moe_clamped_range(moe, e, q0[j], q1[j]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned long long busy = __ballot(q1[j] > q0[j]);
        const int count = __popcll(busy);
        if (found < 0 && slot < seen + count) {
          // The (slot - seen)-th set bit of `busy`.
          unsigned long long m = busy;
          for (int r = slot - seen; r > 0; --r) m &= m - 1;
          found = b + 64 * j + __ffsll(static_cast<long long>(m)) - 1;
          if (b + 64 * j + lane == found) {
            s_expert = found;
            s_p0 = q0[j];
            s_p1 = q1[j];
          }
        }
        seen += count;
      }
    }
  }
  __syncthreads();
  // Workgroup-uniform values: kept in scalar registers (the copy bases built
  // from them must be).
  e_out = __builtin_amdgcn_readfirstlane(s_expert);
  p0_out = __builtin_amdgcn_readfirstlane(s_p0);
  p1_out = __builtin_amdgcn_readfirstlane(s_p1);
}

// Grouped MoE decode, 64-row tiles: workgroup (tile, s) runs tile `tile` of
// the s-th expert with pairs, 8 pairs per pass (decode_tile).
template <int FMT>
__global__ __launch_bounds__(kThreads) void moe_decode_kernel(const GemvArgs base, const MoeArgs moe) {
  int e, p0, p1;
  moe_slot_expert(moe, blockIdx.y, e, p0, p1);
  if (e < 0) return;
  GemvArgs a = base;
  a.codes = base.codes + static_cast<int64_t>(e) * moe.code_stride;
  a.scales = base.scales + static_cast<int64_t>(e) * moe.scale_stride;
  a.gscale[0] = a.gscale[1] = moe.gscales ? moe.gscales[e] : 1.0f;
  a.tokens_total = moe.tokens_total;
  for (int c0 = p0; c0 < p1; c0 += kGemvMaxM) {
    a.row_tokens = moe.tokens + c0;
    a.y = base.y + static_cast<int64_t>(c0) * a.ldy;
    decode_tile<kGemvMaxM, FMT, 1, kDecodeBuffers, 4, true>(a, blockIdx.x, 0,
                                                           p1 - c0 < kGemvMaxM ? p1 - c0 : kGemvMaxM);
    __syncthreads();  // the stage buffers are reused by the next pass
  }
}

// Grouped MoE decode of one or two tokens on the wave-split kernel:
// workgroup (tile, s) runs 16-row tile `tile` of the s-th expert with pairs,
// up to M pairs per pass (M = the token count: one pass per expert for any
// routing of distinct experts per token) -- each pass exactly
// fp4_w4a16_linear's call on that many rows of the expert's weight where that
// call takes the wave-split kernel, so a pair's output equals it bit for bit.
// With one or two tokens the routing activates few experts, whose 64-row
// tiles would leave most CUs idle.
template <int M, int FMT>
__global__ __launch_bounds__(kThreads) void moe_decode_kw_kernel(const GemvArgs base, const MoeArgs moe) {
  int e, p0, p1;
  moe_slot_expert(moe, blockIdx.y, e, p0, p1);
  if (e < 0) return;
  GemvArgs a = base;
  a.codes = base.codes + static_cast<int64_t>(e) * moe.code_stride;
  a.scales = base.scales + static_cast<int64_t>(e) * moe.scale_stride;
  a.gscale[0] = a.gscale[1] = moe.gscales ? moe.gscales[e] : 1.0f;
  a.tokens_total = moe.tokens_total;
  for (int c0 = p0; c0 < p1; c0 += M) {
    a.row_tokens = moe.tokens + c0;
    a.y = base.y + static_cast<int64_t>(c0) * a.ldy;
    kw_tile<M, FMT, kKwBuffers, true>(a, blockIdx.x, p1 - c0 < M ? p1 - c0 : M);
    __syncthreads();  // the stage buffers are reused by the next pass
  }
}

// Launch of the m-row instance on tiles of RB 16-row blocks per wave and W
// waves: m = 3..32 on 64-row tiles (RB = 1, W = 4), m = 3..8 on 96-row (RB =
// 1, W = 6) and 128-row (RB = 2, W = 4) tiles.
template <int M, int FMT, int RB, int W>
hipError_t launch_m(const GemvArgs& a, dim3 grid, hipStream_t stream) {
  constexpr int NB = W == 6 ? decode_buffers_96(FMT) : kDecodeBuffers;
  hipLaunchKernelGGL((decode_mfma_kernel<M, FMT, RB, NB, W>), grid, dim3(64 * W), 0, stream, a);
  return hipGetLastError();
}

template <int FMT, int RB, int W>
hipError_t launch_fmt(const GemvArgs& a, dim3 grid, hipStream_t stream) {
  switch (a.m) {
    case 3: return launch_m<3, FMT, RB, W>(a, grid, stream);
    case 4: return launch_m<4, FMT, RB, W>(a, grid, stream);
    case 5: return launch_m<5, FMT, RB, W>(a, grid, stream);
    case 6: return launch_m<6, FMT, RB, W>(a, grid, stream);
    case 7: return launch_m<7, FMT, RB, W>(a, grid, stream);
    case 8: return launch_m<8, FMT, RB, W>(a, grid, stream);
    default:
      break;
  }
  if constexpr (RB == 1 && W == 4) {
    switch (a.m) {
      case 9: return launch_m<9, FMT, RB, W>(a, grid, stream);
      case 10: return launch_m<10, FMT, RB, W>(a, grid, stream);
      case 11: return launch_m<11, FMT, RB, W>(a, grid, stream);
      case 12: return launch_m<12, FMT, RB, W>(a, grid, stream);
      case 13: return launch_m<13, FMT, RB, W>(a, grid, stream);
      case 14: return launch_m<14, FMT, RB, W>(a, grid, stream);
      case 15: return launch_m<15, FMT, RB, W>(a, grid, stream);
      case 16: return launch_m<16, FMT, RB, W>(a, grid, stream);
      case 17: return launch_m<17, FMT, RB, W>(a, grid, stream);
      case 18: return launch_m<18, FMT, RB, W>(a, grid, stream);
      case 19: return launch_m<19, FMT, RB, W>(a, grid, stream);
      case 20: return launch_m<20, FMT, RB, W>(a, grid, stream);
      case 21: return launch_m<21, FMT, RB, W>(a, grid, stream);
      case 22: return launch_m<22, FMT, RB, W>(a, grid, stream);
      case 23: return launch_m<23, FMT, RB, W>(a, grid, stream);
      case 24: return launch_m<24, FMT, RB, W>(a, grid, stream);
      case 25: return launch_m<25, FMT, RB, W>(a, grid, stream);
      case 26: return launch_m<26, FMT, RB, W>(a, grid, stream);
      case 27: return launch_m<27, FMT, RB, W>(a, grid, stream);
      case 28: return launch_m<28, FMT, RB, W>(a, grid, stream);
      case 29: return launch_m<29, FMT, RB, W>(a, grid, stream);
      case 30: return launch_m<30, FMT, RB, W>(a, grid, stream);
      case 31: return launch_m<31, FMT, RB, W>(a, grid, stream);
      case 32: return launch_m<32, FMT, RB, W>(a, grid, stream);
      default:
        break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_moe_decode(const GemvArgs& a, const MoeArgs& moe, int experts, int tokens_total, int fmt,
                             hipStream_t stream, dim3* grid_out, dim3* block_out) {
  const int slots = experts < moe.pairs ? experts : moe.pairs;
  // One or two tokens: the experts the wave-split kernel takes at that m run on it.
  const bool kw = tokens_total <= 2 && decode_kw_used(a.n_proj, a.k, fmt, tokens_total);
  const dim3 grid(static_cast<unsigned>(a.rows_total / (kw ? kKwRows : kDecodeTileRows)), static_cast<unsigned>(slots));
  if (grid_out) *grid_out = grid;
  if (block_out) *block_out = dim3(kThreads);
  if (kw) {
    if (tokens_total == 1 && fmt == kFmtNvfp4)
      hipLaunchKernelGGL((moe_decode_kw_kernel<1, kFmtNvfp4>), grid, dim3(kThreads), 0, stream, a, moe);
    else if (tokens_total == 1)
      hipLaunchKernelGGL((moe_decode_kw_kernel<1, kFmtMxfp4>), grid, dim3(kThreads), 0, stream, a, moe);
    else if (fmt == kFmtNvfp4)
      hipLaunchKernelGGL((moe_decode_kw_kernel<2, kFmtNvfp4>), grid, dim3(kThreads), 0, stream, a, moe);
    else
      hipLaunchKernelGGL((moe_decode_kw_kernel<2, kFmtMxfp4>), grid, dim3(kThreads), 0, stream, a, moe);
  } else if (fmt == kFmtNvfp4) {
    hipLaunchKernelGGL(moe_decode_kernel<kFmtNvfp4>, grid, dim3(kThreads), 0, stream, a, moe);
  } else {
    hipLaunchKernelGGL(moe_decode_kernel<kFmtMxfp4>, grid, dim3(kThreads), 0, stream, a, moe);
  }
  return hipGetLastError();
}

hipError_t launch_decode_kw(const GemvArgs& a, int fmt, hipStream_t stream, dim3* grid_out, dim3* block_out) {
  if (a.tile_rows != kKwRows || a.splits != 1 || a.act || a.m < 1 || a.m > kKwMaxM ||
      a.rows_total % kKwRows != 0)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(a.rows_total / kKwRows));
  if (grid_out) *grid_out = grid;
  if (block_out) *block_out = dim3(kThreads);
  return fmt == kFmtNvfp4 ? launch_kw_fmt<kFmtNvfp4>(a, grid, stream) : launch_kw_fmt<kFmtMxfp4>(a, grid, stream);
}

hipError_t launch_decode_mfma(const GemvArgs& a, int fmt, hipStream_t stream, dim3* grid_out, dim3* block_out) {
  if (a.tile_rows != 64 && a.tile_rows != 96 && a.tile_rows != 128) return hipErrorInvalidValue;
  if (a.rows_total % a.tile_rows != 0 || (a.tile_rows != 64 && (a.splits != 1 || a.m > 8))) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(a.rows_total / a.tile_rows), static_cast<unsigned>(a.splits));
  const int waves = a.tile_rows == 96 ? 6 : 4;
  if (grid_out) *grid_out = grid;
  if (block_out) *block_out = dim3(64 * waves);
  const bool nv = fmt == kFmtNvfp4;
  if (a.tile_rows == 128) return nv ? launch_fmt<kFmtNvfp4, 2, 4>(a, grid, stream) : launch_fmt<kFmtMxfp4, 2, 4>(a, grid, stream);
  if (a.tile_rows == 96) return nv ? launch_fmt<kFmtNvfp4, 1, 6>(a, grid, stream) : launch_fmt<kFmtMxfp4, 1, 6>(a, grid, stream);
  return nv ? launch_fmt<kFmtNvfp4, 1, 4>(a, grid, stream) : launch_fmt<kFmtMxfp4, 1, 4>(a, grid, stream);
}

}  // namespace fp4
