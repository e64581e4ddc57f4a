// Prefill-shaped W4A16 FP4 GEMM (m > 32 activation rows; SwiGLU gate_up and the
// grouped MoE tile route also below that) on gfx950 bf16 MFMA.
//
// At large m the layer is a dense contraction (2*m*n*k flops over n*k/2 code
// bytes), so it runs on the matrix cores.  The pages run prefill through a
// dequantized bf16 GEMM ("MXFP4 decode-graph + gate_up FUSION default-ON",
// vllm.cpp PR #54, step 3: prefill untouched; "keep the ModelOpt NVFP4 lm_head
// packed", section "Why this row matters": the bf16 head cost 2.37 GiB/step);
// here the packed weight is used directly and decoded in registers.
//
// Tile: a workgroup of kGemmWavesM x 4 waves computes kGemmBM activation rows
// x 256 weight rows of y; wave (wm, wn) owns activation rows [128 wm, +128)
// and weight rows [64 wn, +64).  K advances 64 codes per stage.  Each stage
// holds, in LDS:
//   x       kGemmBM x 64 bf16        (16 KiB per 128 rows)
//   codes   256 rows x 32 bytes      (8 KiB, still packed 4-bit)
//   scales  of those codes           (1 KiB NVFP4, 512 B MXFP4)
// Stages are copied global -> LDS by the load-to-LDS path
// (global_load_lds_dwordx4: each lane's 16 bytes land at lane * 16 after a
// wave-uniform base), so no registers carry them; three stage buffers keep two
// stages in flight while the third is consumed.  The K loop is one body with
// the buffer index computed; results leave through LDS as whole rows
// (gemm_common.hpp), which with a loop unrolled over the three buffers made
// the compiler spill the accumulators.
//
// A wave decodes only its own 64 weight rows, so each code is decoded once per
// workgroup per activation-row block.  E2M1 * S is exact in bf16 (at most 6
// significant bits), so decoding before the MFMA loses nothing; the NVFP4
// global scale multiplies in the epilogue.
//
// v_mfma_f32_32x32x16_bf16 with the weights as the A operand and x as B: lane
// l supplies weight row (l % 32) and activation row (l % 32), each with 8
// consecutive MFMA k-indices 8 * (l / 32) .. +7; result e (0..15) of lane l is
// C[8 * (e / 4) + 4 * (l / 32) + e % 4][l % 32], i.e. four consecutive weight
// rows (output columns) of one activation row.  Within a 64-code stage the
// MFMA k-index 8 * h + e of step kk (0..3) stands for code 32 * h + 8 * kk + e,
// for both operands alike, so a lane's codes for the whole stage are one
// 16-byte read.
#include "fp4_common.hpp"
#include "fp4_device.hpp"
#include "gemm_common.hpp"
#include "lds_copy.hpp"

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kWaves = kGemmWavesM * 4;
constexpr int kThreads = kGemmThreads;
static_assert(kThreads == kWaves * 64, "one wave per 64 threads");
constexpr int kStages = 3;
constexpr int kAChunks = kGemmBM * kGemmBK * 2 / 16;  // 16-byte chunks of an x stage
constexpr int kBChunks = kGemmBN * kGemmBK / 2 / 16;  // 16-byte chunks of a code stage
constexpr int kAPer = kAChunks / kThreads;
constexpr int kBPer = kBChunks / kThreads;
static_assert(kAChunks % kThreads == 0 && kBChunks % kThreads == 0, "stage split");

template <int FMT>
struct Cfg {
  static constexpr int P = scales_per_seg(FMT);
  // 16-byte chunks of a scale stage: 32 P (64 NVFP4, 32 MXFP4), copied by
  // the 64 lanes of wave 0 (MXFP4: lanes 32..63 repeat lanes 0..31 into the
  // second half of a 64-chunk area).
  static constexpr int kSUsed = kGemmBN / kRowGroup * 2 * kRowGroup * P / 16;
  static constexpr int kSChunks = 64;
  static_assert(kSUsed <= kSChunks, "scale stage");
};

template <int FMT>
struct alignas(16) Stage {
  uint4 a[kAChunks];
  uint4 b[kBChunks];
  uint4 s[Cfg<FMT>::kSChunks];
};

static_assert(kGemmBM * kStageYRow <= kStages * sizeof(Stage<kFmtNvfp4>) &&
                  64 * kStagePRow <= kStages * sizeof(Stage<kFmtNvfp4>) &&
                  sizeof(Stage<kFmtNvfp4>) == sizeof(Stage<kFmtMxfp4>),
              "result staging fits in the stage buffers");

union Frag {
  bf16x8_t v;
  uint32_t u[4];
};

// LDS bank layout on gfx950: 64 banks of 4 bytes; a 16-byte-per-lane read is
// served 16 lanes at a time, so it is conflict-free when each group of 16
// lanes touches 16 different 16-byte bank groups (address / 16 mod 16).
//
// x stage: row r holds 8 chunks of 16 bytes (8 k each) at r * 128, chunk c in
// slot c ^ ((r >> 1) & 7).  A fragment read has 16 lanes on 16 consecutive
// rows and one chunk index; their bank groups 8 (r & 1) + slot are distinct.
__device__ __forceinline__ int a_slot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Code stage: row r holds its two 16-byte halves h at r * 32, half h in slot
// h ^ ((r >> 3) & 1).  16 lanes on 16 consecutive rows reading one half hit
// bank groups 2 r + slot (mod 16): rows r and r + 8 take opposite slots.
__device__ __forceinline__ int b_slot(int r, int h) { return 2 * r + (h ^ ((r >> 3) & 1)); }

// FI: 32-row activation blocks a tile computes (4 = all 128 rows; 1 or 2 for
// calls with m <= 32 or 64, whose single row of tiles has no more rows).
// Load-to-LDS copies a wave issues per stage: x (FI per thread for 32 FI
// rows) and codes, plus one for the scales in wave 0.
template <int FI>
constexpr int kLoadsPerStage = FI * kAPer / 4 + kBPer;
static_assert(kAPer == 4, "one x chunk per thread per 32-row block");

// Wait until this wave's copies of all but the newest `stages` stages have
// landed, then join the workgroup barrier.
template <int STAGES, int FI>
__device__ __forceinline__ void wait_stages_barrier(int wave) {
  if (wave == 0)
    wait_vm_barrier<STAGES * (kLoadsPerStage<FI> + 1)>();
  else
    wait_vm_barrier<STAGES * kLoadsPerStage<FI>>();
}

// The stage copies of one workgroup tile.  Chunk positions in LDS are fixed by
// lane order, so the swizzles are applied by choosing which global chunk each
// lane fetches; those choices do not depend on the stage, so each lane keeps
// 32-bit offsets from three wave-uniform tile bases that advance with k.
//   x rows past m repeat row m - 1 (their outputs are never stored).
//   In a stage that straddles k (k an odd multiple of 32), x chunks at or past
//   k are fetched from the zero padding of the prepared code rows instead:
//   every code row then holds at least 32 zero codes, 16 zero bytes, from
//   code k on.  So they are bf16 zeros, whatever x holds beyond its row.
// Every lane issues every copy, so each wave has the same number in flight
// per stage.
// GATHER (grouped MoE): tile row r is the x row of token row_tokens[m0 + r]
// (rows past m repeat row m - 1), fetched through a per-lane address; a
// token id outside [0, tokens_total) fetches row 0 instead, and the kernel
// zeroes that row's sums (zero_rows_of_bad_tokens).
template <int FMT, int FI, bool GATHER = false>
struct Copier {
  static constexpr int P = Cfg<FMT>::P;
  static constexpr int kXPer = FI * kAPer / 4;  // x chunks per thread per stage
  const uint16_t* xt;    // x row m0
  const uint8_t* xrow[GATHER ? kXPer : 1];  // GATHER: this lane's chunk of its row at k = 0
  const uint8_t* ct;     // code row n0
  const uint8_t* st;     // scale row group n0 / 16
  const uint8_t* zeros;  // 16 zero bytes: code row n0 from code k on
  uint32_t xoff[kXPer], coff[kBPer], soff;
  int xk[kXPer];         // first k of this lane's x chunks within a stage
  int k;
  uint32_t lds_wave_a, lds_wave_b;  // this wave's chunk offsets within a stage

  __device__ __forceinline__ Copier(const MfmaArgs& a, int64_t m0, int64_t n0, int t, int wave) {
    const int64_t row_bytes = a.k_pad / 2;
    k = a.k;
    xt = a.x + m0 * a.k;
    ct = a.codes + n0 * row_bytes;
    st = a.scales + (n0 / kRowGroup) * a.ksegs * kRowGroup * P;
    zeros = ct + a.k / 2;
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int p = i * kThreads + t;
      const int r = p >> 3;
      const int c = (p & 7) ^ ((r >> 1) & 7);
      const int64_t rr = m0 + r < a.m ? r : a.m - 1 - m0;
      xk[i] = 8 * c;
      if constexpr (GATHER) {
        int tok = a.row_tokens[m0 + rr];
        if (tok < 0 || tok >= a.tokens_total) tok = 0;
        xrow[i] = reinterpret_cast<const uint8_t*>(a.x + static_cast<int64_t>(tok) * a.k) + 16 * c;
        xoff[i] = 0;
      } else {
        xoff[i] = static_cast<uint32_t>(rr * a.k * 2 + 16 * c);
      }
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int p = i * kThreads + t;
      const int r = p >> 1;
      const int h = (p & 1) ^ ((r >> 3) & 1);
      coff[i] = static_cast<uint32_t>(r * row_bytes + 16 * h);
    }
    // Scales: 16 row groups x 2 segments x 16 rows x P bytes, contiguous per
    // row group in the prepared layout.
    const int lane = t & 63;
    const int ps = lane % Cfg<FMT>::kSUsed;
    soff = static_cast<uint32_t>((ps / (2 * P)) * a.ksegs * kRowGroup * P + 16 * (ps % (2 * P)));
    lds_wave_a = 64 * 16 * wave;
    lds_wave_b = 64 * 16 * wave;
  }

  // Copies of the stage at code k0; `ragged` = the stage straddles k.
  __device__ __forceinline__ void issue(int64_t k0, bool ragged, Stage<FMT>& sb, int wave) const {
    const uint32_t la = lds_addr(sb.a) + lds_wave_a;
    const uint32_t lb = lds_addr(sb.b) + lds_wave_b;
    if constexpr (GATHER) {
#pragma unroll
      for (int i = 0; i < kXPer; ++i) {
        const bool in_k = !ragged || k0 + xk[i] < k;
        copy16_vaddr(in_k ? static_cast<const void*>(xrow[i] + 2 * k0) : static_cast<const void*>(zeros),
                     la + i * kThreads * 16);
      }
    } else if (!ragged) {
      const uint16_t* xb = xt + k0;
#pragma unroll
      for (int i = 0; i < kXPer; ++i) copy16_sbase(xb, xoff[i], la + i * kThreads * 16);
    } else {
#pragma unroll
      for (int i = 0; i < kXPer; ++i) {
        const void* src = k0 + xk[i] < k ? static_cast<const void*>(reinterpret_cast<const uint8_t*>(xt + k0) + xoff[i])
                                         : static_cast<const void*>(zeros);
        copy16_vaddr(src, la + i * kThreads * 16);
      }
    }
    const uint8_t* cb = ct + k0 / 2;
#pragma unroll
    for (int i = 0; i < kBPer; ++i) copy16_sbase(cb, coff[i], lb + i * kThreads * 16);
    if (wave == 0) copy16_sbase(st + (k0 / 32) * kRowGroup * P, soff, lds_addr(sb.s));
  }
};

// The 8 codes of `word` times their block scale, as a bf16 MFMA fragment.
template <int FMT>
__device__ __forceinline__ void decode8(uint32_t word, uint32_t sbyte, Frag& f) {
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

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Register state a wave carries from one stage to the next: the stage's
// codes and scale bytes of its 2 x 32 weight rows, and, for the MFMA step
// about to run, the 4 x fragments and 2 decoded weight fragments.
template <int FMT, int FI>
struct Regs {
  uint4 code[2];
  uint32_t sc[2];
  Frag xf[FI], wf[2];
};

// Read this wave's codes and scale bytes of a stage.
template <int FMT, int FI>
__device__ __forceinline__ void read_codes(const Stage<FMT>& st, int wr0, int lh, Regs<FMT, FI>& r) {
  constexpr int P = Cfg<FMT>::P;
  const uint8_t* sb = reinterpret_cast<const uint8_t*>(st.s);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = wr0 + 32 * j;
    r.code[j] = st.b[b_slot(row, lh)];
    const int so = (((row >> 4) * 2 + lh) * kRowGroup + (row & 15)) * P;
    if constexpr (P == 2)
      r.sc[j] = *reinterpret_cast<const uint16_t*>(sb + so);
    else
      r.sc[j] = sb[so];
  }
}

// Read the x fragments of MFMA step kk (FI activation row blocks).
template <int FMT, int FI>
__device__ __forceinline__ void read_x(const Stage<FMT>& st, int xr0, int lh, int kk, Frag (&f)[FI]) {
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const uint4 q = st.a[a_slot(xr0 + 32 * i, 4 * lh + kk)];
    f[i].u[0] = q.x;
    f[i].u[1] = q.y;
    f[i].u[2] = q.z;
    f[i].u[3] = q.w;
  }
}

// Decode the weight fragments of MFMA step kk from the carried codes.
template <int FMT, int FI>
__device__ __forceinline__ void decode_step(const Regs<FMT, FI>& r, int kk, Frag (&f)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t word = kk == 0 ? r.code[j].x : kk == 1 ? r.code[j].y : kk == 2 ? r.code[j].z : r.code[j].w;
    const uint32_t sbyte = Cfg<FMT>::P == 2 ? (kk < 2 ? r.sc[j] & 0xFFu : r.sc[j] >> 8) : r.sc[j];
    decode8<FMT>(word, sbyte, f[j]);
  }
}

template <int FI>
__device__ __forceinline__ void mfma_step(const Frag (&wf)[2], const Frag (&xf)[FI], f32x16_t (&acc)[FI][2]) {
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j].v, xf[i].v, acc[i][j], 0, 0, 0);
}

// VALU instructions of one MFMA step's weight decode (2 x 8 codes).
template <int FMT>
constexpr int kDecodeValu = FMT == kFmtMxfp4 ? 8 : 36;

// Interleave hint for a run of 8 MFMAs that overlaps `reads` LDS reads and
// one step's decode.
// The run ends with a full scheduling barrier: left free, the scheduler
// merges consecutive steps and issues MFMAs on the same accumulator back to
// back, each then waiting for the previous one's result.
template <int FMT, int READS, int MFMAS>
__device__ __forceinline__ void schedule_step() {
  constexpr int kValuPerMfma = (kDecodeValu<FMT> + MFMAS - 1) / MFMAS;
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, READS, 0);
#pragma unroll
  for (int q = 0; q < MFMAS; ++q) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, kValuPerMfma, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One stage for this wave: 4 MFMA steps of 16 k over its 2 x 32 weight rows
// and 4 activation row blocks.  Entry: r holds the stage's codes and step 0's
// fragments.  Steps 0..2 each read and decode the next step's fragments while
// their 8 MFMAs run.  Then comes the stage's one workgroup barrier, after the
// wave's last LDS read of `cur` and before its last 8 MFMAs: once every wave
// has passed it, `cur` is free and is refilled with stage ks + 3, and stage
// ks + 1 (whose copies the wait before the barrier saw land) is complete in
// `nxt`, so its codes and step-0 fragments are read and decoded under the
// last MFMAs -- the next stage starts with its MFMAs ready to issue.
template <int FMT, int FI, bool GATHER>
__device__ __forceinline__ void pipeline_step(const Copier<FMT, FI, GATHER>& cp, int ks, int k_end, int ragged_ks,
                                              Stage<FMT>& cur, const Stage<FMT>& nxt, int wave, int xr0, int wr0,
                                              int lh, Regs<FMT, FI>& r, f32x16_t (&acc)[FI][2]) {
  Frag xn[FI], wn[2];
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    read_x<FMT, FI>(cur, xr0, lh, kk + 1, xn);
    decode_step<FMT, FI>(r, kk + 1, wn);
    mfma_step<FI>(r.wf, r.xf, acc);
    schedule_step<FMT, FI, 2 * FI>();
#pragma unroll
    for (int i = 0; i < FI; ++i) r.xf[i] = xn[i];
    r.wf[0] = wn[0];
    r.wf[1] = wn[1];
  }
  // Stage ks + 1 landed when at most the copies of stage ks + 2 are in flight.
  if (ks + 2 < k_end)
    wait_stages_barrier<1, FI>(wave);
  else
    wait_stages_barrier<0, FI>(wave);
  if (ks + 3 < k_end) cp.issue(static_cast<int64_t>(ks + 3) * kGemmBK, ks + 3 == ragged_ks, cur, wave);
  // Unconditional, so it shares a basic block (and the interleaved schedule)
  // with the MFMAs; after the last stage it reads a stale buffer, unused.
  read_codes<FMT, FI>(nxt, wr0, lh, r);
  read_x<FMT, FI>(nxt, xr0, lh, 0, xn);
  decode_step<FMT, FI>(r, 0, wn);
  mfma_step<FI>(r.wf, r.xf, acc);
  schedule_step<FMT, 4 + FI, 2 * FI>();
#pragma unroll
  for (int i = 0; i < FI; ++i) r.xf[i] = xn[i];
  r.wf[0] = wn[0];
  r.wf[1] = wn[1];
}

// silu(v) = v / (1 + e^-v), for the SwiGLU epilogue of an interleaved gate_up weight.
__device__ __forceinline__ float act_silu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// acc = the (m0, n0) tile's sums over K steps [k_begin, k_end).
template <int FMT, int FI, bool GATHER = false>
__device__ __forceinline__ void run_tile(const MfmaArgs& a, int64_t m0, int64_t n0, int k_begin, int k_end,
                                         Stage<FMT> (&st)[kStages], f32x16_t (&acc)[FI][2]) {
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int l32 = lane & 31;
  const int lh = lane >> 5;
  const int xr0 = (wave / 4) * 128 + l32;  // x row of this lane's first activation block
  const int wr0 = (wave % 4) * 64 + l32;   // weight row of this lane's first weight block
  // The last stage straddles k when k is an odd multiple of 32.
  const int ragged_ks = (a.k % kGemmBK) != 0 ? a.plan.ksteps - 1 : -1;

#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const Copier<FMT, FI, GATHER> cp(a, m0, n0, t, wave);
  // Prologue: three stages in flight, wait for the first, read its codes
  // and step-0 fragments.
  cp.issue(static_cast<int64_t>(k_begin) * kGemmBK, k_begin == ragged_ks, st[0], wave);
  if (k_begin + 1 < k_end) cp.issue(static_cast<int64_t>(k_begin + 1) * kGemmBK, k_begin + 1 == ragged_ks, st[1], wave);
  if (k_begin + 2 < k_end) cp.issue(static_cast<int64_t>(k_begin + 2) * kGemmBK, k_begin + 2 == ragged_ks, st[2], wave);
  if (k_begin + 2 < k_end)
    wait_stages_barrier<2, FI>(wave);
  else if (k_begin + 1 < k_end)
    wait_stages_barrier<1, FI>(wave);
  else
    wait_stages_barrier<0, FI>(wave);
  Regs<FMT, FI> r;
  read_codes<FMT, FI>(st[0], wr0, lh, r);
  read_x<FMT, FI>(st[0], xr0, lh, 0, r.xf);
  decode_step<FMT, FI>(r, 0, r.wf);
  // One loop body with the buffer index computed, so the accumulators keep
  // their registers from one stage to the next.
  int cur = 0;
  for (int ks = k_begin; ks < k_end; ++ks) {
    const int nxt = cur == kStages - 1 ? 0 : cur + 1;
    pipeline_step<FMT, FI, GATHER>(cp, ks, k_end, ragged_ks, st[cur], st[nxt], wave, xr0, wr0, lh, r, acc);
    cur = nxt;
  }
}

// One launch for all tiles.  Workgroup b < dp_tiles computes data-parallel
// tile b (in XCD order) over all of K and stores bf16 y.  The last `units` =
// tail_tiles x splits workgroups of the grid -- the last round, after their
// own tile if they have one -- then each compute split u % splits of tail tile
// u / splits and store it as an fp32 partial, which tail_reduce_kernel adds.
template <int FMT, bool ACT, int FI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(const MfmaArgs a) {
  __shared__ Stage<FMT> st[kStages];
  const GemmPlan& pl = a.plan;
  const int bid = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  f32x16_t acc[FI][2];
  char* lds = reinterpret_cast<char*>(st);

  if (bid < pl.dp_tiles) {
    int64_t m0, n0;
    tile_coords(pl, dp_tile_of(pl, bid), m0, n0);
    run_tile<FMT, FI>(a, m0, n0, 0, pl.ksteps, st, acc);
    if constexpr (ACT)
      store_tile_swiglu_staged<kGemmBM, kThreads, 64, FI>(a, m0, n0, wave, acc, lds);
    else
      store_tile_bf16_staged<kGemmBM, kThreads, kGemmBM, FI>(a, m0, n0, wave, acc, lds);
  }

  const int units = pl.tail_tiles * pl.splits;
  const int u = bid - (static_cast<int>(gridDim.x) - units);
  if (u < 0) return;
  __syncthreads();  // the stage buffers are reused
  const int split = u % pl.splits;
  int64_t m0, n0;
  tile_coords(pl, pl.dp_tiles + u / pl.splits, m0, n0);
  run_tile<FMT, FI>(a, m0, n0, static_cast<int>(static_cast<int64_t>(split) * pl.ksteps / pl.splits),
                    static_cast<int>(static_cast<int64_t>(split + 1) * pl.ksteps / pl.splits), st, acc);
  store_tile_partial_staged<kGemmBM, kThreads, 64, FI>(a, u, m0, wave, acc, lds);
}

// Grouped MoE prefill: the routed (token, expert) pairs sorted by expert,
// expert e owning pairs [offsets[e], offsets[e + 1]), pair p reading x row
// tokens[p].  Counted in expert order, expert e's c_e pairs form
// ceil(c_e / 128) activation tiles of 128 of its pairs, whose x rows the
// stage copies fetch straight from x (no gathered copy).  With T such tiles
// in all, work item L < T n_tiles is weight-row tile L % n_tiles of the
// (L / n_tiles)-th tile, computed over all of K with that expert's prepared
// weight and stored as bf16 y at the same pair rows.  Items are dealt to the
// workgroups XCD-aware: workgroup b runs on XCD b % X (X = plan.xcds, from the
// device's compute units), and each XCD gets a
// contiguous run of items, so the weight tiles of one activation tile (which
// share its x rows) and an expert's activation tiles (which share its weight)
// meet in one L2; T is counted first, so idle slots leave no XCD short of
// work.  Each tile's sums are the dense GEMM's for those rows (same K steps,
// same MFMA order), so a pair's output does not depend on the other pairs.
// The grid has moe_gemm_slots(pairs, experts) tile slots per weight tile,
// enough for every tile when the offsets are non-decreasing; workgroups past
// the dealt items exit.  Offsets are clamped to [0, pairs] and a token id
// outside [0, tokens_total) gives a zero row, so no routing table can make a
// workgroup touch memory outside x, the weights and y.
// ACT: each expert's weight is an interleaved gate_up pair and y[p] =
// silu(gate) * up (the SwiGLU epilogue of the dense tile GEMM), with the
// expert's two NVFP4 global scales at gscales[2 e], gscales[2 e + 1].
__device__ __forceinline__ void moe_range(const MoeArgs& moe, int e, int& p0, int& p1) {
  p0 = moe.offsets[e];
  p1 = moe.offsets[e + 1];
  p0 = p0 < 0 ? 0 : p0 > moe.pairs ? moe.pairs : p0;
  p1 = p1 < p0 ? p0 : p1 > moe.pairs ? moe.pairs : p1;
}

// The sums of tile rows whose token id is outside [0, tokens_total) become
// zero (their x rows were fetched from row 0): lane l holds activation row
// 32 i + l % 32 of the tile in acc[i].
template <int FI>
__device__ __forceinline__ void zero_rows_of_bad_tokens(const MfmaArgs& a, int64_t m0, f32x16_t (&acc)[FI][2]) {
  const int l32 = threadIdx.x & 31;
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const int64_t m = m0 + 32 * i + l32;
    if (m < a.m) {
      const int tok = a.row_tokens[m];
      if (tok < 0 || tok >= a.tokens_total) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
      }
    }
  }
}

template <int FMT, bool ACT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void moe_gemm_kernel(const MfmaArgs base, const MoeArgs moe) {
  __shared__ Stage<FMT> st[kStages];
  __shared__ int s_expert, s_p0, s_p1, s_tile, s_ntile;
  const int n_tiles = base.plan.n_tiles;
  // Wave 0 counts the tiles of all experts, maps this workgroup to its work
  // item, then finds the item's (expert, tile): 64 experts at a time, each
  // lane takes one expert's tile count, an inclusive scan over the wave gives
  // the tiles before each, and the lane whose range holds the slot records it.
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    if (lane == 0) s_expert = -1;
    int total = 0;  // wave-uniform
    for (int b = 0; b < moe.experts; b += 64) {
      const int e = b + lane;
      int p0 = 0, p1 = 0;
      if (e < moe.experts) moe_range(moe, e, p0, p1);
      int tiles = (p1 - p0 + kGemmBM - 1) / kGemmBM;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) tiles += __shfl_xor(tiles, o);
      total += tiles;
    }
    // Items dealt to XCDs in contiguous runs (XCD x: q or q + 1 items).
    const int64_t items = static_cast<int64_t>(total) * n_tiles;
    const int nx = base.plan.xcds;
    const int xcd = static_cast<int>(blockIdx.x % nx);
    const int64_t q = items / nx, r = items % nx;
    const int64_t j = blockIdx.x / nx;
    const int64_t item = xcd * q + (xcd < r ? xcd : r) + j;
    const bool live = j < q + (xcd < r ? 1 : 0);
    const int slot = live ? static_cast<int>(item / n_tiles) : -1;
    if (lane == 0) s_ntile = live ? static_cast<int>(item % n_tiles) : 0;
    int before = 0;  // tiles of the experts scanned so far (wave-uniform)
    for (int b = 0; b < moe.experts && slot >= 0 && before <= slot; b += 64) {
      const int e = b + lane;
      int p0 = 0, p1 = 0;
      if (e < moe.experts) moe_range(moe, e, p0, p1);
      const int tiles = (p1 - p0 + kGemmBM - 1) / kGemmBM;
      int incl = tiles;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      const int first = before + incl - tiles;
      if (slot >= first && slot < first + tiles) {
        s_expert = e;
        s_p0 = p0;
        s_p1 = p1;
        s_tile = slot - first;
      }
      before += __shfl(incl, 63);
    }
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_expert);
  if (e < 0) return;
  const int p0 = __builtin_amdgcn_readfirstlane(s_p0);
  const int p1 = __builtin_amdgcn_readfirstlane(s_p1);
  const int tile = __builtin_amdgcn_readfirstlane(s_tile);
  const int n_tile = __builtin_amdgcn_readfirstlane(s_ntile);
  MfmaArgs a = base;
  a.row_tokens = moe.tokens + p0;
  a.tokens_total = moe.tokens_total;
  a.y = base.y + static_cast<int64_t>(p0) * a.ldy;
  a.m = p1 - p0;
  a.codes = base.codes + static_cast<int64_t>(e) * moe.code_stride;
  a.scales = base.scales + static_cast<int64_t>(e) * moe.scale_stride;
  a.gscale[0] = moe.gscales ? moe.gscales[ACT ? 2 * e : e] : 1.0f;
  a.gscale[1] = moe.gscales ? moe.gscales[ACT ? 2 * e + 1 : e] : 1.0f;
  const int64_t m0 = static_cast<int64_t>(tile) * kGemmBM;
  const int64_t n0 = static_cast<int64_t>(n_tile) * kGemmBN;
  const int rows = a.m - static_cast<int>(m0);  // >= 1
  const int wave = threadIdx.x >> 6;
  char* lds = reinterpret_cast<char*>(st);
  // A tile with at most 32 (64) rows computes only 1 (2) of its 4 activation
  // blocks, as the dense kernel's instances for small m do.
  if (rows > 64) {
    f32x16_t acc[4][2];
    run_tile<FMT, 4, true>(a, m0, n0, 0, a.plan.ksteps, st, acc);
    zero_rows_of_bad_tokens<4>(a, m0, acc);
    if constexpr (ACT)
      store_tile_swiglu_staged<kGemmBM, kThreads, 64, 4>(a, m0, n0, wave, acc, lds);
    else
      store_tile_bf16_staged<kGemmBM, kThreads, kGemmBM, 4>(a, m0, n0, wave, acc, lds);
  } else if (rows > 32) {
    f32x16_t acc[2][2];
    run_tile<FMT, 2, true>(a, m0, n0, 0, a.plan.ksteps, st, acc);
    zero_rows_of_bad_tokens<2>(a, m0, acc);
    if constexpr (ACT)
      store_tile_swiglu_staged<kGemmBM, kThreads, 64, 2>(a, m0, n0, wave, acc, lds);
    else
      store_tile_bf16_staged<kGemmBM, kThreads, kGemmBM, 2>(a, m0, n0, wave, acc, lds);
  } else {
    f32x16_t acc[1][2];
    run_tile<FMT, 1, true>(a, m0, n0, 0, a.plan.ksteps, st, acc);
    zero_rows_of_bad_tokens<1>(a, m0, acc);
    if constexpr (ACT)
      store_tile_swiglu_staged<kGemmBM, kThreads, 64, 1>(a, m0, n0, wave, acc, lds);
    else
      store_tile_bf16_staged<kGemmBM, kThreads, kGemmBM, 1>(a, m0, n0, wave, acc, lds);
  }
}

// Split-K finish of the tail tiles: y = G * (partial_0 + partial_1 + ... +
// partial_{S-1}), added in split order (a fixed order: the output does not
// depend on timing).  A separate launch, so every partial is complete and
// visible when it starts; each thread takes one (x row, 4 weight rows) item of
// one tail tile and keeps its S loads in flight kBatch at a time.  BM: the
// tile's activation rows (128 for the W4A16 GEMM, 256 for the W4A4 GEMM).
constexpr int kReduceThreads = 256;
template <int BM>
constexpr int kReduceItems = BM * kGemmBN / 4;  // per tail tile
static_assert(kReduceItems<kGemmBM> % kReduceThreads == 0 && kReduceItems<kW4BM> % kReduceThreads == 0,
              "reduce split");

template <int BM>
__global__ __launch_bounds__(kReduceThreads) void tail_reduce_kernel(const MfmaArgs a) {
  const GemmPlan& pl = a.plan;
  const int64_t gi = static_cast<int64_t>(blockIdx.x) * kReduceThreads + threadIdx.x;
  const int tail_tile = static_cast<int>(gi / kReduceItems<BM>);
  const int it = static_cast<int>(gi - static_cast<int64_t>(tail_tile) * kReduceItems<BM>);
  const int mr = it / (kGemmBN / 4);
  const int nr = 4 * (it % (kGemmBN / 4));
  int64_t m0, n0;
  tile_coords<BM>(pl, pl.dp_tiles + tail_tile, m0, n0);
  const int64_t m = m0 + mr;
  if (m >= a.m) return;
  if (a.act) {
    // Interleaved gate_up (every tile runs as a "tail" unit, so all results
    // come through here): items on gate rows also add their up rows (+16)
    // and write y = silu(gate) * up.
    if ((nr & 31) >= 16) return;
    const int64_t grow = n0 + nr;
    const int64_t col = (grow >> 5) * 16 + (grow & 15);
    if (col >= a.n_proj) return;
    const int64_t unit_floats = static_cast<int64_t>(BM) * kGemmBN;
    const float* p = a.partial + static_cast<int64_t>(tail_tile) * pl.splits * unit_floats + mr * kGemmBN + nr;
    f32x4_t gsum = *reinterpret_cast<const f32x4_t*>(p);
    f32x4_t usum = *reinterpret_cast<const f32x4_t*>(p + 16);
    for (int s = 1; s < pl.splits; ++s) {
      gsum += *reinterpret_cast<const f32x4_t*>(p + s * unit_floats);
      usum += *reinterpret_cast<const f32x4_t*>(p + s * unit_floats + 16);
    }
    const float w[4] = {act_silu(gsum.x * a.gscale[0]) * (usum.x * a.gscale[1]),
                        act_silu(gsum.y * a.gscale[0]) * (usum.y * a.gscale[1]),
                        act_silu(gsum.z * a.gscale[0]) * (usum.z * a.gscale[1]),
                        act_silu(gsum.w * a.gscale[0]) * (usum.w * a.gscale[1])};
    uint16_t* dst = a.y + m * a.ldy + col;
    if (col + 4 <= a.n_proj && ((col | a.ldy) & 3) == 0) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(f32x2_to_bf16x2_rne(w[0], w[1]), f32x2_to_bf16x2_rne(w[2], w[3]));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (col + q < a.n_proj) dst[q] = f32_to_bf16_rne(w[q]);
    }
    return;
  }
  int h;
  const int64_t col = out_col(a, n0 + nr, h);
  if (col < 0) return;

  constexpr int kBatch = 8;
  const int64_t unit_floats = static_cast<int64_t>(BM) * kGemmBN;
  const float* p = a.partial + static_cast<int64_t>(tail_tile) * pl.splits * unit_floats + mr * kGemmBN + nr;
  f32x4_t sum = *reinterpret_cast<const f32x4_t*>(p);
  for (int s0 = 1; s0 < pl.splits; s0 += kBatch) {
    f32x4_t v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (s0 + b < pl.splits) v[b] = *reinterpret_cast<const f32x4_t*>(p + (s0 + b) * unit_floats);
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (s0 + b < pl.splits) sum += v[b];
  }
  const float g = a.gscale[h];
  const float w[4] = {sum.x * g, sum.y * g, sum.z * g, sum.w * g};
  const int64_t lr = col - static_cast<int64_t>(h) * a.n_proj;
  uint16_t* dst = a.y + m * a.ldy + col;
  if (lr + 4 <= a.n_proj && ((col | a.ldy) & 3) == 0) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(f32x2_to_bf16x2_rne(w[0], w[1]), f32x2_to_bf16x2_rne(w[2], w[3]));
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lr + q < a.n_proj) dst[q] = f32_to_bf16_rne(w[q]);
  }
}

}  // namespace

// The kernel instance for (format, SwiGLU epilogue, activation blocks).
template <int FMT, bool ACT>
void launch_gemm_fi(const MfmaArgs& a, int fi, dim3 grid, dim3 block, hipStream_t stream) {
  if (fi == 1)
    hipLaunchKernelGGL((gemm_kernel<FMT, ACT, 1>), grid, block, 0, stream, a);
  else if (fi == 2)
    hipLaunchKernelGGL((gemm_kernel<FMT, ACT, 2>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_kernel<FMT, ACT, 4>), grid, block, 0, stream, a);
}

hipError_t launch_mfma(const MfmaArgs& a, int fmt, hipStream_t stream, dim3* grid_out, dim3* block_out) {
  const GemmPlan& p = a.plan;
  const dim3 block(kThreads);
  const int units = p.tail_tiles * p.splits;
  const dim3 grid(static_cast<unsigned>(p.dp_tiles > units ? p.dp_tiles : units));
  if (grid_out) *grid_out = dim3(grid.x, static_cast<unsigned>(units));
  if (block_out) *block_out = block;
  // A call with m <= 32 (64) has one row of tiles with at most 32 (64) rows:
  // its tiles compute 1 (2) of their 4 activation blocks.
  const int fi = a.m <= 32 ? 1 : a.m <= 64 ? 2 : 4;
  if (fmt == kFmtNvfp4) {
    if (a.act)
      launch_gemm_fi<kFmtNvfp4, true>(a, fi, grid, block, stream);
    else
      launch_gemm_fi<kFmtNvfp4, false>(a, fi, grid, block, stream);
  } else {
    if (a.act)
      launch_gemm_fi<kFmtMxfp4, true>(a, fi, grid, block, stream);
    else
      launch_gemm_fi<kFmtMxfp4, false>(a, fi, grid, block, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || units == 0) return e;
  return launch_tail_reduce(a, kGemmBM, stream);
}

hipError_t launch_moe_gemm(const MfmaArgs& a, const MoeArgs& moe, int fmt, hipStream_t stream, dim3* grid_out,
                           dim3* block_out) {
  const int64_t wgs = moe_gemm_slots(moe.pairs, moe.experts) * a.plan.n_tiles;
  if (wgs <= 0 || wgs * kThreads >= (int64_t{1} << 32)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(wgs)), block(kThreads);
  if (grid_out) *grid_out = grid;
  if (block_out) *block_out = block;
  if (fmt == kFmtNvfp4) {
    if (a.act)
      hipLaunchKernelGGL((moe_gemm_kernel<kFmtNvfp4, true>), grid, block, 0, stream, a, moe);
    else
      hipLaunchKernelGGL((moe_gemm_kernel<kFmtNvfp4, false>), grid, block, 0, stream, a, moe);
  } else {
    if (a.act)
      hipLaunchKernelGGL((moe_gemm_kernel<kFmtMxfp4, true>), grid, block, 0, stream, a, moe);
    else
      hipLaunchKernelGGL((moe_gemm_kernel<kFmtMxfp4, false>), grid, block, 0, stream, a, moe);
  }
  return hipGetLastError();
}

hipError_t launch_tail_reduce(const MfmaArgs& a, int bm, hipStream_t stream) {
  if (bm == kW4BM) {
    const unsigned blocks = static_cast<unsigned>(a.plan.tail_tiles * (kReduceItems<kW4BM> / kReduceThreads));
    hipLaunchKernelGGL(tail_reduce_kernel<kW4BM>, dim3(blocks), dim3(kReduceThreads), 0, stream, a);
  } else {
    const unsigned blocks = static_cast<unsigned>(a.plan.tail_tiles * (kReduceItems<kGemmBM> / kReduceThreads));
    hipLaunchKernelGGL(tail_reduce_kernel<kGemmBM>, dim3(blocks), dim3(kReduceThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace fp4
