// Prefill-shaped W4A16 FP4 GEMM (m > 8 activation rows) on gfx950 bf16 MFMA.
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
// stages in flight while the third is consumed.
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

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWaves = kGemmWavesM * 4;
constexpr int kThreads = kWaves * 64;
constexpr int kStages = 3;
constexpr int kGroupM = 8;  // activation-row tiles per tile-order group
constexpr int kAChunks = kGemmBM * kGemmBK * 2 / 16;  // 16-byte chunks of an x stage
constexpr int kBChunks = kGemmBN * kGemmBK / 2 / 16;  // 16-byte chunks of a code stage
constexpr int kAPer = kAChunks / kThreads;
constexpr int kBPer = kBChunks / kThreads;
static_assert(kAChunks % kThreads == 0 && kBChunks % kThreads == 0, "stage split");

template <int FMT>
struct Cfg {
  static constexpr int P = scales_per_seg(FMT);
  static constexpr int kSChunks = kGemmBN / kRowGroup * 2 * kRowGroup * P / 16;  // 64 NVFP4, 32 MXFP4
  static constexpr int kSPerWave = kSChunks / kWaves;
  static_assert(kSChunks % kWaves == 0, "scale split");
};

template <int FMT>
struct alignas(16) Stage {
  uint4 a[kAChunks];
  uint4 b[kBChunks];
  uint4 s[Cfg<FMT>::kSChunks];
};

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

// Wait until at most N of this wave's vector-memory operations are in flight
// and its LDS operations are done, then join the workgroup barrier.  Written
// as one asm statement so the compiler moves no memory access across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Global -> LDS copies of 16 bytes per lane: lane l's bytes land at LDS
// address m0 + 16 l, m0 being the same for the whole wave.  Issued as inline
// asm so that the compiler, which would otherwise guard every later LDS read
// with a wait for all copies in flight, leaves the waits to the pipeline
// (wait_vm_barrier); M0 is restored after.  Device code only: the host pass of
// the compiler cannot parse the asm.
//   copy16_sbase: address = 64-bit base (wave-uniform) + 32-bit lane offset.
//   copy16_vaddr: address = 64-bit per-lane pointer.
__device__ __forceinline__ void copy16_sbase(const void* base, uint32_t off, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
#else
  (void)base;
  (void)off;
  (void)lds;
#endif
}

__device__ __forceinline__ void copy16_vaddr(const void* g, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds)
      : "memory");
#else
  (void)g;
  (void)lds;
#endif
}

// LDS byte address of a __shared__ object (the low half of its generic address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Load-to-LDS copies issued per wave per stage (x, codes, one for scales).
constexpr int kLoadsPerStage = kAPer + kBPer + 1;

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
template <int FMT>
struct Copier {
  static constexpr int P = Cfg<FMT>::P;
  const uint16_t* xt;    // x row m0
  const uint8_t* ct;     // code row n0
  const uint8_t* st;     // scale row group n0 / 16
  const uint8_t* zeros;  // 16 zero bytes: code row n0 from code k on
  uint32_t xoff[kAPer], coff[kBPer], soff;
  int xk[kAPer];         // first k of this lane's x chunks within a stage
  int k;
  uint32_t lds_wave_a, lds_wave_b, lds_wave_s;  // this wave's chunk offsets within a stage

  __device__ __forceinline__ Copier(const MfmaArgs& a, int64_t m0, int64_t n0, int t, int wave) {
    const int64_t row_bytes = a.k_pad / 2;
    k = a.k;
    xt = a.x + m0 * a.k;
    ct = a.codes + n0 * row_bytes;
    st = a.scales + (n0 / kRowGroup) * a.ksegs * kRowGroup * P;
    zeros = ct + a.k / 2;
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int p = i * kThreads + t;
      const int r = p >> 3;
      const int c = (p & 7) ^ ((r >> 1) & 7);
      const int64_t rr = m0 + r < a.m ? r : a.m - 1 - m0;
      xoff[i] = static_cast<uint32_t>(rr * a.k * 2 + 16 * c);
      xk[i] = 8 * c;
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int p = i * kThreads + t;
      const int r = p >> 1;
      const int h = (p & 1) ^ ((r >> 3) & 1);
      coff[i] = static_cast<uint32_t>(r * row_bytes + 16 * h);
    }
    // Scales: 16 row groups x 2 segments x 16 rows x P bytes, contiguous per
    // row group in the prepared layout; lanes past the wave's share idle.
    const int lane = t & 63;
    const int ps = wave * Cfg<FMT>::kSPerWave + (lane < Cfg<FMT>::kSPerWave ? lane : 0);
    soff = static_cast<uint32_t>((ps / (2 * P)) * a.ksegs * kRowGroup * P + 16 * (ps % (2 * P)));
    lds_wave_a = 64 * 16 * wave;
    lds_wave_b = 64 * 16 * wave;
    lds_wave_s = Cfg<FMT>::kSPerWave * 16 * wave;
  }

  __device__ __forceinline__ void issue(int64_t k0, Stage<FMT>& sb, int lane) const {
    const uint32_t la = lds_addr(sb.a) + lds_wave_a;
    const uint32_t lb = lds_addr(sb.b) + lds_wave_b;
    const uint32_t ls = lds_addr(sb.s) + lds_wave_s;
    if (k0 + kGemmBK <= k) {
      const uint16_t* xb = xt + k0;
#pragma unroll
      for (int i = 0; i < kAPer; ++i) copy16_sbase(xb, xoff[i], la + i * kThreads * 16);
    } else {
#pragma unroll
      for (int i = 0; i < kAPer; ++i) {
        const void* src = k0 + xk[i] < k ? static_cast<const void*>(reinterpret_cast<const uint8_t*>(xt + k0) + xoff[i])
                                         : static_cast<const void*>(zeros);
        copy16_vaddr(src, la + i * kThreads * 16);
      }
    }
    const uint8_t* cb = ct + k0 / 2;
#pragma unroll
    for (int i = 0; i < kBPer; ++i) copy16_sbase(cb, coff[i], lb + i * kThreads * 16);
    if (lane < Cfg<FMT>::kSPerWave) copy16_sbase(st + (k0 / 32) * kRowGroup * P, soff, ls);
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

// One stage of the contraction for this wave: 4 MFMA steps of 16 k, each
// over its 2 x 32 weight rows and 4 activation row blocks.  Software
// pipelined: the x fragments and decoded weights of step kk + 1 are read and
// decoded while the MFMAs of step kk run, and the schedule interleaves one
// MFMA with a few VALU decode instructions so decoding hides under the matrix
// core.
template <int FMT>
__device__ __forceinline__ void compute_stage(const Stage<FMT>& st, int xr0, int wr0, int lh, f32x16_t (&acc)[4][2]) {
  constexpr int P = Cfg<FMT>::P;
  const uint8_t* sb = reinterpret_cast<const uint8_t*>(st.s);
  uint4 code[2];
  uint32_t sc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wr0 + 32 * j;
    code[j] = st.b[b_slot(r, lh)];
    const int so = (((r >> 4) * 2 + lh) * kRowGroup + (r & 15)) * P;
    if constexpr (P == 2)
      sc[j] = *reinterpret_cast<const uint16_t*>(sb + so);
    else
      sc[j] = sb[so];
  }
  Frag xf[2][4], wf[2][2];
  auto load_x = [&](int kk, Frag (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = st.a[a_slot(xr0 + 32 * i, 4 * lh + kk)];
      f[i].u[0] = q.x;
      f[i].u[1] = q.y;
      f[i].u[2] = q.z;
      f[i].u[3] = q.w;
    }
  };
  auto decode = [&](int kk, Frag (&f)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t word = kk == 0 ? code[j].x : kk == 1 ? code[j].y : kk == 2 ? code[j].z : code[j].w;
      const uint32_t sbyte = P == 2 ? (kk < 2 ? sc[j] & 0xFFu : sc[j] >> 8) : sc[j];
      decode8<FMT>(word, sbyte, f[j]);
    }
  };
  load_x(0, xf[0]);
  decode(0, wf[0]);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk < 3) {
      load_x(kk + 1, xf[(kk + 1) & 1]);
      decode(kk + 1, wf[(kk + 1) & 1]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[kk & 1][j].v, xf[kk & 1][i].v, acc[i][j], 0, 0, 0);
  }
  // Schedule: the stage's first LDS reads and decode, then per MFMA step its
  // successor's four x reads and eight (MFMA, VALU) pairs.
  constexpr int kDecodeValu = FMT == kFmtMxfp4 ? 8 : 36;  // VALU per step's decode
  constexpr int kValuPerMfma = (kDecodeValu + 7) / 8;
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
  __builtin_amdgcn_sched_group_barrier(kSchedValu, kDecodeValu, 0);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk < 3) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (kk < 3) __builtin_amdgcn_sched_group_barrier(kSchedValu, kValuPerMfma, 0);
    }
  }
}

// Pipeline step for the stage `ks` held in buffer `cur`: wait for it to land
// (leaving the next stage's copies in flight), then refill buffer `nxt2` --
// read two stages ago, which the barrier just proved every wave has finished
// with -- with stage ks + 2, and consume `cur`.
template <int FMT>
__device__ __forceinline__ void pipeline_step(const Copier<FMT>& cp, int ks, int k_end, const Stage<FMT>& cur,
                                              Stage<FMT>& nxt2, int lane, int xr0, int wr0, int lh,
                                              f32x16_t (&acc)[4][2]) {
  if (ks + 1 < k_end)
    wait_vm_barrier<kLoadsPerStage>();
  else
    wait_vm_barrier<0>();
  if (ks + 2 < k_end) cp.issue(static_cast<int64_t>(ks + 2) * kGemmBK, nxt2, lane);
  compute_stage<FMT>(cur, xr0, wr0, lh, acc);
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));
// Buffer descriptor word 3 for raw (unformatted) 32-bit accesses.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Output column of prepared weight row `row`, or -1 for a padding row.
__device__ __forceinline__ int64_t out_col(const MfmaArgs& a, int64_t row, int& h) {
  h = static_cast<int>(row / a.n_proj_pad);
  const int64_t lr = row - static_cast<int64_t>(h) * a.n_proj_pad;
  return lr < a.n_proj ? static_cast<int64_t>(h) * a.n_proj + lr : -1;
}


// TAIL = false: workgroup b computes data-parallel tile b (in XCD order) over
// all of K.  TAIL = true: workgroup u computes split u % splits of tail tile
// u / splits and stores it as an fp32 partial.  Two kernels rather than one with a
// branch keep the register allocation of the data-parallel loop free of the
// finish code.
template <int FMT, bool TAIL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(const MfmaArgs a) {
  __shared__ Stage<FMT> st0, st1, st2;

  const GemmPlan& pl = a.plan;
  const int bid = blockIdx.x;
  int tile, k_begin, k_end;
  if constexpr (!TAIL) {
    // XCD-aware order: workgroup b runs on XCD b % 8, so XCD x gets the ids
    // x, x + 8, ...; give it the contiguous run of tiles starting at
    // x * q + min(x, r) (q = tiles / 8, r = tiles % 8).  Tiles are numbered
    // weight-tile-major, so a run shares weight and x tiles in that XCD's L2.
    const int xcd = bid % 8;
    const int q = pl.dp_tiles / 8;
    const int r = pl.dp_tiles % 8;
    tile = xcd * q + (xcd < r ? xcd : r) + bid / 8;
    k_begin = 0;
    k_end = pl.ksteps;
  } else {
    const int split = bid % pl.splits;
    tile = pl.dp_tiles + bid / pl.splits;
    k_begin = static_cast<int>(static_cast<int64_t>(split) * pl.ksteps / pl.splits);
    k_end = static_cast<int>(static_cast<int64_t>(split + 1) * pl.ksteps / pl.splits);
  }
  // Tile order: groups of kGroupM activation-row tiles, weight-tile-major
  // inside a group, so the 64 tiles an XCD holds at once form an 8 x 8 block
  // that shares 8 x tiles and 8 weight tiles in its L2 (x is re-read from
  // outside the XCD once per 8 weight tiles instead of once per 2).
  const int group = tile / (kGroupM * pl.n_tiles);
  const int in_group = tile - group * kGroupM * pl.n_tiles;
  const int rows = pl.m_tiles - group * kGroupM < kGroupM ? pl.m_tiles - group * kGroupM : kGroupM;
  const int n_tile = in_group / rows;
  const int m_tile = group * kGroupM + (in_group - n_tile * rows);
  const int64_t m0 = static_cast<int64_t>(m_tile) * kGemmBM;
  const int64_t n0 = static_cast<int64_t>(n_tile) * kGemmBN;

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int l32 = lane & 31;
  const int lh = lane >> 5;
  const int wm = wave / 4;
  const int wn = wave % 4;

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const Copier<FMT> cp(a, m0, n0, t, wave);
  const int xr0 = wm * 128 + l32;  // x row of this lane's first activation block
  const int wr0 = wn * 64 + l32;   // weight row of this lane's first weight block
  cp.issue(static_cast<int64_t>(k_begin) * kGemmBK, st0, lane);
  if (k_begin + 1 < k_end) cp.issue(static_cast<int64_t>(k_begin + 1) * kGemmBK, st1, lane);
  for (int ks = k_begin; ks < k_end; ks += kStages) {
    pipeline_step<FMT>(cp, ks, k_end, st0, st2, lane, xr0, wr0, lh, acc);
    if (ks + 1 >= k_end) break;
    pipeline_step<FMT>(cp, ks + 1, k_end, st1, st0, lane, xr0, wr0, lh, acc);
    if (ks + 2 >= k_end) break;
    pipeline_step<FMT>(cp, ks + 2, k_end, st2, st1, lane, xr0, wr0, lh, acc);
  }

  if constexpr (!TAIL) {
    // Whole tile: scale by the projection's global scale and store bf16 y,
    // four consecutive output columns (weight rows) of one activation row per
    // lane and (i, j, e4).
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
            for (int q = 0; q < 4; ++q)
              if (lr + q < a.n_proj) dst[q] = f32_to_bf16_rne(w[q]);
          }
        }
      }
    return;
  }

  // Tail unit: store this K range's fp32 partial tile [x row][weight row];
  // tail_reduce_kernel, the next launch, adds the splits.  Written with
  // buffer stores: with plain stores here the compiler's register allocation
  // of the K loop above spills.
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      a.partial + static_cast<int64_t>(bid) * kGemmBM * kGemmBN, 0, kGemmBM * kGemmBN * 4, kBufferRsrcWord3);
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

// Split-K finish of the tail tiles: y = G * (partial_0 + partial_1 + ... +
// partial_{S-1}), added in split order (a fixed order: the output does not
// depend on timing).  A separate launch, so every partial is complete and
// visible when it starts; each thread takes one (x row, 4 weight rows) item of
// one tail tile and keeps its S loads in flight kBatch at a time.
constexpr int kReduceThreads = 256;
constexpr int kReduceItems = kGemmBM * kGemmBN / 4;  // per tail tile
static_assert(kReduceItems % kReduceThreads == 0, "reduce split");

__global__ __launch_bounds__(kReduceThreads) void tail_reduce_kernel(const MfmaArgs a) {
  const GemmPlan& pl = a.plan;
  const int64_t gi = static_cast<int64_t>(blockIdx.x) * kReduceThreads + threadIdx.x;
  const int tail_tile = static_cast<int>(gi / kReduceItems);
  const int it = static_cast<int>(gi - static_cast<int64_t>(tail_tile) * kReduceItems);
  const int mr = it / (kGemmBN / 4);
  const int nr = 4 * (it % (kGemmBN / 4));
  const int tile = pl.dp_tiles + tail_tile;
  const int group = tile / (kGroupM * pl.n_tiles);
  const int in_group = tile - group * kGroupM * pl.n_tiles;
  const int rows = pl.m_tiles - group * kGroupM < kGroupM ? pl.m_tiles - group * kGroupM : kGroupM;
  const int n_tile = in_group / rows;
  const int m_tile = group * kGroupM + (in_group - n_tile * rows);
  const int64_t m = static_cast<int64_t>(m_tile) * kGemmBM + mr;
  if (m >= a.m) return;
  int h;
  const int64_t col = out_col(a, static_cast<int64_t>(n_tile) * kGemmBN + nr, h);
  if (col < 0) return;

  constexpr int kBatch = 8;
  const int64_t unit_floats = static_cast<int64_t>(kGemmBM) * kGemmBN;
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

hipError_t launch_mfma(const MfmaArgs& a, int fmt, hipStream_t stream, dim3* grid_out, dim3* block_out) {
  const GemmPlan& p = a.plan;
  const dim3 block(kThreads);
  const unsigned units = static_cast<unsigned>(p.tail_tiles * p.splits);
  if (grid_out) *grid_out = dim3(static_cast<unsigned>(p.dp_tiles), units);
  if (block_out) *block_out = block;
  if (p.dp_tiles > 0) {
    if (fmt == kFmtNvfp4)
      hipLaunchKernelGGL((gemm_kernel<kFmtNvfp4, false>), dim3(p.dp_tiles), block, 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_kernel<kFmtMxfp4, false>), dim3(p.dp_tiles), block, 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (units > 0) {
    if (fmt == kFmtNvfp4)
      hipLaunchKernelGGL((gemm_kernel<kFmtNvfp4, true>), dim3(units), block, 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_kernel<kFmtMxfp4, true>), dim3(units), block, 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned reduce_blocks = static_cast<unsigned>(p.tail_tiles * (kReduceItems / kReduceThreads));
    hipLaunchKernelGGL(tail_reduce_kernel, dim3(reduce_blocks), dim3(kReduceThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace fp4
