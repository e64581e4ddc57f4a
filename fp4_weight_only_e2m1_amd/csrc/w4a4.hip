// W4A4 MXFP4 linear on gfx950's block-scaled MFMA: the activations are
// quantized at call time to MXFP4 (E2M1 codes, one E8M0 scale per 32 k), then
// contracted with the prepared MXFP4 weight by
// v_mfma_scale_f32_32x32x64_f8f6f4, which takes both operands as 4-bit codes
// and applies both block scales itself.
//
// This is the variant the pages keep apart from the weight-only default: the
// compressed-tensors MXFP4 scheme with quantized activations, run by a GEMM
// over 4-bit operands with block-32 E8M0 scales ("native MXFP4 keep-quant",
// vllm.cpp PR #38, commit list, the W0 vehicle and the W1 kernel).  It is an
// entry point of its own with its own numerics contract; the weight-only path
// never calls it.
//
// Activation quantizer (the OCP MX v1.0 conversion; the pages name the
// scheme, not its rule): per row and 32-code block, the scale byte is
// max(E - 2, 0), E the biased exponent of the block's largest |x| as a bf16,
// i.e. X = 2^(floor(log2 amax) - 2) clamped to at least 2^-127; each element
// becomes the E2M1 code nearest to x / X, ties to the even code, saturating
// at 6, with the sign bit of x.  A block holding an Inf or NaN gets scale
// byte 0xFF and zero codes.  x / X is exact in float32 (a power-of-two
// scaling that stays below 8), so every decision matches an exact one.
//
// GEMM tile: a workgroup of 8 waves computes 256 activation rows x 256
// weight rows, wave w = 4 wm + wn owning activation rows [128 wm, +128) and
// weight rows [64 wn, +64).  K advances 128 codes per stage; a stage holds in
// LDS
//   activation codes   256 rows x 64 bytes                    16 KiB
//   weight codes       256 rows x 64 bytes                    16 KiB
//   activation scales  16 row groups x 4 blocks x 16 rows      1 KiB
//   weight scales      16 row groups x 4 blocks x 16 rows      1 KiB
// copied by the load-to-LDS path into four stage buffers (136 KiB: one
// workgroup per CU), three stages in flight.  Results leave through LDS as
// whole rows (gemm_common.hpp).  Tiles past the last full round of
// workgroups either run as two 128-row halves over all of K (where the plan
// would split them two ways along K) or as K ranges whose partials a reduce
// launch adds; a tile with at most 128 rows below m computes its upper half
// only.  Measured on MI355X at the gate_up shape (m = 1024): 128 x 256 tiles
// with direct stores 1.66 PFLOP/s, 256 x 256 tiles 1.78, results through LDS
// 2.22, tail tiles as row halves 2.64.
//
// Operand layout of the instruction with 4-bit A and B (checked on MI355X
// against a host product): lane l supplies row l % 32 of A and column l % 32
// of B, each as the 32 codes k = 32 (l / 32) .. +31 of the 64-k step in 16
// bytes (low nibble first), with one E8M0 byte each for that row / column
// and 32-code block; result e of lane l is C[8 (e / 4) + 4 (l / 32) + e % 4]
// [l % 32].  The weights are the A operand, so the result layout -- and the
// stores -- are the W4A16 GEMM's.
#include "fp4_common.hpp"
#include "fp4_device.hpp"
#include "gemm_common.hpp"
#include "lds_copy.hpp"

namespace fp4 {
namespace {

// ---------------------------------------------------------------------------
// Activation quantizer: four lanes per (row, 32-code block), each taking 8
// consecutive values (one 16-byte load); consecutive lanes read consecutive
// bytes of a row.  The block's amax is combined across the four lanes, each
// lane writes its 8 codes (4 bytes) and the block's first lane its scale.

constexpr int kQuantThreads = 256;

__global__ __launch_bounds__(kQuantThreads) void act_quant_kernel(const uint16_t* __restrict__ x, int m, int k,
                                                                  int64_t act_k, uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales) {
  const int64_t kb = act_k / 32;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kQuantThreads + threadIdx.x;
  const int q = static_cast<int>(i & 3);   // quarter of the block
  const int64_t rb = i >> 2;               // (row, block)
  const int64_t row = rb / kb;
  const int64_t blk = rb - row * kb;
  // Every lane of a 4-lane group has the same (row, block), so the group
  // leaves together and the shuffles below see only active partners.
  if (row >= m) return;
  const bool real = blk * 32 < k;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (real) v = *reinterpret_cast<const uint4*>(x + row * k + blk * 32 + 8 * q);
  const uint32_t h[4] = {v.x, v.y, v.z, v.w};
  uint32_t amax = 0;
  uint32_t nonfinite = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t b = (h[j / 2] >> (16 * (j & 1))) & 0xFFFFu;
    const uint32_t mag = b & 0x7FFFu;  // bf16 magnitudes order as integers
    amax = mag > amax ? mag : amax;
    nonfinite |= (b & 0x7F80u) == 0x7F80u;
  }
#pragma unroll
  for (int d = 1; d < 4; d <<= 1) {
    const uint32_t oa = static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), d, 4));
    const uint32_t on = static_cast<uint32_t>(__shfl_xor(static_cast<int>(nonfinite), d, 4));
    amax = oa > amax ? oa : amax;
    nonfinite |= on;
  }
  uint32_t sbyte = 0;
  uint32_t word = 0;
  if (real) {
    if (nonfinite) {
      sbyte = 0xFFu;
    } else {
      const uint32_t e = amax >> 7;
      sbyte = e > 2 ? e - 2 : 0;
      const float inv = __uint_as_float((254u - sbyte) << 23);  // 1 / X = 2^(127 - sbyte)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t b = (h[j / 2] >> (16 * (j & 1))) & 0xFFFFu;
        const float f = __uint_as_float((b & 0x7FFFu) << 16) * inv;
        // Nearest E2M1 magnitude: each threshold is a midpoint of the grid;
        // at a midpoint the even code wins (> keeps the lower, >= takes the upper).
        uint32_t c = (f > 0.25f) + (f >= 0.75f) + (f > 1.25f) + (f >= 1.75f) + (f > 2.5f) + (f >= 3.5f) + (f > 5.0f);
        c |= (b >> 12) & 8u;  // sign
        word |= c << (4 * j);
      }
    }
  }
  *reinterpret_cast<uint32_t*>(codes + row * (act_k / 2) + blk * 16 + 4 * q) = word;
  if (q == 0) scales[((row >> 4) * kb + blk) * kRowGroup + (row & 15)] = static_cast<uint8_t>(sbyte);
}

// ---------------------------------------------------------------------------
// Tile GEMM.

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;
constexpr int kStages = 4;
constexpr int kRowBytes = kW4BK / 2;             // code bytes of a row per stage
constexpr int kRowChunks = kRowBytes / 16;       // 16-byte chunks (32-code blocks) of a row per stage
constexpr int kAChunks = kW4BM * kRowChunks;     // activation code chunks per stage (whole tile)
constexpr int kBChunks = kGemmBN * kRowChunks;   // weight code chunks per stage
constexpr int kBPer = kBChunks / kThreads;
// Activation code chunks each thread copies per stage when the tile has
// 64 FI activation rows (FI = 4: whole tiles; FI = 2: the half tiles of the
// tail).
template <int FI>
constexpr int kAPer = 64 * FI * kRowChunks / kThreads;
static_assert(kAChunks % kThreads == 0 && kBChunks % kThreads == 0 && kAPer<2> >= 1, "stage split");
static_assert(kThreads == 64 * 8 && kW4BM == 256 && kGemmBN == 256, "two rows of four waves");

struct alignas(16) Stage {
  uint4 a[kAChunks];
  uint4 b[kBChunks];
  uint4 sa[64];  // [row group 0..15][block 0..3][16 rows] (half tiles: row groups 0..7, then a repeat)
  uint4 sb[64];  // [row group 0..15][block 0..3][16 rows]
};
static_assert(kStages * sizeof(Stage) <= 160 * 1024, "one workgroup of four stages per CU");
static_assert(kW4BM * kStageYRow <= kStages * sizeof(Stage) && 128 * kStagePRow <= kStages * sizeof(Stage),
              "result staging fits in the stage buffers");

// Code stages: row r holds its 4 chunks at 16-byte slots 4 r .. 4 r + 3,
// chunk c in slot 4 r + (c ^ ((r >> 2) & 3)).  A fragment read has 16 lanes
// on 16 consecutive rows and one chunk; their bank groups (16-byte units
// mod 16) 4 (r & 3) + (c ^ ((r >> 2) & 3)) are distinct.

// The stage copies of one tile: chunk positions in LDS are fixed by lane
// order (lane l's 16 bytes land at 16 l past the wave's base), so the swizzle
// is applied by choosing which global chunk each lane fetches.  Each lane keeps
// 32-bit offsets from wave-uniform bases that advance with the stage.  Wave 0
// also copies the weight scales, wave 1 the activation scales (one 16-byte
// chunk per lane: row group lane / 4, block lane % 4 of the stage).
template <int FI>
struct Copier {
  const uint8_t* xa;  // activation code row m0
  const uint8_t* wb;  // weight code row n0
  const uint8_t* xs;  // activation scale row group m0 / 16
  const uint8_t* ws;  // weight scale row group n0 / 16
  uint32_t aoff[kAPer<FI>], boff[kBPer], soff;

  __device__ __forceinline__ Copier(const MfmaArgs& a, int64_t m0, int64_t n0, int t, int wave) {
    const int64_t arow = a.act_k / 2;
    const int64_t brow = a.k_pad / 2;
    xa = a.xq_codes + m0 * arow;
    wb = a.codes + n0 * brow;
    xs = a.xq_scales + (m0 / kRowGroup) * (a.act_k / 32) * kRowGroup;
    ws = a.scales + (n0 / kRowGroup) * a.ksegs * kRowGroup;
#pragma unroll
    for (int i = 0; i < kAPer<FI>; ++i) {
      const int p = i * kThreads + t;
      const int r = p >> 2;
      const int c = (p & 3) ^ ((r >> 2) & 3);
      aoff[i] = static_cast<uint32_t>(r * arow + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int p = i * kThreads + t;
      const int r = p >> 2;
      const int c = (p & 3) ^ ((r >> 2) & 3);
      boff[i] = static_cast<uint32_t>(r * brow + 16 * c);
    }
    const int lane = t & 63;
    // Activation scales: 4 FI row groups; with FI = 2 lanes 32..63 repeat
    // lanes 0..31 (into chunks 32..63, unused), so no lane reads past the
    // tile's rows.
    const int arg = FI == 4 ? lane >> 2 : (lane & 31) >> 2;
    soff = wave == 0 ? static_cast<uint32_t>((lane >> 2) * a.ksegs * kRowGroup + 16 * (lane & 3))
                     : static_cast<uint32_t>(arg * (a.act_k / 32) * kRowGroup + 16 * (lane & 3));
  }

  __device__ __forceinline__ void issue(int ks, Stage& sb, int wave) const {
    const uint32_t la = lds_addr(sb.a) + 64 * 16 * wave;
    const uint32_t lb = lds_addr(sb.b) + 64 * 16 * wave;
    const uint8_t* xb = xa + static_cast<int64_t>(ks) * kRowBytes;
#pragma unroll
    for (int i = 0; i < kAPer<FI>; ++i) copy16_sbase(xb, aoff[i], la + i * kThreads * 16);
    const uint8_t* wbk = wb + static_cast<int64_t>(ks) * kRowBytes;
#pragma unroll
    for (int i = 0; i < kBPer; ++i) copy16_sbase(wbk, boff[i], lb + i * kThreads * 16);
    if (wave == 0)
      copy16_sbase(ws + static_cast<int64_t>(ks) * kRowChunks * kRowGroup, soff, lds_addr(sb.sb));
    else if (wave == 1)
      copy16_sbase(xs + static_cast<int64_t>(ks) * kRowChunks * kRowGroup, soff, lds_addr(sb.sa));
  }
};

// Wait until this wave's copies of all but the newest `STAGES` stages have
// landed, then join the workgroup barrier.
template <int STAGES, int FI>
__device__ __forceinline__ void wait_stages_barrier(int wave) {
  if (wave < 2)
    wait_vm_barrier<STAGES * (kAPer<FI> + kBPer + 1)>();
  else
    wait_vm_barrier<STAGES * (kAPer<FI> + kBPer)>();
}

// The operands of one 64-k MFMA step: 2 weight and FI activation fragments
// with their scale bytes.
template <int FI>
struct Frags {
  i32x8_t w[2], x[FI];
  int ws[2], xs[FI];
};

__device__ __forceinline__ i32x8_t as_operand(uint4 q) {
  const i32x8_t v = {static_cast<int>(q.x), static_cast<int>(q.y), static_cast<int>(q.z), static_cast<int>(q.w),
                     0, 0, 0, 0};
  return v;
}

// This lane's byte offsets inside a stage for one MFMA step: its code chunk
// of activation row 128 wm + l % 32 (xo) and weight row 64 wn + l % 32 (wo),
// and its scale bytes (xso, wso).  Fragment i / j adds 32 rows: 2048 bytes of codes,
// 128 bytes of scales.
struct LaneOffsets {
  uint32_t xo, wo, xso, wso;
};

template <int FI>
__device__ __forceinline__ void read_step(const Stage& st, const LaneOffsets& o, Frags<FI>& f) {
  const char* ca = reinterpret_cast<const char*>(st.a) + o.xo;
  const char* cb = reinterpret_cast<const char*>(st.b) + o.wo;
  const uint8_t* sa = reinterpret_cast<const uint8_t*>(st.sa) + o.xso;
  const uint8_t* sb = reinterpret_cast<const uint8_t*>(st.sb) + o.wso;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    f.w[j] = as_operand(*reinterpret_cast<const uint4*>(cb + 2048 * j));
    f.ws[j] = sb[128 * j];
  }
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    f.x[i] = as_operand(*reinterpret_cast<const uint4*>(ca + 2048 * i));
    f.xs[i] = sa[128 * i];
  }
}

template <int FI>
__device__ __forceinline__ void mfma_step(const Frags<FI>& f, f32x16_t (&acc)[FI][2]) {
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[j], f.x[i], acc[i][j], 4, 4, 0, f.ws[j], 0,
                                                                  f.xs[i]);
}

// acc = the (m0, n0) tile's sums over stages [k_begin, k_end).  Stage ks
// lives in buffer (ks - k_begin) % 4.  Each iteration waits for stage ks
// (and, through the barrier, for every wave to be done with stage ks - 1,
// whose buffer it then refills with stage ks + 3) and runs the stage's two
// MFMA steps.  One loop body, so the accumulators keep their registers.
template <int FI>
__device__ __forceinline__ void run_tile(const MfmaArgs& a, int64_t m0, int64_t n0, int k_begin, int k_end,
                                         Stage (&st)[kStages], f32x16_t (&acc)[FI][2]) {
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int l32 = lane & 31;
  const int lh = lane >> 5;
  const int xr0 = (wave >> 2) * 32 * FI + l32;  // activation row of this lane's first fragment
  const int wr0 = (wave & 3) * 64 + l32;     // weight row of this lane's first fragment
  // Step s uses block c = 2 s + lh of the stage, in slot c ^ sw of the row
  // (sw = (row >> 2) & 3, the same for every row of this lane): step 1's
  // slot is step 0's with bit 1 flipped.
  const int sw = (l32 >> 2) & 3;
  LaneOffsets o0, o1;
  o0.xo = static_cast<uint32_t>(16 * (4 * xr0 + (lh ^ sw)));
  o0.wo = static_cast<uint32_t>(16 * (4 * wr0 + (lh ^ sw)));
  o0.xso = static_cast<uint32_t>((xr0 >> 4) * 64 + 16 * lh + (xr0 & 15));
  o0.wso = static_cast<uint32_t>((wr0 >> 4) * 64 + 16 * lh + (wr0 & 15));
  o1.xo = o0.xo ^ 32u;
  o1.wo = o0.wo ^ 32u;
  o1.xso = o0.xso + 32;
  o1.wso = o0.wso + 32;
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  const Copier<FI> cp(a, m0, n0, t, wave);
  cp.issue(k_begin, st[0], wave);
  if (k_begin + 1 < k_end) cp.issue(k_begin + 1, st[1], wave);
  if (k_begin + 2 < k_end) cp.issue(k_begin + 2, st[2], wave);
  int buf = 0;
  for (int ks = k_begin; ks < k_end; ++ks) {
    // Stage ks landed when at most the copies of the (up to two) stages
    // after it are in flight.
    if (ks + 2 < k_end)
      wait_stages_barrier<2, FI>(wave);
    else if (ks + 1 < k_end)
      wait_stages_barrier<1, FI>(wave);
    else
      wait_stages_barrier<0, FI>(wave);
    const int fill = buf == 0 ? kStages - 1 : buf - 1;
    if (ks + 3 < k_end) cp.issue(ks + 3, st[fill], wave);
    Frags<FI> f;
    read_step(st[buf], o0, f);
    mfma_step(f, acc);
    read_step(st[buf], o1, f);
    mfma_step(f, acc);
    buf = buf == kStages - 1 ? 0 : buf + 1;
  }
}

// One launch for all tiles, planned as the W4A16 GEMM: workgroup b <
// dp_tiles computes data-parallel tile b (in XCD order) over all of K and
// stores bf16 y; the last tail_tiles x splits workgroups then each compute one
// K range of a tail tile into an fp32 partial, which the reduce launch adds.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void w4a4_gemm_kernel(const MfmaArgs a) {
  __shared__ Stage st[kStages];
  const GemmPlan& pl = a.plan;
  const int bid = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  char* lds = reinterpret_cast<char*>(st);
  if (bid < pl.dp_tiles) {
    int64_t m0, n0;
    tile_coords<kW4BM>(pl, dp_tile_of(pl, bid), m0, n0);
    if (a.m - m0 <= kW4BM / 2) {
      // A tile with at most 128 rows below m (small m, or the last row of
      // tiles): only its upper half is computed.
      f32x16_t acc[2][2];
      run_tile<2>(a, m0, n0, 0, pl.ksteps, st, acc);
      store_tile_bf16_staged<kW4BM / 2, kThreads, kW4BM / 2, 2>(a, m0, n0, wave, acc, lds);
    } else {
      f32x16_t acc[4][2];
      run_tile<4>(a, m0, n0, 0, pl.ksteps, st, acc);
      store_tile_bf16_staged<kW4BM, kThreads, kW4BM>(a, m0, n0, wave, acc, lds);
    }
  }
  // The last `units` workgroups run the tail units.  Row halves over all of
  // K are numbered XCD by XCD, so that both halves of a tail tile and the
  // tiles of neighbouring activation-row tiles (the same weight tile) share
  // an XCD's L2: dealt in launch order, each weight tile of such a tail was
  // fetched from HBM by every XCD (measured on MI355X for the 2 x 12288 x
  // 4096 gate_up at m = 1024: the GEMM's HBM reads 198 -> 89 MB per call,
  // 80.4 -> 79.7 us).  K ranges keep launch order (numbered XCD by XCD, the
  // 17408 x 5120 layer at m = 1024 and 4096 was 1-2% slower).
  const int units = pl.tail_tiles * pl.splits;
  const int first = static_cast<int>(gridDim.x) - units;
  if (bid < first) return;
  const int u = pl.mhalf ? xcd_major_index(bid, first, static_cast<int>(gridDim.x), pl.xcds) : bid - first;
  __syncthreads();  // the stage buffers are reused
  int64_t m0, n0;
  tile_coords<kW4BM>(pl, pl.dp_tiles + u / pl.splits, m0, n0);
  if (pl.mhalf) {
    // Half u % 2 of the tail tile's rows, over all of K, stored as bf16 y.
    m0 += (kW4BM / 2) * (u % 2);
    if (m0 >= a.m) return;
    f32x16_t acc[2][2];
    run_tile<2>(a, m0, n0, 0, pl.ksteps, st, acc);
    store_tile_bf16_staged<kW4BM / 2, kThreads, kW4BM / 2, 2>(a, m0, n0, wave, acc, lds);
    return;
  }
  const int split = u % pl.splits;
  f32x16_t acc[4][2];
  run_tile<4>(a, m0, n0, static_cast<int>(static_cast<int64_t>(split) * pl.ksteps / pl.splits),
              static_cast<int>(static_cast<int64_t>(split + 1) * pl.ksteps / pl.splits), st, acc);
  store_tile_partial_staged<kW4BM, kThreads, 128>(a, u, m0, wave, acc, lds);
}

}  // namespace

hipError_t launch_act_quant_mxfp4(const uint16_t* x, int m, int k, uint8_t* codes, uint8_t* scales,
                                  hipStream_t stream) {
  const int64_t act_k = w4a4_act_k(k);
  const int64_t items = static_cast<int64_t>(m) * (act_k / 32) * 4;
  const unsigned blocks = static_cast<unsigned>((items + kQuantThreads - 1) / kQuantThreads);
  hipLaunchKernelGGL(act_quant_kernel, dim3(blocks), dim3(kQuantThreads), 0, stream, x, m, k, act_k, codes, scales);
  return hipGetLastError();
}

hipError_t launch_w4a4(const MfmaArgs& a, hipStream_t stream, dim3* grid_out, dim3* block_out) {
  const GemmPlan& p = a.plan;
  const int units = p.tail_tiles * p.splits;
  const dim3 grid(static_cast<unsigned>(p.dp_tiles > units ? p.dp_tiles : units));
  const dim3 block(kThreads);
  if (grid_out) *grid_out = dim3(grid.x, static_cast<unsigned>(units));
  if (block_out) *block_out = block;
  hipLaunchKernelGGL(w4a4_gemm_kernel, grid, block, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || units == 0 || p.mhalf) return e;
  return launch_tail_reduce(a, kW4BM, stream);
}

}  // namespace fp4
