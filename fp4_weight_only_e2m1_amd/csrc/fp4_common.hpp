// Shared host/device definitions of the prepared weight layout and the launch
// interface between the C ABI (api.cpp) and the kernels (*.hip).
#pragma once

#include <cstddef>
#include <cstdint>
#include <hip/hip_runtime.h>

namespace fp4 {

constexpr int kFmtNvfp4 = 0;
constexpr int kFmtMxfp4 = 1;

// Prepared layout granules.  Rows are padded to kRowAlign so every kernel tile
// is full; k is padded to kSlabK, the k-extent one 32-lane GEMV team covers per
// step (32 lanes x 32 codes = 16 bytes per lane).
constexpr int kRowAlign = 256;
constexpr int kSlabK = 1024;
constexpr int kRowGroup = 16;        // rows whose scale bytes are interleaved
constexpr int kGemvTeams = 8;        // 32-lane teams per 256-thread GEMV workgroup
constexpr int kDecodeTileRows = 64;  // rows of an MFMA-decode workgroup
constexpr int kDecodeThreads = 256;  // threads of a decode workgroup (GEMV and MFMA decode)
constexpr int kGemvMaxSlabsPerSplit = 4;  // x staged in LDS: 8 rows * 4096 k * 2 B = 64 KiB
constexpr int kGemvMaxM = 8;
constexpr int kTargetCUs = 256;      // MI355X compute units: the nominal machine of every plan
// Compute units per XCD on MI355X (8 XCDs of 32 CUs).  Workgroup b of a launch
// is dispatched to XCD b % (number of XCDs).
constexpr int kCUsPerXcd = 32;
// XCDs of a device (or partition) of `cus` compute units, 1..8.
inline int xcds_of(int cus) {
  const int x = cus / kCUsPerXcd;
  return x < 1 ? 1 : x > 8 ? 8 : x;
}
// m from which the decode path contracts on MFMA instead of VALU v_dot2
// (measured crossover on MI355X: the VALU GEMV is faster at m = 1, 2).
constexpr int kDecodeMfmaMinM = 3;
// Largest m the decode path serves.  The MFMA decode kernel's 16x16x32 MFMA
// computes 16 activation rows whatever m is (the rows past m read zeros), so
// m = 9..16 costs it the same matrix-core work as m = 8 and only more x
// copies per stage (x stages of 16 rows instead of 8); m = 17..32 runs two
// MFMAs per decoded weight fragment (two 16-row groups, x stages of 32 rows).
// The SwiGLU epilogue of the decode kernels serves up to kDecodeActMaxM rows
// (its float32 tile in LDS would cost the 32-row instances a workgroup per
// CU); SwiGLU calls with more rows take the tile GEMM.
constexpr int kDecodeMaxM = 32;
constexpr int kDecodeActMaxM = 16;
// k-extent of one stage of the MFMA decode kernel (codes), and its LDS stage
// buffers (all but one in flight).
constexpr int kDecodeStageK = 256;
constexpr int kDecodeBuffers = 3;
// Stage buffers of the 96-row MFMA decode tiles, whose launches give each CU
// one workgroup, so LDS leaves room for a deeper pipeline: 4 for MXFP4, 3 for
// NVFP4.  Measured on MI355X on the 24576 x 4096 fused gate_up (HIP-graph
// replay, medians of repeated runs, us, 3 / 4 / 5 buffers): MXFP4 m = 4
// 12.5 / 12.1 / 12.6, m = 8 12.5 / 12.1 / 12.7; NVFP4 m = 4 16.7 / 17.2 /
// 17.5, m = 8 16.6 / 17.2 / 17.4.
inline constexpr int decode_buffers_96(int fmt) { return fmt == kFmtMxfp4 ? 4 : kDecodeBuffers; }

inline constexpr int group_size(int fmt) { return fmt == kFmtNvfp4 ? 16 : 32; }
// Scale bytes per 32-code segment of a row: 2 for NVFP4, 1 for MXFP4.
inline constexpr int scales_per_seg(int fmt) { return 32 / group_size(fmt); }
inline constexpr int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Byte offset of the scale of (row, k-group kg) in the prepared scale layout
// [n_pad/16][k_pad/32][16][P], P = scales_per_seg: for every 16-row group and
// every 32-code segment, the 16 rows' P scale bytes are adjacent.
__host__ __device__ inline int64_t scale_offset(int64_t row, int64_t kg, int64_t ksegs, int p) {
  return (((row >> 4) * ksegs + kg / p) * kRowGroup + (row & 15)) * p + (kg % p);
}

struct PreparedShape {
  int n, k, fmt;
  int64_t n_pad, k_pad;
  int64_t code_bytes, scale_bytes;
  int64_t kgroups;  // k_pad / g: scale bytes per row
  int64_t ksegs;    // k_pad / 32: 32-code segments per row
};

inline PreparedShape prepared_shape(int n, int k, int fmt) {
  PreparedShape s;
  s.n = n;
  s.k = k;
  s.fmt = fmt;
  s.n_pad = round_up(n, kRowAlign);
  s.k_pad = round_up(k, kSlabK);
  s.kgroups = s.k_pad / group_size(fmt);
  s.ksegs = s.k_pad / 32;
  s.code_bytes = s.n_pad * s.k_pad / 2;
  s.scale_bytes = s.n_pad * s.kgroups;
  return s;
}

// Rows one 32-lane GEMV team processes at once (its workgroup owns 8 teams'
// rows): 8 for layers of at least 512 such 64-row tiles, else 4 (twice the
// workgroups; measured faster on MI355X for the 24576-, 12288- and 5120-row
// decode layers, slightly slower for the 248320-row head).  It changes which
// rows a workgroup holds, never an output's summation order.
inline int gemv_rows_per_team(int64_t rows_total) { return rows_total / 64 >= 512 ? 8 : 4; }

// Workspace of a decode call with `tile_rows` rows per workgroup: the split-K
// partials [splits][m][rows_total] fp32, then the arrival flags
// [rows_total / tile_rows][splits].
inline int64_t decode_workspace_bytes(int64_t splits, int m, int64_t rows_total, int tile_rows) {
  if (splits <= 1) return 0;
  return splits * m * rows_total * 4 + (rows_total / tile_rows) * splits * 8;
}

// Number of K splits of the GEMV: as few as the LDS budget for x allows (4
// slabs of 1024 codes per split).  Splitting further only adds the
// cross-workgroup finish; measured on MI355X it never paid for the extra
// parallelism at the decode shapes.  A function of k alone, so summation order
// -- and every output bit -- is the same at every m a kernel serves and in the
// fused gate_up launch as in the separate ones.
inline int gemv_splits(int n_proj, int k, int fmt) {
  (void)n_proj;
  (void)fmt;
  const int64_t nslab = round_up(k, kSlabK) / kSlabK;
  return static_cast<int>((nslab + kGemvMaxSlabsPerSplit - 1) / kGemvMaxSlabsPerSplit);
}

// K splits of the MFMA decode kernel.  Layers of at least 128 64-row tiles
// (8192 rows) run unsplit: the split-K finish costs a few microseconds of
// round trips, more than the extra workgroups win there (measured on MI355X:
// gate_up m=4 13.7 -> 12.4 us unsplit).  Smaller layers (5120 rows: 80 tiles)
// split K so that one projection has about 512 workgroups, keeping at least 4
// stages of 256 codes per split.  (Measured on MI355X for the 5120 x 6144
// layer: 6 splits of 4 stages 8.8 to 9.9 us at m = 3..8, 3 splits of 8
// stages 9.8 to 10.5; more than 512 workgroups or fewer than 4 stages per
// split were slower.)  A function of (rows per projection, k) only, so the
// summation order is the same at every m the kernel serves and in the fused
// gate_up launch as in the separate ones.
inline int decode_mfma_splits(int n_proj, int k) {
  const int64_t tiles = round_up(n_proj, kRowAlign) / kDecodeTileRows;
  if (tiles >= 128) return 1;
  const int ksteps = static_cast<int>((k + kDecodeStageK - 1) / kDecodeStageK);
  int s = static_cast<int>(512 / tiles);
  if (s > ksteps / 4) s = ksteps / 4;
  return s < 1 ? 1 : s;
}

// Wave-split decode (decode_kw_kernel): a 256-thread workgroup owns 16 rows
// and its 4 waves split K, each streaming its quarter through kKwBuffers
// stage buffers of its own (two in flight; measured on MI355X, 4 or 5 buffers
// were slower).  16-row tiles give a 5120-row layer 320 workgroups with no
// cross-workgroup split-K finish, at the price of staging x once per 16 rows
// instead of once per 64 (at m = 8, twice the code bytes per stage).
constexpr int kKwWaves = 4;
constexpr int kKwRows = 16;
constexpr int kKwMaxM = 8;
constexpr int kKwBuffers = 3;
constexpr int kKwMaxSteps = 32;
// Whether a decode call of m rows without the SwiGLU epilogue runs on the
// wave-split kernel: at most kKwMaxSteps stages of 256 codes (8 per wave),
// and either m <= 8 on a layer of fewer than 128 64-row tiles per projection
// (those the 64-row kernels split along K across workgroups, or leave with
// few workgroups), or, for MXFP4, m <= 2 on fewer than 256 such tiles.
// Measured on MI355X (HIP-graph replay, in us, wave-split against the VALU
// GEMV or the 64-row MFMA decode):
//   NVFP4 n = 5120, k = 1024,  m = 1 / 4: 3.5 / 4.0   against 4.1 / 5.4
//   NVFP4 n = 2048, k = 4096,  m = 1 / 4: 4.4 / 4.7   against 6.0 / 7.0
//   NVFP4 n = 5120, k = 6144,  m = 1 / 4: 7.3 / 8.4   against 9.1 / 8.9
//   NVFP4 n = 7168, k = 8192,  m = 1 / 4: 9.3 / 11.2  against 10.8 / 12.3
//   MXFP4 n = 12288, k = 4096, m = 1 / 2: 6.6 / 7.2   against 7.9 / 8.9
//   MXFP4 fused gate_up 2 x 12288 x 4096, m = 1 / 2: 11.3-11.7 / 11.9 against
//     11.9-12.6 / 12.7-12.9
// and not taken where it lost:
//   NVFP4 n = 5120, k = 12288, m = 1 / 4: 12.1-12.8 / 13.7 against 11.2 / 12.4
//   NVFP4 n = 5120, k = 17408, m = 1 / 4: 16.3 / 18.8 against 14.6 / 15.8
//   (16 or more stages per wave: the 320 workgroups on 256 CUs, a fifth of
//   the CUs running two, cost more than the finish saves);
//   MXFP4 fused gate_up 2 x 12288 x 4096, m = 4 / 8: 13.6 / 17.3 against
//   13.0 / 13.3 (x staged per 16 rows costs twice the code bytes at m = 8);
//   NVFP4 fused gate_up 2 x 12288 x 4096, m = 1: 15.0-15.6 against 12.3-12.5
//   (the NVFP4 decode's VALU work over 1536 workgroups);
//   the 248320-row head at m = 1 / 4: 126 / 148 against 109 / 132.
// A function of (rows per projection, k, format, m): the fused gate_up
// launch and the separate ones take the same kernel.
inline bool decode_kw_used(int n_proj, int k, int fmt, int m) {
  const int64_t tiles = round_up(n_proj, kRowAlign) / kDecodeTileRows;
  const int ksteps = static_cast<int>((k + kDecodeStageK - 1) / kDecodeStageK);
  const bool small_layer = m <= kKwMaxM && tiles < 128;
  const bool mxfp4_gemv_rows = fmt == kFmtMxfp4 && m <= 2 && tiles < 256;
  return m >= 1 && ksteps <= kKwMaxSteps && (small_layer || mxfp4_gemv_rows);
}

// Rows of an MFMA-decode workgroup: 64 (four waves of one 16-row block), 96
// (six such waves) or 128 (four waves of two blocks, each x fragment read
// from LDS feeding two MFMAs: half the x copies per weight byte).
//  - 128 for layers of at least 2048 64-row tiles, where 128-row tiles still
//    leave thousands of workgroups.  Such layers are never split along K
//    (decode_mfma_splits).
//  - 96 for unsplit layers whose 64-row tiles would give some CUs more
//    workgroups than others and whose 96-row tiles put fewer rows on the
//    busiest CU (the 24576-row fused gate_up: 384 64-row tiles leave half of
//    the 256 CUs two, 256 96-row tiles give each CU one), with a third less
//    x staged per weight byte than 64-row tiles.
//  - 64 otherwise, and for calls of more than 8 rows: their 16-row x stages
//    would leave larger tiles one workgroup per CU.
// The tile size changes which rows a workgroup holds, never an output's
// summation order (every wave streams its rows' stages in order), so the
// choice may follow the total rows of a launch.
inline int decode_mfma_tile_rows(int64_t rows_total, int m, int splits) {
  if (m > 8) return 64;
  if (rows_total / kDecodeTileRows >= 2048) return 128;
  if (splits == 1 && rows_total % 96 == 0) {
    const int64_t busiest64 = (rows_total / 64 + kTargetCUs - 1) / kTargetCUs * 64;
    const int64_t busiest96 = (rows_total / 96 + kTargetCUs - 1) / kTargetCUs * 96;
    if (busiest96 < busiest64) return 96;
  }
  return 64;
}

struct GemvArgs {
  const uint16_t* x;      // bf16 [m][k]
  const uint8_t* codes;   // prepared codes
  const uint8_t* scales;  // prepared scales
  uint16_t* y;            // bf16 [m][ldy]
  float* partial;         // fp32 [splits][m][rows_total] when splits > 1
  uint64_t* flags;        // [rows_total / tile_rows][splits] split-K arrival flags
  uint64_t token;         // unique per call; tags this call's flags
  uint64_t* keys;         // greedy argmax: [tiles][m] best key per tile, or null
  int act;                // 1: interleaved gate_up weight, y = silu(gate) * up [m][n_proj]
  int m, k;
  int64_t k_pad;          // prepared row length in codes
  int64_t kgroups;        // prepared scale bytes per row
  int64_t ksegs;          // 32-code segments per prepared row
  int nslab;              // k_pad / kSlabK
  int splits;
  int n_proj;             // real rows per projection
  int64_t n_proj_pad;     // padded rows per projection
  int projections;        // 1 (linear) or 2 (gate_up)
  int64_t rows_total;     // projections * n_proj_pad
  int64_t ldy;            // projections * n_proj
  float gscale[2];        // global scale per projection (1 for MXFP4)
  int tile_rows;          // rows per workgroup (the split-K finish tile)
  // Grouped MoE decode: activation row r of a pass is x row row_tokens[r]
  // (a token id outside [0, tokens_total) gives zero outputs); null: row r
  // of x.
  const int32_t* row_tokens;
  int tokens_total;
};

// Grouped MoE decode: routed (token, expert) pairs sorted by expert.
struct MoeArgs {
  const int32_t* offsets;    // [experts + 1]: expert e's pairs are [offsets[e], offsets[e + 1])
  const int32_t* tokens;     // [pairs]: x row of each pair (both routes read x directly)
  int tokens_total;          // rows of x
  const float* gscales;      // [experts] NVFP4 global scales, or null (MXFP4)
  int64_t code_stride;       // bytes between experts' prepared codes
  int64_t scale_stride;      // bytes between experts' prepared scales
  int pairs;
  int experts;
};

// Prefill GEMM tiling.  A workgroup of kGemmWavesM x 4 waves computes a
// kGemmBM (activation rows) x kGemmBN (weight rows) tile of y, each wave a
// 128 x 64 block of it, stepping K by kGemmBK.  kGemmSlots workgroups are
// resident on the chip at once (two per CU for a 4-wave workgroup).
constexpr int kGemmWavesM = 1;
constexpr int kGemmBM = 128 * kGemmWavesM;
constexpr int kGemmBN = 256;
constexpr int kGemmBK = 64;
constexpr int kGemmThreads = kGemmWavesM * 4 * 64;
constexpr int kGemmSlots = kTargetCUs * (kGemmWavesM == 1 ? 2 : 1);
// Fewest K steps a split of a tail tile is given: 20 (1280 codes).  Measured
// on MI355X for the 17408 x 5120 prefill GEMM, 4 splits of its 80 steps beat
// 8 to 10 shorter ones by 1.5 to 2.5 % at m = 1024 and 2048: the shorter tail
// saves less than writing, reading back and adding more partial tiles costs.
constexpr int kGemmMinSplitSteps = 20;

// How a prefill call's tiles are spread over the resident workgroups.  Tiles
// are taken whole while they fill complete rounds of kGemmSlots workgroups
// ("data-parallel" tiles); the remaining tail tiles, too few to fill the last
// round, are each cut into `splits` K ranges run by separate workgroups, whose
// fp32 partial tiles a final launch adds in split order.
struct GemmPlan {
  int m_tiles, n_tiles, tiles;
  int dp_tiles;    // tiles computed whole
  int tail_tiles;  // tiles computed as `splits` K ranges
  int splits;
  int ksteps;      // K steps of a whole tile
  int mhalf;       // W4A4 only: tail tiles run as two halves of their rows over all of K instead of K ranges
  int xcds;        // XCDs the tile order deals the data-parallel tiles over
};

// Plan over tiles of `bm` activation rows, K steps of `step_k` codes, `slots`
// resident workgroups, splits of at least `min_split_steps`.
inline GemmPlan tile_plan(int m, int64_t rows_total, int k, int step_k, int min_split_steps, int bm, int slots) {
  GemmPlan p;
  p.mhalf = 0;
  p.xcds = 8;
  p.m_tiles = static_cast<int>((m + bm - 1) / bm);
  p.n_tiles = static_cast<int>(rows_total / kGemmBN);
  p.tiles = p.m_tiles * p.n_tiles;
  p.ksteps = static_cast<int>((k + step_k - 1) / step_k);
  const int tail = p.tiles % slots;
  int s = tail > 0 ? slots / tail : 1;
  const int by_k = p.ksteps / min_split_steps;
  if (s > by_k) s = by_k;
  if (s <= 1) {
    p.dp_tiles = p.tiles;
    p.tail_tiles = 0;
    p.splits = 1;
  } else {
    p.dp_tiles = p.tiles - tail;
    p.tail_tiles = tail;
    p.splits = s;
  }
  return p;
}

// A tail that would be split only two ways runs as whole tiles instead, one
// per CU beside an idle workgroup slot.  Measured on MI355X this beats both
// the two K halves (partials and a reduce launch) and the two 64-row halves
// over all of K (each decoding the whole weight tile): 17408 x 5120 at
// m = 1408: 1112 vs 1007 TFLOP/s; 5120 x 17408 at m = 1280 (200 tiles):
// 926 vs 790; 24576 x 4096 at m = 1024: 5 to 9 % faster.
// The tiling, the tail and its split count come from the nominal 256-CU
// machine (kGemmSlots) whatever the device, so an output's summation order
// never depends on the device; only the XCD deal of the tile order (`xcds`,
// from the device's CU count) does.
inline GemmPlan gemm_plan(int m, int64_t rows_total, int k, int xcds = 8) {
  GemmPlan p = tile_plan(m, rows_total, k, kGemmBK, kGemmMinSplitSteps, kGemmBM, kGemmSlots);
  if (p.splits == 2) {
    p.dp_tiles = p.tiles;
    p.tail_tiles = 0;
    p.splits = 1;
  }
  p.xcds = xcds;
  return p;
}

// W4A4 tile GEMM (MXFP4 activations x MXFP4 weights on the block-scaled
// MFMA): 256 x 256 tiles, one 8-wave workgroup per CU, K stepping 128 codes
// per stage, tail splits of at least 4 stages (512 codes).
constexpr int kW4BM = 256;
constexpr int kW4BK = 128;
constexpr int kW4Slots = kTargetCUs;
constexpr int kW4MinSplitSteps = 4;

// Where the plan would split each tail tile in two along K, the W4A4 GEMM
// runs the two 128-row halves of the tile over all of K instead: the same
// MFMA work per workgroup, no partial tiles to write, read back and add.
// Unlike the W4A16 GEMM's, its half tiles decode no weights, and running the
// tail whole instead measured slower on MI355X (5120 x 17408 at m = 1536:
// 1790 vs 2090 TFLOP/s; 12288 x 4096 at m = 2048: 2240 vs 2350).
inline GemmPlan w4a4_plan(int m, int64_t rows_total, int k, int xcds = 8) {
  GemmPlan p = tile_plan(m, rows_total, k, kW4BK, kW4MinSplitSteps, kW4BM, kW4Slots);
  if (p.splits == 2) p.mhalf = 1;
  p.xcds = xcds;
  return p;
}

// The quantized activations of a W4A4 call: codes [act_rows][act_k / 2]
// (two codes per byte, low nibble first) and E8M0 scales in the prepared
// weight's row-group layout [act_rows / 16][act_k / 32][16].  act_rows covers
// whole 256-row tiles; rows from m on are never written (their results are
// never stored), codes and scales from k to act_k are zero.
inline int64_t w4a4_act_k(int k) { return round_up(k, kW4BK); }
inline int64_t w4a4_act_rows(int m) { return round_up(m, kW4BM); }
inline int64_t w4a4_act_code_bytes(int m, int k) { return w4a4_act_rows(m) * w4a4_act_k(k) / 2; }
inline int64_t w4a4_act_scale_bytes(int m, int k) { return w4a4_act_rows(m) * w4a4_act_k(k) / 32; }

// Workspace of a prefill call: fp32 partial tiles [tail_tiles][splits][bm][BN].
// Grouped MoE tile GEMM: an upper bound on the 128-row activation tiles of
// all experts together, sum over experts e of ceil(c_e / 128) with c_e
// routed pairs summing to `pairs`: at most pairs / 128 + (experts with
// pairs), and no more experts than pairs can have pairs.
inline int64_t moe_gemm_slots(int pairs, int experts) {
  return (static_cast<int64_t>(pairs) + kGemmBM - 1) / kGemmBM + (experts < pairs ? experts : pairs);
}

inline int64_t gemm_workspace_bytes(const GemmPlan& p, int bm = kGemmBM) {
  if (p.mhalf) return 0;
  return static_cast<int64_t>(p.tail_tiles) * p.splits * bm * kGemmBN * 4;
}

struct MfmaArgs {
  const uint16_t* x;      // bf16 [m][k]
  const uint8_t* codes;
  const uint8_t* scales;
  uint16_t* y;
  float* partial;         // tail partial tiles (workspace)
  int m, k;
  int64_t k_pad, kgroups, ksegs;
  int n_proj;
  int64_t n_proj_pad;
  int projections;
  int64_t rows_total, ldy;
  float gscale[2];
  GemmPlan plan;
  int act;                // 1: interleaved gate_up weight, y = silu(gate) * up [m][n_proj]
  // W4A4 only: the quantized activations (w4a4_act_* layout), act_k codes per row.
  const uint8_t* xq_codes;
  const uint8_t* xq_scales;
  int64_t act_k;
  // Grouped MoE tile route only: tile row r reads x row row_tokens[r] (rows of x: tokens_total).
  const int32_t* row_tokens;
  int tokens_total;
};

// Launchers (defined in the .hip files).  Each returns the hipError_t of its
// launch; the grid/block it used is written to *grid / *block when non-null.
hipError_t launch_prepare(const uint8_t* codes, const uint8_t* scales, int n, int k, int fmt,
                          uint8_t* prep_codes, uint8_t* prep_scales, hipStream_t stream);
hipError_t launch_prepare_interleaved(const uint8_t* gate_codes, const uint8_t* gate_scales, const uint8_t* up_codes,
                                      const uint8_t* up_scales, int n, int k, int fmt, uint8_t* prep_codes,
                                      uint8_t* prep_scales, hipStream_t stream);
hipError_t launch_gemv(const GemvArgs& a, int fmt, hipStream_t stream, dim3* grid, dim3* block);
hipError_t launch_decode_mfma(const GemvArgs& a, int fmt, hipStream_t stream, dim3* grid, dim3* block);
hipError_t launch_decode_kw(const GemvArgs& a, int fmt, hipStream_t stream, dim3* grid, dim3* block);
hipError_t launch_moe_decode(const GemvArgs& a, const MoeArgs& moe, int experts, int tokens_total, int fmt,
                             hipStream_t stream, dim3* grid, dim3* block);
hipError_t launch_mfma(const MfmaArgs& a, int fmt, hipStream_t stream, dim3* grid, dim3* block);
hipError_t launch_moe_gemm(const MfmaArgs& a, const MoeArgs& moe, int fmt, hipStream_t stream, dim3* grid,
                           dim3* block);
hipError_t launch_tail_reduce(const MfmaArgs& a, int bm, hipStream_t stream);
hipError_t launch_act_quant_mxfp4(const uint16_t* x, int m, int k, uint8_t* codes, uint8_t* scales,
                                  hipStream_t stream);
hipError_t launch_w4a4(const MfmaArgs& a, hipStream_t stream, dim3* grid, dim3* block);
// NVFP4 activation quantizer with per-tensor scale gx: xhat non-null writes
// the quantized activations as bf16 [m][k] (E2M1(code) * S, no gx); else
// codes [m][k/2] (two per byte, low nibble first) and E4M3FN scales [m][k/16].
hipError_t launch_act_nvfp4(const uint16_t* x, int m, int k, float gx, uint16_t* xhat, uint8_t* codes,
                            uint8_t* scales, hipStream_t stream);
hipError_t launch_argmax_reduce(const uint64_t* keys, int tiles, int m, int32_t* idx, uint16_t* val,
                                hipStream_t stream);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int n, int k, int fmt,
                          float gscale, float* out, hipStream_t stream);

}  // namespace fp4
