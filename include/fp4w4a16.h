/*
 * fp4w4a16.h - W4A16 FP4 weight-only linear layer for AMD Instinct MI355X (gfx950).
 *
 * The layer: y[m, n] = sum_k x[m, k] * w[n, k], with x bf16 and w stored as
 * packed 4-bit E2M1 codes plus block scales, dequantized in registers:
 *
 *   w[n, k] = E2M1(code[n, k]) * S(n, k / g) * G
 *
 *   NVFP4: g = 16, S is an FP8 E4M3FN byte, G is a float32 global scale that
 *          multiplies ("re-verify 27B NVFP4 on the nvidia ModelOpt checkpoint",
 *          vllm.cpp PR #178, section "Layer 3 - ModelOpt NVFP4 naming").
 *   MXFP4: g = 32, S is an E8M0 byte (2^(b-127)), no global scale
 *          ("native MXFP4 keep-quant", vllm.cpp PR #38, commit list).
 *
 * Canonical packed input (what a checkpoint holds; "keep the ModelOpt NVFP4
 * lm_head packed", vllm.cpp PR #263, section "Why this row matters"):
 *   codes  uint8 [n][k/2], row-major; byte j of a row holds element 2j in
 *          bits 3..0 and element 2j+1 in bits 7..4;
 *   scales uint8 [n][k/g], row-major; element k of a row uses scale k/g.
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device pointers owned by the caller; the library
 *     never allocates, frees or caches device memory.  Its only state is a
 *     process-wide atomic call counter (host memory) whose values tag the
 *     split-K arrival flags a call writes into its workspace, so calls are
 *     reentrant and may come from several host threads.  Out-parameters named
 *     *_out are host pointers.
 *   - Device pointers must be 16-byte aligned.
 *   - Work is enqueued on `stream` and is asynchronous; argument checks happen
 *     on the host before anything is enqueued, and an invalid call enqueues
 *     nothing.  After a launch the library checks hipGetLastError.
 *   - Sizes: 1 <= n <= FP4_MAX_N, 32 <= k <= FP4_MAX_K with k % 32 == 0,
 *     0 <= m <= FP4_MAX_M (m == 0 is valid and does nothing).
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - A workspace is never assumed to hold anything (it need not be zeroed).
 *   - Return value: FP4_OK or a negative fp4_status.
 */
#ifndef FP4W4A16_H
#define FP4W4A16_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats. */
enum fp4_fmt {
  FP4_FMT_NVFP4 = 0, /* group 16, E4M3FN block scale, float32 global scale */
  FP4_FMT_MXFP4 = 1  /* group 32, E8M0 block scale, no global scale */
};

/* Status codes. */
enum fp4_status {
  FP4_OK = 0,
  FP4_EINVAL = -1,     /* null pointer, size out of range, k not a multiple of 32 */
  FP4_EFMT = -2,       /* unknown format */
  FP4_EALIGN = -3,     /* a device pointer is not 16-byte aligned */
  FP4_EWORKSPACE = -4, /* workspace smaller than fp4_workspace_bytes() asks for */
  FP4_EHIP = -5        /* the HIP runtime reported an error for a launch */
};

#define FP4_MAX_N (1 << 24)
#define FP4_MAX_K (1 << 20)
#define FP4_MAX_M (1 << 20)

/* Which kernel a call ran (filled when the caller passes a non-null pointer). */
typedef struct fp4_dispatch_info {
  int kernel;  /* 0 = VALU decode GEMV (m = 1, 2), 2 = MFMA decode GEMV
                  (m = 3..32; SwiGLU gate_up: m = 3..16; row tiles of 64
                  rows, or at m <= 8 of 128 rows on launches of at least
                  131072 rows and of 96 rows, 384 threads, on unsplit
                  launches whose rows are a multiple of 96 that 64-row
                  tiles would spread unevenly over 256 CUs, such as the
                  2 x 12288-row gate_up), 1 = MFMA tile GEMM
                  (m > 32; SwiGLU gate_up: m > 16), 3 = grouped MoE decode,
                  4 = W4A4 MXFP4 tile GEMM (any m),
                  5 = grouped MoE tile GEMM (prefill),
                  6 = wave-split MFMA decode GEMV, instead of kernels 0 and
                  2 where k <= 8192: m = 1..8 on layers of fewer than 8192
                  rows per projection (n rounded up to 256), and for MXFP4
                  also m = 1, 2 on fewer than 16384 (not for the SwiGLU
                  gate_up); 16-row workgroups whose four waves split K and
                  add their sums in the workgroup */
  int splits;  /* K splits: decode kernels split every tile, the tile GEMMs only
                  their tail tiles (1 = no split; W4A4 tail tiles run as row
                  halves over all of K also report 1) */
  int grid_x;  /* decode: workgroups along the output rows; tile GEMMs:
                  workgroups of the launch */
  int grid_y;  /* decode / MoE: workgroups along the second grid axis; tile
                  GEMMs: workgroups that run the tail tiles (tail tiles x
                  splits for K ranges, x 2 for W4A4 row halves; 0 if none) */
  int block;   /* threads per workgroup */
  int xcds;    /* tile GEMMs: the XCDs their tile order was dealt over, from the
                  device's compute-unit count (1 to 8; 32 CUs per XCD); 0 for
                  the decode kernels, whose workgroups own fixed row tiles */
} fp4_dispatch_info;

/*
 * The launch plan a W4A16 call would use on a device (or partition) with
 * `cus` compute units, without running it: what fp4_w4a16_linear
 * (projections = 1, n rows) or fp4_w4a16_gate_up (projections = 2, n rows per
 * half) fills into its fp4_dispatch_info on such a device.  Tile sizes and
 * K-split counts are those of the full 256-CU MI355X on every device, so an
 * output's summation order (and every output bit) never depends on the
 * device; only the XCD deal of the tile GEMMs' tile order follows `cus`.
 * Host utility (no passage defines it): pure host function, never touches
 * the GPU.  FP4_EINVAL for sizes out of range, cus < 1 or a null out.
 */
int fp4_plan(int m, int n, int k, int fmt, int projections, int cus, fp4_dispatch_info* info_out);

/*
 * Size of a prepared weight of n rows and k columns.
 * The prepared layout (written by fp4_prepare, read by every compute call):
 *   codes: uint8 [n_pad][k_pad/2], the canonical code bytes, zero padded,
 *          with n_pad = n rounded up to 256 and k_pad = k rounded up to 1024;
 *   scales: uint8 [n_pad/16][k_pad/32][16][32/g]: for each group of 16 rows
 *          and each 32-code segment, the 16 rows' scale bytes of the segment
 *          (2 per row for NVFP4, 1 for MXFP4) are contiguous; zero padded.
 * A prepared gate_up weight is a prepared gate weight followed by a prepared
 * up weight, in both buffers (twice these sizes).
 * Host utility (no passage defines it): sizes the prepared buffers; pure host
 * function, never touches the GPU.
 */
int fp4_prepared_bytes(int n, int k, int fmt, size_t* code_bytes_out, size_t* scale_bytes_out);

/*
 * Repack a canonical packed weight (codes_dev [n][k/2], scales_dev [n][k/g])
 * into the prepared layout (prep_codes_dev, prep_scales_dev, sized by
 * fp4_prepared_bytes).  Integer byte moves only; run once per weight.
 * The canonical buffers are only read and may be released after the stream
 * reaches this call.  Input and output must not overlap.
 * Cite: the packed weight is consumed as is, never expanded to bf16 ("keep the
 * ModelOpt NVFP4 lm_head packed", section "Round-2 findings resolved": the
 * prepare step may only write state it owns).
 */
int fp4_prepare(const uint8_t* codes_dev, const uint8_t* scales_dev, int n, int k, int fmt,
                uint8_t* prep_codes_dev, uint8_t* prep_scales_dev, hipStream_t stream);

/*
 * Prepare a fused gate_up weight: gate rows then up rows, each n_half x k.
 * Equivalent to two fp4_prepare calls into the two halves of the output.
 * Cite: "MXFP4 decode-graph + gate_up FUSION default-ON" (vllm.cpp PR #54),
 * step 2: one GEMM over the concatenated [gate; up] weight.
 */
int fp4_prepare_gate_up(const uint8_t* gate_codes_dev, const uint8_t* gate_scales_dev,
                        const uint8_t* up_codes_dev, const uint8_t* up_scales_dev,
                        int n_half, int k, int fmt,
                        uint8_t* prep_codes_dev, uint8_t* prep_scales_dev, hipStream_t stream);

/*
 * Workspace a compute call needs, in bytes (0 when none), for split-K fp32
 * partials and arrival flags: the m = 1, 2 decode GEMV with k > 4096, the
 * m = 3..32 MFMA decode on layers of fewer than 8192 rows per projection
 * (except where the wave-split kernel runs, kernel 6 of fp4_dispatch_info), and
 * the m > 32 tile GEMM when its 128 x 256 output tiles do not fill whole
 * rounds of the 512 workgroups resident on the chip (the tail tiles are then
 * split along K; at most 64 MiB).  It never needs zeroing.  `projections` is 1 for
 * fp4_w4a16_linear (n = output features) and 2 for fp4_w4a16_gate_up
 * (n = n_half).
 * Host utility (no passage defines it): sizes the workspace argument of the
 * compute calls; pure host function, never touches the GPU.
 */
int fp4_workspace_bytes(int m, int n, int k, int fmt, int projections, size_t* bytes_out);

/*
 * y = x * w^T.
 *   x_dev   bf16 [m][k] row-major;
 *   prep_*  the prepared weight of n rows (fp4_prepare);
 *   global_scale  G for NVFP4 (a multiplier, applied after the sum over k);
 *                 ignored for MXFP4;
 *   y_dev   bf16 [m][n] row-major, rounded to nearest even from float32;
 *   workspace_dev / workspace_bytes  scratch of fp4_workspace_bytes(m, n, k, fmt, 1);
 *   info_out  optional, may be NULL.
 * Accumulation is float32.  The order of every sum depends only on (k, fmt, n)
 * and on which kernel m selects (fp4_dispatch_info.kernel) -- for the tile
 * GEMM (m > 32) also on m, which decides the tiles summed in K splits -- so
 * results are deterministic run to run, and for m <= 32 a row's result does
 * not depend on the other rows of the call as long as m selects the same
 * kernel (m = 1, 2: the VALU GEMV; m = 3..32: the MFMA decode; on the layers
 * the wave-split kernel serves, m = 1..8 on it and m = 9..32 on the MFMA
 * decode).
 * Cite: "native MXFP4 keep-quant" (vllm.cpp PR #38), commit list (the W4A16
 * entry points take bf16 x and the packed weight to bf16 y); "keep the ModelOpt
 * NVFP4 lm_head packed" (vllm.cpp PR #263), section "Why this row matters"
 * (the 248320 x 5120 head run as a W4A16 GEMM).
 */
int fp4_w4a16_linear(const uint16_t* x_dev, int m, int k,
                     const uint8_t* prep_codes_dev, const uint8_t* prep_scales_dev, int n,
                     float global_scale, int fmt,
                     uint16_t* y_dev, void* workspace_dev, size_t workspace_bytes,
                     hipStream_t stream, fp4_dispatch_info* info_out);

/*
 * fp4_w4a16_linear without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, checks, kernels, plan and
 * results as fp4_w4a16_linear -- bit for bit -- except that the split-K
 * partials and arrival flags (or the tile GEMM's tail partials) live in a
 * scratch array the library owns: FP4_NOALLOC_SCRATCH_BYTES of device memory
 * per GPU, reserved when the library's code is loaded and held until the
 * process ends.  The call allocates nothing (no hipMalloc or hipFree).
 *   - A call whose fp4_workspace_bytes(m, n, k, fmt, 1) exceeds the scratch
 *     size returns FP4_EWORKSPACE and enqueues nothing (the decode shapes
 *     need at most a few MiB; the tile GEMM's tail partials at most 64 MiB).
 *   - Nothing in the scratch has to start at zero: the split-K flags carry a
 *     per-call token and every partial is written before it is read.
 *   - All calls on one GPU share its scratch: calls that may run at the same
 *     time on that GPU (on different streams, or from several host threads
 *     without ordering) race and give undefined results.  Calls ordered on
 *     one stream are safe.
 *   - The first call on a device looks up the scratch address for that
 *     device (the current device); a failure returns FP4_EHIP.
 */
#define FP4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fp4_w4a16_linear_noalloc(const uint16_t* x_dev, int m, int k,
                             const uint8_t* prep_codes_dev, const uint8_t* prep_scales_dev, int n,
                             float global_scale, int fmt, uint16_t* y_dev,
                             hipStream_t stream, fp4_dispatch_info* info_out);

/*
 * Fused gate_up: y[:, 0:n_half] = x * gate^T, y[:, n_half:2 n_half] = x * up^T,
 * in one launch over the prepared [gate; up] weight (fp4_prepare_gate_up).
 * global_gate / global_up are the two NVFP4 global scales (ignored for MXFP4).
 * y_dev is bf16 [m][2 n_half].  Workspace: fp4_workspace_bytes(m, n_half, k, fmt, 2).
 * Bitwise equal to two fp4_w4a16_linear calls on the halves.
 * Cite: "MXFP4 decode-graph + gate_up FUSION default-ON" (vllm.cpp PR #54), step 2.
 */
int fp4_w4a16_gate_up(const uint16_t* x_dev, int m, int k,
                      const uint8_t* prep_codes_dev, const uint8_t* prep_scales_dev, int n_half,
                      float global_gate, float global_up, int fmt,
                      uint16_t* y_dev, void* workspace_dev, size_t workspace_bytes,
                      hipStream_t stream, fp4_dispatch_info* info_out);

/*
 * SwiGLU gate_up: y[m][j] = bf16(silu(g) * u), g = x * gate[j]^T * global_gate,
 * u = x * up[j]^T * global_up (float32 sums, as fp4_w4a16_gate_up computes
 * them before rounding), silu(v) = v / (1 + e^-v), one rounding to bf16;
 * y_dev is bf16 [m][n_half].  The weight is prepared by
 * fp4_prepare_gate_up_interleaved (same buffer sizes as fp4_prepare_gate_up:
 * twice fp4_prepared_bytes(n_half, k, fmt)), which interleaves gate and up
 * rows in groups of 16 (prepared row R: gate row 16 (R / 32) + R % 16 when
 * R % 32 < 16, else the up row with that index) so that both operands of an
 * output are computed by one workgroup.  m <= 16: the decode kernels 0 and 2
 * form y in their epilogue (never the wave-split kernel 6, whose 16-row
 * workgroups would hold only gate or only up rows); m > 16: the tile GEMM
 * forms y in the epilogue of every whole tile, and its reduce launch forms y
 * for the tail tiles split along K.
 * Workspace: fp4_swiglu_workspace_bytes.  At m <= 16 it is the split-K
 * partials and flags of kernels 0 and 2 for the 2 n_half rows -- equal to
 * fp4_workspace_bytes(m, n_half, k, fmt, 2) except where fp4_w4a16_gate_up
 * runs the wave-split kernel, which needs none; at m = 17..32 the SwiGLU call
 * runs the tile GEMM while fp4_w4a16_gate_up runs the decode kernel, so the
 * two sizes differ there.
 * silu uses the hardware exp and reciprocal (about 1 ulp each).
 * Reading taken: the pages name the MLP block after the fused gate_up but not
 * its activation; silu(gate) * up is the gated MLP of the model family they
 * run ("MXFP4 decode-graph + gate_up FUSION default-ON", vllm.cpp PR #54,
 * step 2: gate_up feeds the MLP of Qwen3-8B-MXFP4).
 */
int fp4_prepare_gate_up_interleaved(const uint8_t* gate_codes_dev, const uint8_t* gate_scales_dev,
                                    const uint8_t* up_codes_dev, const uint8_t* up_scales_dev,
                                    int n_half, int k, int fmt,
                                    uint8_t* prep_codes_dev, uint8_t* prep_scales_dev, hipStream_t stream);
int fp4_swiglu_workspace_bytes(int m, int n_half, int k, int fmt, size_t* bytes_out);
int fp4_w4a16_gate_up_swiglu(const uint16_t* x_dev, int m, int k,
                             const uint8_t* prep_codes_dev, const uint8_t* prep_scales_dev, int n_half,
                             float global_gate, float global_up, int fmt,
                             uint16_t* y_dev, void* workspace_dev, size_t workspace_bytes,
                             hipStream_t stream, fp4_dispatch_info* info_out);

/*
 * Greedy token of a decode call: idx_out_dev[i] (int32) = the index j of the
 * largest logit y[i][j] -- the bf16 value fp4_w4a16_linear gives for the same
 * arguments -- and the lowest such j when several are equal; -0 equals +0
 * and a NaN counts as larger than every number.  m = 1..32 only (the decode
 * kernels; FP4_EINVAL otherwise).  The argmax is the epilogue of the decode
 * kernel fp4_w4a16_linear picks for the same arguments (0, 2 or 6): each workgroup
 * reduces its logits to one (value, index) per activation row, a second
 * launch reduces those over the workgroups.  A maximum under that total
 * order does not depend on the reduction order, so the result is
 * deterministic and equals the argmax of fp4_w4a16_linear's y.
 *   y_dev        NULL, or bf16 [m][n] to receive the logits as well;
 *   idx_out_dev  int32 [m], 4-byte aligned;
 *   val_out_dev  NULL, or bf16 [m]: the winning logits;
 *   workspace_dev / workspace_bytes  scratch of fp4_argmax_workspace_bytes(m, n, k, fmt).
 * Cite: "re-verify 27B NVFP4 on the nvidia ModelOpt checkpoint" (vllm.cpp
 * PR #178), section on the 35B correctness result (exact logit ties go to the
 * lowest token id; an argmax reduction is order-independent).
 */
int fp4_argmax_workspace_bytes(int m, int n, int k, int fmt, size_t* bytes_out);
int fp4_w4a16_linear_argmax(const uint16_t* x_dev, int m, int k,
                            const uint8_t* prep_codes_dev, const uint8_t* prep_scales_dev, int n,
                            float global_scale, int fmt, uint16_t* y_dev,
                            int32_t* idx_out_dev, uint16_t* val_out_dev,
                            void* workspace_dev, size_t workspace_bytes,
                            hipStream_t stream, fp4_dispatch_info* info_out);

/*
 * Grouped MoE decode: for each routed (token, expert) pair p,
 *   y[p][:] = x[pair_tokens[p]] * w_e^T   (e = the expert of pair p),
 * computed as fp4_w4a16_linear would for that expert's weight (float32
 * accumulation, the expert's NVFP4 global scale applied after the sum,
 * bf16 round to nearest even).  Routing and the weighted combine of the
 * pairs are the caller's.
 *   x_dev              bf16 [tokens][k];
 *   prep_codes_dev / prep_scales_dev  the experts' prepared weights (n rows
 *                      each, fp4_prepare) stacked: expert e at e times the
 *                      sizes fp4_prepared_bytes(n, k, fmt) gives;
 *   global_scales_dev  float32 [experts] NVFP4 global scales (device memory);
 *                      ignored and may be NULL for MXFP4;
 *   expert_offsets_dev int32 [experts + 1]: the pairs are sorted by expert,
 *                      expert e's are [offsets[e], offsets[e + 1]);
 *   pair_tokens_dev    int32 [pairs]: the token (row of x) of each pair;
 *   y_dev              bf16 [pairs][n];
 *   workspace_dev / workspace_bytes  unused (fp4_moe_workspace_bytes reports
 *                      0 bytes); may be NULL / 0.
 * Device-side routing data is not validated on the host: offsets are clamped
 * to [0, pairs] and a token id outside [0, tokens) reads a zero row, so no
 * table can make the kernels access memory outside these buffers.  One
 * launch: a workgroup per (row tile, expert with pairs) on the matrix cores,
 * whose stage copies fetch each pair's x row by its token id: the m = 3..8
 * decode kernel on
 * 64-row tiles, up to 8 pairs of an expert per pass; with one or two tokens
 * (tokens <= 2), on experts the wave-split kernel takes at m = tokens, that
 * kernel on 16-row tiles, up to `tokens` pairs per pass, each pair's output
 * then equal to fp4_w4a16_linear's output for that token on its expert's
 * weight bit for bit (when the expert's pairs are the same tokens).  The
 * grid has min(experts, pairs) expert slots, enough for every expert with
 * pairs when the offsets are non-decreasing (with other tables some experts
 * may be skipped); dispatch info kernel 3, grid_x = row tiles.  The sum order
 * of an output depends only on (n, k, fmt) and on whether tokens <= 2: a
 * pair's result does not depend on the other pairs.
 * Cite: "MXFP4 decode-graph + gate_up FUSION default-ON" (vllm.cpp PR #54),
 * the later commit on the dense-template marlin port: the dense projections
 * had run as the single-expert case of the grouped MoE W4A16 route, the same
 * per-expert product; "re-verify 27B NVFP4 on the nvidia ModelOpt checkpoint"
 * (vllm.cpp PR #178), section on the 35B result: the MoE model's grouped
 * W4A16 operations have their own test gates.
 */
/*
 * Workspace of fp4_w4a16_moe_decode for `pairs` routed pairs of k values:
 * 0 bytes, since the kernels fetch each pair's x row by its token id.
 * FP4_EINVAL for pairs or k out of range or k not a multiple of 32.
 * Host utility (no passage defines it): pure host function, never touches the
 * GPU.
 */
int fp4_moe_workspace_bytes(int pairs, int k, size_t* bytes_out);
int fp4_w4a16_moe_decode(const uint16_t* x_dev, int tokens, int k,
                         const uint8_t* prep_codes_dev, const uint8_t* prep_scales_dev, int n, int experts,
                         const float* global_scales_dev, int fmt,
                         const int32_t* expert_offsets_dev, const int32_t* pair_tokens_dev, int pairs,
                         uint16_t* y_dev, void* workspace_dev, size_t workspace_bytes,
                         hipStream_t stream, fp4_dispatch_info* info_out);

/*
 * Grouped MoE prefill: the same operation, arguments, checks and containment
 * of routing data as fp4_w4a16_moe_decode, for routings that give experts
 * many pairs (prefill batches): one launch of the MFMA tile GEMM over 128-row
 * tiles of each expert's pairs, so an expert's weight is read once per 128 of
 * its pairs instead of once per 8.  The tile's stage copies fetch each pair's
 * x row straight from x_dev, so no workspace is used: workspace_dev and
 * workspace_bytes are ignored (NULL and 0 are fine).
 * Workgroup slots: the tiles of all experts in expert order, at most
 * ceil(pairs / 128) + min(experts, pairs) of them (every tile, when the
 * offsets are non-decreasing), times ceil(n / 256) weight tiles; FP4_EINVAL
 * when that grid would exceed 2^32 threads.  A tile's sums are the tile
 * GEMM's (K in order, the dense call's MFMA accumulation), so a pair's result
 * does not depend on the other pairs, and equals the dense fp4_w4a16_linear
 * output of that expert where the dense call computes the row in a whole tile.
 * Dispatch info: kernel 5, grid_x = workgroups launched.
 * Cite: as fp4_w4a16_moe_decode; the pages' MoE model runs its grouped W4A16
 * route at prefill sizes too ("MXFP4 decode-graph + gate_up FUSION
 * default-ON" (vllm.cpp PR #54), step 3: prefill keeps its own path).
 */
int fp4_w4a16_moe_prefill(const uint16_t* x_dev, int tokens, int k,
                          const uint8_t* prep_codes_dev, const uint8_t* prep_scales_dev, int n, int experts,
                          const float* global_scales_dev, int fmt,
                          const int32_t* expert_offsets_dev, const int32_t* pair_tokens_dev, int pairs,
                          uint16_t* y_dev, void* workspace_dev, size_t workspace_bytes,
                          hipStream_t stream, fp4_dispatch_info* info_out);

/*
 * Grouped MoE prefill with the SwiGLU epilogue: each expert's weight is an
 * interleaved gate_up pair (fp4_prepare_gate_up_interleaved of n_half rows
 * per projection; experts stacked at twice fp4_prepared_bytes(n_half, k, fmt)
 * apart), and for every routed pair p
 *   y[p][j] = bf16(silu(g) * u),  g = x[pair_tokens[p]] . gate_e[j] * G_gate,
 *                                 u = x[pair_tokens[p]] . up_e[j] * G_up,
 * silu(v) = v / (1 + e^-v), as fp4_w4a16_gate_up_swiglu forms it.
 *   global_scales_dev  float32 [experts][2] (gate, up) for NVFP4; ignored
 *                      and may be NULL for MXFP4;
 *   y_dev              bf16 [pairs][n_half].
 * Other arguments, checks and the containment of routing data are
 * fp4_w4a16_moe_prefill's; no workspace.  Dispatch info: kernel 5.
 * Cite: the MLP step after the fused gate_up ("MXFP4 decode-graph + gate_up
 * FUSION default-ON" (vllm.cpp PR #54), step 2) on the experts of the MoE
 * model's grouped route (as fp4_w4a16_moe_decode); the activation is the
 * reading fp4_w4a16_gate_up_swiglu takes.
 */
int fp4_w4a16_moe_prefill_swiglu(const uint16_t* x_dev, int tokens, int k,
                                 const uint8_t* prep_codes_dev, const uint8_t* prep_scales_dev, int n_half,
                                 int experts, const float* global_scales_dev, int fmt,
                                 const int32_t* expert_offsets_dev, const int32_t* pair_tokens_dev, int pairs,
                                 uint16_t* y_dev, hipStream_t stream, fp4_dispatch_info* info_out);

/*
 * W4A4 MXFP4 variant: activations quantized to MXFP4 at call time and
 * contracted with an MXFP4 weight on the block-scaled MFMA.  A separate,
 * opt-in numerics contract: the weight-only entry points above never use it.
 * Cite: "native MXFP4 keep-quant" (vllm.cpp PR #38), commit list, W0 and W1:
 * the compressed-tensors MXFP4 scheme with quantized input activations, run
 * by a GEMM over 4-bit operands with block-32 E8M0 scales; the pages keep the
 * weight-only GEMM as the default path ("re-verify 27B NVFP4 on the nvidia
 * ModelOpt checkpoint" (vllm.cpp PR #178): the fp4-activation GEMM stays
 * behind an opt-in switch).
 *
 * Activation quantization (per row, per 32 consecutive k; the OCP MX v1.0
 * conversion, as the pages do not print the rule): scale byte
 * s = max(E - 2, 0), E the biased exponent of the block's largest |x| as a
 * bf16 (X = 2^(s - 127) = 2^(floor(log2 amax) - 2), at least 2^-127); code =
 * nearest E2M1 value to x / X, ties to the even code, saturating at 6, sign
 * bit of x.  A block holding an Inf or NaN gets s = 0xFF and zero codes (the
 * y of such a row is unspecified).
 *
 * Quantized activation layout (fp4_w4a4_act_bytes): with
 * R = round_up(m, 256) and K = round_up(k, 128),
 *   codes  [R][K / 2]: two codes per byte, low nibble first;
 *   scales [R / 16][K / 32][16]: for every group of 16 rows and every 32-code
 *          block, the 16 rows' E8M0 bytes (the prepared weight's scale layout);
 * rows m .. R-1 are not written; blocks at or past k get zero codes and byte 0.
 */
int fp4_w4a4_act_bytes(int m, int k, size_t* code_bytes_out, size_t* scale_bytes_out);

/*
 * Quantize bf16 x [m][k] (row-major) into codes_dev / scales_dev (layout
 * above; buffers of fp4_w4a4_act_bytes(m, k) bytes, 16-byte aligned).  The
 * quantizer fp4_w4a4_linear runs; exposed so its output can be checked.
 */
int fp4_quantize_act_mxfp4(const uint16_t* x_dev, int m, int k, uint8_t* codes_dev, uint8_t* scales_dev,
                           hipStream_t stream);

/*
 * Workspace of fp4_w4a4_linear (projections 1) / fp4_w4a4_gate_up
 * (projections 2, n = n_half): the quantized activations, then the tile
 * GEMM's tail partials when its 256 x 256 tiles do not fill whole rounds of
 * the chip (one tile per CU).  Never needs zeroing.  Pure host function.
 */
int fp4_w4a4_workspace_bytes(int m, int n, int k, int projections, size_t* bytes_out);

/*
 * y = Q(x) * w^T with Q the activation quantization above and w the MXFP4
 * weight prepared by fp4_prepare (fmt must be FP4_FMT_MXFP4; any other
 * format is rejected with FP4_EFMT: the block-scaled MFMA takes only E8M0
 * block-32 scales).  x_dev bf16 [m][k]; y_dev bf16 [m][n], rounded to nearest
 * even from the float32 sums; workspace of fp4_w4a4_workspace_bytes(m, n, k, 1).
 * Two launches (quantizer, tile GEMM) plus the tail reduce when the plan
 * splits tail tiles.  Each 64-k block product of the MFMA is accumulated in
 * float32; sums are in a fixed order given (m, n, k), so results are
 * deterministic run to run.
 */
int fp4_w4a4_linear(const uint16_t* x_dev, int m, int k, const uint8_t* prep_codes_dev,
                    const uint8_t* prep_scales_dev, int n, int fmt, uint16_t* y_dev, void* workspace_dev,
                    size_t workspace_bytes, hipStream_t stream, fp4_dispatch_info* info_out);

/*
 * Fused gate_up of the W4A4 variant over the prepared [gate; up] weight
 * (fp4_prepare_gate_up): y = [Q(x) gate^T | Q(x) up^T], bf16 [m][2 n_half].
 * Workspace: fp4_w4a4_workspace_bytes(m, n_half, k, 2).
 */
int fp4_w4a4_gate_up(const uint16_t* x_dev, int m, int k, const uint8_t* prep_codes_dev,
                     const uint8_t* prep_scales_dev, int n_half, int fmt, uint16_t* y_dev, void* workspace_dev,
                     size_t workspace_bytes, hipStream_t stream, fp4_dispatch_info* info_out);

/*
 * NVFP4 W4A4 variant (ModelOpt's): an NVFP4 checkpoint's per-tensor
 * activation scale input_scale (G_x) sets alpha = G_x * G_w and routes the
 * layer to a GEMM over 4-bit activations; the pages keep that arm behind an
 * opt-in switch ("keep the ModelOpt NVFP4 lm_head packed", vllm.cpp PR #263,
 * section "Round-1 findings resolved", item 1; "re-verify 27B NVFP4 on the
 * nvidia ModelOpt checkpoint", vllm.cpp PR #178, section "W4A16 is the
 * default for ModelOpt").  Separate, opt-in entry points; the weight-only
 * path never calls them.
 *
 * Activation quantizer Q (the weights' two-level NVFP4 rule with G_x; the
 * pages name the scale, not the rule): per row and block of 16 k,
 *   s = fl32(fl32(amax / 6) / G_x), S = E4M3FN(s) nearest-even saturating at
 *   448, q = fl32(S * G_x), code = E2M1(fl32(x / q)) nearest-even saturating
 *   at 6 with the sign of x (code 0 where q == 0); a block holding an Inf or
 *   NaN gets scale byte 0x7F and codes 0.  Correctly rounded float32 steps.
 *
 * fp4_quantize_act_nvfp4 writes Q(x) as codes_dev uint8 [m][k/2] (two codes
 * per byte, low nibble first) and scales_dev uint8 [m][k/16] (E4M3FN bytes,
 * row-major); it is the quantizer the products run, exposed so its output can
 * be checked.  input_scale must be finite and > 0 (else FP4_EINVAL); k % 32 == 0.
 */
int fp4_quantize_act_nvfp4(const uint16_t* x_dev, int m, int k, float input_scale, uint8_t* codes_dev,
                           uint8_t* scales_dev, hipStream_t stream);

/*
 * Workspace of fp4_w4a4_nvfp4_linear (projections 1) / fp4_w4a4_nvfp4_gate_up
 * (projections 2, n = n_half): the quantized activations as bf16 [m][k]
 * (rounded up to 256 bytes), then the W4A16 call's workspace
 * (fp4_workspace_bytes with FP4_FMT_NVFP4).  Never needs zeroing.  Pure host
 * function.
 */
int fp4_w4a4_nvfp4_workspace_bytes(int m, int n, int k, int projections, size_t* bytes_out);

/*
 * y = alpha * (Q(x) w^T), alpha = fl32(input_scale * global_scale), with Q
 * as above (without G_x) and w the NVFP4 weight prepared by fp4_prepare
 * (without G_w).  x_dev bf16 [m][k]; y_dev bf16 [m][n] rounded to nearest even
 * from the float32 results.
 * gfx950's block-scaled MFMA takes E8M0 scales per 32 elements only, not
 * NVFP4's E4M3 scales per 16, so Q(x) is written to the workspace as bf16
 * E2M1(code) * S -- exact -- and the W4A16 kernels (the kernel m selects,
 * reported in info_out) contract it with the weight and apply alpha after the
 * sum: the same products and float32 accumulation as a GEMM over the 4-bit
 * operands.  Two or more launches (quantizer, then the W4A16 call).
 * Errors as fp4_w4a16_linear, plus FP4_EINVAL for an input_scale that is not
 * finite and > 0; the weight is NVFP4 (no format argument).
 */
int fp4_w4a4_nvfp4_linear(const uint16_t* x_dev, int m, int k, const uint8_t* prep_codes_dev,
                          const uint8_t* prep_scales_dev, int n, float global_scale, float input_scale,
                          uint16_t* y_dev, void* workspace_dev, size_t workspace_bytes, hipStream_t stream,
                          fp4_dispatch_info* info_out);

/*
 * Fused gate_up of the NVFP4 W4A4 variant over the prepared [gate; up] NVFP4
 * weight (fp4_prepare_gate_up): y = [alpha_g Q(x) gate^T | alpha_u Q(x) up^T],
 * bf16 [m][2 n_half], alpha_g = fl32(input_scale * gate_global_scale),
 * alpha_u likewise.  Workspace: fp4_w4a4_nvfp4_workspace_bytes(m, n_half, k, 2).
 */
int fp4_w4a4_nvfp4_gate_up(const uint16_t* x_dev, int m, int k, const uint8_t* prep_codes_dev,
                           const uint8_t* prep_scales_dev, int n_half, float gate_global_scale,
                           float up_global_scale, float input_scale, uint16_t* y_dev, void* workspace_dev,
                           size_t workspace_bytes, hipStream_t stream, fp4_dispatch_info* info_out);

/*
 * Dequantize a prepared weight to float32 out_dev [n][k]:
 * out = fl32(fl32(E2M1 * S) * G), G = 1 for MXFP4.  It decodes with the
 * instruction sequences of the compute kernels' weight decode (NVFP4: E2M1 to
 * f32 at unit scale, times the E4M3 scale; MXFP4: E2M1 times 2^(b-127) to
 * bf16 in one conversion with the E8M0 byte as its scale operand), then
 * multiplies by G, which the compute kernels apply after the sum over k
 * instead.  The compute kernels' own decode is pinned separately: a one-hot
 * x makes each output a single decoded weight.
 * Cite: "native MXFP4 keep-quant" (vllm.cpp PR #38), commit list (the CPU
 * dequant reference the device GEMM is checked against).
 */
int fp4_dequantize(const uint8_t* prep_codes_dev, const uint8_t* prep_scales_dev, int n, int k,
                   float global_scale, int fmt, float* out_dev, hipStream_t stream);

/* A static, human-readable name for a status code.  Host utility (no passage
 * defines it); never touches the GPU. */
const char* fp4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP4W4A16_H */
