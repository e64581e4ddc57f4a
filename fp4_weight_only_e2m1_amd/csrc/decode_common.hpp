// Pieces shared by the two decode kernels (VALU GEMV and MFMA decode):
// staging x in LDS, and the single-launch, lock-free split-K finish.
#pragma once

#include "fp4_common.hpp"
#include "fp4_device.hpp"

namespace fp4 {

constexpr int kChunksPerSlab = kSlabK / 8;  // 16-byte chunks of x (8 bf16) per slab

// First and one-past-last slab of K split `split`.
struct SlabRange {
  int first, count;
};
__device__ __forceinline__ SlabRange split_slabs(const GemvArgs& a, int split) {
  const int s0 = static_cast<int>(static_cast<int64_t>(split) * a.nslab / a.splits);
  const int s1 = static_cast<int>(static_cast<int64_t>(split + 1) * a.nslab / a.splits);
  return {s0, s1 - s0};
}

// Copy x[0:M, 1024*slab0 : 1024*(slab0+nsl)) into xs (16-byte chunks, zero
// beyond k), chunk q of row m at index Swz(m, q).  All global loads are issued
// before the first LDS store, so the copy costs one L2 round trip rather than
// one per chunk.  Ends with a workgroup barrier.
template <int M, typename Swz>
__device__ __forceinline__ void stage_x(const GemvArgs& a, int slab0, int nsl,
                                        uint4 (*xs)[kGemvMaxSlabsPerSplit * kChunksPerSlab], Swz swz) {
  constexpr int kPer = kGemvMaxSlabsPerSplit * kChunksPerSlab / kDecodeThreads;
  const int chunks = nsl * kChunksPerSlab;
  const int64_t k0 = static_cast<int64_t>(slab0) * kSlabK;
  uint4 v[M][kPer];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int cc = threadIdx.x + i * kDecodeThreads;
      const int64_t kk = k0 + cc * 8;
      v[m][i] = make_uint4(0u, 0u, 0u, 0u);
      if (cc < chunks && kk < a.k) v[m][i] = *reinterpret_cast<const uint4*>(a.x + static_cast<int64_t>(m) * a.k + kk);
    }
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int cc = threadIdx.x + i * kDecodeThreads;
      if (cc < chunks) xs[m][swz(m, cc)] = v[m][i];
    }
  __syncthreads();
}

// Output column of prepared row `row` (projection h, local row lr), or -1 for
// a padding row.
__device__ __forceinline__ int64_t out_col(const GemvArgs& a, int64_t row, int& h) {
  h = static_cast<int>(row / a.n_proj_pad);
  const int64_t lr = row - static_cast<int64_t>(h) * a.n_proj_pad;
  return lr < a.n_proj ? static_cast<int64_t>(h) * a.n_proj + lr : -1;
}

// Greedy argmax over a call's logits (the decode epilogue's optional output).
// Each logit -- the bf16 value y would hold -- becomes a 64-bit key that is
// larger exactly when the (value, index) pair wins: the value's bits mapped
// to an unsigned order (negative values flipped, -0 made +0, every NaN made
// the largest) in the top half, the inverted output index in the bottom half,
// so equal values prefer the lower index.  A maximum under this total order
// does not depend on the order of the reduction ("re-verify 27B NVFP4 on the
// nvidia ModelOpt checkpoint", section on the 35B correctness result: exact
// ties go to the lowest token id).
__device__ __forceinline__ uint64_t argmax_key(uint16_t b, int64_t col) {
  if ((b & 0x7FFFu) == 0) b = 0;                              // -0 == +0
  if ((b & 0x7F80u) == 0x7F80u && (b & 0x7Fu) != 0) b = 0x7FC0u;  // any NaN: largest
  const uint32_t o = (b & 0x8000u) ? (~static_cast<uint32_t>(b) & 0xFFFFu) : (b | 0x8000u);
  return (static_cast<uint64_t>(o) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(col));
}

// Workgroup-wide argmax of one tile.  Between tile_argmax_begin and
// tile_argmax_end (both reached by every thread) each thread folds the keys
// it produces into its own running maximum per activation row
// (tile_argmax_offer); the end takes the maximum over each wave by lane
// exchanges, over the waves by one LDS 64-bit max per wave and row, and
// writes the tile's best key per row to keys[tile][m].  Every step is a
// maximum, so the order does not matter.
struct TileArgmax {
  unsigned long long best[kDecodeMaxM];
};
template <int M>
struct ArgmaxLocal {
  uint64_t best[M];
};
template <int M>
__device__ __forceinline__ void tile_argmax_begin(TileArgmax& ta, ArgmaxLocal<M>& l) {
#pragma unroll
  for (int mm = 0; mm < M; ++mm) l.best[mm] = 0;
  if (threadIdx.x < kDecodeMaxM) ta.best[threadIdx.x] = 0ull;
  __syncthreads();
}
template <int M>
__device__ __forceinline__ void tile_argmax_offer(ArgmaxLocal<M>& l, int m, uint64_t key) {
#pragma unroll
  for (int mm = 0; mm < M; ++mm)
    if (mm == m && key > l.best[mm]) l.best[mm] = key;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const int lo = __shfl_xor(static_cast<int>(static_cast<uint32_t>(v)), o);
  const int hi = __shfl_xor(static_cast<int>(static_cast<uint32_t>(v >> 32)), o);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}
template <int M>
__device__ __forceinline__ void tile_argmax_end(TileArgmax& ta, ArgmaxLocal<M>& l, uint64_t* keys, int64_t tile) {
#pragma unroll
  for (int mm = 0; mm < M; ++mm) {
    uint64_t v = l.best[mm];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t w = shfl_xor_u64(v, o);
      v = w > v ? w : v;
    }
    if ((threadIdx.x & 63) == 0) atomicMax(&ta.best[mm], static_cast<unsigned long long>(v));
  }
  __syncthreads();
  if (threadIdx.x < M) keys[tile * M + threadIdx.x] = ta.best[threadIdx.x];
}

// SwiGLU epilogue of a fused gate_up call on the interleaved weight (prepared
// row R: gate row 16 (R / 32) + R % 16 if R % 32 < 16, else the up row with
// that index).  A tile's float32 results (global scale applied) go to LDS;
// then y[m][j] = bf16(silu(gate[m][j]) * up[m][j]), silu(v) = v / (1 + e^-v)
// (hardware exp and reciprocal, about 1 ulp each), with one rounding to bf16.  Tiles hold whole 32-row blocks, so both operands of an
// output are in the same workgroup.
__device__ __forceinline__ int il_proj(int64_t row) { return static_cast<int>((row >> 4) & 1); }
__device__ __forceinline__ int64_t il_col(int64_t row) { return (row >> 5) * 16 + (row & 15); }
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// [activation row][row within the tile], up to 128-row tiles; a placeholder
// for the instances above kDecodeActMaxM rows, which never run the epilogue.
template <int M>
struct ActTile {
  float v[M <= kDecodeActMaxM ? M : 1][M <= kDecodeActMaxM ? 128 : 1];
};
// y for the tile of `tile_rows` rows starting at prepared row row0, after
// every thread has stored its results; all threads must call it.
template <int M>
__device__ __forceinline__ void act_store(ActTile<M>& at, const GemvArgs& a, int64_t row0, int tile_rows, int mrows) {
  static_assert(M <= kDecodeActMaxM, "SwiGLU epilogue rows");
  __syncthreads();
  const int pairs = tile_rows / 2;
  for (int i = threadIdx.x; i < M * pairs; i += blockDim.x) {
    const int m = i / pairs;
    const int p = i - m * pairs;
    const int gl = 32 * (p >> 4) + (p & 15);  // the gate row; its up row is gl + 16
    const int64_t col = il_col(row0 + gl);
    if (m < mrows && col < a.n_proj)
      a.y[static_cast<int64_t>(m) * a.ldy + col] = f32_to_bf16_rne(silu(at.v[m][gl]) * at.v[m][gl + 16]);
  }
}

// Split-K partial sums and arrival flags are exchanged between workgroups that
// may sit on different XCDs, whose L2 caches are not coherent with each other.
// They are therefore written and read with device-coherent (sc1) accesses --
// relaxed atomics at agent scope -- which go to the coherence point instead of
// a local L2 line.  Ordering comes from waiting for those stores to complete
// (s_waitcnt 0) before the next step, not from device-scope fences, which on
// this target write back and invalidate the whole L2.
//
// Why this is a correct publication under the AMDGPU memory model (the LLVM
// AMDGPUUsage code sequences for the GFX942 family, which gfx950 follows):
// an agent-scope monotonic load or store is the plain instruction with sc1
// set; an agent-scope release store adds "buffer_wbl2 sc1; s_waitcnt
// vmcnt(0)" before it, and an agent-scope acquire load adds "s_waitcnt
// vmcnt(0); buffer_inv sc1" after it.  The wbl2 writes back L2 lines dirtied
// by non-atomic stores, and the inv drops L2 lines that non-atomic loads could
// otherwise hit stale; both exist only to make non-atomic data coherent.  Here
// every store a reader depends on (partials, flags) and every load that
// depends on a flag (partials) is itself an sc1 agent-scope access, so no
// non-atomic data is published and the two cache operations have nothing to
// do.  What remains of release/acquire is the ordering, and it is explicit:
// a workgroup's partial stores are complete (s_waitcnt vmcnt(0)) before its
// flag store is issued, and the partial loads are issued only after the flag
// loads have returned and been compared (s_waitcnt, then a branch on their
// values), so a workgroup that sees every flag reads every partial from the
// coherence point after it was written.
__device__ __forceinline__ void store_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Split-K finish for one tile (a.tile_rows rows), called by every thread of the
// workgroup after it has stored (store_partial) this split's sums
// partial[split][m][row].
//
// Each (tile, split) workgroup publishes a flag = the call's 64-bit token once
// its partials are complete, then reads the flags of all splits of its tile.
// Store, wait for completion, then load: the last workgroup to publish sees
// every flag (two may both see them; they then compute the same bytes).  A
// workgroup that sees all flags adds the partials in split order 0, 1, ...,
// S-1 -- a fixed order, so the output does not depend on which workgroup
// finishes last -- applies the global scale, writes bf16 y and clears the
// tile's flags.  Flags left by earlier calls either were cleared or hold older
// tokens, so they never match: the workspace needs no zeroing, a captured
// graph can replay the same token, and no workgroup ever waits for another.
//
// Every step is one memory round trip: the flags are read by one lane each
// (wave 0), and each thread issues all the partial loads of its outputs before
// it adds them.  The loads go through a buffer descriptor with the sc1
// (device-coherent) policy -- the policy of the agent-scope atomics above --
// because atomic loads would be issued one after another.
constexpr int kCoherentPolicy = 16;           // sc1
constexpr int kBufferRsrcWord3 = 0x00020000;  // raw 32-bit buffer accesses

template <int M>
__device__ __forceinline__ void splitk_finish(const GemvArgs& a, int64_t tile, int split) {
  __shared__ int s_last;
  wait_memory();
  __syncthreads();
  uint64_t* flags = a.flags + tile * a.splits;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    if (lane == 0) __hip_atomic_store(flags + split, a.token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_memory();
    bool mine = true;
    for (int s = lane; s < a.splits; s += 64)
      mine = mine && __hip_atomic_load(flags + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.token;
    const bool all = __all(mine);
    if (lane == 0) s_last = all ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  for (int s = threadIdx.x; s < a.splits; s += blockDim.x)
    __hip_atomic_store(flags + s, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __shared__ TileArgmax ta;
  __shared__ ActTile<M> at;
  ArgmaxLocal<M> al;
  if (a.keys) tile_argmax_begin(ta, al);
  // One buffer descriptor per split: partial[split] is [M][rows_total] with
  // M <= kDecodeMaxM = 32 and rows_total < 2^24 (FP4_MAX_N), i.e. under 2^29
  // floats = 2^31 bytes, so 32-bit byte offsets suffice within it.
  const int64_t split_floats = static_cast<int64_t>(M) * a.rows_total;
  constexpr int kBatch = 8;
  for (int i = threadIdx.x; i < M * a.tile_rows; i += blockDim.x) {
    const int m = i / a.tile_rows;
    const int64_t row = tile * a.tile_rows + (i - m * a.tile_rows);
    int h = 0;
    const int64_t col = a.act ? 0 : out_col(a, row, h);
    if (col < 0) continue;
    const int off = static_cast<int>((static_cast<int64_t>(m) * a.rows_total + row) * 4);
    float s = 0.0f;
    for (int s0 = 0; s0 < a.splits; s0 += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        v[b] = 0.0f;
        if (s0 + b < a.splits) {
          const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
              a.partial + (s0 + b) * split_floats, 0, static_cast<int>(split_floats * 4), kBufferRsrcWord3);
          v[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, kCoherentPolicy));
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        if (s0 + b < a.splits) s = s0 + b == 0 ? v[b] : s + v[b];
    }
    if constexpr (M <= kDecodeActMaxM) {
      if (a.act) {
        at.v[m][row - tile * a.tile_rows] = s * (il_proj(row) == 0 ? a.gscale[0] : a.gscale[1]);
        continue;
      }
    }
    const uint16_t yb = f32_to_bf16_rne(s * (h == 0 ? a.gscale[0] : a.gscale[1]));
    if (a.y) a.y[static_cast<int64_t>(m) * a.ldy + col] = yb;
    if (a.keys) tile_argmax_offer(al, m, argmax_key(yb, col));
  }
  if (a.keys) tile_argmax_end(ta, al, a.keys, tile);
  if constexpr (M <= kDecodeActMaxM) {
    if (a.act) act_store(at, a, tile * a.tile_rows, a.tile_rows, M);
  }
}

}  // namespace fp4
