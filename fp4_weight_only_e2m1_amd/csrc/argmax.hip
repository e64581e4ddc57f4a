// Second step of the greedy argmax of a decode call: the decode kernels leave
// one key per (tile, activation row) -- the best (value, index) of the tile's
// logits as a 64-bit key, larger exactly when the pair wins (argmax_key) --
// and this launch takes the maximum over the tiles for each activation row.
// A maximum under a total order: any reduction order gives the same (value,
// index), so the result is deterministic ("re-verify 27B NVFP4 on the nvidia
// ModelOpt checkpoint", section on the 35B correctness result: the argmax
// reduction with lowest-index ties is order-independent).
#include "fp4_common.hpp"

namespace fp4 {
namespace {

constexpr int kThreads = 1024;
constexpr int kPerThread = 4;  // keys per thread per pass, loaded before any is compared

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  const uint32_t l2 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), o));
  const uint32_t h2 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), o));
  return (static_cast<uint64_t>(h2) << 32) | l2;
}

// The bf16 bits of a key's value (argmax_key's order mapping undone; a NaN
// comes back as the canonical 0x7FC0, -0 as +0).
__device__ __forceinline__ uint16_t key_value(uint64_t key) {
  const uint32_t o = static_cast<uint32_t>(key >> 32) & 0xFFFFu;
  return static_cast<uint16_t>((o & 0x8000u) ? (o & 0x7FFFu) : (~o & 0xFFFFu));
}

// Workgroup `row`: the maximum of keys[t][row] over t < tiles.  Each pass
// issues kPerThread independent loads per thread before comparing, so a
// layer of up to kThreads * kPerThread tiles takes one memory round trip.
__global__ __launch_bounds__(kThreads) void argmax_reduce_kernel(const uint64_t* keys, int tiles, int m,
                                                                 int32_t* idx, uint16_t* val) {
  const int row = blockIdx.x;
  uint64_t best = 0;
  for (int t0 = 0; t0 < tiles; t0 += kThreads * kPerThread) {
    uint64_t v[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int t = t0 + i * kThreads + static_cast<int>(threadIdx.x);
      v[i] = t < tiles ? keys[static_cast<int64_t>(t) * m + row] : 0ull;
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) best = max_u64(best, v[i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = max_u64(best, shfl_xor_u64(best, o));
  __shared__ uint64_t wave_best[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_best[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) best = max_u64(best, wave_best[w]);
    idx[row] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(best));
    if (val) val[row] = key_value(best);
  }
}

}  // namespace

hipError_t launch_argmax_reduce(const uint64_t* keys, int tiles, int m, int32_t* idx, uint16_t* val,
                                hipStream_t stream) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(static_cast<unsigned>(m)), dim3(kThreads), 0, stream, keys, tiles,
                     m, idx, val);
  return hipGetLastError();
}

}  // namespace fp4
