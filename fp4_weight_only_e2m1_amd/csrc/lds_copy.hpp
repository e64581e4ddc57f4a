// Asynchronous global -> LDS copies (the load-to-LDS path of gfx950) and the
// wait + workgroup barrier that consumes them, shared by the MFMA kernels.
#pragma once

#include <cstdint>
#include <hip/hip_runtime.h>

namespace fp4 {

// Wait until at most N of this wave's vector-memory operations are in flight
// and its LDS operations are done, then join the workgroup barrier.  Written
// as one asm statement so the compiler moves no memory access across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Global -> LDS copies of 16 bytes per lane: lane l's bytes land at LDS
// address M0 + 16 l, M0 being the same for the whole wave.  Issued as inline
// asm so that the compiler, which would otherwise guard every later LDS read
// with a wait for all copies in flight, leaves the waits to the pipeline
// (wait_vm_barrier).  M0 is left holding the last LDS address: nothing else in
// these kernels reads M0 (no LDS-DMA builtins, no s_movrel or GWS).  Device
// code only: the host pass of the compiler cannot parse the asm.
//   copy16_sbase: address = 64-bit base (wave-uniform) + 32-bit lane offset.
//   copy16_vaddr: address = 64-bit per-lane pointer.
__device__ __forceinline__ void copy16_sbase(const void* base, uint32_t off, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
#else
  (void)base;
  (void)off;
  (void)lds;
#endif
}

// copy16_sbase with the non-temporal hint: for a stream read once (decode
// weights), so it does not displace lines that are re-read.  Measured on
// MI355X for the 64-row decode tiles: ~5% less time per call than the default
// policy.
__device__ __forceinline__ void copy16_sbase_nt(const void* base, uint32_t off, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %0, %1 nt"
      :
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
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
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

}  // namespace fp4
