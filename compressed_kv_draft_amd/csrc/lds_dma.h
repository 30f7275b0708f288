// Direct global -> LDS loads (gfx950 global_load_lds_dwordx4) and the waits
// that go with them.
//
// One load instruction moves 16 bytes per lane; lane i's bytes land at LDS
// address M0 + 16 i, so a wavefront fills 1 KiB.  Exec-masked lanes write
// nothing.  No register receives the data, so a kernel can keep several tiles
// in flight without spending VGPRs on them.
//
// The loads are issued from inline assembly so that the compiler does not see
// them: it would otherwise wait for all of them (vmcnt(0)) before any LDS read
// it cannot prove disjoint, which serialises a prefetch ring.  The kernels wait
// explicitly instead.  Loads complete in order, so "at most N outstanding"
// means every load instruction but the last N has written LDS; any vector-
// memory instruction the compiler adds after them only makes such a wait
// stricter, never weaker.  M0 is saved and restored around each load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vc {

// load instructions needed for `bytes` bytes (16 per lane, 64 lanes)
constexpr int lds_dma_count(int bytes) { return (bytes + 1023) / 1024; }

// LDS address (for M0) of a shared-memory pointer, as a wave-uniform value
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  using lptr = __attribute__((address_space(3))) const void*;
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lptr)p);
}

// 16 bytes from base + voff (base wave-uniform, in scalar registers; voff the
// lane's byte offset) to LDS lds_addr + 16 * lane.
__device__ __forceinline__ void lds_dma16(const unsigned char* base, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "memory");
}

// 16 bytes from the lane's own address src to LDS lds_addr + 16 * lane.
__device__ __forceinline__ void lds_dma16(const unsigned char* src, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_addr)
      : "memory");
}

// BYTES (a multiple of 16) from the wave-uniform address gbase to the
// wave-uniform LDS address lds; voff = 16 * lane.
template <int BYTES>
__device__ __forceinline__ void lds_dma(const unsigned char* gbase, uint32_t voff, uint32_t lds, int lane) {
  static_assert(BYTES % 16 == 0, "");
#pragma unroll
  for (int k = 0; k < BYTES / 1024; ++k) lds_dma16(gbase + 1024 * k, voff, lds + 1024 * k);
  if constexpr (BYTES % 1024 != 0) {
    constexpr int k = BYTES / 1024;
    if (lane < (BYTES % 1024) / 16) lds_dma16(gbase + 1024 * k, voff, lds + 1024 * k);
  }
}

// Wait until at most N vector-memory instructions of this wavefront are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait for every load the compiler itself has issued so far, through its own
// s_waitcnt intrinsic (vmcnt 0; expcnt and lgkmcnt left free), so that its
// wait-insertion pass knows those loads are done.  The pass cannot see the
// direct loads above: a value it loaded before a loop that issues direct loads
// and first uses inside it would get its wait inside the loop, where the
// hardware counter also holds the direct loads, so every iteration would stall
// until they land.  Call this after such loads and before the loop.
__device__ __forceinline__ void settle_compiler_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait for this wavefront's outstanding LDS reads (before a load may overwrite
// the LDS they read).
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

}  // namespace vc
