// Device helpers shared by the libkq kernels (gfx950): global->LDS DMA issued from inline
// asm, LDS addresses, and explicit memory-counter waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define KQ_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

namespace {

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0]+[15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int kWaitVm0 = 0x0F70;     // vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;   // lgkmcnt(0)

// Wait, and keep both the compiler and the scheduler from moving memory accesses across.
template <int IMM>
__device__ __forceinline__ void wait_and_fence() {
  __builtin_amdgcn_s_waitcnt(IMM);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// One global -> LDS DMA of 16 bytes per lane (global_load_lds_dwordx4): lane i reads
// base + voff_i and its bytes land at lds_base + 16 i; base and lds_base must be
// wave-uniform. NT selects the non-temporal cache policy (data read once).
// Issued from inline asm on purpose: the compiler's wait insertion cannot tell which LDS
// bytes a DMA writes, so for a builtin DMA it makes every later LDS read wait for it, and
// with stores in flight it turns that into a wait for all vector-memory traffic (stores
// included). The kernels order their DMAs with explicit s_waitcnt instead. m0 is saved
// and restored so that no value the compiler keeps there is lost; the s_nop gives the m0
// write and a VALU write of the base (readfirstlane) the wait states a vector-memory
// read of them needs.
template <bool NT>
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(lds_base)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(lds_base)
        : "memory");
  }
}

// The same DMA with a full 64-bit address per lane (rows that are not one stride apart).
template <bool NT>
__device__ __forceinline__ void dma16_addr(const void *gaddr, uint32_t lds_base) {
  uint32_t saved;
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gaddr), "s"(lds_base)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gaddr), "s"(lds_base)
        : "memory");
  }
}

__device__ __forceinline__ void dma16_nt(const void *base, uint32_t voff, uint32_t lds_base) {
  dma16<true>(base, voff, lds_base);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)KQ_LDS_PTR(p);
}

// s_waitcnt immediate for vmcnt(n), 0 <= n < 64 (gfx9: vmcnt in bits [3:0] and [15:14];
// expcnt and lgkmcnt at their maxima, so not waited for)
constexpr int wait_vm_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

// Copy `bytes` (a multiple of 1 KiB) from global memory to LDS by DMA, the waves of the
// workgroup taking the 1 KiB instructions in turn (lane i of instruction j moves bytes
// 1024 j + 16 i). Waiting for it takes this wave's vmcnt; the copy is complete for the
// workgroup after every wave has waited and passed a barrier.
__device__ __forceinline__ void dma_copy(const void *src, void *dst, int bytes, int wave,
                                         int waves, int lane) {
  for (int j = wave; j < bytes / 1024; j += waves)
    dma16<false>(src, (uint32_t)(j * 1024 + lane * 16),
                 lds_addr(static_cast<unsigned char *>(dst) + j * 1024));
}

}  // namespace
