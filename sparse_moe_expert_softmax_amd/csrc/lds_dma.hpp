// Global -> LDS loads through the buffer unit (LDS-DMA) and the waits and
// barriers around them, shared by the prefill GEMMs on gfx950.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ft {

// s_waitcnt vmcnt(n) alone (expcnt and lgkmcnt at their no-wait maxima)
#define BG_VMWAIT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))
// A workgroup barrier without the memory fence that __syncthreads() carries:
// the fence would wait for every LDS-DMA load in flight.  The empty asm keeps
// the compiler from moving memory accesses across it.
#define BG_BARRIER()                          \
  do {                                        \
    asm volatile("" ::: "memory");            \
    __builtin_amdgcn_s_barrier();             \
    asm volatile("" ::: "memory");            \
  } while (0)

// Buffer descriptor word 3 for untyped 32-bit accesses on gfx9-family parts.
constexpr int GM_RSRC_WORD3 = 0x00020000;

typedef int bg_i32x4_t __attribute__((ext_vector_type(4)));

// Buffer load of 16 (or 12) bytes per lane straight into LDS: lane l's bytes
// land at lds + size * l.  Written as inline asm so that the compiler does not
// add its own waits for these loads (its LDS-DMA tracking falls back to
// waiting for all of them before any LDS read); the kernel waits for them
// explicitly before each barrier.
__device__ __forceinline__ void bg_dma16(bg_i32x4_t rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void bg_dma12(bg_i32x4_t rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx3 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ bg_i32x4_t bg_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return (bg_i32x4_t){(int)(uint32_t)a, (int)(uint32_t)((a >> 32) & 0xFFFFu), (int)bytes, GM_RSRC_WORD3};
}
__device__ __forceinline__ uint32_t bg_lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

}  // namespace ft
