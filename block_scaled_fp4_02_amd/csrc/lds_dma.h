// lds_dma.h -- gfx950 direct-to-LDS loads and the explicit waits that go with them.
//
// global_load_lds_* copy from memory straight into LDS (no staging registers).
// They are issued from asm blocks with no output registers: the hardware writes
// lane l's 16 bytes at M0 + 16 l (dwordx4), its 2 or 1 bytes zero-extended into
// the dword at M0 + 4 l (ushort, ubyte); M0 (the wave's LDS address) is set in
// the same block. The compiler does not see these as LDS writes, so it adds no
// waits of its own between them and reads of other LDS buffers; a kernel waits
// for them itself (vmcnt) before the barrier that makes a buffer visible.
// Addresses are a wave-uniform 64-bit base (SGPRs) plus a 32-bit lane offset.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang diagnostic ignored "-Winline-asm"   // M0 is named as clobbered on purpose

namespace nvfp4 {

__device__ inline void dma16s(const void *base, uint32_t off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds_addr), "v"(off), "s"(base) : "memory", "m0");
}
__device__ inline void dma2s(const void *base, uint32_t off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_ushort %1, %2"
                 :: "s"(lds_addr), "v"(off), "s"(base) : "memory", "m0");
}
__device__ inline void dma1s(const void *base, uint32_t off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_ubyte %1, %2"
                 :: "s"(lds_addr), "v"(off), "s"(base) : "memory", "m0");
}
// 32-bit LDS address of a pointer into shared memory (wave-uniform)
__device__ inline uint32_t lds_addr_of(const void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p);
}

}  // namespace nvfp4

// s_waitcnt with vmcnt <= n (n < 64) and the other counters left alone, and with
// lgkmcnt == 0 and the others left alone (gfx9 encoding: vmcnt low bits 3:0 and
// high bits 15:14, expcnt 6:4, lgkmcnt 11:8)
#define DMA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (0x7 << 4) | (0xF << 8))
#define DMA_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4))
