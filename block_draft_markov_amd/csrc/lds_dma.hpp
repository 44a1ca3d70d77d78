// Buffer loads that write LDS directly (gfx950 buffer_load_dwordx4 ... lds), shared by
// the kernels that stage their operands through LDS.
//
// Each instruction moves 16 bytes per lane: lane l's bytes land at LDS byte m0 + 16 l,
// so one instruction fills a contiguous 1 KB block.  Eight lanes per 128-byte line
// fetch eight whole lines; choosing which 16-byte chunk of its line each lane fetches
// lays the block out with chunk c of row q at chunk c ^ swz(q), which keeps the
// fragment reads of 32 rows at one chunk free of bank conflicts without padding.
// An offset past the described buffer range reads as zeros and moves no memory.
#pragma once

#include "common.hpp"

namespace dflash {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kBufWord3 = 0x00020000;   // gfx9 buffer descriptor word 3 for raw dword access
constexpr int kBig = 0x40000000;        // buffer offset past every described range (ranges stay < 2^29)
constexpr int64_t kDmaRange = 1 << 29;  // largest range a descriptor of sbuf describes

__device__ __forceinline__ constexpr int waitcnt_vm(int n) {
    // s_waitcnt immediate: vmcnt <= n; expcnt and lgkmcnt unconstrained
    return (n & 0xf) | (0x7 << 4) | (0xf << 8) | ((n >> 4) << 14);
}

// Raw buffer descriptor (base, stride 0, size in bytes) in scalar registers.
__device__ __forceinline__ u32x4 sbuf(const void* base, int64_t bytes) {
    const uint64_t p = (uint64_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane((uint32_t)(bytes < kDmaRange ? bytes : kDmaRange));
    r[3] = kBufWord3;
    return r;
}

// buffer_load_dwordx4 ... lds: lane l's 16 bytes at offset voff + soff land at LDS byte lds + 16 l.
// Issued from inline assembly, so the compiler neither reorders it nor waits for it: every
// wait for these loads is an explicit s_waitcnt vmcnt of the kernel.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// LDS chunk swizzle of a row of 128-byte lines
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

}  // namespace dflash
