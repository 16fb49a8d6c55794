// lds_dma.hpp -- gfx950 global -> LDS asynchronous copies shared by the MFMA kernels.
//
// global_load_lds_dwordx4 copies 16 bytes per lane straight into LDS: lane i writes at
// M0 + 16*i, so one wave instruction fills 1 KB contiguously.  No registers hold the
// data in flight.  The copies are issued through inline assembly and awaited with an
// explicit s_waitcnt vmcnt(n): issued through the compiler builtin, every LDS read
// after such a copy is preceded by a full vmcnt(0) wait, which would serialise the
// pipeline.  Lanes whose source lies outside the tensor (padding, ragged tiles) copy a
// 16-byte zero page instead.
//
// M0: each copy sets M0 to its LDS base in the same asm block, right before the
// instruction that reads it, and lists M0 as clobbered.  The compiler warns that it may
// not preserve a reserved register across such a block; that would only matter if it
// kept a value of its own in M0 across one.  In these kernels it never uses M0 at all
// (no indirect register indexing, messages, GWS or LDS-DMA builtins), so every M0 write
// in the built code is one of these blocks, immediately followed by its copy;
// tests/test_isa_cpu.py checks exactly that on the built library.
#pragma once

#include "common.hpp"

namespace convmi {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ const uint4 kZero16 = {0u, 0u, 0u, 0u};

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr_t)(p); }

// The M0 clobber warning is silenced for these two blocks only (see above for why it
// is safe and which test guards it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// 16 bytes per lane, global -> LDS; lds_base must be wave-uniform.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base) : "memory", "m0");
}

// The same copy through a raw buffer resource: lane i copies the 16 bytes at byte offset
// voff of the buffer.  A 16-byte piece whose offset lies at or past the buffer's size
// (including "negative" offsets, which wrap to huge unsigned values) is written as zeros,
// so a buffer per tensor segment turns every padding and ragged-edge test into the
// hardware's range check.
typedef int dma_rsrc __attribute__((ext_vector_type(4)));

// Raw buffer of `bytes` bytes at `base` (both wave-uniform; stride 0, no swizzle).
__device__ __forceinline__ dma_rsrc make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    dma_rsrc r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xFFFFu));
    r.z = __builtin_amdgcn_readfirstlane((int)bytes);
    r.w = __builtin_amdgcn_readfirstlane(0x00020000);
    return r;
}

__device__ __forceinline__ void dma16_buf(uint32_t voff, dma_rsrc rsrc, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds_base)
                 : "memory", "m0");
}

#pragma clang diagnostic pop

// Wait until at most n of this wave's copies are outstanding (n wave-uniform; values
// above 31 wait for 31, which is only more conservative).
__device__ __forceinline__ void wait_dma(int n) {
#define CONVMI_W(N) case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
    switch (n) {
        CONVMI_W(0) CONVMI_W(1) CONVMI_W(2) CONVMI_W(3) CONVMI_W(4) CONVMI_W(5) CONVMI_W(6) CONVMI_W(7)
        CONVMI_W(8) CONVMI_W(9) CONVMI_W(10) CONVMI_W(11) CONVMI_W(12) CONVMI_W(13) CONVMI_W(14) CONVMI_W(15)
        CONVMI_W(16) CONVMI_W(17) CONVMI_W(18) CONVMI_W(19) CONVMI_W(20) CONVMI_W(21) CONVMI_W(22) CONVMI_W(23)
        CONVMI_W(24) CONVMI_W(25) CONVMI_W(26) CONVMI_W(27) CONVMI_W(28) CONVMI_W(29) CONVMI_W(30)
        default: asm volatile("s_waitcnt vmcnt(31)" ::: "memory"); break;
    }
#undef CONVMI_W
}

__device__ __forceinline__ int xcd_tile(int bid, int nb) {
    // Hardware places block b on XCD b % 8.  Give each XCD a contiguous run of tiles.
    const int full = nb & ~7;
    if (bid >= full) return bid;
    const int per = full >> 3;
    return (bid & 7) * per + (bid >> 3);
}

}  // namespace
}  // namespace convmi
