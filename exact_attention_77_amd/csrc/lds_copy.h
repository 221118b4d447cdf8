// lds_copy.h -- direct global -> LDS tile copies for gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Copies 16 bytes per lane from global memory straight into LDS (lane l fills
// LDS bytes lds + 16 l .. +15; `lds` must be wave-uniform), without passing
// through registers.  The copy is issued so that the compiler does not track
// it: while a direct-to-LDS copy it knows of is pending, it makes every LDS
// read wait for all outstanding LDS operations (lgkmcnt(0)), which defeats
// operand prefetching.  Callers therefore (1) never copy into a buffer that
// any wave may still read, and (2) wait for the copies explicitly
// (s_waitcnt vmcnt(0), then a workgroup barrier) before any wave reads the
// buffer.  Writing M0 needs one wait state before the LDS-DMA load.
__device__ __forceinline__ void copy16_to_lds(const void* src, const void* lds) {
    typedef __attribute__((address_space(3))) const void lds_cvoid;
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cvoid*)lds));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(src) : "memory", "m0");
}

// The same with the source split into a base and a 32-bit per-lane byte
// offset (the address is base + off, the offset zero-extended): one vector
// register per copy instead of a 64-bit address.  `base` must be the same in
// every lane of the wave; it is read from the first active lane into scalar
// registers (a no-op when the compiler already holds it there).
__device__ __forceinline__ void copy16_to_lds_off(const void* base, uint32_t off, const void* lds) {
    typedef __attribute__((address_space(3))) const void lds_cvoid;
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cvoid*)lds));
    const uint64_t b = reinterpret_cast<uintptr_t>(base);
    const uint64_t sb = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b)))) |
                        (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b >> 32)))) << 32);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(off), "s"(sb) : "memory", "m0");
}

// The same for 4 bytes per lane (lane l fills lds + 4 l .. +3).
__device__ __forceinline__ void copy4_to_lds(const void* src, const void* lds) {
    typedef __attribute__((address_space(3))) const void lds_cvoid;
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cvoid*)lds));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(src) : "memory", "m0");
}

}  // namespace fa
