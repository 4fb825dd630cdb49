// Direct global -> LDS loads for gfx950 (the load-to-LDS forms of
// global_load_dword / global_load_dwordx4), shared by the attention, its
// backward and the INT8-weight linear.
//
// Lane l's bytes land at lds_base + size * l, where lds_base is wave-uniform
// and travels in M0. The loads are issued from inline assembly so that the
// compiler records no pending LDS write: with its builtin it cannot tell the
// kernels' LDS buffers apart and drains every such load (s_waitcnt vmcnt(0))
// before each later LDS read of another buffer. The kernels therefore await
// completion themselves with s_waitcnt vmcnt(n).
//
// M0 is a reserved register, and clang warns that clobbering it in inline
// assembly is not preserved for the compiler's own use. Here that is the
// intent: each helper sets M0 itself (one wait state after the SALU write
// before the load), and no compiler-generated instruction in these kernels
// reads or writes M0 (no LDS-DMA builtins, GWS, message or relative-move
// instructions; checked in the generated gfx950 assembly), so the warning is
// silenced for these helpers only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace segc {

// A generic pointer into LDS holds the LDS byte address in its low 32 bits
// (the shared aperture is 4 GB aligned; the address-space cast would add a
// null check per use, which these never-null tile pointers do not need).
__device__ inline uint32_t lds_addr(const char* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// A wave-uniform address as a pair of SGPRs (each half widened as unsigned).
__device__ inline uint64_t uniform_addr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from a per-lane 64-bit address.
__device__ inline void dload16(const void* g, const char* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds_addr(lds_base)) : "memory", "m0");
}
// 4 bytes per lane.
__device__ inline void dload4(const void* g, const char* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(lds_addr(lds_base)) : "memory", "m0");
}
// 16 bytes per lane with a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset (the load's scalar-base form: no per-lane 64-bit
// address arithmetic).
__device__ inline void dload16_s(uint32_t voff, uint64_t sbase, const char* lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr(lds_base)) : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace segc
