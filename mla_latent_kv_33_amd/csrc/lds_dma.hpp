// Direct-to-LDS copies and the explicit waits and barriers around them.
//
// The compiler tracks direct-to-LDS loads conservatively (it would wait for
// every copy in flight before each LDS read, serialising copy and compute),
// so the copies, their vmcnt waits and the barriers are written out.  None
// of these statements returns a register, and each is a compiler memory
// barrier ("memory" clobber), so LDS accesses stay between the waits and
// barriers they are written between.  Kernels that use them issue no other
// vector-memory loads while copies are counted, so vmcnt counts copies only.
#pragma once

#include "mla_common.hpp"

namespace mla {

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// The wave's 64 lanes copy 16 bytes each from sbase + voff (lane's offset)
// to LDS address lds_addr + 16 * lane.  M0 carries the LDS address; one
// wait state separates its write from the load that reads it.  Both
// addresses are wave-uniform; readfirstlane makes that explicit so that they
// sit in scalar registers.  readfirstlane returns a signed int: converting
// through uint32_t zero-extends the low word into the 64-bit address.
// NT: a non-temporal load, for data read once per step (streamed weights,
// the cache rows of a large decode), which then does not displace what the
// Infinity Cache holds.
template <bool NT = false>
__device__ __forceinline__ void dma16(uint32_t lds_addr, const void* sbase,
                                      uint32_t voff) {
  const uint64_t b = (uint64_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %1 nt"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "s"((const char*)sb),
          "v"(voff)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %1"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "s"((const char*)sb),
          "v"(voff)
        : "memory", "m0");
}
template <int IMM, bool NT = false>
__device__ __forceinline__ void dma16_off(uint32_t lds_addr, const void* sbase,
                                          uint32_t voff) {
  static_assert(IMM >= 0 && IMM < 4096, "offset field range");
  lds_addr -= IMM;
  const uint64_t b = (uint64_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %1 offset:%3 nt"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "s"((const char*)sb),
          "v"(voff), "n"(IMM)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %1 offset:%3"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "s"((const char*)sb),
          "v"(voff), "n"(IMM)
        : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() {
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
}
__device__ __forceinline__ void barrier() {
  asm volatile("s_barrier" : : : "memory");
}

// Swizzle of a 16-byte chunk position inside a 128-byte row, keyed by the
// row index mod 8: rows r = 0..7 reading the same chunk hit 8 distinct bank
// groups, and so do the 8 chunks of one row.
__device__ __forceinline__ int swz(int t8) { return ((2 * t8) & 7) | (t8 >> 2); }

}  // namespace mla
