// Shared device/host helpers for the gfx950 MLA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

#define MLA_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediates (gfx9 encoding): vmcnt in [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]; an all-ones field means "do not wait".
__device__ __forceinline__ constexpr int waitcnt_vm(int n) {
  return (n & 15) | ((n >> 4) << 14) | 0x0F70;
}
__device__ __forceinline__ constexpr int waitcnt_lgkm(int n) {
  return 0xC07F | ((n & 15) << 8);
}

// bf16 <-> fp32.  Stores round to nearest, ties to even.
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu))
    return (uint16_t)0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// Two floats -> packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

template <typename T>
struct DT;
template <>
struct DT<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) {
    return p[i];
  }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) {
    p[i] = v;
  }
};
template <>
struct DT<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) {
    return bf2f(p[i]);
  }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i,
                                               float v) {
    p[i] = f2bf(v);
  }
};

inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

}  // namespace mla
