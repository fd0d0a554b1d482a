// Shared device/host helpers for the gfx950 MLA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/mla.h"

namespace mla {

// Raises a kernel's dynamic-LDS limit to `bytes` once per device (the
// setting belongs to the current device).  `done` is that kernel's set of
// devices already configured; concurrent callers may both set it, which is
// harmless, and the flag itself is race-free.
inline hipError_t set_lds_limit_once(const void* kernel, int bytes,
                                     std::atomic<unsigned long long>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
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

// fp32 x -> bf16 hi + bf16 lo with hi + lo = x to about 16 significant bits
// (hi rounded to nearest by the hardware conversion, lo the rounded
// remainder): eight values a[0..3], b[0..3] into hi[0..7], lo[0..7].  Two
// bf16 products against the same weight then reproduce an fp32 activation.
__device__ __forceinline__ void split_hi_lo_hw(const f32x4& a, const f32x4& b,
                                               bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t hp = __builtin_bit_cast(
        uint32_t, __builtin_convertvector((f32x2){x[2 * e], x[2 * e + 1]},
                                          bf16x2));
    const float r0 = x[2 * e] - __uint_as_float(hp << 16);
    const float r1 = x[2 * e + 1] - __uint_as_float(hp & 0xFFFF0000u);
    h[e] = hp;
    l[e] = __builtin_bit_cast(
        uint32_t, __builtin_convertvector((f32x2){r0, r1}, bf16x2));
  }
  hi = __builtin_bit_cast(bf16x8, (u32x4){h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, (u32x4){l[0], l[1], l[2], l[3]});
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
