// Machine-rate kernels: what this MI355X reaches on a plain HBM read stream
// and on a loop of bf16 matrix-core operations, measured on the same box and
// under the same power state as the kernels they are compared with.  They
// compute nothing of the layer; the decode measurement divides by these
// rates next to the datasheet peaks.
//
// stream_read_kernel: every workgroup reads its own contiguous chunk of a
// buffer larger than the 256 MB Infinity Cache in 16-byte vectors, eight
// loads in flight per lane, and folds them into one word so that the loads
// cannot be removed.
//
// mfma_loop_kernel: every wave issues independent v_mfma_f32_32x32x16_bf16
// on register operands (eight accumulators, so no MFMA waits for another),
// four waves per compute unit per workgroup and two workgroups per compute
// unit.  The operands are hashed lane values, not zeros, so the multipliers
// toggle as they do on real data.

#include "mla_common.hpp"
#include "../../include/mla_peaks.h"

namespace mla {
namespace {

constexpr int SR_THREADS = 256;
constexpr int SR_UNROLL = 8;

// Workgroup w reads its own contiguous chunk of the buffer (the access
// pattern of a kernel that streams whole cache blocks per workgroup); each
// wave reads 1 KiB per load, SR_UNROLL loads in flight per lane.
__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(
    const u32x4* __restrict__ buf, size_t per_wg, uint32_t* __restrict__ sink) {
  const u32x4* p = buf + (size_t)blockIdx.x * per_wg;
  uint32_t acc = 0;
  size_t i = threadIdx.x;
  for (; i + (SR_UNROLL - 1) * SR_THREADS < per_wg; i += SR_UNROLL * SR_THREADS) {
    u32x4 v[SR_UNROLL];
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u)
      v[u] = __builtin_nontemporal_load(p + i + u * SR_THREADS);
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < per_wg; i += SR_THREADS) {
    const u32x4 v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // one word per workgroup, written only when the fold is a value no
  // buffer of this test produces, so the store almost never happens but the
  // compiler must keep every load
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// A bf16 pair with exponent in [2^-2, 2^1) and random mantissa and sign.
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t seed) {
  const uint32_t h = hash32(seed);
  const uint32_t lo = 0x3E80u | (h & 0x807Fu) | ((h >> 7) & 0x0100u);
  const uint32_t hi = 0x3E80u | ((h >> 16) & 0x807Fu) | ((h >> 23) & 0x0100u);
  return lo | (hi << 16);
}

constexpr int MF_ACC = 8;

__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(
    int iters, float* __restrict__ sink) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[2], b[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const u32x4 ua = {rand_bf16x2(4 * t + 8 * k), rand_bf16x2(4 * t + 8 * k + 1),
                      rand_bf16x2(4 * t + 8 * k + 2), rand_bf16x2(4 * t + 8 * k + 3)};
    const u32x4 ub = {rand_bf16x2(~(4 * t + 8 * k)), rand_bf16x2(~(4 * t + 8 * k + 1)),
                      rand_bf16x2(~(4 * t + 8 * k + 2)), rand_bf16x2(~(4 * t + 8 * k + 3))};
    a[k] = __builtin_bit_cast(bf16x8, ua);
    b[k] = __builtin_bit_cast(bf16x8, ub);
  }
  f32x16 acc[MF_ACC];
#pragma unroll
  for (int j = 0; j < MF_ACC; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < MF_ACC; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 1], b[(j >> 1) & 1],
                                                       acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < MF_ACC; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  sink[t] = s;
}

}  // namespace
}  // namespace mla

extern "C" {

mla_status mla_peak_stream_read(const void* buf, size_t bytes, void* sink,
                                int32_t workgroups, mla_stream_t stream) {
  if (!buf || !sink) return MLA_ERR_NULL;
  if (bytes < 16 || bytes % 16 || workgroups <= 0 ||
      (bytes / 16) % (size_t)workgroups)
    return MLA_ERR_SHAPE;
  hipLaunchKernelGGL(mla::stream_read_kernel, dim3(workgroups),
                     dim3(mla::SR_THREADS), 0, (hipStream_t)stream,
                     (const mla::u32x4*)buf, bytes / 16 / workgroups,
                     (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_DEVICE;
}

size_t mla_peak_mfma_sink_bytes(int32_t workgroups) {
  return workgroups > 0 ? (size_t)workgroups * 256 * sizeof(float) : 0;
}

double mla_peak_mfma_flops(int32_t workgroups, int32_t iters) {
  // 4 waves per workgroup, MF_ACC MFMAs of 32 x 32 x 16 per wave per
  // iteration, 2 flops per multiply-add
  return (double)workgroups * 4 * iters * mla::MF_ACC * (2.0 * 32 * 32 * 16);
}

mla_status mla_peak_mfma_loop(int32_t workgroups, int32_t iters, void* sink,
                              mla_stream_t stream) {
  if (!sink) return MLA_ERR_NULL;
  if (workgroups <= 0 || iters <= 0) return MLA_ERR_SHAPE;
  hipLaunchKernelGGL(mla::mfma_loop_kernel, dim3(workgroups), dim3(256), 0,
                     (hipStream_t)stream, iters, (float*)sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_DEVICE;
}

}  // extern "C"
