// Query-side pre-merged absorption ('MLA：潜在表示压缩与解耦 RoPE', section
// 4: W^UQ^T W^UK can be merged ahead of time; section 5: the RoPE part
// cannot, so q_R keeps its own projection).
//
// The merged matrix of head h is M_h = W_UK_h^T W_UQ_h, d_c x d_cq (W_UK_h
// and W_UQ_h are rows h d_h .. h d_h + d_h - 1 of W_UK [n_h d_h][d_c] and
// W_UQ [n_h d_h][d_cq]), so that q_lat_h = W_UK_h^T (W_UQ_h c_Q) = M_h c_Q.
// merge_kernel builds all n_h of them once (fp32 accumulation over the d_h
// products, one rounding to the weight dtype); the step then needs one
// projection of c_Q onto [M_0; ...; M_{n_h-1}; W_QR] instead of W_UQ
// followed by the per-head absorption.  Per layer that is n_h d_c d_cq
// weights against n_h d_h (d_c + d_cq) unmerged (100.7 M against 33.6 M at
// DeepSeek-V2 dims).

#include "mla_common.hpp"
#include "mla_kernels.hpp"

namespace mla {
namespace {

// out[h][c][j] = sum_i W_UK[h d_h + i][c] W_UQ[h d_h + i][j]; block (j
// chunk of 256, c, h); the W_UK element of a step is the same for the whole
// block, the W_UQ row piece is read coalesced.
template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(
    const T* __restrict__ w_uq, const T* __restrict__ w_uk, int d_h, int d_c,
    int d_cq, T* __restrict__ out) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y, h = blockIdx.z;
  if (j >= d_cq) return;
  const T* uk = w_uk + (size_t)h * d_h * d_c + c;
  const T* uq = w_uq + (size_t)h * d_h * d_cq + j;
  float acc = 0.0f;
  for (int i = 0; i < d_h; ++i)
    acc = __builtin_fmaf(DT<T>::load(uk, (size_t)i * d_c),
                         DT<T>::load(uq, (size_t)i * d_cq), acc);
  DT<T>::store(out, ((size_t)h * d_c + c) * d_cq + j, acc);
}

}  // namespace

hipError_t launch_merge_uq_uk(const mla_dims& d, const void* w_uq,
                              const void* w_uk, void* out,
                              hipStream_t stream) {
  const dim3 grid((d.d_cq + 255) / 256, d.d_c, d.n_h);
  if (d.dtype == MLA_BF16)
    hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       (const uint16_t*)w_uq, (const uint16_t*)w_uk, d.d_h,
                       d.d_c, d.d_cq, (uint16_t*)out);
  else
    hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(256), 0, stream,
                       (const float*)w_uq, (const float*)w_uk, d.d_h, d.d_c,
                       d.d_cq, (float*)out);
  return hipGetLastError();
}

}  // namespace mla
