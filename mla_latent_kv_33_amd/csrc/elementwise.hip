// Element-wise epilogues of the projections: summing K-chunk partials,
// RoPE, rounding to the layer dtype and the scatter of latent rows into the
// paged cache.
//
// RoPE ('MLA：潜在表示压缩与解耦 RoPE', sections 5-6): position p rotates the
// pair (x_j, x_{j + d_r/2}) by the angle p * theta_j, with cos/sin taken
// from host-built fp32 tables [max_pos][d_r/2].  A position outside the
// table (a caller error) yields NaN in the rotated columns instead of a read
// past the table.

#include "mla_common.hpp"
#include "mla_kernels.hpp"

namespace mla {
namespace {

// Sum of the parts at i; four independent loads in flight per round.
__device__ __forceinline__ float sum_parts(const float* p, int nparts,
                                           long stride, long i) {
  const float* q = p + i;
  float v0 = 0.0f, v1 = 0.0f, v2 = 0.0f, v3 = 0.0f;
  int k = 0;
  for (; k + 4 <= nparts; k += 4) {
    v0 += q[k * stride];
    v1 += q[(k + 1) * stride];
    v2 += q[(k + 2) * stride];
    v3 += q[(k + 3) * stride];
  }
  for (; k < nparts; ++k) v0 += q[k * stride];
  return (v0 + v1) + (v2 + v3);
}

__global__ void reduce_parts_kernel(const float* __restrict__ src, int nparts,
                                    long part_stride, long n,
                                    float* __restrict__ dst) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n;
       i += (long)gridDim.x * blockDim.x)
    dst[i] = sum_parts(src, nparts, part_stride, i);
}

// Token t's cache row from acc (row t at t * ld_acc, d_c + d_r columns):
// items j < d_c are copied columns, the rest rotate the d_r RoPE columns in
// pairs; this thread takes items j0, j0 + jstep, ...
template <typename T>
__device__ __forceinline__ void scatter_row(
    const float* __restrict__ acc, int nparts, long part_stride, long ld_acc,
    int t, int j0, int jstep, int d_c, int d_r,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const float* __restrict__ rcos, const float* __restrict__ rsin,
    int max_pos, const int32_t* __restrict__ block_table, int max_blocks,
    int block_size, T* __restrict__ cache) {
  const int width = d_c + d_r;
  const int half = d_r / 2;
  const int p = pos[t];
  const int blk = block_table[(long)seq_idx[t] * max_blocks + p / block_size];
  T* row = cache + ((long)blk * block_size + (p % block_size)) * width;
  const long base = (long)t * ld_acc;
  for (int j = j0; j < d_c + half; j += jstep) {
    if (j < d_c) {
      DT<T>::store(row, j, sum_parts(acc, nparts, part_stride, base + j));
    } else {
      const int jj = j - d_c;
      const float x1 = sum_parts(acc, nparts, part_stride, base + d_c + jj);
      const float x2 =
          sum_parts(acc, nparts, part_stride, base + d_c + jj + half);
      const bool ok = p >= 0 && p < max_pos;
      const float c = ok ? rcos[(long)p * half + jj] : NAN;
      const float s = ok ? rsin[(long)p * half + jj] : NAN;
      DT<T>::store(row, d_c + jj, x1 * c - x2 * s);
      DT<T>::store(row, d_c + jj + half, x1 * s + x2 * c);
    }
  }
}

// Workgroup (token, slice of 256 items) of the rows acc [T][d_c + d_r].
template <typename T>
__global__ void append_scatter_kernel(
    const float* __restrict__ acc, int nparts, long part_stride, int d_c,
    int d_r, const int32_t* __restrict__ seq_idx,
    const int32_t* __restrict__ pos, const float* __restrict__ rcos,
    const float* __restrict__ rsin, int max_pos,
    const int32_t* __restrict__ block_table, int max_blocks, int block_size,
    T* __restrict__ cache) {
  scatter_row<T>(acc, nparts, part_stride, d_c + d_r, blockIdx.x,
                 blockIdx.y * blockDim.x + threadIdx.x, gridDim.y * blockDim.x,
                 d_c, d_r, seq_idx, pos, rcos, rsin, max_pos, block_table,
                 max_blocks, block_size, cache);
}

template <typename T>
__global__ void query_rope_kernel(const float* __restrict__ qr, int nparts,
                                  long part_stride, long ld_qr,
                                  int n_h, int d_c, int d_r,
                                  const int32_t* __restrict__ pos,
                                  const float* __restrict__ rcos,
                                  const float* __restrict__ rsin, int max_pos,
                                  T* __restrict__ q_out) {
  const int t = blockIdx.x;
  const int half = d_r / 2;
  const int p = pos[t];
  const float* src = qr + (long)t * ld_qr;
  for (int i = blockIdx.y * blockDim.x + threadIdx.x; i < n_h * half;
       i += gridDim.y * blockDim.x) {
    const int h = i / half, jj = i - h * half;
    const float x1 = sum_parts(src, nparts, part_stride, h * d_r + jj);
    const float x2 = sum_parts(src, nparts, part_stride, h * d_r + jj + half);
    const bool ok = p >= 0 && p < max_pos;
    const float c = ok ? rcos[(long)p * half + jj] : NAN;
    const float s = ok ? rsin[(long)p * half + jj] : NAN;
    T* dst = q_out + ((long)t * n_h + h) * (d_c + d_r) + d_c;
    DT<T>::store(dst, jj, x1 * c - x2 * s);
    DT<T>::store(dst, jj + half, x1 * s + x2 * c);
  }
}

template <typename T>
// Source row r sits at (r / grp) * lds_grp + (r % grp) * lds: groups of grp
// rows, lds apart inside a group and lds_grp between groups.
__global__ void convert_kernel(const float* __restrict__ src, long lds,
                               int grp, long lds_grp, int nparts,
                               long part_stride, int rows, int cols,
                               T* __restrict__ dst, long ldd) {
  const long n = (long)rows * cols;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n;
       i += (long)gridDim.x * blockDim.x) {
    const long r = i / cols, c = i - r * cols;
    const long g = r / grp;
    DT<T>::store(dst, r * ldd + c,
                 sum_parts(src, nparts, part_stride,
                           g * lds_grp + (r - g * grp) * lds + c));
  }
}

inline int grid_for(long n, int threads) {
  long g = (n + threads - 1) / threads;
  return (int)(g < 8192 ? (g < 1 ? 1 : g) : 8192);
}

}  // namespace

// Value i of rows of `cols` values (cols % 8 == 0), summed from rows ld_src
// apart: hi to 16 (i / 8) + i % 8 (bf16 units), lo 8 further.
__device__ __forceinline__ void reduce_hl_item(const float* __restrict__ src,
                                               int nparts, long part_stride,
                                               long ld_src, int cols, long i,
                                               uint16_t* __restrict__ dst) {
  const long r = i / cols;
  const float x = sum_parts(src, nparts, part_stride, i + r * (ld_src - cols));
  const uint16_t hi = f2bf(x);
  const long at = 16 * (i >> 3) + (i & 7);
  dst[at] = hi;
  dst[at + 8] = f2bf(x - bf2f(hi));
}

// One thread per value.
__global__ void reduce_parts_hl_kernel(const float* __restrict__ src,
                                       int nparts, long part_stride, long n,
                                       int cols, uint16_t* __restrict__ dst) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n;
       i += (long)gridDim.x * blockDim.x)
    reduce_hl_item(src, nparts, part_stride, cols, cols, i, dst);
}

// The epilogue of the stacked down-projection [W_DQ; W_DKV; W_KR] h of a
// decode batch, one launch for both consumers of its K parts (rows of
// ld_acc = d_cq + d_c + d_r floats): workgroups below nq_blocks write c_Q
// (the first d_cq columns) in the pre-split hi|lo layout, the next
// T * nsl workgroups the cache rows (the other columns, RoPE on k_R), nsl
// slices of 256 items per token, one item per thread (every item is a sum
// over the K parts, a chain of dependent loads: one per thread keeps the
// chains short).
template <typename T>
__global__ __launch_bounds__(256) void project_epilogue_kernel(
    const float* __restrict__ acc, int nparts, long part_stride, int d_cq,
    int ntok, int nq_blocks, int nsl, uint16_t* __restrict__ cq, int d_c,
    int d_r,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const float* __restrict__ rcos, const float* __restrict__ rsin,
    int max_pos, const int32_t* __restrict__ block_table, int max_blocks,
    int block_size, T* __restrict__ cache) {
  const long ld_acc = (long)d_cq + d_c + d_r;
  if ((int)blockIdx.x < nq_blocks) {
    const long n = (long)ntok * d_cq;
    for (long i = blockIdx.x * 256L + threadIdx.x; i < n;
         i += (long)nq_blocks * 256)
      reduce_hl_item(acc, nparts, part_stride, ld_acc, d_cq, i, cq);
    return;
  }
  const int w = (int)blockIdx.x - nq_blocks;
  const int t = w / nsl;
  scatter_row<T>(acc + d_cq, nparts, part_stride, ld_acc, t,
                 (w - t * nsl) * 256 + threadIdx.x, nsl * 256, d_c, d_r,
                 seq_idx, pos, rcos, rsin, max_pos, block_table, max_blocks,
                 block_size, cache);
}

hipError_t launch_reduce_parts_hl(const float* src, int nparts,
                                  long part_stride, long n, int ld, void* dst,
                                  hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (ld % 8 != 0 || n % ld != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reduce_parts_hl_kernel, dim3(grid_for(n, 256)),
                     dim3(256), 0, stream, src, nparts, part_stride, n, ld,
                     (uint16_t*)dst);
  return hipGetLastError();
}

hipError_t launch_project_epilogue(const mla_dims& d, int T, const float* acc,
                                   int nparts, long part_stride, void* cq,
                                   const int32_t* seq_idx, const int32_t* pos,
                                   const float* rope_cos,
                                   const float* rope_sin, int max_pos,
                                   const int32_t* block_table, int max_blocks,
                                   void* cache, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  // bf16 layers (the pre-split c_Q feeds the weight-streaming kernel)
  if (d.dtype != MLA_BF16 || d.d_cq % 8 != 0) return hipErrorInvalidValue;
  const int nq = grid_for((long)T * d.d_cq, 256);
  const int nsl = (d.d_c + d.d_r / 2 + 255) / 256;
  hipLaunchKernelGGL(project_epilogue_kernel<uint16_t>, dim3(nq + T * nsl),
                     dim3(256), 0, stream, acc, nparts, part_stride, d.d_cq,
                     T, nq, nsl, (uint16_t*)cq, d.d_c, d.d_r, seq_idx, pos,
                     rope_cos, rope_sin, max_pos, block_table, max_blocks,
                     d.block_size, (uint16_t*)cache);
  return hipGetLastError();
}

hipError_t launch_reduce_parts(const float* src, int nparts, long part_stride,
                               long n, float* dst, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_parts_kernel, dim3(grid_for(n, 256)), dim3(256), 0,
                     stream, src, nparts, part_stride, n, dst);
  return hipGetLastError();
}

// Latent RMSNorm variant ('MiniMind 学习笔记 10', section 9: the latent
// half of the down-projection goes through kv_norm before it is cached; the
// RoPE key does not): one workgroup (4 waves) per token.  Pass 1 sums the
// squares of the d_c latent values (fp32, the K-split parts summed first),
// reduced across the workgroup; pass 2 writes
//   c_j = w_j x_j / sqrt(mean(x^2) + eps)
// rounded once to the cache dtype, and rotates the RoPE pairs as above.
template <typename T>
__global__ __launch_bounds__(256) void append_norm_scatter_kernel(
    const float* __restrict__ acc, int nparts, long part_stride, int d_c,
    int d_r, const T* __restrict__ kv_norm_w, float eps,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const float* __restrict__ rcos, const float* __restrict__ rsin,
    int max_pos, const int32_t* __restrict__ block_table, int max_blocks,
    int block_size, T* __restrict__ cache) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int width = d_c + d_r;
  const int half = d_r / 2;
  const long base = (long)t * width;
  float ss = 0.0f;
  for (int j = threadIdx.x; j < d_c; j += 256) {
    const float x = sum_parts(acc, nparts, part_stride, base + j);
    ss = __builtin_fmaf(x, x, ss);
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float inv =
      1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d_c + eps);
  const int p = pos[t];
  const int blk = block_table[(long)seq_idx[t] * max_blocks + p / block_size];
  T* row = cache + ((long)blk * block_size + (p % block_size)) * width;
  for (int j = threadIdx.x; j < d_c + half; j += 256) {
    if (j < d_c) {
      const float x = sum_parts(acc, nparts, part_stride, base + j);
      DT<T>::store(row, j, DT<T>::load(kv_norm_w, j) * (x * inv));
    } else {
      const int jj = j - d_c;
      const float x1 = sum_parts(acc, nparts, part_stride, base + d_c + jj);
      const float x2 =
          sum_parts(acc, nparts, part_stride, base + d_c + jj + half);
      const bool ok = p >= 0 && p < max_pos;
      const float c = ok ? rcos[(long)p * half + jj] : NAN;
      const float s = ok ? rsin[(long)p * half + jj] : NAN;
      DT<T>::store(row, d_c + jj, x1 * c - x2 * s);
      DT<T>::store(row, d_c + jj + half, x1 * s + x2 * c);
    }
  }
}

hipError_t launch_append_norm_scatter(const mla_dims& d, int T,
                                      const float* acc, int nparts,
                                      long part_stride, const void* kv_norm_w,
                                      float eps, const int32_t* seq_idx,
                                      const int32_t* pos,
                                      const float* rope_cos,
                                      const float* rope_sin, int max_pos,
                                      const int32_t* block_table,
                                      int max_blocks, void* cache,
                                      hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (d.dtype == MLA_BF16)
    hipLaunchKernelGGL(append_norm_scatter_kernel<uint16_t>, dim3(T),
                       dim3(256), 0, stream, acc, nparts, part_stride, d.d_c,
                       d.d_r, (const uint16_t*)kv_norm_w, eps, seq_idx, pos,
                       rope_cos, rope_sin, max_pos, block_table, max_blocks,
                       d.block_size, (uint16_t*)cache);
  else
    hipLaunchKernelGGL(append_norm_scatter_kernel<float>, dim3(T), dim3(256),
                       0, stream, acc, nparts, part_stride, d.d_c, d.d_r,
                       (const float*)kv_norm_w, eps, seq_idx, pos, rope_cos,
                       rope_sin, max_pos, block_table, max_blocks,
                       d.block_size, (float*)cache);
  return hipGetLastError();
}

hipError_t launch_append_scatter(const mla_dims& d, int T, const float* acc,
                                 int nparts, long part_stride,
                                 const int32_t* seq_idx, const int32_t* pos,
                                 const float* rope_cos, const float* rope_sin,
                                 int max_pos, const int32_t* block_table,
                                 int max_blocks, void* cache,
                                 hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const dim3 grid(T, (d.d_c + d.d_r / 2 + 255) / 256);
  if (d.dtype == MLA_BF16)
    hipLaunchKernelGGL(append_scatter_kernel<uint16_t>, grid, dim3(256), 0,
                       stream, acc, nparts, part_stride, d.d_c, d.d_r, seq_idx,
                       pos, rope_cos, rope_sin, max_pos, block_table,
                       max_blocks, d.block_size, (uint16_t*)cache);
  else
    hipLaunchKernelGGL(append_scatter_kernel<float>, grid, dim3(256), 0,
                       stream, acc, nparts, part_stride, d.d_c, d.d_r, seq_idx,
                       pos, rope_cos, rope_sin, max_pos, block_table,
                       max_blocks, d.block_size, (float*)cache);
  return hipGetLastError();
}

hipError_t launch_query_rope(const mla_dims& d, int T, const float* qr,
                             int nparts, long part_stride, long ld_qr,
                             const int32_t* pos, const float* rope_cos,
                             const float* rope_sin, int max_pos, void* q_out,
                             hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const dim3 grid(T, (d.n_h * (d.d_r / 2) + 255) / 256);
  if (d.dtype == MLA_BF16)
    hipLaunchKernelGGL(query_rope_kernel<uint16_t>, grid, dim3(256), 0,
                       stream, qr, nparts, part_stride, ld_qr, d.n_h, d.d_c,
                       d.d_r, pos, rope_cos, rope_sin, max_pos,
                       (uint16_t*)q_out);
  else
    hipLaunchKernelGGL(query_rope_kernel<float>, grid, dim3(256), 0,
                       stream, qr, nparts, part_stride, ld_qr, d.n_h, d.d_c,
                       d.d_r, pos, rope_cos, rope_sin, max_pos,
                       (float*)q_out);
  return hipGetLastError();
}

hipError_t launch_convert(const mla_dims& d, int rows, int cols,
                          const float* src, long lds, int nparts,
                          long part_stride, void* dst, long ldd,
                          hipStream_t stream, int grp, long lds_grp) {
  const long n = (long)rows * cols;
  if (n <= 0) return hipSuccess;
  if (grp <= 0) {
    grp = rows;
    lds_grp = 0;
  }
  if (d.dtype == MLA_BF16)
    hipLaunchKernelGGL(convert_kernel<uint16_t>, dim3(grid_for(n, 256)),
                       dim3(256), 0, stream, src, lds, grp, lds_grp, nparts,
                       part_stride, rows, cols, (uint16_t*)dst, ldd);
  else
    hipLaunchKernelGGL(convert_kernel<float>, dim3(grid_for(n, 256)),
                       dim3(256), 0, stream, src, lds, grp, lds_grp, nparts,
                       part_stride, rows, cols, (float*)dst, ldd);
  return hipGetLastError();
}

}  // namespace mla
