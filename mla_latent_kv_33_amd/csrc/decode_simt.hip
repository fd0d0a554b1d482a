// General split-KV latent decode (any d_c, d_r, block size; fp32 or bf16)
// and the split combine shared by both decode kernels.
//
// Same computation as the matrix-core kernel ('MLA：潜在表示压缩与解耦 RoPE',
// sections 4, 6 and 7): per (sequence, query, head, split), scores against
// the shared cache rows, an online softmax in base 2 and the weighted sum of
// the c_KV columns.  One workgroup handles one head; its threads score one
// key each per round, then share the weights through LDS to accumulate the
// d_c output columns.  Used for dims the matrix-core kernel does not cover
// (including fp32 layers).
//
// Combine: for splits j with states (acc_j, m_j, l_j) in log2 units,
//   M = max_j m_j,  w_j = 2^(m_j - M),  o = sum_j w_j acc_j / sum_j w_j l_j,
//   lse = (M + log2 sum_j w_j l_j) * ln 2.
// Splits with no keys carry m = -inf and are skipped.

#include "mla_common.hpp"
#include "mla_kernels.hpp"

namespace mla {
namespace {

constexpr int NT = 128;

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename T>
__global__ __launch_bounds__(NT) void decode_simt_kernel(
    const T* __restrict__ q, const T* __restrict__ cache,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ kv_lens, int n_q, int n_h, int d_c, int d_r,
    int bs, int n_split, float scale_log2,
    float* __restrict__ o_part, float* __restrict__ m_part,
    float* __restrict__ l_part, float* __restrict__ o_final,
    float* __restrict__ lse_final) {
  extern __shared__ float sh[];
  const int width = d_c + d_r;
  float* qs = sh;             // [width]
  float* acc = qs + width;    // [d_c]
  float* ps = acc + d_c;      // [NT]
  int* rows = (int*)(ps + NT);  // [NT] cache row index of each key
  __shared__ float red[NT / 64];

  const int tid = threadIdx.x;
  const int bq = blockIdx.x, split = blockIdx.y, h = blockIdx.z;
  const int b = bq / n_q, qi = bq - b * n_q;
  const int visible = kv_lens[b] - n_q + qi + 1;
  // Split j covers blocks [j nblk / n_split, (j + 1) nblk / n_split).
  const int nblk = (visible + bs - 1) / bs;
  const int tok0 = (int)((long)split * nblk / n_split) * bs;
  const int tok1 = min(visible, (int)((long)(split + 1) * nblk / n_split) * bs);
  const size_t row_id = ((size_t)bq * n_split + split) * n_h + h;
  if (tok0 >= tok1) {
    // No visible key (an empty split, or kv_len < n_q): weight zero in the
    // combine.  With one split there are no partials; the row's output is
    // written as zeros with lse = -inf instead.
    if (n_split == 1) {
      float* dst = o_final + ((size_t)bq * n_h + h) * d_c;
      for (int j = tid; j < d_c; j += NT) dst[j] = 0.0f;
      if (tid == 0 && lse_final) lse_final[(size_t)bq * n_h + h] = -INFINITY;
    } else if (tid == 0) {
      m_part[row_id] = -INFINITY;
      l_part[row_id] = 0.0f;
    }
    return;
  }
  const T* qrow = q + ((size_t)bq * n_h + h) * width;
  for (int k = tid; k < width; k += NT) qs[k] = DT<T>::load(qrow, k);
  for (int j = tid; j < d_c; j += NT) acc[j] = 0.0f;
  const int32_t* bt = block_table + (size_t)b * max_blocks;
  float m_run = -INFINITY, l_run = 0.0f;
  __syncthreads();

  for (int start = tok0; start < tok1; start += NT) {
    const int t = start + tid;
    float s = -INFINITY;
    if (t < tok1) {
      const int r = bt[t / bs] * bs + (t % bs);
      rows[tid] = r;
      const T* kr = cache + (size_t)r * width;
      float dot = 0.0f;
      for (int k = 0; k < width; ++k) dot = fmaf(qs[k], DT<T>::load(kr, k), dot);
      s = dot * scale_log2;
    }
    float cmax = wave_max(s);
    if ((tid & 63) == 0) red[tid >> 6] = cmax;
    __syncthreads();
    cmax = red[0];
    for (int w = 1; w < NT / 64; ++w) cmax = fmaxf(cmax, red[w]);
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = exp2f(m_run - m_new);
    const float p = t < tok1 ? exp2f(s - m_new) : 0.0f;
    ps[tid] = p;
    __syncthreads();  // red[] reads done, ps/rows visible
    float psum = wave_sum(p);
    if ((tid & 63) == 0) red[tid >> 6] = psum;
    __syncthreads();
    psum = 0.0f;
    for (int w = 0; w < NT / 64; ++w) psum += red[w];
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const int cnt = min(NT, tok1 - start);
    for (int j = tid; j < d_c; j += NT) {
      float a = acc[j] * alpha;
      for (int u = 0; u < cnt; ++u)
        a = fmaf(ps[u], DT<T>::load(cache + (size_t)rows[u] * width, j), a);
      acc[j] = a;
    }
    __syncthreads();
  }

  if (n_split == 1) {
    float* dst = o_final + ((size_t)bq * n_h + h) * d_c;
    const float inv = 1.0f / l_run;
    for (int j = tid; j < d_c; j += NT) dst[j] = acc[j] * inv;
    if (tid == 0 && lse_final)
      lse_final[(size_t)bq * n_h + h] =
          (m_run + log2f(l_run)) * 0.69314718055994531f;
  } else {
    float* dst = o_part + row_id * d_c;
    for (int j = tid; j < d_c; j += NT) dst[j] = acc[j];
    if (tid == 0) {
      m_part[row_id] = m_run;
      l_part[row_id] = l_run;
    }
  }
}

// One workgroup per (row, head); threads over the d_c columns.
// Split combine ('MLA：潜在表示压缩与解耦 RoPE', section 7: the softmax over
// the whole key range from per-split maxima and sums).  For each head,
// M = max_j m_j, w_j = 2^(m_j - M) (0 for an empty split, m_j = -inf),
// L = sum_j w_j l_j, o_lat = sum_j w_j o_j / L, lse = (M + log2 L) ln 2.
//
// combine_rows_kernel (d_c a multiple of 4, at most 512 wide; with fp16
// partials a multiple of 8): workgroup = (query row, 16 heads), 16 threads
// per head, thread q of a head owning the column vectors q, q + 16, ...
// (NB of them; 4 fp32 columns, or 8 fp16 columns for fp16 partials).  Every
// thread loads the m and l of its head with its partial columns, CS splits
// at a time, so the workgroup has no barrier and one round of load latency
// per split chunk; the chunks merge online (running maximum, earlier sums
// rescaled).  An empty split never wrote its partial, so its columns enter
// through a select on w = 0, never a product.
//
// fp32 partials hold the unnormalised O_j (weight w_j); fp16 partials hold
// O_j / (l_j s_j) with s_j the row's scale stored after the fp16 rows
// (weight w_j l_j s_j), as the matrix-core decode writes them.
// Shapes: TPH = 16 threads per head and CS = 4 splits per chunk for many
// query rows.  For few rows (a grid of a few dozen workgroups) TPH = 64,
// CS = 16 and SG = 4 split groups: a head takes the whole workgroup, each
// group of 64 threads merges its own quarter of the splits (one round of
// loads for up to 64 splits), and group 0 merges the four partial results
// through LDS with the same formula.
template <int NB, bool P16, int TPH, int CS, int SG = 1, int CSPL = 1>
__global__ __launch_bounds__(256) void combine_rows_kernel(
    int n_h, int d_c, int n_split, int slots, const int2* __restrict__ plan,
    const float* __restrict__ o_part, const float* __restrict__ m_part,
    const float* __restrict__ l_part, float* __restrict__ o_lat,
    float* __restrict__ lse) {
  constexpr int VW = P16 ? 8 : 4;  // columns per vector
  constexpr int HPW = 256 / (TPH * SG);  // heads per workgroup
  static_assert(HPW >= 1 && HPW * TPH * SG == 256, "thread split");
  const int bq = blockIdx.x;
  const int hl = threadIdx.x / (TPH * SG);
  const int sg = (threadIdx.x / TPH) % SG;
  const int h = blockIdx.y * HPW + hl;
  const int q = threadIdx.x % TPH;
  // (with SG > 1 the grid has exactly n_h / HPW columns: no thread leaves
  // before the barrier below)
  if (SG == 1 && h >= n_h) return;
  // the row's splits: slots slot0 .. slot0 + n_split - 1 (balanced plan, or
  // n_split per row)
  int slot0 = bq * n_split;
  if (plan) {
    const int2 pl = plan[bq];
    slot0 = pl.x;
    n_split = pl.y;
    if (n_split == 1) return;  // written final by the decode
  }
  // this workgroup's column vectors: cv0 .. cv0 + cvn - 1 (part
  // blockIdx.z of CSPL)
  const int cvn = d_c / VW / CSPL;
  const int cv0 = CSPL > 1 ? (int)blockIdx.z * cvn : 0;
  const size_t row0 = (size_t)slot0 * n_h + h;  // + j n_h
  const uint16_t* const p16 = (const uint16_t*)o_part;
  const float* const sc_part =
      (const float*)(p16 + (size_t)slots * n_h * d_c);
  float M = -INFINITY, L = 0.0f;
  f32x4 acc[NB][VW / 4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int hh = 0; hh < VW / 4; ++hh)
      acc[b][hh] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  // this group's splits: [j_lo, j_hi)
  const int per = (n_split + SG - 1) / SG;
  const int j_lo = min(sg * per, n_split);
  const int j_hi = min(j_lo + per, n_split);
  for (int j0 = j_lo; j0 < j_hi; j0 += CS) {
    float m[CS], l[CS], ps[CS];
    f32x4 v[CS][NB][VW / 4];
    // Every load is issued unconditionally from an in-range address (split
    // and column clamped) and masked afterwards, so that all of them are in
    // flight together: a load under a condition becomes a branch that waits
    // for it on the spot.
    uint4 raw[CS][NB];
    f32x4 rawf[CS][NB];
#pragma unroll
    for (int u = 0; u < CS; ++u) {
      const size_t r = row0 + (size_t)min(j0 + u, j_hi - 1) * n_h;
      m[u] = m_part[r];
      l[u] = l_part[r];
      ps[u] = P16 ? sc_part[r] : 1.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int cv = cv0 + min(q + TPH * b, cvn - 1);
        if (P16)
          raw[u][b] = *(const uint4*)(p16 + r * d_c + 8 * cv);
        else
          rawf[u][b] = *(const f32x4*)(o_part + r * d_c + 4 * cv);
      }
    }
#pragma unroll
    for (int u = 0; u < CS; ++u) {
      const bool ok = j0 + u < j_hi;
      m[u] = ok ? m[u] : -INFINITY;
      l[u] = ok ? l[u] : 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const bool in = ok && q + TPH * b < cvn;
        if (P16) {
          const f32x8 f = __builtin_convertvector(
              __builtin_bit_cast(f16x8, raw[u][b]), f32x8);
#pragma unroll
          for (int hh = 0; hh < VW / 4; ++hh)
            v[u][b][hh] = in ? (f32x4){f[4 * hh], f[4 * hh + 1],
                                       f[4 * hh + 2], f[4 * hh + 3]}
                             : (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        } else {
          v[u][b][0] = in ? rawf[u][b] : (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        }
      }
    }
    float mc = M;
#pragma unroll
    for (int u = 0; u < CS; ++u) mc = fmaxf(mc, m[u]);
    if (mc == -INFINITY) continue;  // only empty splits so far
    const float sc = M == -INFINITY ? 0.0f : exp2f(M - mc);
    L *= sc;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int hh = 0; hh < VW / 4; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[b][hh][e] *= sc;
#pragma unroll
    for (int u = 0; u < CS; ++u) {
      const bool live = m[u] != -INFINITY;
      const float w = live ? exp2f(m[u] - mc) : 0.0f;
      const float wl = w * l[u];
      L += live ? wl : 0.0f;
      const float wv = P16 ? wl * ps[u] : w;  // weight of the stored partial
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int hh = 0; hh < VW / 4; ++hh)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[b][hh][e] =
                live ? __builtin_fmaf(wv, v[u][b][hh][e], acc[b][hh][e])
                     : acc[b][hh][e];
    }
    M = mc;
  }
  if constexpr (SG > 1) {
    // groups 1 .. SG-1 hand (M, L, columns) to group 0, which merges them
    // as one more chunk of splits (a group without splits has M = -inf)
    __shared__ float sm_ml[HPW][SG][2];
    __shared__ f32x4 sm_acc[HPW][SG][TPH][NB * VW / 4];
    if (sg > 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int hh = 0; hh < VW / 4; ++hh)
          sm_acc[hl][sg][q][b * (VW / 4) + hh] = acc[b][hh];
      if (q == 0) {
        sm_ml[hl][sg][0] = M;
        sm_ml[hl][sg][1] = L;
      }
    }
    __syncthreads();
    if (sg > 0) return;
    float mc = M;
#pragma unroll
    for (int g2 = 1; g2 < SG; ++g2) mc = fmaxf(mc, sm_ml[hl][g2][0]);
    const float sc = M == -INFINITY ? 0.0f : exp2f(M - mc);
    L *= sc;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int hh = 0; hh < VW / 4; ++hh) acc[b][hh] *= sc;
#pragma unroll
    for (int g2 = 1; g2 < SG; ++g2) {
      const float mg = sm_ml[hl][g2][0];
      const bool live = mg != -INFINITY;
      const float w = live ? exp2f(mg - mc) : 0.0f;
      L += live ? w * sm_ml[hl][g2][1] : 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int hh = 0; hh < VW / 4; ++hh) {
          const f32x4 a = sm_acc[hl][g2][q][b * (VW / 4) + hh];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[b][hh][e] =
                live ? __builtin_fmaf(w, a[e], acc[b][hh][e]) : acc[b][hh][e];
        }
    }
    M = mc;
  }
  const float il = 1.0f / L;
  float* dst = o_lat + ((size_t)bq * n_h + h) * d_c;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int cv = q + TPH * b;
    if (cv < cvn)
#pragma unroll
      for (int hh = 0; hh < VW / 4; ++hh)
        *(f32x4*)(dst + VW * (cv0 + cv) + 4 * hh) =
            (f32x4){acc[b][hh][0] * il, acc[b][hh][1] * il,
                    acc[b][hh][2] * il, acc[b][hh][3] * il};
  }
  if (q == 0 && lse && (CSPL == 1 || blockIdx.z == 0))
    lse[(size_t)bq * n_h + h] = (M + log2f(L)) * 0.69314718055994531f;
}

// Other widths: workgroup = (query row, ch heads).  The weights of its
// heads are computed in parallel (one thread per head), then each thread
// owns CB float4 columns and reads their partials CMB_CS splits at a time.
// Splits of weight 0 are not read: an empty split never wrote its partial.
constexpr int CMB_CH = 16, CMB_CB = 8, CMB_CS = 4;
constexpr size_t CMB_LDS_MAX = 160 * 1024;

__global__ __launch_bounds__(256) void combine_kernel(
    int n_h, int d_c, int n_split, int ch, const float* __restrict__ o_part,
    const float* __restrict__ m_part, const float* __restrict__ l_part,
    float* __restrict__ o_lat, float* __restrict__ lse) {
  extern __shared__ float wsh[];  // [ch][n_split] weights, [ch] 1/L
  float* inv_l = wsh + ch * n_split;
  const int bq = blockIdx.x;
  const int h0 = blockIdx.y * ch;
  const int nh = min(ch, n_h - h0);
  const size_t rows = (size_t)bq * n_split * n_h + h0;  // + j n_h + h
  // weights: one thread per head
  for (int h = threadIdx.x; h < nh; h += blockDim.x) {
    float M = -INFINITY;
    for (int j = 0; j < n_split; ++j)
      M = fmaxf(M, m_part[rows + (size_t)j * n_h + h]);
    float L = 0.0f;
    for (int j = 0; j < n_split; ++j) {
      const float m = m_part[rows + (size_t)j * n_h + h];
      const float w = m == -INFINITY ? 0.0f : exp2f(m - M);
      wsh[h * n_split + j] = w;
      L += w * l_part[rows + (size_t)j * n_h + h];
    }
    inv_l[h] = 1.0f / L;
    if (lse)
      lse[(size_t)bq * n_h + h0 + h] = (M + log2f(L)) * 0.69314718055994531f;
  }
  __syncthreads();
  if (d_c % 4) {  // rows not float4-aligned: plain loop
    for (int idx = threadIdx.x; idx < nh * d_c; idx += blockDim.x) {
      const int h = idx / d_c, c = idx - h * d_c;
      float acc = 0.0f;
      for (int j = 0; j < n_split; ++j) {
        const float w = wsh[h * n_split + j];
        if (w != 0.0f)
          acc += w * o_part[(rows + (size_t)j * n_h + h) * d_c + c];
      }
      o_lat[((size_t)bq * n_h + h0 + h) * d_c + c] = acc * inv_l[h];
    }
    return;
  }
  const int c4n = d_c / 4;
  const int total = nh * c4n;
  for (int base = threadIdx.x; base < total; base += blockDim.x * CMB_CB) {
    f32x4 acc[CMB_CB];
#pragma unroll
    for (int b = 0; b < CMB_CB; ++b) acc[b] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    for (int j0 = 0; j0 < n_split; j0 += CMB_CS) {
      f32x4 v[CMB_CS][CMB_CB];
      float w[CMB_CS][CMB_CB];
#pragma unroll
      for (int u = 0; u < CMB_CS; ++u)
#pragma unroll
        for (int b = 0; b < CMB_CB; ++b) {
          const int idx = base + b * blockDim.x;
          const int h = idx / c4n, c4 = idx - h * c4n;
          const int j = j0 + u;
          w[u][b] = (j < n_split && idx < total) ? wsh[h * n_split + j] : 0.0f;
          v[u][b] = w[u][b] != 0.0f
                        ? *(const f32x4*)(o_part +
                                          (rows + (size_t)j * n_h + h) * d_c +
                                          4 * c4)
                        : (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
      for (int u = 0; u < CMB_CS; ++u)
#pragma unroll
        for (int b = 0; b < CMB_CB; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[b][e] += w[u][b] * v[u][b][e];
    }
#pragma unroll
    for (int b = 0; b < CMB_CB; ++b) {
      const int idx = base + b * blockDim.x;
      if (idx < total) {
        const int h = idx / c4n, c4 = idx - h * c4n;
        const float il = inv_l[h];
        *(f32x4*)(o_lat + ((size_t)bq * n_h + h0 + h) * d_c + 4 * c4) =
            (f32x4){acc[b][0] * il, acc[b][1] * il, acc[b][2] * il,
                    acc[b][3] * il};
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_simt(const mla_dims& d, int B, int n_q,
                              const void* q, const void* cache,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* kv_lens, int n_split,
                              float* o_part, float* m_part,
                              float* l_part, float* o_final, float* lse_final,
                              hipStream_t stream) {
  const float scale_log2 =
      (float)(1.4426950408889634 / __builtin_sqrt((double)(d.d_h + d.d_r)));
  const size_t lds = (size_t)(d.d_c + d.d_r + d.d_c + NT) * sizeof(float) +
                     NT * sizeof(int);
  dim3 grid(B * n_q, n_split, d.n_h);
  if (d.dtype == MLA_BF16)
    hipLaunchKernelGGL(decode_simt_kernel<uint16_t>, grid, dim3(NT), lds,
                       stream, (const uint16_t*)q, (const uint16_t*)cache,
                       block_table, max_blocks, kv_lens, n_q, d.n_h, d.d_c,
                       d.d_r, d.block_size, n_split, scale_log2, o_part,
                       m_part, l_part, o_final, lse_final);
  else
    hipLaunchKernelGGL(decode_simt_kernel<float>, grid, dim3(NT), lds, stream,
                       (const float*)q, (const float*)cache, block_table,
                       max_blocks, kv_lens, n_q, d.n_h, d.d_c, d.d_r,
                       d.block_size, n_split, scale_log2, o_part, m_part,
                       l_part, o_final, lse_final);
  return hipGetLastError();
}

hipError_t launch_combine(const mla_dims& d, int rows, int n_split,
                          const float* o_part, bool f16_parts,
                          const float* m_part, const float* l_part,
                          float* o_lat, float* lse, hipStream_t stream,
                          const int2* plan, int slots) {
  if (rows <= 0) return hipSuccess;
  if (plan && !f16_parts) return hipErrorInvalidValue;
  if (!plan) slots = rows * n_split;
  // Many rows: 16 threads per head (16 heads per workgroup), 4 splits per
  // chunk.  Few rows: one head per workgroup in four split groups of 64
  // threads, 16 splits per chunk, so that a small batch still spreads over
  // hundreds of waves and up to 64 splits take one round of loads.
  const bool wide = (long)rows * ((d.n_h + 15) / 16) < 256;
#define MLA_CMB(NB, P16, TPH, CS)                                             \
  hipLaunchKernelGGL((combine_rows_kernel<NB, P16, TPH, CS>),                  \
                     dim3(rows, (d.n_h + 256 / TPH - 1) / (256 / TPH)),        \
                     dim3(256), 0, stream, d.n_h, d.d_c, n_split, slots,      \
                     plan, o_part, m_part, l_part, o_lat, lse)
  if (f16_parts) {
    if (d.d_c % 8 != 0 || d.d_c > 8 * 16 * 4) return hipErrorInvalidValue;
    if (wide && (long)rows * d.n_h < 256 && d.d_c % 16 == 0) {
      // fewer (row, head) pairs than compute units (one sequence): each
      // head's columns in two workgroups of eight split groups (32 threads
      // x 8 columns cover half of d_c <= 512), so that the grid fills the
      // chip (B = 1: 6.1 -> 5.1 us)
      hipLaunchKernelGGL((combine_rows_kernel<1, true, 32, 8, 8, 2>),
                         dim3(rows, d.n_h, 2), dim3(256), 0, stream, d.n_h,
                         d.d_c, n_split, slots, plan, o_part, m_part, l_part,
                         o_lat, lse);
    } else if (wide) {
      // one head per workgroup (64 threads x 8 columns cover d_c <= 512),
      // four split groups
      hipLaunchKernelGGL((combine_rows_kernel<1, true, 64, 16, 4>),
                         dim3(rows, d.n_h), dim3(256), 0, stream, d.n_h,
                         d.d_c, n_split, slots, plan, o_part, m_part, l_part,
                         o_lat, lse);
    } else
      MLA_CMB(4, true, 16, 4);
    return hipGetLastError();
  }
  if (d.d_c % 4 == 0 && d.d_c <= 4 * 16 * 8) {
    const int c4n = d.d_c / 4;
    const int nb = (c4n + 15) / 16;
    if (nb <= 1)
      MLA_CMB(1, false, 16, 4);
    else if (nb <= 2)
      MLA_CMB(2, false, 16, 4);
    else if (nb <= 4)
      MLA_CMB(4, false, 16, 4);
    else
      MLA_CMB(8, false, 16, 4);
    return hipGetLastError();
  }
#undef MLA_CMB
  static std::atomic<unsigned long long> lds_set{0};
  {
    const hipError_t e = set_lds_limit_once((const void*)combine_kernel,
                                            (int)CMB_LDS_MAX, lds_set);
    if (e != hipSuccess) return e;
  }
  // heads per workgroup: their weights must fit the LDS
  const size_t per_head = (size_t)(n_split + 1) * sizeof(float);
  int ch = (int)(CMB_LDS_MAX / per_head);
  if (ch > CMB_CH) ch = CMB_CH;
  if (ch < 1) return hipErrorInvalidValue;
  dim3 grid(rows, (d.n_h + ch - 1) / ch);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), ch * per_head, stream,
                     d.n_h, d.d_c, n_split, ch, o_part, m_part, l_part, o_lat,
                     lse);
  return hipGetLastError();
}

}  // namespace mla
