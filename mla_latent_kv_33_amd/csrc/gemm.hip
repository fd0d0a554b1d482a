// C = A . B^T for the projections of the MLA layer (W_DKV, W_KR, W_DQ, W_UQ,
// W_QR, W_UK, W_UV, W_O).  Layouts follow a PyTorch Linear: B is the weight,
// [N][K] row-major ("NT"); W_UK enters the absorption as [K][N] ("NN").
//
// bf16 layers run on the matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulate).  Activations that are kept in fp32 between steps (c_Q, q_C,
// o_lat, v) enter the MFMA as a pair of bf16 values hi + lo with
// hi = bf16(x), lo = bf16(x - hi), i.e. two MFMAs per fragment; this keeps
// those intermediates at ~16 significant bits instead of 8.
//
// Two kernels:
//   * skinny (M <= 64, NT): decode batches.  The weight stream dominates, so
//     B fragments are loaded straight from HBM into registers in MFMA
//     layout; the four waves of a workgroup interleave their 16-wide k-steps
//     so that together they read each weight row in 128-byte runs, and sum
//     their partial tiles through LDS.  Workgroups may further split K; each
//     K chunk writes its own partial C (summed by the consumer), which keeps
//     results deterministic.
//   * tiled (any M, NT or NN): 128x128x32 tiles staged through padded LDS,
//     2x2 waves of 64x64; NN weights are read with ds_read_b64_tr_b16 so the
//     MFMA still sees k-contiguous B fragments.
// fp32 layers use a plain SIMT kernel (small shapes only).

#include "mla_common.hpp"
#include "mla_kernels.hpp"

namespace mla {
namespace {

__device__ __forceinline__ void split_hi_lo(const float* x, bf16x8& hi,
                                            bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t h0 = f2bf(x[2 * e]), h1 = f2bf(x[2 * e + 1]);
    h[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[e] = pack_bf2(x[2 * e] - bf2f(h0), x[2 * e + 1] - bf2f(h1));
  }
  hi = __builtin_bit_cast(bf16x8, (u32x4){h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, (u32x4){l[0], l[1], l[2], l[3]});
}

// Guarded 8-element loads along k (zero outside [0, K)).
__device__ __forceinline__ bf16x8 load8_bf16(const uint16_t* row, int k,
                                             int K, bool row_ok) {
  if (row_ok && k + 8 <= K) return *(const bf16x8*)(row + k);
  uint32_t w[4] = {0, 0, 0, 0};
  if (row_ok)
    for (int e = 0; e < 8; ++e)
      if (k + e < K) w[e >> 1] |= (uint32_t)row[k + e] << (16 * (e & 1));
  return __builtin_bit_cast(bf16x8, (u32x4){w[0], w[1], w[2], w[3]});
}
__device__ __forceinline__ void load8_f32(const float* row, int k, int K,
                                          bool row_ok, float* x) {
  if (row_ok && k + 8 <= K) {
    const f32x4 a = *(const f32x4*)(row + k);
    const f32x4 b = *(const f32x4*)(row + k + 4);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
    return;
  }
  for (int e = 0; e < 8; ++e) x[e] = (row_ok && k + e < K) ? row[k + e] : 0.0f;
}

// B row n of a possibly two-part weight: rows < nb1 from B, others from B2.
__device__ __forceinline__ const uint16_t* brow(const uint16_t* B,
                                                const uint16_t* B2, int nb1,
                                                long ldb, int n) {
  return n < nb1 ? B + (long)n * ldb : B2 + (long)(n - nb1) * ldb;
}

// ---------------------------------------------------------------- skinny
constexpr int SK_WAVES = 4;
constexpr int SK_UNROLL = 4;

template <int MT, bool AF32>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(
    const void* __restrict__ Av, long lda, long a_bs,
    const uint16_t* __restrict__ B, const uint16_t* __restrict__ B2, int nb1,
    long ldb, long b_bs, float* __restrict__ C, long ldc, long c_bs, long c_ks,
    int M, int N, int K, int k_chunk) {
  __shared__ float red[SK_WAVES - 1][MT][16][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int col = lane & 31;
  const int n0 = blockIdx.x * 32;
  const int kz = blockIdx.y;
  const int z = blockIdx.z;
  const int kbeg = kz * k_chunk;
  const int kend = min(K, kbeg + k_chunk);

  const int n = n0 + col;
  const bool n_ok = n < N;
  const uint16_t* bz = B + z * b_bs;
  const uint16_t* b2z = B2 ? B2 + z * b_bs : nullptr;
  const uint16_t* brow_p = n_ok ? brow(bz, b2z, nb1, ldb, n) : bz;

  f32x16 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

  // wave w takes k-steps kbeg + 16 (w + 4 j)
  for (int k0 = kbeg + 16 * wave; k0 < kend; k0 += 16 * SK_WAVES * SK_UNROLL) {
    bf16x8 bf[SK_UNROLL];
#pragma unroll
    for (int u = 0; u < SK_UNROLL; ++u) {
      const int k = k0 + 16 * SK_WAVES * u + 8 * g;
      bf[u] = load8_bf16(brow_p, k, kend, n_ok && k0 + 16 * SK_WAVES * u < kend);
    }
#pragma unroll
    for (int u = 0; u < SK_UNROLL; ++u) {
      const int k = k0 + 16 * SK_WAVES * u + 8 * g;
      if (k0 + 16 * SK_WAVES * u >= kend) break;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = 32 * mt + col;
        const bool m_ok = m < M;
        if (AF32) {
          const float* ar = (const float*)Av + z * a_bs + (long)m * lda;
          float x[8];
          load8_f32(ar, k, kend, m_ok, x);
          bf16x8 hi, lo;
          split_hi_lo(x, hi, lo);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, bf[u], acc[mt],
                                                            0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, bf[u], acc[mt],
                                                            0, 0, 0);
        } else {
          const uint16_t* ar = (const uint16_t*)Av + z * a_bs + (long)m * lda;
          const bf16x8 a = load8_bf16(ar, k, kend, m_ok);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf[u], acc[mt],
                                                            0, 0, 0);
        }
      }
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave - 1][mt][r][lane] = acc[mt][r];
  }
  __syncthreads();
  if (wave == 0) {
    float* cz = C + z * c_bs + kz * c_ks;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = acc[mt][r];
#pragma unroll
        for (int w = 0; w < SK_WAVES - 1; ++w) v += red[w][mt][r][lane];
        const int m = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
        if (m < M && n_ok) cz[(long)m * ldc + n] = v;
      }
  }
}

// ----------------------------------------------------------------- tiled
constexpr int TB_M = 128, TB_N = 128, TB_K = 32;
constexpr int A_LD = TB_K + 8;     // bf16 elements per LDS row of A / NT B
constexpr int BNN_LD = TB_N + 16;  // bf16 elements per LDS row of NN B

template <bool AF32, bool BNN>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(
    const void* __restrict__ Av, long lda, long a_bs,
    const uint16_t* __restrict__ B, const uint16_t* __restrict__ B2, int nb1,
    long ldb, long b_bs, float* __restrict__ C, long ldc, long c_bs, long c_ks,
    int M, int N, int K, int k_chunk, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t a_hi[TB_M * A_LD];
  __shared__ __attribute__((aligned(16))) uint16_t a_lo[AF32 ? TB_M * A_LD : 8];
  __shared__ __attribute__((aligned(16)))
  uint16_t b_s[BNN ? TB_K * BNN_LD : TB_N * A_LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int col = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;  // 2x2 waves of 64x64
  const int tile_m = blockIdx.x / tiles_n;
  const int tile_n = blockIdx.x - tile_m * tiles_n;
  const int m0 = tile_m * TB_M, n0 = tile_n * TB_N;
  const int kz = blockIdx.y, z = blockIdx.z;
  const int kbeg = kz * k_chunk;
  const int kend = min(K, kbeg + k_chunk);

  const uint16_t* bz = B + z * b_bs;
  const uint16_t* b2z = B2 ? B2 + z * b_bs : nullptr;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // loader roles
  const int la_row = tid >> 1, la_k = (tid & 1) * 16;  // A and NT B
  const int lb_k = tid >> 3, lb_n = (tid & 7) * 16;    // NN B

  for (int k0 = kbeg; k0 < kend; k0 += TB_K) {
    // ---- global -> registers -> LDS ----
    {
      const int m = m0 + la_row;
      const bool ok = m < M;
      if (AF32) {
        const float* ar = (const float*)Av + z * a_bs + (long)m * lda;
        float x[8];
        bf16x8 hi, lo;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          load8_f32(ar, k0 + la_k + 8 * h, kend, ok, x);
          split_hi_lo(x, hi, lo);
          *(bf16x8*)&a_hi[la_row * A_LD + la_k + 8 * h] = hi;
          *(bf16x8*)&a_lo[la_row * A_LD + la_k + 8 * h] = lo;
        }
      } else {
        const uint16_t* ar = (const uint16_t*)Av + z * a_bs + (long)m * lda;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *(bf16x8*)&a_hi[la_row * A_LD + la_k + 8 * h] =
              load8_bf16(ar, k0 + la_k + 8 * h, kend, ok);
      }
    }
    if (BNN) {
      const int k = k0 + lb_k;
      const bool kok = k < kend;
      const uint16_t* br = bz + (long)k * ldb;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int nn = n0 + lb_n + 8 * h;
        bf16x8 v;
        if (kok && nn + 8 <= N) {
          v = *(const bf16x8*)(br + nn);
        } else {
          uint32_t w[4] = {0, 0, 0, 0};
          for (int e = 0; e < 8; ++e)
            if (kok && nn + e < N)
              w[e >> 1] |= (uint32_t)br[nn + e] << (16 * (e & 1));
          v = __builtin_bit_cast(bf16x8, (u32x4){w[0], w[1], w[2], w[3]});
        }
        *(bf16x8*)&b_s[lb_k * BNN_LD + lb_n + 8 * h] = v;
      }
    } else {
      const int nn = n0 + la_row;
      const bool ok = nn < N;
      const uint16_t* br = ok ? brow(bz, b2z, nb1, ldb, nn) : bz;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *(bf16x8*)&b_s[la_row * A_LD + la_k + 8 * h] =
            load8_bf16(br, k0 + la_k + 8 * h, kend, ok);
    }
    __syncthreads();

    // ---- MFMA over the 32-wide k slice: 2 k-steps ----
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[2], al[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + 32 * i + col;
        af[i] = *(const bf16x8*)&a_hi[r * A_LD + 16 * ks + 8 * g];
        if (AF32) al[i] = *(const bf16x8*)&a_lo[r * A_LD + 16 * ks + 8 * g];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (BNN) {
          // lane L of 16-lane group q gets B[k0 + j'][n] for 4 k's per read
          const int q16 = lane >> 4, s16 = lane & 15;
          const int kr = 16 * ks + 8 * (q16 >> 1) + (s16 >> 2);
          const int nc = wn * 64 + 32 * j + 16 * (q16 & 1) + 4 * (s16 & 3);
          const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (s16x4 __attribute__((address_space(3)))*)(
                  (__attribute__((address_space(3))) uint16_t*)&b_s[kr * BNN_LD + nc]));
          const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (s16x4 __attribute__((address_space(3)))*)(
                  (__attribute__((address_space(3))) uint16_t*)&b_s[(kr + 4) * BNN_LD + nc]));
          const s16x8 v = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5,
                                                  6, 7);
          bf[j] = __builtin_bit_cast(bf16x8, v);
        } else {
          const int r = wn * 64 + 32 * j + col;
          bf[j] = *(const bf16x8*)&b_s[r * A_LD + 16 * ks + 8 * g];
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j],
                                                              acc[i][j], 0, 0, 0);
          if (AF32)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                al[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  float* cz = C + z * c_bs + kz * c_ks;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        const int nn = n0 + wn * 64 + 32 * j + col;
        if (m < M && nn < N) cz[(long)m * ldc + nn] = acc[i][j][r];
      }
}

// ------------------------------------------------------------------ SIMT
__global__ void gemm_simt_kernel(const float* __restrict__ A, long lda,
                                 long a_bs, const float* __restrict__ B,
                                 const float* __restrict__ B2, int nb1,
                                 long ldb, long b_bs, int b_nn,
                                 float* __restrict__ C, long ldc, long c_bs,
                                 long c_ks, int M, int N, int K, int k_chunk) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int m = blockIdx.y;
  const int z = blockIdx.z;
  if (n >= N) return;
  const float* a = A + z * a_bs + (long)m * lda;
  const float* bz = B + z * b_bs;
  float acc = 0.0f;
  if (b_nn) {
    for (int k = 0; k < K; ++k) acc = fmaf(a[k], bz[(long)k * ldb + n], acc);
  } else {
    const float* br = n < nb1 ? bz + (long)n * ldb
                              : B2 + z * b_bs + (long)(n - nb1) * ldb;
    for (int k = 0; k < K; ++k) acc = fmaf(a[k], br[k], acc);
  }
  C[z * c_bs + (long)m * ldc + n] = acc;
}

}  // namespace

int gemm_pick_k_split(const mla_dims& d, const GemmArgs& g) {
  if (d.dtype != MLA_BF16 || g.b_nn || g.M > 64) return 1;
  // Skinny path: aim for >= ~1024 workgroups, each with >= 512 of K.
  const long tiles = (long)((g.N + 31) / 32) * g.batch;
  int ks = 1;
  while (tiles * ks < 1024 && (long)g.K / (ks * 2) >= 512) ks *= 2;
  return ks;
}

hipError_t launch_gemm(const mla_dims& d, const GemmArgs& g,
                       hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.batch <= 0) return hipSuccess;
  const int ks = g.k_split < 1 ? 1 : g.k_split;
  long k_chunk = (g.K + ks - 1) / ks;
  if (d.dtype != MLA_BF16) {
    dim3 grid((g.N + 127) / 128, g.M, g.batch);
    hipLaunchKernelGGL(gemm_simt_kernel, grid, dim3(128), 0, stream,
                       (const float*)g.A, g.lda, g.a_bs, (const float*)g.B,
                       (const float*)g.B2, g.nb1, g.ldb, g.b_bs, g.b_nn, g.C,
                       g.ldc, g.c_bs, g.c_ks, g.M, g.N, g.K, (int)g.K);
    return hipGetLastError();
  }
  const uint16_t* B = (const uint16_t*)g.B;
  const uint16_t* B2 = (const uint16_t*)g.B2;
  if (!g.b_nn && g.M <= 64) {
    k_chunk = (k_chunk + 63) / 64 * 64;
    dim3 grid((g.N + 31) / 32, ks, g.batch);
#define MLA_SK(MT, AF)                                                       \
  hipLaunchKernelGGL((gemm_skinny_kernel<MT, AF>), grid, dim3(256), 0,       \
                     stream, g.A, g.lda, g.a_bs, B, B2, g.nb1, g.ldb, g.b_bs, \
                     g.C, g.ldc, g.c_bs, g.c_ks, g.M, g.N, g.K, (int)k_chunk)
    if (g.M <= 32) {
      if (g.a_f32) MLA_SK(1, true); else MLA_SK(1, false);
    } else {
      if (g.a_f32) MLA_SK(2, true); else MLA_SK(2, false);
    }
#undef MLA_SK
    return hipGetLastError();
  }
  k_chunk = (k_chunk + TB_K - 1) / TB_K * TB_K;
  const int tiles_n = (g.N + TB_N - 1) / TB_N;
  const int tiles_m = (g.M + TB_M - 1) / TB_M;
  dim3 grid(tiles_m * tiles_n, ks, g.batch);
#define MLA_TL(AF, NN)                                                       \
  hipLaunchKernelGGL((gemm_tiled_kernel<AF, NN>), grid, dim3(256), 0, stream, \
                     g.A, g.lda, g.a_bs, B, B2, g.nb1, g.ldb, g.b_bs, g.C,    \
                     g.ldc, g.c_bs, g.c_ks, g.M, g.N, g.K, (int)k_chunk,      \
                     tiles_n)
  if (g.a_f32) {
    if (g.b_nn) MLA_TL(true, true); else MLA_TL(true, false);
  } else {
    if (g.b_nn) MLA_TL(false, true); else MLA_TL(false, false);
  }
#undef MLA_TL
  return hipGetLastError();
}

}  // namespace mla
