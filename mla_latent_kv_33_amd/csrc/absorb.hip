// Query absorption for decode batches on gfx950 matrix cores.
//
// What is computed ('MLA：潜在表示压缩与解耦 RoPE', section 6, absorbing the
// key up-projection into the query): for every query row m and head h,
//   q_lat[m, h, :] = W_UK_h^T q_C[m, h, :]
// with W_UK_h stored [d_h][d_c] (row k holds the d_c latent weights of
// query feature k), and q_C[m, h, :] the sum of the K-split parts of the
// query up-projection (fp32).  The result is rounded to bf16 into the first
// d_c columns of the head's query row.  The same launch rotates the head's
// decoupled RoPE query (section 5: q_R = RoPE(W_QR c_Q), half-split pairs
// (j, j + d_r / 2) at angle pos theta_j from the cos / sin tables) into the
// last d_r columns: the workgroups of a head share its query rows, after
// their MFMA work.
//
// Shape this kernel serves: bf16 weights, d_h = 128, d_r = 64, d_c a multiple of 256,
// at most 64 query rows and at most two fp32 parts.  Workgroup = (head,
// 256 latent columns), 4 waves; wave w owns latent columns 64 w .. 64 w + 63
// and every query row.  The transposed product C^T[n][m] is accumulated, so
// that W fragments are the MFMA A operand (read with transposing LDS loads,
// as the key/value tiles of the decode kernel) and each lane ends with 4
// consecutive latent columns of one row, stored as 8 bytes.
//
// All operands reach LDS by direct-to-LDS copies, so vmcnt counts copies
// only: first the activation parts, then the W rows 0..63, then 64..127;
// the first half of the k loop runs while the second half of W lands.
//
// LDS (bytes):
//   [0, 64 KiB)  W tile: 1 KiB groups (chunk group cg = 64 columns, k group
//     kg = 8 rows) at 1024 (16 cg + kg); inside, k row 8 kg + t8 at 128 t8,
//     16-byte chunk c at position c ^ swz(t8) ^ 2 (kg % 2) (conflict free for
//     the 64-bank LDS: the transposing reads of 32 lanes cover 32 distinct
//     8-byte slots of a 256-byte bank row).
//   [64 KiB, +32 KiB per part)  activation rows, 512 bytes each (128 fp32);
//     16-byte piece p of row m at position p ^ (m % 16).
#include "lds_dma.hpp"
#include "mla_common.hpp"
#include "mla_kernels.hpp"

namespace mla {
namespace {

constexpr int AB_K = 128;                  // d_h
constexpr int AB_N = 256;                  // latent columns per workgroup
constexpr int AB_W_BYTES = AB_K * AB_N * 2;  // 64 KiB
constexpr int AB_ROWS = 64;                // query rows held
constexpr int AB_A_BYTES = AB_ROWS * AB_K * 4;  // 32 KiB per part
constexpr int AB_MAX_PARTS = 2;
constexpr int AB_DR = 64;                  // d_r

__global__ __launch_bounds__(256) void absorb_kernel(
    const float* __restrict__ parts, int nparts, long part_stride, long lda,
    const uint16_t* __restrict__ w_uk, int d_c, int row_elems, int M,
    uint16_t* __restrict__ q_out, long ldq, long qr_col,
    const int32_t* __restrict__ pos, const float* __restrict__ rcos,
    const float* __restrict__ rsin, int max_pos) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;
  const int h = blockIdx.x;
  const int ns = blockIdx.y;
  const uint32_t l0 = lds_u32(lds);

  // ---- copies: activation parts (8 per wave per part) -------------------
  // Copy i (0..31) of a part: rows 2 i and 2 i + 1; lane l writes row
  // r = 2 i + l / 32, position x = l % 32, which holds piece x ^ (r % 16).
  // Rows at or past M repeat row M - 1 (their results are not stored).
  for (int p = 0; p < nparts; ++p) {
    const char* ab = (const char*)(parts + (size_t)p * part_stride +
                                   (size_t)h * AB_K);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int i = wave * 8 + c;
      const int r = 2 * i + (lane >> 5);
      const int x = lane & 31;
      const uint32_t voff =
          (uint32_t)((size_t)min(r, M - 1) * lda * 4) + 16 * (x ^ (r & 15));
      dma16(l0 + AB_W_BYTES + p * AB_A_BYTES + i * 1024, ab, voff);
    }
  }
  // ---- copies: W tile in two halves of k (8 per wave each) --------------
  // Group j = 4 c + wave of a half: chunk group j / 8, k group 8 s + j % 8;
  // lane l fetches k row 8 kg + l / 8, chunk (l % 8) ^ swz(l / 8) ^ 2 (kg % 2).
  const uint16_t* wh = w_uk + (size_t)h * AB_K * d_c + (size_t)ns * AB_N;
  uint32_t wvo[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int t8 = lane >> 3;
    const int c8 = (lane & 7) ^ swz(t8) ^ (2 * par);
    wvo[par] = (uint32_t)(t8 * d_c * 2 + c8 * 16);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int j = 4 * c + wave;
      const int cg = j / 8, kg = 8 * s + j % 8;
      // W_UK is read once per step: non-temporal
      dma16<true>(l0 + 1024 * (16 * cg + kg),
                  (const char*)(wh + (size_t)8 * kg * d_c + 64 * cg),
                  wvo[kg & 1]);
    }

  // ---- fragment offsets -------------------------------------------------
  // W (A operand), tile nt of the wave (32 columns), k-step kk: two
  // transposing reads of k groups 2 kk and 2 kk + 1 (the second with the
  // group-parity term, byte offset ^ 32); lane L ends with column L % 32 of
  // the tile for k = 16 kk + 8 (e / 4) + 4 (L / 32) + e % 4, e = 0..7.
  int a_w[2];
  {
    const int q16 = lane >> 4, s16 = lane & 15;
    const int vt = 4 * (q16 >> 1) + (s16 >> 2);
    const int vc = 2 * (q16 & 1) + ((s16 & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      a_w[e] = vt * 128 + 16 * ((4 * e + vc) ^ swz(vt)) + 8 * (s16 & 1) +
               16384 * wave;
  }
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  const lds_char* L = (const lds_char*)lds;
  auto wfrag = [&](int nt, int kk) __attribute__((always_inline)) {
    const int off = a_w[nt] + 2048 * kk;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(L + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(L + ((off ^ 32) + 1024)));
    return __builtin_bit_cast(
        bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Activations (B operand), rows 32 mt + L % 32, the same k order: pieces
  // 4 kk + g (k slots 0..3) and 4 kk + 2 + g (slots 4..7), summed over the
  // parts and split into bf16 hi + lo.
  const int am = lane & 31;
  auto afrag = [&](int mt, int kk, bf16x8& hi, bf16x8& lo)
      __attribute__((always_inline)) {
    const int m = 32 * mt + am;
    const lds_char* row = L + AB_W_BYTES + m * 512;
    const int p0 = 16 * ((4 * kk + g) ^ (m & 15));
    const int p1 = 16 * ((4 * kk + 2 + g) ^ (m & 15));
    f32x4 x0 = *(const lds_f32x4*)(row + p0);
    f32x4 x1 = *(const lds_f32x4*)(row + p1);
    if (nparts > 1) {
      x0 += *(const lds_f32x4*)(row + AB_A_BYTES + p0);
      x1 += *(const lds_f32x4*)(row + AB_A_BYTES + p1);
    }
    split_hi_lo_hw(x0, x1, hi, lo);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nt][mt][r] = 0.0f;
  const bool two_m = M > 32;
  auto ksteps = [&](int kk0) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = kk0; kk < kk0 + 4; ++kk) {
      const bf16x8 w0 = wfrag(0, kk), w1 = wfrag(1, kk);
      bf16x8 hi, lo;
      afrag(0, kk, hi, lo);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w0, hi, acc[0][0], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1, hi, acc[1][0], 0, 0, 0);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w0, lo, acc[0][0], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1, lo, acc[1][0], 0, 0, 0);
      if (two_m) {
        afrag(1, kk, hi, lo);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w0, hi, acc[0][1], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1, hi, acc[1][1], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w0, lo, acc[0][1], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1, lo, acc[1][1], 0, 0, 0);
      }
    }
  };
  // Activations and the first half of W landed (own copies), then everyone's.
  wait_vm<8>();
  barrier();
  ksteps(0);
  wait_vm<0>();
  barrier();
  ksteps(4);

  // ---- store: C^T register r of lane L is latent column
  // 8 (r / 4) + 4 (L / 32) + r % 4 of the tile, query row 32 mt + L % 32.
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int m = 32 * mt + am;
    if (m >= M) continue;
    uint16_t* dst = q_out + (size_t)m * ldq + (size_t)h * row_elems +
                    (size_t)ns * AB_N + 64 * wave + 4 * g;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x16& a = acc[nt][mt];
        const bf16x2 p0 = __builtin_convertvector(
            (f32x2){a[4 * i], a[4 * i + 1]}, bf16x2);
        const bf16x2 p1 = __builtin_convertvector(
            (f32x2){a[4 * i + 2], a[4 * i + 3]}, bf16x2);
        *(uint2*)(dst + 32 * nt + 8 * i) =
            make_uint2(__builtin_bit_cast(uint32_t, p0),
                       __builtin_bit_cast(uint32_t, p1));
      }
  }

  // ---- RoPE query of head h: rows [r0, r1) of this workgroup, 4 pairs per
  // item.  Every copy has landed (vmcnt 0 above), so these loads are the
  // only ones in flight.  An out-of-range position yields NaN, as for the
  // cache rows.
  constexpr int HALF = AB_DR / 2;
  const int rows_per = (AB_ROWS + gridDim.y - 1) / gridDim.y;
  const int r0 = ns * rows_per, r1 = min(M, r0 + rows_per);
  for (int it = threadIdx.x; it < (r1 - r0) * (HALF / 4); it += 256) {
    const int m = r0 + it / (HALF / 4);
    const int j0 = 4 * (it % (HALF / 4));
    const int p = pos[m];
    const bool ok = p >= 0 && p < max_pos;
    const size_t src = (size_t)m * lda + qr_col + (size_t)h * AB_DR + j0;
    f32x4 x1 = *(const f32x4*)(parts + src);
    f32x4 x2 = *(const f32x4*)(parts + src + HALF);
    for (int pp = 1; pp < nparts; ++pp) {
      x1 += *(const f32x4*)(parts + pp * part_stride + src);
      x2 += *(const f32x4*)(parts + pp * part_stride + src + HALF);
    }
    const f32x4 c = ok ? *(const f32x4*)(rcos + (size_t)p * HALF + j0)
                       : (f32x4){NAN, NAN, NAN, NAN};
    const f32x4 s = ok ? *(const f32x4*)(rsin + (size_t)p * HALF + j0)
                       : (f32x4){NAN, NAN, NAN, NAN};
    uint16_t* dst = q_out + (size_t)m * ldq + (size_t)h * row_elems + d_c + j0;
    const f32x4 y1 = x1 * c - x2 * s;
    const f32x4 y2 = x1 * s + x2 * c;
    *(uint2*)dst = make_uint2(pack_bf2(y1[0], y1[1]), pack_bf2(y1[2], y1[3]));
    *(uint2*)(dst + HALF) =
        make_uint2(pack_bf2(y2[0], y2[1]), pack_bf2(y2[2], y2[3]));
  }
}

}  // namespace

bool absorb_fast_supported(const mla_dims& d, int T, int nparts) {
  return d.dtype == MLA_BF16 && d.d_h == AB_K && d.d_c % AB_N == 0 &&
         d.d_r == AB_DR && T >= 1 && T <= AB_ROWS && nparts >= 1 &&
         nparts <= AB_MAX_PARTS;
}

hipError_t launch_absorb_fast(const mla_dims& d, int T, const float* parts,
                              int nparts, long part_stride, long lda,
                              const void* w_uk, const int32_t* pos,
                              const float* rope_cos, const float* rope_sin,
                              int max_pos, void* q_out, hipStream_t stream) {
  static std::atomic<unsigned long long> lds_set{0};
  {
    const hipError_t e = set_lds_limit_once(
        (const void*)absorb_kernel, AB_W_BYTES + AB_MAX_PARTS * AB_A_BYTES,
        lds_set);
    if (e != hipSuccess) return e;
  }
  const int row_elems = d.d_c + d.d_r;
  const dim3 grid(d.n_h, d.d_c / AB_N);
  const size_t lds = AB_W_BYTES + (size_t)nparts * AB_A_BYTES;
  hipLaunchKernelGGL(absorb_kernel, grid, dim3(256), lds, stream, parts,
                     nparts, part_stride, lda, (const uint16_t*)w_uk, d.d_c,
                     row_elems, T, (uint16_t*)q_out,
                     (long)d.n_h * row_elems, (long)d.n_h * d.d_h, pos,
                     rope_cos, rope_sin, max_pos);
  return hipGetLastError();
}

}  // namespace mla
