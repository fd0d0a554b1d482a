// Projections of a decode step with at most GV_MAXT (4) new tokens, as
// matrix-vector products ('MLA：潜在表示压缩与解耦 RoPE', sections 3, 4, 6
// and 7: c_KV = W_DKV h, k_R = RoPE(W_KR h), c_Q = W_DQ h, q_C = W_UQ c_Q,
// q_R = RoPE(W_QR c_Q), q_lat_h = W_UK_h^T q_C_h, v_h = W_UV_h o_lat_h,
// u = W_O v).
//
// With one to four tokens every projection only streams its weights once;
// the matrix cores would compute 32-row tiles for one real row, and a K
// split would need a second pass to sum its parts.  Here one wave owns R
// whole weight rows: its 64 lanes read each row in 1 KiB runs (16 bytes
// per lane per load, two register sets of loads in flight), multiply them
// by the activations with fp32 accumulation (the activations are read
// through the L1 cache, shared by the waves of a compute unit), and reduce
// across the lanes.  No partial results leave the wave, so each projection
// is one kernel whose epilogue writes the final form: cache rows with the
// RoPE key rotated, c_Q and v as bf16 hi|lo pairs and q_C in fp32 for the
// next projection, the rotated q_R into the query row, u in bf16.  The
// append serves up to four tokens; the query and output projections, whose
// products grow with the token count, serve up to two (GV_QO_MAXT).
//
// Cache policy of the weight reads.  A step streams 299 MB of weights, more
// than the 256 MB Infinity Cache, so with ordinary loads each weight is
// evicted before the next step needs it again.  W_O and [W_UQ; W_QR]
// (168 + 75.5 MB) keep ordinary loads; the other weights use non-temporal
// loads, which do not displace cached lines.  The two large weights then
// stay largely resident between steps, and so do the 4.7 MB of cache rows
// at B = 1.  B = 1 at 4K context, same box: 86.0 us per step with every
// weight read ordinarily, 83.1 with every one non-temporal except W_O,
// 82.1 with W_UQ / W_QR ordinary as well; W_O alone ordinary and the rest
// cached measured 83.6.
//
// The absorption q_lat_h = W_UK_h^T q_C_h reads W_UK_h [d_h][d_c] by rows:
// two workgroups per head (256 latent columns each), each of their 8 waves
// accumulates 16 rows (lanes own 8 latent columns) and the sums meet in
// LDS.

#include "mla_common.hpp"
#include "mla_kernels.hpp"

namespace mla {
namespace {

// 16-byte weight loads per row and lane in one register set: a whole row of
// the 5120-wide projections (10 loads, 2 rows per wave, one set), a
// sixteenth of W_O's 16384-wide rows (2 loads, 4 rows per wave, two sets of
// 8 in flight), a third of the 1536-wide W_UQ / W_QR rows (1 load, 4 rows
// per wave, two sets of 4 in flight).  Measured at one token against 5, 4
// and 3 loads: 1.4 us less over the three projections; these kernels are
// bound by the HBM stream, not by the depth.
constexpr int GV_U_WIDE = 2;
constexpr int GV_U_D = 10;
constexpr int GV_U_UQ = 1;

// Activation forms a row routine reads (per token row, along k):
//   XB16: bf16 values;
//   XHL:  fp32 values stored pre-split as bf16 pairs, hi = bf16(x) and
//         lo = bf16(x - hi): for every 8 consecutive values (one 16-byte
//         weight piece) 16 bytes of hi then 16 bytes of lo;
//   XF32: fp32 values.
// bf16 activations meet the weights in v_dot2c_f32_bf16 (two products per
// instruction, fp32 accumulate), the pre-split ones in two of them (hi and
// lo), fp32 ones in fp32 fused multiply-adds.
enum { XB16 = 0, XHL = 1, XF32 = 2 };

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, x), acc,
                                         false);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Activations of token row t at weight piece p (8 values along k), in the
// registers the multiply reads: 4 words (XB16) or 8 (XHL: hi then lo; XF32).
template <int XM>
struct XPiece {
  u32x4 a, b;
};
template <int T, int XM>
__device__ __forceinline__ void load_x(const void* x, long ldx, int p,
                                       XPiece<XM> (&xv)[T]) {
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (XM == XB16) {
      xv[t].a = *(const u32x4*)((const uint16_t*)x + t * ldx + 8L * p);
    } else if (XM == XHL) {
      // token row t of the pre-split layout: 2 ldx bf16 values
      const u32x4* xp =
          (const u32x4*)((const uint16_t*)x + 2 * t * ldx + 16L * p);
      xv[t].a = xp[0];
      xv[t].b = xp[1];
    } else {
      const u32x4* xp = (const u32x4*)((const float*)x + t * ldx + 8L * p);
      xv[t].a = xp[0];
      xv[t].b = xp[1];
    }
  }
}

// Weight piece (16 bytes, 8 values along k) of every row times the token
// rows' activations at the same k, accumulated into acc[t][r].
template <int T, int R, int XM>
__device__ __forceinline__ void mul_piece(const u32x4 (&wv)[R],
                                          const XPiece<XM> (&xv)[T],
                                          float (&acc)[T][R]) {
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (XM == XB16) {
          acc[t][r] = dot2(wv[r][e], xv[t].a[e], acc[t][r]);
        } else if (XM == XHL) {
          acc[t][r] = dot2(wv[r][e], xv[t].a[e], acc[t][r]);
          acc[t][r] = dot2(wv[r][e], xv[t].b[e], acc[t][r]);
        } else {
          const float x0 = __uint_as_float(e < 2 ? xv[t].a[2 * e] : xv[t].b[2 * e - 4]);
          const float x1 = __uint_as_float(e < 2 ? xv[t].a[2 * e + 1] : xv[t].b[2 * e - 3]);
          acc[t][r] = __builtin_fmaf(__uint_as_float(wv[r][e] << 16), x0,
                                     acc[t][r]);
          acc[t][r] = __builtin_fmaf(__uint_as_float(wv[r][e] & 0xFFFF0000u),
                                     x1, acc[t][r]);
        }
      }
}

// acc[t][r] = sum_k W[row r][k] x[t][k] over this lane's 16-byte pieces
// p = lane, lane + 64, ..., then summed over the wave (every lane holds the
// totals).  K % 512 == 0 (whole 64-lane piece groups).  Whole sets of U
// groups run in two register sets: a set's activations are loaded, then the
// next set's weights are issued, then the set is multiplied, so that the
// wait for the activations leaves the next weights in flight.  A remainder
// of fewer than U groups follows one group at a time.  NT: the weights are
// read with non-temporal loads (see the kernels below).
template <int T, int R, int XM, int U, bool NT = true>
__device__ __forceinline__ void gemv_rows(const uint16_t* const (&w)[R],
                                          const void* x, long ldx, int K,
                                          int lane, float (&acc)[T][R]) {
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[t][r] = 0.0f;
  const int np = K / 8;  // pieces per row, a multiple of 64
  constexpr int STEP = 64 * U;
  const int nsets = np / STEP;
  auto load_w = [&](u32x4 (&wv)[U][R], int q0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
        wv[u][r] = NT ? __builtin_nontemporal_load(
                            (const u32x4*)(w[r] + 8 * (q0 + 64 * u + lane)))
                      : *(const u32x4*)(w[r] + 8 * (q0 + 64 * u + lane));
  };
  auto load_xs = [&](XPiece<XM> (&xv)[U][T], int q0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) load_x<T, XM>(x, ldx, q0 + 64 * u + lane, xv[u]);
  };
  auto mul = [&](const u32x4 (&wv)[U][R], const XPiece<XM> (&xv)[U][T])
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) mul_piece<T, R, XM>(wv[u], xv[u], acc);
  };
  if (nsets > 0) {
    // No load in the loop body is conditional: a wait after a conditional
    // load would have to assume it absent and drain the queue.
    u32x4 wa[U][R], wb[U][R];
    XPiece<XM> xs[U][T];
    load_w(wa, 0);
    int s = 0;
    for (; s + 2 < nsets; s += 2) {
      load_xs(xs, s * STEP);
      load_w(wb, (s + 1) * STEP);
      mul(wa, xs);
      load_xs(xs, (s + 1) * STEP);
      load_w(wa, (s + 2) * STEP);
      mul(wb, xs);
    }
    load_xs(xs, s * STEP);
    if (s + 1 < nsets) {
      load_w(wb, (s + 1) * STEP);
      mul(wa, xs);
      load_xs(xs, (s + 1) * STEP);
      mul(wb, xs);
    } else {
      mul(wa, xs);
    }
  }
  for (int q0 = nsets * STEP; q0 < np; q0 += 64) {
    u32x4 wv[R];
    XPiece<XM> xv[T];
#pragma unroll
    for (int r = 0; r < R; ++r) wv[r] = *(const u32x4*)(w[r] + 8 * (q0 + lane));
    load_x<T, XM>(x, ldx, q0 + lane, xv);
    mul_piece<T, R, XM>(wv, xv, acc);
  }
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[t][r] = wave_sum(acc[t][r]);
}

// Writes value y of (token t, column n) in the pre-split layout of a row of
// ld values: hi at 16 (n / 8) + n % 8 (bf16 units), lo 8 further.
__device__ __forceinline__ void store_hl(uint16_t* y, long ld, int t, long n,
                                         float v) {
  const uint16_t hi = f2bf(v);
  uint16_t* row = y + 2 * t * ld + 16 * (n >> 3) + (n & 7);
  row[0] = hi;
  row[8] = f2bf(v - bf2f(hi));
}

// RoPE of the pair (x1, x2) = (x_j, x_{j + d_r/2}) at position p: NaN for a
// position outside the table (the documented behaviour of every path).
__device__ __forceinline__ void rope_pair(float x1, float x2, int p, int j,
                                          int half, int max_pos,
                                          const float* __restrict__ rcos,
                                          const float* __restrict__ rsin,
                                          float& y1, float& y2) {
  const bool ok = p >= 0 && p < max_pos;
  const float c = ok ? rcos[(long)p * half + j] : NAN;
  const float s = ok ? rsin[(long)p * half + j] : NAN;
  y1 = x1 * c - x2 * s;
  y2 = x1 * s + x2 * c;
}

// ---- append: c_KV rows (pairs of rows) and k_R pairs (j, j + d_r/2) ----
// task < d_c / 2: rows 2 task, 2 task + 1 of W_DKV; then k_R task
// j = task - d_c / 2: rows j and j + d_r/2 of W_KR (one RoPE pair).
template <int T>
__device__ __forceinline__ void append_task(
    int task, const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_dkv,
    const uint16_t* __restrict__ w_kr, int d, int d_c, int d_r,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const float* __restrict__ rcos, const float* __restrict__ rsin,
    int max_pos, const int32_t* __restrict__ block_table, int max_blocks,
    int block_size, uint16_t* __restrict__ cache) {
  const int lane = threadIdx.x;
  const int width = d_c + d_r, half = d_r / 2;
  const bool is_kv = task < d_c / 2;
  const int c0 = is_kv ? 2 * task : task - d_c / 2;
  const int c1 = is_kv ? c0 + 1 : c0 + half;
  const uint16_t* wm = is_kv ? w_dkv : w_kr;
  const uint16_t* w[2] = {wm + (size_t)c0 * d, wm + (size_t)c1 * d};
  float acc[T][2];
  gemv_rows<T, 2, XB16, GV_U_D>(w, h, d, d, lane, acc);
  if (lane >= T) return;
  // lane t writes token t's values (after the sums every lane holds all)
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (t != lane) continue;
    const int p = pos[t];
    const int blk =
        block_table[(long)seq_idx[t] * max_blocks + p / block_size];
    uint16_t* row = cache + ((long)blk * block_size + (p % block_size)) * width;
    if (is_kv) {
      row[c0] = f2bf(acc[t][0]);
      row[c1] = f2bf(acc[t][1]);
    } else {
      float y1, y2;
      rope_pair(acc[t][0], acc[t][1], p, c0, half, max_pos, rcos, rsin, y1,
                y2);
      row[d_c + c0] = f2bf(y1);
      row[d_c + c1] = f2bf(y2);
    }
  }
}

template <int T>
__global__ __launch_bounds__(64) void gemv_append_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_dkv,
    const uint16_t* __restrict__ w_kr, int d, int d_c, int d_r,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const float* __restrict__ rcos, const float* __restrict__ rsin,
    int max_pos, const int32_t* __restrict__ block_table, int max_blocks,
    int block_size, uint16_t* __restrict__ cache) {
  append_task<T>(blockIdx.x, h, w_dkv, w_kr, d, d_c, d_r, seq_idx, pos, rcos,
                 rsin, max_pos, block_table, max_blocks, block_size, cache);
}

// ---- the three down-projections of h in one launch ----------------------
// [W_DQ; W_DKV; W_KR] h: tasks < d_cq / 2 take rows 2 task, 2 task + 1 of
// W_DQ and write c_Q as hi|lo pairs (ldcq values per token row) for the
// query up-projection; the next d_c / 2 + d_r / 2 tasks are the append's.
template <int T>
__global__ __launch_bounds__(64) void gemv_down_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_dq,
    int d_cq, uint16_t* __restrict__ cq, const uint16_t* __restrict__ w_dkv,
    const uint16_t* __restrict__ w_kr, int d, int d_c, int d_r,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const float* __restrict__ rcos, const float* __restrict__ rsin,
    int max_pos, const int32_t* __restrict__ block_table, int max_blocks,
    int block_size, uint16_t* __restrict__ cache) {
  const int nq = d_cq / 2;
  if ((int)blockIdx.x >= nq) {
    append_task<T>(blockIdx.x - nq, h, w_dkv, w_kr, d, d_c, d_r, seq_idx, pos,
                   rcos, rsin, max_pos, block_table, max_blocks, block_size,
                   cache);
    return;
  }
  const int lane = threadIdx.x;
  const int n0 = 2 * blockIdx.x;
  const uint16_t* w[2] = {w_dq + (size_t)n0 * d, w_dq + (size_t)(n0 + 1) * d};
  float acc[T][2];
  gemv_rows<T, 2, XB16, GV_U_D>(w, h, d, d, lane, acc);
  // lane 2 t + r writes (t, row r)
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < 2; ++r)
      if (lane == 2 * t + r) store_hl(cq, d_cq, t, n0 + r, acc[t][r]);
}

// ---- plain rows: y[t][n] = W[n] . x[t] ----------------------------------
// Rows R task .. R task + R - 1 (< N); d_h_sel > 0: per-head activations
// (W_UV: x of row n is x + (n / d_h_sel) xhead values; d_h_sel % R == 0).
// Output: fp32, bf16, or the pre-split hi|lo pairs the next projection
// reads (ldy values per token row).
enum { YF32 = 0, YB16 = 1, YHL = 2 };
template <int T, int XM, int YM, int R, int U, bool NT = true>
__global__ __launch_bounds__(64) void gemv_plain_kernel(
    const uint16_t* __restrict__ W, int N, int K, const void* __restrict__ x,
    long ldx, int d_h_sel, long xhead, void* __restrict__ y, long ldy) {
  const int lane = threadIdx.x;
  const int n0 = R * blockIdx.x;
  const uint16_t* w[R];
#pragma unroll
  for (int r = 0; r < R; ++r) w[r] = W + (size_t)min(n0 + r, N - 1) * K;
  const void* xs = x;
  if (d_h_sel > 0)
    xs = (const char*)x +  // 2 bytes per bf16 value, 4 per fp32 or hi|lo pair
         (size_t)(n0 / d_h_sel) * xhead * (XM == XB16 ? 2 : 4);
  float acc[T][R];
  gemv_rows<T, R, XM, U, NT>(w, xs, ldx, K, lane, acc);
  // lane R t + r writes (t, row r)
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lane == R * t + r && n0 + r < N) {
        if (YM == YB16)
          ((uint16_t*)y)[(size_t)t * ldy + n0 + r] = f2bf(acc[t][r]);
        else if (YM == YHL)
          store_hl((uint16_t*)y, ldy, t, n0 + r, acc[t][r]);
        else
          ((float*)y)[(size_t)t * ldy + n0 + r] = acc[t][r];
      }
}

// ---- split combine fused with v_h = W_UV_h o_lat_h (one or two rows) ---
// For a decode of one or two query rows whose keys were split by the
// matrix-core decode (scaled fp16 partials, m and l per split):
// workgroup (head h, half z) first issues its 64 rows of W_UV_h (wave w:
// rows 64 z + 16 w .. + 15; lane l: latent columns 8 l .. 8 l + 7 of
// each), then merges the head's splits for every query row with the split
// combine's formula (wave w takes a quarter of the splits, lane l the same
// 8 columns; the quarters meet in LDS), keeps the merged o_lat_h row in
// LDS and takes its rows' dot products with it.  The weight stream thus
// runs under the combine's loads instead of after them in a second kernel.
// Half 0 also writes o_lat and lse.  The two workgroups of a head are n_h
// apart in launch order, so with n_h % 8 == 0 they run on one XCD and the
// second finds the partials in its L2.  Shapes: d_c = 512, d_h = 128.
constexpr int CU_DC = 512, CU_DH = 128, CU_RW = 16, CU_CS = 16;

// Wave totals of 16 values per lane in 17 exchanges instead of 16 x 6: at
// each of the offsets 32, 16, 8, 4 a lane keeps the half of its values
// whose row bit matches its lane bit and adds the partner's copy of that
// half, then the last two offsets sum plainly.  Lane l ends with the total
// of value (l >> 2) & 15.
__device__ __forceinline__ float wave_sum16(const float (&a)[16], int lane) {
  float b[8];
  const bool p5 = lane & 32, p4 = lane & 16, p3 = lane & 8, p2 = lane & 4;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    b[i] = (p5 ? a[i + 8] : a[i]) + __shfl_xor(p5 ? a[i] : a[i + 8], 32);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    b[i] = (p4 ? b[i + 4] : b[i]) + __shfl_xor(p4 ? b[i] : b[i + 4], 16);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    b[i] = (p3 ? b[i + 2] : b[i]) + __shfl_xor(p3 ? b[i] : b[i + 2], 8);
  float c = (p2 ? b[1] : b[0]) + __shfl_xor(p2 ? b[0] : b[1], 4);
  c += __shfl_xor(c, 2);
  c += __shfl_xor(c, 1);
  return c;
}

template <int T>
__global__ __launch_bounds__(256) void combine_uv_kernel(
    int n_h, int n_split, const uint16_t* __restrict__ o_part,
    const float* __restrict__ m_part, const float* __restrict__ l_part,
    const uint16_t* __restrict__ w_uv, float* __restrict__ o_lat,
    float* __restrict__ lse, uint16_t* __restrict__ v) {
  static_assert(CU_RW == 16 && T <= 4, "wave_sum16 and the store lanes");
  const int h = blockIdx.x, z = blockIdx.y;
  const int lane = threadIdx.x % 64;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  // this wave's rows of W_UV_h, one 16-byte piece per lane and row (read
  // once per step: non-temporal)
  const int r0 = z * (CU_DH / 2) + wv * CU_RW;
  const uint16_t* wb = w_uv + ((size_t)h * CU_DH + r0) * CU_DC + 8 * lane;
  u32x4 wr[CU_RW];
#pragma unroll
  for (int k = 0; k < CU_RW; ++k)
    wr[k] = __builtin_nontemporal_load((const u32x4*)(wb + (size_t)k * CU_DC));

  __shared__ float sm_ml[4][2];
  __shared__ f32x4 sm_o[4][64][2];
  __shared__ f32x4 xs[T][64][2];
  // the scales follow the T n_split n_h fp16 partial rows
  const float* sc_part =
      (const float*)(o_part + (size_t)T * n_split * n_h * CU_DC);
  const int per = (n_split + 3) / 4;
  const int j_lo = min(wv * per, n_split);
  const int j_hi = min(j_lo + per, n_split);
  for (int t = 0; t < T; ++t) {
    const size_t row0 = (size_t)t * n_split * n_h + h;  // + j n_h
    float M = -INFINITY, L = 0.0f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    for (int j0 = j_lo; j0 < j_hi; j0 += CU_CS) {
      // every load from an in-range split (clamped), masked afterwards, so
      // that all of them are in flight together
      float m[CU_CS], l[CU_CS], ps[CU_CS];
      u32x4 raw[CU_CS];
#pragma unroll
      for (int u = 0; u < CU_CS; ++u) {
        const size_t r = row0 + (size_t)min(j0 + u, j_hi - 1) * n_h;
        m[u] = m_part[r];
        l[u] = l_part[r];
        ps[u] = sc_part[r];
        raw[u] = *(const u32x4*)(o_part + r * CU_DC + 8 * lane);
      }
      float mc = M;
#pragma unroll
      for (int u = 0; u < CU_CS; ++u) {
        m[u] = j0 + u < j_hi ? m[u] : -INFINITY;
        mc = fmaxf(mc, m[u]);
      }
      if (mc == -INFINITY) continue;  // only empty splits so far
      const float sc = M == -INFINITY ? 0.0f : exp2f(M - mc);
      L *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
      for (int u = 0; u < CU_CS; ++u) {
        const bool live = m[u] != -INFINITY;
        const float w = live ? exp2f(m[u] - mc) : 0.0f;
        const float wl = w * l[u];
        L += live ? wl : 0.0f;
        const float wp = wl * ps[u];  // weight of the stored partial
        const f32x8 f = __builtin_convertvector(
            __builtin_bit_cast(f16x8, raw[u]), f32x8);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[e] = live ? __builtin_fmaf(wp, f[e], acc[e]) : acc[e];
      }
      M = mc;
    }
    // waves 1..3 hand (M, L, columns) to wave 0, which merges them as one
    // more chunk of splits (a wave without splits has M = -inf)
    if (wv > 0) {
      sm_o[wv][lane][0] = (f32x4){acc[0], acc[1], acc[2], acc[3]};
      sm_o[wv][lane][1] = (f32x4){acc[4], acc[5], acc[6], acc[7]};
      if (lane == 0) {
        sm_ml[wv][0] = M;
        sm_ml[wv][1] = L;
      }
    }
    __syncthreads();
    if (wv == 0) {
      float mc = M;
#pragma unroll
      for (int g = 1; g < 4; ++g) mc = fmaxf(mc, sm_ml[g][0]);
      const float sc = M == -INFINITY ? 0.0f : exp2f(M - mc);
      L *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
      for (int g = 1; g < 4; ++g) {
        const float mg = sm_ml[g][0];
        const bool live = mg != -INFINITY;
        const float w = live ? exp2f(mg - mc) : 0.0f;
        L += live ? w * sm_ml[g][1] : 0.0f;
        const f32x4 a0 = sm_o[g][lane][0], a1 = sm_o[g][lane][1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] = live ? __builtin_fmaf(w, a0[e], acc[e]) : acc[e];
          acc[e + 4] = live ? __builtin_fmaf(w, a1[e], acc[e + 4]) : acc[e + 4];
        }
      }
      const float il = 1.0f / L;
      const f32x4 o0 = {acc[0] * il, acc[1] * il, acc[2] * il, acc[3] * il};
      const f32x4 o1 = {acc[4] * il, acc[5] * il, acc[6] * il, acc[7] * il};
      xs[t][lane][0] = o0;
      xs[t][lane][1] = o1;
      if (z == 0) {
        float* dst = o_lat + ((size_t)t * n_h + h) * CU_DC + 8 * lane;
        *(f32x4*)dst = o0;
        *(f32x4*)(dst + 4) = o1;
        if (lane == 0 && lse)
          lse[(size_t)t * n_h + h] = (mc + log2f(L)) * 0.69314718055994531f;
      }
    }
    // publishes xs[t]; sm_o and sm_ml are free again for the next row
    __syncthreads();
  }
  // v rows: the wave's rows of W_UV_h times the merged rows, fp32 products
  // of the bf16 weights (as the matrix-vector W_UV with fp32 activations)
  float a[T][CU_RW];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const f32x4 x0 = xs[t][lane][0], x1 = xs[t][lane][1];
    const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
    for (int k = 0; k < CU_RW; ++k) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = __builtin_fmaf(__uint_as_float(wr[k][e] << 16), x[2 * e], s);
        s = __builtin_fmaf(__uint_as_float(wr[k][e] & 0xFFFF0000u), x[2 * e + 1], s);
      }
      a[t][k] = s;
    }
  }
  // lane 4 k + t writes (t, row r0 + k), pre-split for the W_O kernel
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const float tot = wave_sum16(a[t], lane);
    if ((lane & 3) == t)
      store_hl(v, (long)n_h * CU_DH, t, (long)h * CU_DH + r0 + (lane >> 2),
               tot);
  }
}

// ---- query up-projection: q_C rows (fp32 out) and q_R pairs (rotated,
// bf16 into the query row), from c_Q in pre-split pairs ------------------
// task < n_h d_h / 4: rows 4 task .. + 3 of W_UQ -> qc[t][n]; then task
// jt = task - n_h d_h / 4 of the RoPE part: head hh = jt / (d_r / 4), rows
// j, j + 1, j + d_r/2, j + 1 + d_r/2 of W_QR_hh (j = 2 (jt % (d_r / 4))).
template <int T>
__global__ __launch_bounds__(64) void gemv_uq_kernel(
    const uint16_t* __restrict__ cq, int d_cq,
    const uint16_t* __restrict__ w_uq,
    const uint16_t* __restrict__ w_qr, int n_h, int d_h, int d_c, int d_r,
    float* __restrict__ qc, const int32_t* __restrict__ pos,
    const float* __restrict__ rcos, const float* __restrict__ rsin,
    int max_pos, uint16_t* __restrict__ q_out) {
  const int lane = threadIdx.x;
  const int task = blockIdx.x;
  const int nqc = n_h * d_h, half = d_r / 2;
  const bool is_c = task < nqc / 4;
  const uint16_t* w[4];
  int hh = 0, j = 0;
  if (is_c) {
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = w_uq + (size_t)(4 * task + r) * d_cq;
  } else {
    const int jt = task - nqc / 4;
    hh = jt / (d_r / 4);
    j = 2 * (jt % (d_r / 4));
    const uint16_t* wh = w_qr + (size_t)hh * d_r * d_cq;
    w[0] = wh + (size_t)j * d_cq;
    w[1] = wh + (size_t)(j + 1) * d_cq;
    w[2] = wh + (size_t)(j + half) * d_cq;
    w[3] = wh + (size_t)(j + 1 + half) * d_cq;
  }
  float acc[T][4];
  gemv_rows<T, 4, XHL, GV_U_UQ, false>(w, cq, d_cq, d_cq, lane, acc);
  if (is_c) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (lane == 4 * t + r) qc[(size_t)t * nqc + 4 * task + r] = acc[t][r];
  } else {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (lane != t) continue;
      uint16_t* dst =
          q_out + ((size_t)t * n_h + hh) * (d_c + d_r) + d_c;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        float y1, y2;
        rope_pair(acc[t][k], acc[t][k + 2], pos[t], j + k, half, max_pos,
                  rcos, rsin, y1, y2);
        dst[j + k] = f2bf(y1);
        dst[j + k + half] = f2bf(y2);
      }
    }
  }
}

// ---- absorption: q_lat_h = W_UK_h^T q_C_h -------------------------------
// Workgroup = (head hh, 256 latent columns: blockIdx.y), 8 waves, so that
// the 128 heads fill all compute units with two workgroups each.  Wave w
// takes rows i = w, w + 8, ... of W_UK_h (d_h rows of d_c): lane half g
// (lanes 32 g .. 32 g + 31) reads every other one of them, 512 contiguous
// bytes per row and instruction, lane l owning latent columns
// 256 y + 8 (l % 32) + 512 c (c = 0 .. d_c / 512 - 1).  The 16 partial sums
// of a column (8 waves x 2 lane halves) are added in LDS and written as
// bf16 into the first d_c columns of each token's query row.
constexpr int AB_WAVES = 8;
constexpr int AB_PARTS = 2 * AB_WAVES;  // partial sums per column
template <int T>
__global__ __launch_bounds__(64 * AB_WAVES) void gemv_absorb_kernel(
    const float* __restrict__ qc, const uint16_t* __restrict__ w_uk,
    int n_h, int d_h, int d_c, int d_r, uint16_t* __restrict__ q_out) {
  extern __shared__ float red[];  // [AB_PARTS][T][256]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int hh = blockIdx.x;
  const int nch = d_c / 512;  // 512-column chunks (d_c % 512 == 0)
  const uint16_t* wh = w_uk + (size_t)hh * d_h * d_c;
  const float* qh = qc + (size_t)hh * d_h;
  for (int c = 0; c < nch; ++c) {
    float acc[T][8];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[t][e] = 0.0f;
    const int col0 = 512 * c + 256 * blockIdx.y;
    const int col = col0 + 8 * (lane & 31);
    // all of the lane half's rows in flight at once (8 for d_h = 128)
    constexpr int AU = 8;
    for (int i0 = wave + AB_WAVES * g; i0 < d_h; i0 += AB_PARTS * AU) {
      u32x4 wv[AU];
#pragma unroll
      for (int u = 0; u < AU; ++u) {
        const int i = i0 + AB_PARTS * u;
        wv[u] = i < d_h ? __builtin_nontemporal_load(
                              (const u32x4*)(wh + (size_t)i * d_c + col))
                        : (u32x4){0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < AU; ++u) {
        const int i = i0 + AB_PARTS * u;
        if (i >= d_h) break;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const float s = qh[(size_t)t * n_h * d_h + i];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[t][2 * e] = __builtin_fmaf(
                __uint_as_float(wv[u][e] << 16), s, acc[t][2 * e]);
            acc[t][2 * e + 1] = __builtin_fmaf(
                __uint_as_float(wv[u][e] & 0xFFFF0000u), s,
                acc[t][2 * e + 1]);
          }
        }
      }
    }
    const int part = 2 * wave + g;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        red[((size_t)part * T + t) * 256 + 8 * (lane & 31) + e] = acc[t][e];
    __syncthreads();
    for (int k = threadIdx.x; k < T * 256; k += 64 * AB_WAVES) {
      const int t = k / 256, cc = k % 256;
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < AB_PARTS; ++w) s += red[((size_t)w * T + t) * 256 + cc];
      q_out[((size_t)t * n_h + hh) * (d_c + d_r) + col0 + cc] = f2bf(s);
    }
    __syncthreads();
  }
}

}  // namespace

bool gemv_supported(const mla_dims& d, int T, int t_max) {
  // every contraction length a multiple of 512 (whole 64-lane piece sets)
  return d.dtype == MLA_BF16 && T >= 1 && T <= t_max && T <= GV_MAXT &&
         d.d % 512 == 0 &&
         d.d_cq % 512 == 0 && d.d_c % 512 == 0 && d.d_r % 4 == 0 &&
         d.d_h % 4 == 0 && (d.n_h * d.d_h) % 512 == 0;
}

#define MLA_GV_T(T, CALL) \
  switch (T) {            \
    case 1: CALL(1); break; \
    case 2: CALL(2); break; \
    case 3: CALL(3); break; \
    default: CALL(4); break; \
  }
// the query and output projections take this path up to GV_QO_MAXT tokens
static_assert(GV_QO_MAXT == 2, "token-count dispatch below");
#define MLA_GV_T2(T, CALL) \
  switch (T) {             \
    case 1: CALL(1); break;  \
    default: CALL(2); break; \
  }

hipError_t launch_gemv_append(const mla_dims& d, int T, const void* h,
                              const void* w_dkv, const void* w_kr,
                              const int32_t* seq_idx, const int32_t* pos,
                              const float* rope_cos, const float* rope_sin,
                              int max_pos, const int32_t* block_table,
                              int max_blocks, void* cache,
                              hipStream_t stream) {
  if (T < 1 || T > GV_MAXT) return hipErrorInvalidValue;
  const int tasks = d.d_c / 2 + d.d_r / 2;
#define MLA_APP(TT)                                                          \
  hipLaunchKernelGGL(gemv_append_kernel<TT>, dim3(tasks), dim3(64), 0,       \
                     stream, (const uint16_t*)h, (const uint16_t*)w_dkv,      \
                     (const uint16_t*)w_kr, d.d, d.d_c, d.d_r, seq_idx, pos, \
                     rope_cos, rope_sin, max_pos, block_table, max_blocks,   \
                     d.block_size, (uint16_t*)cache)
  MLA_GV_T(T, MLA_APP)
#undef MLA_APP
  return hipGetLastError();
}

hipError_t launch_gemv_query(const mla_dims& d, int T, const void* h,
                             const void* w_dq, const void* w_uq,
                             const void* w_qr, const void* w_uk,
                             const int32_t* pos, const float* rope_cos,
                             const float* rope_sin, int max_pos, float* cq,
                             float* qc, void* q_out, hipStream_t stream) {
  if (T < 1 || T > GV_QO_MAXT) return hipErrorInvalidValue;
  // c_Q = W_DQ h, pre-split into hi|lo pairs for the next projection
  const int t1 = (d.d_cq + 1) / 2;
#define MLA_DQ(TT)                                                           \
  hipLaunchKernelGGL((gemv_plain_kernel<TT, XB16, YHL, 2, GV_U_D>),          \
                     dim3(t1),                                               \
                     dim3(64), 0, stream, (const uint16_t*)w_dq, d.d_cq, d.d, \
                     h, (long)d.d, 0, 0L, (void*)cq, (long)d.d_cq)
  MLA_GV_T2(T, MLA_DQ)
#undef MLA_DQ
  return launch_gemv_query_tail(d, T, w_uq, w_qr, w_uk, pos, rope_cos,
                                rope_sin, max_pos, cq, qc, q_out, stream);
}

hipError_t launch_gemv_query_tail(const mla_dims& d, int T, const void* w_uq,
                                  const void* w_qr, const void* w_uk,
                                  const int32_t* pos, const float* rope_cos,
                                  const float* rope_sin, int max_pos,
                                  const float* cq, float* qc, void* q_out,
                                  hipStream_t stream) {
  if (T < 1 || T > GV_QO_MAXT) return hipErrorInvalidValue;
  // q_C (fp32) and RoPE(q_R) into the query rows
  const int t2 = d.n_h * d.d_h / 4 + d.n_h * (d.d_r / 4);
#define MLA_UQ(TT)                                                           \
  hipLaunchKernelGGL(gemv_uq_kernel<TT>, dim3(t2), dim3(64), 0, stream,      \
                     (const uint16_t*)cq,                                    \
                     d.d_cq, (const uint16_t*)w_uq, (const uint16_t*)w_qr,    \
                     d.n_h, d.d_h, d.d_c, d.d_r, qc, pos,                     \
                     rope_cos, rope_sin, max_pos, (uint16_t*)q_out)
  MLA_GV_T2(T, MLA_UQ)
#undef MLA_UQ
  // q_lat_h = W_UK_h^T q_C_h
#define MLA_AB(TT)                                                          \
  hipLaunchKernelGGL(gemv_absorb_kernel<TT>, dim3(d.n_h, 2),                \
                     dim3(64 * AB_WAVES), AB_PARTS * TT * 256 * 4, stream, qc, \
                     (const uint16_t*)w_uk, d.n_h, d.d_h, d.d_c, d.d_r,      \
                     (uint16_t*)q_out)
  MLA_GV_T2(T, MLA_AB)
#undef MLA_AB
  return hipGetLastError();
}

hipError_t launch_gemv_down(const mla_dims& d, int T, const void* h,
                            const void* w_dq, const void* w_dkv,
                            const void* w_kr, const int32_t* seq_idx,
                            const int32_t* pos, const float* rope_cos,
                            const float* rope_sin, int max_pos,
                            const int32_t* block_table, int max_blocks,
                            void* cache, float* cq, hipStream_t stream) {
  if (T < 1 || T > GV_QO_MAXT || d.d_cq % 2) return hipErrorInvalidValue;
  const int tasks = d.d_cq / 2 + d.d_c / 2 + d.d_r / 2;
#define MLA_DN(TT)                                                           \
  hipLaunchKernelGGL(gemv_down_kernel<TT>, dim3(tasks), dim3(64), 0, stream, \
                     (const uint16_t*)h, (const uint16_t*)w_dq, d.d_cq,       \
                     (uint16_t*)cq, (const uint16_t*)w_dkv,                  \
                     (const uint16_t*)w_kr, d.d, d.d_c, d.d_r, seq_idx, pos,  \
                     rope_cos, rope_sin, max_pos, block_table, max_blocks,   \
                     d.block_size, (uint16_t*)cache)
  MLA_GV_T2(T, MLA_DN)
#undef MLA_DN
  return hipGetLastError();
}

hipError_t launch_gemv_out(const mla_dims& d, int T, const float* o_lat,
                           const void* w_uv, const void* w_o, float* v,
                           void* u, hipStream_t stream) {
  if (T < 1 || T > GV_QO_MAXT) return hipErrorInvalidValue;
  const int nv = d.n_h * d.d_h;
  // v_h = W_UV_h o_lat_h, pre-split into hi|lo pairs: rows of head h read
  // x = o_lat[t][h]
#define MLA_UV(TT)                                                           \
  hipLaunchKernelGGL((gemv_plain_kernel<TT, XF32, YHL, 4, 1>),              \
                     dim3(nv / 4),                                           \
                     dim3(64), 0, stream, (const uint16_t*)w_uv, nv, d.d_c,   \
                     (const void*)o_lat, (long)d.n_h * d.d_c, d.d_h,          \
                     (long)d.d_c, (void*)v, (long)nv)
  MLA_GV_T2(T, MLA_UV)
#undef MLA_UV
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gemv_wo(d, T, v, w_o, u, stream);
}

hipError_t launch_gemv_wo(const mla_dims& d, int T, const float* v,
                          const void* w_o, void* u, hipStream_t stream) {
  if (T < 1 || T > GV_QO_MAXT) return hipErrorInvalidValue;
  const int nv = d.n_h * d.d_h;
  // u = W_O v (bf16)
#define MLA_O(TT)                                                            \
  hipLaunchKernelGGL((gemv_plain_kernel<TT, XHL, YB16, 4, GV_U_WIDE, false>), \
                     dim3((d.d + 3) / 4),                                    \
                     dim3(64), 0, stream, (const uint16_t*)w_o, d.d, nv,      \
                     (const void*)v, (long)nv, 0, 0L, u, (long)d.d)
  MLA_GV_T2(T, MLA_O)
#undef MLA_O
  return hipGetLastError();
}

bool combine_uv_supported(const mla_dims& d, int T) {
  return d.dtype == MLA_BF16 && d.d_c == CU_DC && d.d_h == CU_DH && T >= 1 &&
         T <= GV_QO_MAXT;
}

hipError_t launch_combine_uv(const mla_dims& d, int T, int n_split,
                             const float* o_part, const float* m_part,
                             const float* l_part, const void* w_uv,
                             float* o_lat, float* lse, float* v,
                             hipStream_t stream) {
  if (!combine_uv_supported(d, T) || n_split < 2) return hipErrorInvalidValue;
#define MLA_CUV(TT)                                                          \
  hipLaunchKernelGGL(combine_uv_kernel<TT>, dim3(d.n_h, 2), dim3(256), 0,    \
                     stream, d.n_h, n_split, (const uint16_t*)o_part, m_part, \
                     l_part, (const uint16_t*)w_uv, o_lat, lse, (uint16_t*)v)
  MLA_GV_T2(T, MLA_CUV)
#undef MLA_CUV
  return hipGetLastError();
}

#undef MLA_GV_T
#undef MLA_GV_T2

}  // namespace mla
