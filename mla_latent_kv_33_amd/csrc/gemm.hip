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
// Kernels (gemm_plan picks one):
//   * lds (M <= 64, NT, K % 64 == 0): decode batches, bound by streaming the
//     weights once.  Activation rows and 128 or 256 weight rows arrive in
//     64-k steps by direct-to-LDS copies into a 3-4 slot ring; workgroups
//     split K, each K chunk writing its own partial C (summed by the
//     consumer), which keeps results deterministic.  It also reads and
//     writes fp32 activations pre-split into bf16 hi|lo pairs.
//   * tiled (any M, NT or NN; the fallback for shapes the others do not
//     take): 128x128x32 tiles staged through padded LDS,
//     2x2 waves of 64x64; NN weights are read with ds_read_b64_tr_b16 so the
//     MFMA still sees k-contiguous B fragments.
//   * big (M >= 128; NT, K >= 256): 128x128 tiles (64x128 with fp32
//     activations) in 64-k steps through a two-slot direct-to-LDS ring, two
//     workgroups per compute unit, one K chunk per tile.
// fp32 layers use a plain SIMT kernel (small shapes only).

#include "lds_dma.hpp"
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

// ------------------------------------------------------------------ ldsk
// LDS-staged weight-streaming kernel for M <= 64, NT, K % 64 == 0, with a
// weight of up to three parts stacked by rows (rows < nb1 from B, < nb2
// from B2, the rest from B3; both boundaries multiples of 32 rows).  Workgroup = 4 waves over
// 128 NTW output columns and 32 MT rows (row block gridDim.z / batch of a
// row split: a small grid can run each half of the rows in its own
// workgroup, the pair sharing the weights through L2),
// wave w owning column tiles w NTW .. w NTW + NTW-1;
// all waves walk the workgroup's K chunk together in super-steps of 64 k.
// Each super-step's activation rows (shared by the waves) and weight rows
// are copied HBM -> LDS by direct-to-LDS loads, whole 128-byte line runs per
// instruction, into a ring of NBUF slots, so that NBUF - 1 super-steps are
// in flight while one is consumed; MFMA operands are read back with
// ds_read_b128 from swizzled positions (conflict free).  No cross-wave
// reduction: each wave writes its own tiles; each K chunk writes its own
// partial C.
template <int MT, int NTW, bool AF32>
struct LdsCfg {
  static constexpr int MROWS = 32 * MT;
  static constexpr int RB = AF32 ? 256 : 128;      // A bytes per row per 64 k
  static constexpr int PPR = RB / 16;              // 16-byte pieces per row
  static constexpr int RPI = 64 / PPR;             // A rows per copy
  static constexpr int A_BYTES = MROWS * RB;
  static constexpr int A_PER = A_BYTES / 1024 / 4; // A copies per wave
  static constexpr int B_PER = 4 * NTW;            // B copies per wave
  static constexpr int D_PER = A_PER + B_PER;      // copies per wave per step
  static constexpr int B_OFF = A_BYTES;
  static constexpr int SLOT = A_BYTES + 4 * NTW * 4096;
  static constexpr int NB0 = (160 * 1024) / SLOT;
  static constexpr int NBUF = NB0 > 4 ? 4 : NB0;
  static_assert(A_PER >= 1 && A_BYTES % 4096 == 0, "A copy split");
  static_assert(NBUF >= 2, "LDS ring");
  static_assert((NBUF - 2) * D_PER <= 63, "vmcnt range");
  static constexpr int LDS = NBUF * SLOT;
  // A row swizzle (see the copy offsets)
  static __device__ __forceinline__ int sw(int r) {
    return PPR == 16 ? (r & 15) : ((r >> 1) & 7);
  }
};

// HL: A holds pre-split hi|lo pairs (AF32 layout, no split in the kernel);
// c_hl: C is written as pre-split pairs (one K chunk).
template <int MT, int NTW, bool AF32, bool HL>
__global__ __launch_bounds__(256) void gemm_lds_kernel(
    const void* __restrict__ Av, long lda, long a_bs,
    const uint16_t* __restrict__ B, const uint16_t* __restrict__ B2, int nb1,
    const uint16_t* __restrict__ B3, int nb2,
    long ldb, long b_bs, float* __restrict__ C, long ldc, long c_bs, long c_ks,
    int M, int N, int K, int k_chunk, int m_split, int c_hl, int w_nt) {
  static_assert(!HL || AF32, "pre-split A uses the fp32 layout");
  using L = LdsCfg<MT, NTW, AF32>;
  constexpr int NBUF = L::NBUF;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;
  const int col = lane & 31;
  // K chunk fastest in the launch order (see gemm_stream_kernel).
  const int kz = blockIdx.x;
  const int n_wg = blockIdx.y * 128 * NTW;
  const int nbatch = gridDim.z / m_split;
  const int z = blockIdx.z % nbatch;
  const int m0 = (blockIdx.z / nbatch) * L::MROWS;  // first row of the block
  M = min(L::MROWS, M - m0);
  if (M <= 0) return;  // empty row block (whole workgroup, before any barrier)
  C += (size_t)m0 * ldc;
  const int kbeg = kz * k_chunk;
  const int kend = min(K, kbeg + k_chunk);
  const int nss = max(0, (kend - kbeg) / 64);
  const int esz = AF32 ? 4 : 2;

  // ---- per-lane copy offsets (bytes from the per-super-step scalar base)
  // A: copy i (= wave A_PER + a) covers rows i RPI .. i RPI + RPI - 1; lane l
  // takes row r = i RPI + l / PPR and piece (l % PPR) ^ sw(r) of it, so that
  // LDS position p of row r holds piece p ^ sw(r).  A 256-byte fp32 row
  // spans all 16 bank groups of 16 bytes: sw = r % 16.  Two 128-byte bf16
  // rows share a bank row (r % 2 picks the half): sw = (r / 2) % 8.  Either
  // way the 16 rows a ds_read_b128 cycle serves hit 16 distinct groups.
  const char* a_base = (const char*)Av + (size_t)z * a_bs * esz +
                       (size_t)m0 * lda * esz + (size_t)kbeg * esz;
  uint32_t a_off[L::A_PER];
#pragma unroll
  for (int a = 0; a < L::A_PER; ++a) {
    const int r = (wave * L::A_PER + a) * L::RPI + lane / L::PPR;
    const int pos = lane % L::PPR;
    a_off[a] = (uint32_t)((size_t)min(r, M - 1) * lda * esz) +
               16 * (pos ^ L::sw(r));
  }
  // B: column tile t = wave NTW + nt (32 rows), copies q = 0..3 of 8 rows
  // (1 KiB groups); lane l takes row 8 q + l / 8 and chunk
  // (l % 8) ^ swz(l / 8) ^ 2 (q % 2): the group parity term moves odd groups
  // onto the other half of each 256-byte bank row, so that rows t and t + 8
  // of a tile (1 KiB apart, the same banks otherwise) do not collide.
  const char* b_base[NTW];
  uint32_t b_off[NTW][4];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int row0 = min(n_wg + 32 * (wave * NTW + nt), N - 1);
    const uint16_t* bb =
        row0 < nb1   ? B + z * b_bs + (long)row0 * ldb
        : row0 < nb2 ? B2 + z * b_bs + (long)(row0 - nb1) * ldb
                     : B3 + z * b_bs + (long)(row0 - nb2) * ldb;
    b_base[nt] = (const char*)(bb + kbeg);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = min(row0 + 8 * q + (lane >> 3), N - 1) - row0;
      b_off[nt][q] = (uint32_t)(rr * ldb * 2) +
                     16 * ((lane & 7) ^ swz(lane >> 3) ^ (2 * (q & 1)));
    }
  }
  const uint32_t lds0 = lds_u32(lds);
  // The workgroup walks its K chunk starting at a column-slice-dependent
  // super-step and wrapping around, so that at any moment the slices stream
  // different k offsets of their rows.  With a power-of-two row stride
  // (W_O: 16384 bf16 = 32 KiB) the rows at one k offset all fall on a few
  // HBM channels; staggering the offsets spreads them (W_O at 64 rows:
  // 42.1 -> 38.0 us).  The sum over the chunk is the same, in another
  // (fixed) order.
  const int rot = nss > 0 ? (int)(blockIdx.y % (unsigned)nss) : 0;
  auto issue = [&](int ss) __attribute__((always_inline)) {
    const uint32_t slot = lds0 + (ss % NBUF) * L::SLOT;
    const int ks_ = ss + rot < nss ? ss + rot : ss + rot - nss;
#pragma unroll
    for (int a = 0; a < L::A_PER; ++a)
      dma16(slot + (wave * L::A_PER + a) * 1024, a_base + (size_t)ks_ * L::RB,
            a_off[a]);
    // weights: non-temporal when w_nt (a uniform branch around the copies)
    if (w_nt) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dma16<true>(slot + L::B_OFF + (wave * NTW + nt) * 4096 + q * 1024,
                      b_base[nt] + (size_t)ks_ * 128, b_off[nt][q]);
    } else {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dma16(slot + L::B_OFF + (wave * NTW + nt) * 4096 + q * 1024,
                b_base[nt] + (size_t)ks_ * 128, b_off[nt][q]);
    }
  };

  // ---- per-lane read offsets inside a slot
  // A operand (mt, ks): row m = 32 mt + col; fp32 pieces 4 ks + 2 g and
  // 4 ks + 2 g + 1, bf16 piece 2 ks + g.
  // B operand (nt, ks): row col of tile (wave NTW + nt), chunk 2 ks + g.
  const int ar = col;  // row within an M tile; (32 mt + col) % 8 == col % 8
  auto a_read = [&](const lds_char* sl, int mt, int piece) __attribute__((always_inline)) {
    const int m = 32 * mt + ar;
    return *(const __attribute__((address_space(3))) u32x4*)(
        sl + m * L::RB + 16 * (piece ^ L::sw(m)));
  };
  const int b_row_off = (col >> 3) * 1024 + (col & 7) * 128;
  auto b_read = [&](const lds_char* sl, int nt, int ks) __attribute__((always_inline)) {
    const int c = 2 * ks + g;
    return *(const __attribute__((address_space(3))) bf16x8*)(
        sl + L::B_OFF + (wave * NTW + nt) * 4096 + b_row_off +
        16 * (c ^ swz(col & 7) ^ (2 * ((col >> 3) & 1))));
  };

  f32x16 acc[MT][NTW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.0f;

#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (i < nss) issue(i);
  for (int ss = 0; ss < nss; ++ss) {
    // Own copies of super-step ss done (later ones may stay in flight),
    // then everybody's; the slot of ss - 1 is free after the barrier.
    const int later = min(NBUF - 2, nss - 1 - ss);
    if (later >= 2 && NBUF >= 4) wait_vm<(NBUF >= 4 ? 2 : 0) * L::D_PER>();
    else if (later >= 1 && NBUF >= 3) wait_vm<(NBUF >= 3 ? 1 : 0) * L::D_PER>();
    else wait_vm<0>();
    barrier();
    if (ss + NBUF - 1 < nss) issue(ss + NBUF - 1);
    const lds_char* sl = (const lds_char*)lds + (ss % NBUF) * L::SLOT;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 ahi[MT], alo[MT], bf[NTW];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (AF32) {
          // values 16 ks + 8 g .. + 7: fp32 pieces 4 ks + 2 g and + 1, or
          // their pre-split hi and lo pieces at the same places
          const u32x4 x0 = a_read(sl, mt, 4 * ks + 2 * g);
          const u32x4 x1 = a_read(sl, mt, 4 * ks + 2 * g + 1);
          if (HL) {
            ahi[mt] = __builtin_bit_cast(bf16x8, x0);
            alo[mt] = __builtin_bit_cast(bf16x8, x1);
          } else {
            split_hi_lo_hw(__builtin_bit_cast(f32x4, x0),
                           __builtin_bit_cast(f32x4, x1), ahi[mt], alo[mt]);
          }
        } else {
          ahi[mt] = __builtin_bit_cast(bf16x8, a_read(sl, mt, 2 * ks + g));
        }
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) bf[nt] = b_read(sl, nt, ks);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              ahi[mt], bf[nt], acc[mt][nt], 0, 0, 0);
          if (AF32)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                alo[mt], bf[nt], acc[mt][nt], 0, 0, 0);
        }
    }
    wait_lgkm0();  // this slot's reads returned before the next barrier
  }

  // Accumulator register r of lane (col, g): row 32 mt + 8 (r / 4) + 4 g +
  // r % 4, column 32 (wave NTW + nt) + col.
  float* cz = C + z * c_bs + kz * c_ks;
  if (c_hl) {
    // value (m, n) -> hi at 2 m ldc + 16 (n / 8) + n % 8 (bf16 units), lo
    // 8 further (the batch offset z c_bs is a multiple of 8 values)
    uint16_t* ch = (uint16_t*)cz;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int n = n_wg + 32 * (wave * NTW + nt) + col;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
          if (m < M && n < N) {
            const float x = acc[mt][nt][r];
            const uint16_t hi = f2bf(x);
            const long at = 2 * (long)m * ldc + 16 * (n >> 3) + (n & 7);
            ch[at] = hi;
            ch[at + 8] = f2bf(x - bf2f(hi));
          }
        }
    }
    return;
  }
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int n = n_wg + 32 * (wave * NTW + nt) + col;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
        if (m < M && n < N) cz[(long)m * ldc + n] = acc[mt][nt][r];
      }
  }
}

// ------------------------------------------------------------------- big
// Large-M GEMM (prefill chunks): C = A B^T with A [M][K] (bf16, or fp32 as
// hi + lo bf16 terms), B [N][K] bf16 (NT), K % 64 == 0, one K chunk.
//
// Workgroup tile BM x 128 (BM = 128 for bf16 A, 64 for fp32 A, so that the
// A tile is 16 KiB either way) in 64-k steps, 4 waves as 2 x 2 of
// (BM / 2) x 64.  Each step's A and B tiles (32 KiB) arrive by direct-to-LDS
// copies of whole 128/256-byte row runs into a two-slot ring (64 KiB): the
// next step is in flight while one is computed, and two workgroups per
// compute unit cover each other's waits, ring fill and epilogue.  LDS rows
// hold their
// 16-byte pieces XOR-swizzled by the row index (bf16 rows of 128 B: piece ^
// (row / 2) % 8; fp32 rows of 256 B: piece ^ row % 16), so the 16 lanes of
// one ds_read_b128 phase, 16 consecutive rows at the same piece, hit
// distinct banks.  The wave computes C^T tiles (A operand = weight rows,
// B operand = activation rows) so that each lane ends with 4 consecutive
// output columns of one row: 16-byte fp32 or 8-byte bf16 stores.
//
// Tile order: the ids dealt to one XCD (round-robin) form a contiguous run of
// the grouped order (groups of 8 row tiles, column tiles outer), so the
// workgroups one XCD runs together share A row bands and B column bands
// through its L2.
constexpr int BG_BN = 128;
constexpr int BG_GROUP = 8;

// Tiles of 128 x 128 (64 x 128 with fp32 activations, so that the
// activation tile is 16 KiB either way) and a two-slot ring of 32 KiB
// slots, 64 KiB in all: two workgroups share a compute unit, and one's ring
// fill and epilogue overlap the other's k-steps.  (Tiles of 256 x 128 with a
// three-slot ring and one workgroup per compute unit measured 8 - 20 %
// slower on every shape, and 1.8x slower at K = 512.)
template <bool AF32>
struct BigCfg {
  static constexpr int BM = AF32 ? 64 : 128;
  static constexpr int RB = AF32 ? 256 : 128;   // A bytes per row per 64 k
  static constexpr int PPR = RB / 16;           // pieces per A row
  static constexpr int RPC = 1024 / RB;         // A rows per copy
  static constexpr int MT = BM / 64;            // 32-row tiles per wave
  static constexpr int A_BYTES = BM * RB;       // 16 KiB
  static_assert(MT >= 1, "at least one 32-row tile per wave");
  static constexpr int SLOT = A_BYTES + BG_BN * 128;
  static constexpr int NSLOT = 2;
  static constexpr int LDS = NSLOT * SLOT;      // 64 KiB
  static constexpr int A_PER = A_BYTES / 1024 / 4;     // A copies per wave
  static constexpr int B_PER = BG_BN * 128 / 1024 / 4; // 4 B copies per wave
  static constexpr int PER = A_PER + B_PER;
  static_assert((NSLOT - 1) * PER <= 63, "vmcnt range");
};

// Position of piece p of A row r in the LDS row.
template <bool AF32>
__device__ __forceinline__ int big_apos(int r, int p) {
  return AF32 ? p ^ (r & 15) : p ^ ((r >> 1) & 7);
}

template <bool AF32>
__global__ __launch_bounds__(256, 2) void gemm_big_kernel(
    const void* __restrict__ Av, long lda, const uint16_t* __restrict__ B,
    const uint16_t* __restrict__ B2, int nb1, long ldb,
    float* __restrict__ C, uint16_t* __restrict__ C16, long ldc, int M,
    int N, int K, int tiles_m, int tiles_n) {
  using L = BigCfg<AF32>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;
  const int col = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int esz = AF32 ? 4 : 2;

  // block id -> (tm, tn)
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int w = xcd * (nwg >> 3) + min(xcd, nwg & 7) + (blockIdx.x >> 3);
  const int gsize = BG_GROUP * tiles_n;
  const int first_m = (w / gsize) * BG_GROUP;
  const int gm = min(tiles_m - first_m, BG_GROUP);
  const int wi = w - (w / gsize) * gsize;
  const int tm = first_m + wi % gm;
  const int tn = wi / gm;
  const int m0 = tm * L::BM, n0 = tn * BG_BN;

  // ---- copy offsets (bytes from the per-step scalar bases) ---------------
  // A copy i = wave A_PER + a covers rows i RPC .. i RPC + RPC - 1; lane l
  // takes row r = i RPC + l / PPR, LDS position l % PPR, i.e. the piece
  // that belongs there.  Rows past M repeat row M - 1 (results unused).
  const char* a_base = (const char*)Av + (size_t)m0 * lda * esz;
  uint32_t a_off[L::A_PER];
#pragma unroll
  for (int a = 0; a < L::A_PER; ++a) {
    const int r = (wave * L::A_PER + a) * L::RPC + lane / L::PPR;
    const int piece = big_apos<AF32>(r, lane % L::PPR);
    a_off[a] = (uint32_t)((size_t)min(r, M - 1 - m0) * lda * esz) +
               16 * piece;
  }
  // B copy j = wave B_PER + b covers rows 8 j .. 8 j + 7 (128 B each).  The
  // tile lies wholly in B or wholly in B2 (nb1 % 128 == 0 or nb1 >= N).
  const uint16_t* bt = n0 < nb1 ? B + (size_t)n0 * ldb
                                : B2 + (size_t)(n0 - nb1) * ldb;
  uint32_t b_off[L::B_PER];
#pragma unroll
  for (int b = 0; b < L::B_PER; ++b) {
    const int r = 8 * (wave * L::B_PER + b) + (lane >> 3);
    const int piece = (lane & 7) ^ ((r >> 1) & 7);
    b_off[b] = (uint32_t)(min(r, N - 1 - n0) * ldb * 2) + 16 * piece;
  }
  const uint32_t lds0 = lds_u32(lds);
  auto issue = [&](int kt) __attribute__((always_inline)) {
    const uint32_t slot = lds0 + (kt % L::NSLOT) * L::SLOT;
    const char* ab = a_base + (size_t)kt * 64 * esz;
    const char* bb = (const char*)bt + (size_t)kt * 128;
#pragma unroll
    for (int a = 0; a < L::A_PER; ++a)
      dma16(slot + (wave * L::A_PER + a) * 1024, ab, a_off[a]);
#pragma unroll
    for (int b = 0; b < L::B_PER; ++b)
      dma16(slot + L::A_BYTES + (wave * L::B_PER + b) * 1024, bb, b_off[b]);
  };

  // ---- fragment reads -----------------------------------------------------
  // weight fragment (A operand) nt, k-step ks: row wn 64 + 32 nt + col,
  // piece 2 ks + g; activation fragment (B operand) mt: row
  // wm BM / 2 + 32 mt + col, bf16 piece 2 ks + g or fp32 pieces 4 ks + 2 g
  // and 4 ks + 2 g + 1.
  auto w_read = [&](const lds_char* sl, int nt, int ks) __attribute__((always_inline)) {
    const int r = wn * 64 + 32 * nt + col;
    return *(const __attribute__((address_space(3))) bf16x8*)(
        sl + L::A_BYTES + r * 128 + 16 * ((2 * ks + g) ^ ((r >> 1) & 7)));
  };
  auto a_read = [&](const lds_char* sl, int mt, int piece) __attribute__((always_inline)) {
    const int r = wm * (L::BM / 2) + 32 * mt + col;
    return *(const __attribute__((address_space(3))) u32x4*)(
        sl + r * L::RB + 16 * big_apos<AF32>(r, piece));
  };

  f32x16 acc[2][L::MT];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < L::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nt][mt][r] = 0.0f;

  const int nk = K / 64;
#pragma unroll
  for (int i = 0; i < L::NSLOT - 1; ++i)
    if (i < nk) issue(i);
  for (int kt = 0; kt < nk; ++kt) {
    // own copies of step kt done, then everybody's; the slot of step kt - 1
    // is free after the barrier
    wait_vm<0>();
    barrier();
    if (kt + L::NSLOT - 1 < nk) issue(kt + L::NSLOT - 1);
    const lds_char* sl = (const lds_char*)lds + (kt % L::NSLOT) * L::SLOT;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 wf[2], ahi[L::MT], alo[L::MT];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) wf[nt] = w_read(sl, nt, ks);
#pragma unroll
      for (int mt = 0; mt < L::MT; ++mt) {
        if (AF32) {
          const u32x4 x0 = a_read(sl, mt, 4 * ks + 2 * g);
          const u32x4 x1 = a_read(sl, mt, 4 * ks + 2 * g + 1);
          split_hi_lo_hw(__builtin_bit_cast(f32x4, x0),
                         __builtin_bit_cast(f32x4, x1), ahi[mt], alo[mt]);
        } else {
          ahi[mt] = __builtin_bit_cast(bf16x8, a_read(sl, mt, 2 * ks + g));
        }
      }
#pragma unroll
      for (int mt = 0; mt < L::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              wf[nt], ahi[mt], acc[nt][mt], 0, 0, 0);
          if (AF32)
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                wf[nt], alo[mt], acc[nt][mt], 0, 0, 0);
        }
    }
    wait_lgkm0();  // this slot's reads returned before it is refilled
  }

  // C^T accumulator register r of lane (col, g), tiles (nt, mt): column
  // n0 + wn 64 + 32 nt + 8 (r / 4) + 4 g + r % 4 of row
  // m0 + wm BM / 2 + 32 mt + col.  N % 4 == 0, so a group of 4 columns is
  // wholly inside or outside.
#pragma unroll
  for (int mt = 0; mt < L::MT; ++mt) {
    const int m = m0 + wm * (L::BM / 2) + 32 * mt + col;
    if (m >= M) continue;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + wn * 64 + 32 * nt + 8 * i + 4 * g;
        if (n >= N) continue;
        const f32x4 v = {acc[nt][mt][4 * i], acc[nt][mt][4 * i + 1],
                         acc[nt][mt][4 * i + 2], acc[nt][mt][4 * i + 3]};
        if (C16) {
          const uint32_t lo = pack_bf2(v[0], v[1]), hi = pack_bf2(v[2], v[3]);
          *(uint2*)(C16 + (size_t)m * ldc + n) = make_uint2(lo, hi);
        } else {
          *(f32x4*)(C + (size_t)m * ldc + n) = v;
        }
      }
  }
}

template <bool AF32>
hipError_t launch_big(const GemmArgs& g, hipStream_t stream) {
  using L = BigCfg<AF32>;
  static std::atomic<unsigned long long> lds_set{0};
  {
    const hipError_t e = set_lds_limit_once(
        (const void*)gemm_big_kernel<AF32>, L::LDS, lds_set);
    if (e != hipSuccess) return e;
  }
  const int tiles_m = (g.M + L::BM - 1) / L::BM;
  const int tiles_n = (g.N + BG_BN - 1) / BG_BN;
  hipLaunchKernelGGL((gemm_big_kernel<AF32>), dim3(tiles_m * tiles_n),
                     dim3(256), L::LDS, stream, g.A, g.lda,
                     (const uint16_t*)g.B, (const uint16_t*)g.B2, g.nb1,
                     g.ldb, g.C, (uint16_t*)g.c16, g.ldc, g.M, g.N, g.K,
                     tiles_m, tiles_n);
  return hipGetLastError();
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
    int M, int N, int K, int k_chunk, int tiles_n,
    uint16_t* __restrict__ C16) {
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

  // fp32 partial per K chunk, or (C16, one K chunk) the result rounded to
  // bf16 straight into its destination.
  float* cz = C16 ? nullptr : C + z * c_bs + kz * c_ks;
  uint16_t* cz16 = C16 ? C16 + z * c_bs : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        const int nn = n0 + wn * 64 + 32 * j + col;
        if (m < M && nn < N) {
          if (C16)
            cz16[(long)m * ldc + nn] = f2bf(acc[i][j][r]);
          else
            cz[(long)m * ldc + nn] = acc[i][j][r];
        }
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

template <int MT, int NTW, bool AF, bool HL>
hipError_t launch_lds(const GemmArgs& g, dim3 grid, int k_chunk,
                      hipStream_t stream) {
  constexpr int lds = LdsCfg<MT, NTW, AF>::LDS;
  static std::atomic<unsigned long long> lds_set{0};
  {
    const hipError_t e = set_lds_limit_once(
        (const void*)gemm_lds_kernel<MT, NTW, AF, HL>, lds, lds_set);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((gemm_lds_kernel<MT, NTW, AF, HL>), grid, dim3(256), lds,
                     stream, g.A, g.lda, g.a_bs, (const uint16_t*)g.B,
                     (const uint16_t*)g.B2, g.nb1, (const uint16_t*)g.B3,
                     g.nb2, g.ldb, g.b_bs, g.C, g.ldc, g.c_bs, g.c_ks, g.M,
                     g.N, g.K, k_chunk, g.m_split, g.c_hl, g.w_nt);
  return hipGetLastError();
}

}  // namespace

void gemm_plan(const mla_dims& d, GemmArgs& g, int max_split) {
  g.ntw = 0;
  g.k_split = 1;
  g.m_split = 1;
  g.big = 0;
  // Many rows (prefill chunks): the large-tile kernel, one K chunk.  Decode
  // batches (M <= 64) stay on the K-split weight-streaming kernel below: one
  // K chunk per tile would leave W_O's 40 column tiles on 40 compute units.
  const int esz = g.a_f32 ? 4 : 2;
  if (d.dtype == MLA_BF16 && !g.b_nn && g.batch == 1 &&
      g.M >= 128 && g.K >= 256 && g.K % 64 == 0 &&
      g.N % 4 == 0 &&
      g.ldc % 4 == 0 && (g.lda * esz) % 16 == 0 && g.ldb % 8 == 0 &&
      (g.nb1 >= g.N || g.nb1 % BG_BN == 0) && g.nb2 >= g.N) {
    g.big = 1;
    return;
  }
  if (d.dtype != MLA_BF16 || g.b_nn || g.M > 64 || g.M <= 0 || g.N <= 0 ||
      g.K <= 0)
    return;
  if (g.K % 64 == 0 && (g.nb1 >= g.N || g.nb1 % 32 == 0) &&
      (g.nb2 >= g.N || g.nb2 % 32 == 0)) {
    // LDS-staged kernel: 128 or 256 columns per workgroup and a K split
    // (64-multiple chunks) with at most one workgroup per compute unit.
    // Cost = weights (padded to whole column slices) + half the activation
    // bytes (one chunk per workgroup, mostly L2 hits) + half the partial
    // tiles written and read back, over the fraction of the 256 compute
    // units the grid occupies (weights fitted to measured decode shapes).
    const double a_el = g.a_f32 ? 4.0 : 2.0;
    double best = 1e300;
    for (int ntw = 2; ntw >= 1; --ntw) {
      const long slices =
          (long)((g.N + 128 * ntw - 1) / (128 * ntw)) * g.batch;
      for (int s = 1; s <= max_split; ++s) {
        const int kc = ((g.K + s - 1) / s + 63) / 64 * 64;
        const int se = (g.K + kc - 1) / kc;
        if (se != s) continue;
        const long wgs = slices * se;
        if (wgs > 256 && s > 1) break;
        const double eff = wgs <= 256 ? wgs / 256.0
                                      : wgs / (((wgs + 255) / 256) * 256.0);
        const double wbytes = 2.0 * slices * 128.0 * ntw * g.K;
        const double abytes = 0.5 * slices * g.M * (double)g.K * a_el;
        const double parts =
            se > 1 ? 0.5 * 2.0 * se * g.M * (double)g.N * 4.0 * g.batch : 0.0;
        const double cost = (wbytes + abytes + parts) / eff;
        if (cost < best * 0.999) {
          best = cost;
          g.ntw = -ntw;
          g.k_split = se;
        }
      }
    }
    // A grid that leaves half the compute units idle runs its two 32-row
    // blocks in separate workgroups (same XCD, weights shared through L2).
    const long wgs = (long)((g.N + 128 * -g.ntw - 1) / (128 * -g.ntw)) *
                     g.batch * g.k_split;
    g.m_split = (g.M > 32 && 2 * wgs <= 256) ? 2 : 1;
    return;
  }
  // Other decode-batch shapes take the tiled kernel.
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
  // a third weight part: LDS-staged kernel only
  if (g.nb2 < g.N && (g.big || g.ntw >= 0)) return hipErrorInvalidValue;
  if (g.big) {
    if (ks != 1 || g.batch != 1) return hipErrorInvalidValue;
    return g.a_f32 ? launch_big<true>(g, stream) : launch_big<false>(g, stream);
  }
  const uint16_t* B = (const uint16_t*)g.B;
  const uint16_t* B2 = (const uint16_t*)g.B2;
  if (g.c16 && (ks != 1 || g.ntw != 0 || (!g.b_nn && g.M <= 64)))
    return hipErrorInvalidValue;  // bf16 output: tiled kernel, one K chunk
  // pre-split layouts: LDS-staged kernel only; written C needs one K chunk
  if ((g.a_hl && (g.ntw >= 0 || !g.a_f32)) ||
      (g.c_hl && (g.ntw >= 0 || ks != 1 || g.c_bs % 8 != 0)))
    return hipErrorInvalidValue;
  if (g.ntw < 0) {  // LDS-staged kernel, -ntw column tiles per wave
    const int kc = (g.K + ks - 1) / ks;
    k_chunk = (kc + 63) / 64 * 64;
    const int ntw = -g.ntw;
    dim3 grid(ks, (g.N + 128 * ntw - 1) / (128 * ntw), g.batch * g.m_split);
#define MLA_LK(MT, NTW, AF, HL) \
  return launch_lds<MT, NTW, AF, HL>(g, grid, (int)k_chunk, stream)
#define MLA_LK_NTW(MT, AF, HL)                \
  if (ntw == 1) MLA_LK(MT, 1, AF, HL);        \
  else MLA_LK(MT, 2, AF, HL);
#define MLA_LK_A(MT)                                           \
  if (g.a_hl) { MLA_LK_NTW(MT, true, true) }                   \
  else if (g.a_f32) { MLA_LK_NTW(MT, true, false) }            \
  else { MLA_LK_NTW(MT, false, false) }
    if (g.M <= 32 || g.m_split > 1) {
      MLA_LK_A(1)
    } else {
      MLA_LK_A(2)
    }
#undef MLA_LK_A
#undef MLA_LK_NTW
#undef MLA_LK
  }
  k_chunk = (k_chunk + TB_K - 1) / TB_K * TB_K;
  const int tiles_n = (g.N + TB_N - 1) / TB_N;
  const int tiles_m = (g.M + TB_M - 1) / TB_M;
  dim3 grid(tiles_m * tiles_n, ks, g.batch);
#define MLA_TL(AF, NN)                                                       \
  hipLaunchKernelGGL((gemm_tiled_kernel<AF, NN>), grid, dim3(256), 0, stream, \
                     g.A, g.lda, g.a_bs, B, B2, g.nb1, g.ldb, g.b_bs, g.C,    \
                     g.ldc, g.c_bs, g.c_ks, g.M, g.N, g.K, (int)k_chunk,      \
                     tiles_n, (uint16_t*)g.c16)
  if (g.a_f32) {
    if (g.b_nn) MLA_TL(true, true); else MLA_TL(true, false);
  } else {
    if (g.b_nn) MLA_TL(false, true); else MLA_TL(false, false);
  }
#undef MLA_TL
  return hipGetLastError();
}

}  // namespace mla
