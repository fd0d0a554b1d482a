// Split-KV MLA decode on gfx950 matrix cores, latent width 512 + RoPE 64.
//
// What is computed ('MLA：潜在表示压缩与解耦 RoPE', sections 4, 6 and 7;
// 'Latent 压缩', MLA section): for one (sequence b, query i) and every head h,
//   score_s = (q_lat_h . c_KV_s + q_R_h . k_R_s) / sqrt(d_h + d_r)
//   o_lat_h = sum_s softmax(score)_s c_KV_s
// over the key range of one split.  In the latent space every head uses the
// same key (the 576-wide cache row) and the same value (its first 512
// columns), so one workgroup serves all heads and each cache row crosses
// HBM once.  (Grids too small to fill the chip, e.g. one sequence, split the
// heads over two workgroups instead; the second read of each row is an L2
// hit.)
//
// Work decomposition (one workgroup = NW waves, NW * 32 heads, one split of
// one query row; either n_split splits per row, or a balanced plan that the
// kernel derives from kv_lens so that long rows get more splits than short
// ones, see balanced_work):
//   * keys stream in half tiles of 32 tokens (half a 64-token cache block),
//     copied HBM -> LDS by direct-to-LDS loads into a ring of four buffers:
//     while a wave computes on halves j and j+1, halves j+2 and j+3 are in
//     flight.
//   * scores: wave w owns heads 32w .. 32w+31.  Its query slice Q[32][576]
//     lives in VGPRs as 36 MFMA B operands; the scores S^T[32 tok][32 heads]
//     of a half are 36 MFMA 32x32x16 (A = key rows from LDS) accumulated in
//     two independent chains.
//   * softmax in base 2 against a reference maximum m_ref per head, taken
//     from the split's first half tile: P = 2^(s - m_ref), rounded to bf16;
//     l and O accumulate with no rescaling, so O is never touched by vector
//     ALU code inside the loop.  Keys far below m_ref underflow to 0 as in
//     any softmax; a half tile whose maximum exceeds m_ref by more than 2^64
//     (still finite, but beyond the range trusted for P and the sums) makes
//     the workgroup restart the split with a raised m_ref.  Real scores never
//     span that range; the restart keeps the result exact for inputs that do.
//   * values: the owner wave writes its P^T to LDS, and wave w accumulates
//     O^T[latent tiles of wave w][all heads of the workgroup] += V^T P^T,
//     32 MFMAs per half, so each value element is read from LDS once per
//     workgroup (through ds_read_b64_tr_b16 transposing loads) rather than
//     once per wave.  The MFMA k slots are mapped to tokens the way the score
//     accumulator lays them out, so P needs no transposition on its way.
//   * software pipeline, one barrier per half: step j interleaves the score
//     MFMAs of half j+1 with the first half of the value MFMAs of half j,
//     then runs the rest of the value MFMAs with the softmax of half j+1
//     spread over them, then stores P of half j+1.
//   * the workgroup writes its partial O / l as fp16 under a power-of-two
//     scale per head (half the bytes of fp32, 11 significant bits), with
//     m_ref (log2 units), l and the scale, or the final o_lat and lse when
//     there is one split.
//
// LDS (NW = 4): 4 half-tile buffers of 36 KiB, then two P buffers of
// 128 heads x 32 tokens bf16 (8 KiB each): 160 KiB, the whole LDS.

#include "lds_dma.hpp"
#include "mla_common.hpp"
#include "mla_kernels.hpp"

namespace mla {
namespace {

constexpr int DC = 512;
constexpr int DR = 64;
constexpr int ROW = DC + DR;          // elements per cache row
constexpr int ROWB = ROW * 2;         // bytes per cache row
constexpr int BS = 64;                // tokens per cache block
constexpr int BLOCK_BYTES = BS * ROWB;
constexpr int HT = 32;                // tokens per half tile
constexpr int HALF_BYTES = HT * ROWB; // 36864
constexpr int HGROUPS = HALF_BYTES / 1024;  // 36 DMA groups per half tile
constexpr int NBUF = 4;               // half-tile ring
constexpr int KSTEPS = ROW / 16;      // 36 k-steps of the score MFMA
constexpr int MT_LAT = DC / 32;       // 16 latent tiles of the value MFMA
constexpr float REF_SLACK = 64.0f;    // log2 headroom above m_ref
constexpr int SDEPTH = 3;             // score fragments in flight
// Epilogue staging of the fp16 partial rows: one padded row per head (the
// 16-byte pad moves consecutive heads to other banks), after the per-head
// maxima at the start of LDS.
constexpr int EPI_OFF = 2048;
constexpr int EPI_STRIDE = DC * 2 + 16;

template <int NW>
struct Cfg {
  static constexpr int HEADS = 32 * NW;
  static constexpr int MTW = MT_LAT / NW;          // latent tiles per wave
  static constexpr int PER_HALF = HGROUPS / NW;    // copies per wave per half
  static constexpr int PBYTES = HEADS * HT * 2;    // P of one half tile
  static constexpr int P_OFF = NBUF * HALF_BYTES;
  static constexpr int LDS = P_OFF + 2 * PBYTES;
  static constexpr int AR = NW == 4 ? 3 : NW == 2 ? 4 : 8;  // V^T ring
  static_assert(HGROUPS % NW == 0, "half-tile groups must split evenly");
  static_assert(PER_HALF <= 63, "outstanding copies must fit vmcnt");
  static_assert(MTW % 2 == 0, "latent tiles per wave must be even");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(EPI_OFF >= NW * HEADS * 4 &&
                    EPI_OFF + HEADS * EPI_STRIDE <= P_OFF,
                "epilogue staging lies between the maxima and the P buffers");
};

// Value of lane l ^ 32.  permlane32_swap(x, x) returns {[x_lo, x_lo],
// [x_hi, x_hi]} (upper half of the first operand exchanged with the lower
// half of the second), so the partner sits in the second result for the
// lower 32 lanes and in the first for the upper 32.
__device__ __forceinline__ float lane_xor32(float x, int g) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                   __float_as_uint(x), false,
                                                   false);
  return __uint_as_float(g ? sw[0] : sw[1]);
}


// Score MFMAs with the accumulator pinned to VGPRs.  The output O^T of a
// wave fills all 256 accumulation registers, so the score accumulators must
// live in the other register file; the compiler picks one file for every
// MFMA of a function, so these few are written out.  Hazards the compiler
// cannot see through the asm: the first MFMA of a chain takes a literal 0 as
// accumulator (no VALU write feeds it), accumulation into exactly the same
// registers as an earlier MFMA needs no wait states, and mfma_v_drain adds
// the wait states a 32x32x16 result needs before VALU reads it (>= 18).
__device__ __forceinline__ f32x16 mfma_v_first(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
               : "=&v"(d)
               : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma_v_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
               : "+v"(d)
               : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_drain(f32x16& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d));
}

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;


// Copy half `hf` (tokens 32 hf .. 32 hf + 31) of a cache block into an LDS
// half-tile buffer.  LDS layout: 16-byte chunk c (of 72 per row) of token t
// lives in group (c / 8, t / 8) of 64 chunks (1 KiB) at 1024 (4 (c / 8) +
// t / 8), position 8 (t % 8) + x, x = (c % 8) ^ swz(t % 8) ^ 2 ((t / 8) % 2).
// One copy fills one group, i.e. 8 tokens x 128 contiguous bytes.  The LDS
// has 64 four-byte banks and serves 16 lanes of a 16-byte read (32 of an
// 8-byte read) per cycle; the score reads take tokens 0..15 in one such
// step, so swz spreads the 8 tokens of a group over all chunk positions of
// two bank rows and the parity term moves the next group onto the other
// half of each row.  Every score, value and copy access is conflict free.
// Wave `wave` issues groups k = wave, wave + NW, ...; lane l fetches token
// 8 (k % 4) + l / 8, chunk 8 (k / 4) + ((l % 8) ^ swz(l / 8) ^ 2 (k % 2)).
// Rows at or past `nvalid` (only in the
// last, partial half of a sequence) are filled from the last valid row:
// their scores are masked, and finite data keeps 0 * value at zero.
//
// The lane's byte offset depends on k only through k % 4 (the token group)
// and k / 4 (128 bytes per chunk group, the copy's immediate offset), so a
// half needs at most four lane offsets, computed once per half.
template <int NW, bool NTC>
struct HalfCopy {
  static constexpr int PER = Cfg<NW>::PER_HALF;
  static constexpr int NQ = NW >= 4 ? 1 : 4 / NW;  // distinct k % 4 per wave
  uint32_t lane_off[NQ];
  uint32_t lds_buf;
  const char* blk;

  __device__ __forceinline__ HalfCopy(const char* blk_, int hf, uint32_t buf,
                                      int nvalid, int wave, int lane)
      : lds_buf(buf), blk(blk_) {
    int tl = lane >> 3;
    // Opaque, so that the offsets are computed here, once per half, and not
    // hoisted into long-lived registers.
    asm volatile("" : "+v"(tl));
    const uint32_t ch = ((lane & 7) ^ swz(tl)) * 16;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int k = q * NW + wave;  // k % 4 for copies i = q, q + NQ, ...
      const int t = min(8 * (k & 3) + tl, nvalid - 1);
      lane_off[q] = (HT * hf + t) * ROWB + (ch ^ (32 * (k & 1)));
    }
  }
  // Copy i (0 .. PER - 1) of this wave: group k = i NW + wave.
  template <int I>
  __device__ __forceinline__ void copy(int wave) const {
    static_assert(I < PER, "copy index");
    constexpr int Q = I % NQ;
    // group k = I NW + wave; k / 4 = (I NW) / 4 since wave < NW <= 4 and
    // (I NW) % 4 + wave < 4 for every wave when NW divides 4.
    constexpr int CG = (I * NW) / 4;
    dma16_off<CG * 128, NTC>(lds_buf + (I * NW + wave) * 1024, blk,
                             lane_off[Q]);
  }
};

// All PER copies of a half, in order (the offsets are template arguments).
template <int I, int N>
struct CopyAll {
  template <class HC>
  static __device__ __forceinline__ void run(const HC& hc, int wave) {
    hc.template copy<I>(wave);
    CopyAll<I + 1, N>::run(hc, wave);
  }
};
template <int N>
struct CopyAll<N, N> {
  template <class HC>
  static __device__ __forceinline__ void run(const HC&, int) {}
};

// The copies that go with group g (0 .. NG - 1) of a step: copy c is issued
// in group (c NG) / PER, so the PER copies spread evenly over the groups.
template <int PER, int NG, int C = 0, class HC>
__device__ __forceinline__ void copy_group(const HC& hc, int wave, int g,
                                           bool on) {
  if constexpr (C < PER) {
    // g is a constant here (the step is fully unrolled).
    if ((C * NG) / PER == g && on) hc.template copy<C>(wave);
    copy_group<PER, NG, C + 1>(hc, wave, g, on);
  }
}

// ---- balanced splits ------------------------------------------------------
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

struct BalWork {
  int row, split, count, slot0;  // row < 0: no work for this workgroup
};

// Work item w of the balanced plan (see DecodeBalance): query row r has
// nb_r visible blocks (at least one), the chunk c is the smallest value >=
// max(BAL_MIN_CHUNK, ceil(sum nb / slots)) with sum ceil(nb_r / c) <= slots
// (binary search; c = max nb gives one split per row, rows <= slots), and
// row r's ceil(nb_r / c) splits take consecutive items.  Every wave
// computes the same values; lane l holds rows l, l + 64, ...
__device__ BalWork balanced_work(const int32_t* __restrict__ kv_lens,
                                 int rows, int n_q, int slots, int w,
                                 int lane) {
  constexpr int RPL = BAL_SLOTS / 64;
  int nb[RPL];
  int total = 0, nbmax = 0;
#pragma unroll
  for (int c = 0; c < RPL; ++c) {
    const int r = 64 * c + lane;
    int v = 0;
    if (r < rows) {
      const int b = r / n_q, qi = r - b * n_q;
      v = max((kv_lens[b] - n_q + qi + 1 + BS - 1) / BS, 1);
    }
    nb[c] = v;
    total += v;
    nbmax = max(nbmax, v);
  }
  total = wave_sum_i(total);
  nbmax = wave_max_i(nbmax);
  auto items = [&](int ch) {
    int n = 0;
#pragma unroll
    for (int c = 0; c < RPL; ++c) n += (nb[c] + ch - 1) / ch;
    return wave_sum_i(n);
  };
  int lo = max(BAL_MIN_CHUNK, (total + slots - 1) / slots);
  if (items(lo) > slots) {
    int hi = max(lo, nbmax);  // items(hi) = rows <= slots
    while (hi - lo > 1) {     // items(lo) > slots >= items(hi)
      const int mid = lo + (hi - lo) / 2;
      if (items(mid) <= slots)
        hi = mid;
      else
        lo = mid;
    }
    lo = hi;
  }
  const int chunk = lo;
  int base = 0;
#pragma unroll
  for (int c = 0; c < RPL; ++c) {
    const int n = (nb[c] + chunk - 1) / chunk;  // 0 past the last row
    const int incl = wave_incl_scan(n, lane);
    const int tot = __shfl(incl, 63);
    if (w < base + tot) {
      const unsigned long long m = __ballot(base + incl > w);
      const int L = __builtin_ctzll(m);
      const int cnt = __shfl(n, L), slot0 = base + __shfl(incl, L) - cnt;
      return {64 * c + L, w - slot0, cnt, slot0};
    }
    base += tot;
  }
  return {-1, 0, 0, 0};
}

template <int NW, bool NTC>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(1, 1))) void
decode_mfma_kernel(
    const uint16_t* __restrict__ q, const char* __restrict__ cache,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ kv_lens, int n_q, int n_h, int n_split,
    int rows, int slots, int2* __restrict__ plan, float scale_log2,
    float* __restrict__ o_part, float* __restrict__ m_part,
    float* __restrict__ l_part, float* __restrict__ o_final,
    float* __restrict__ lse_final) {
  using C = Cfg<NW>;
  constexpr int MTW = C::MTW;
  constexpr int PER = C::PER_HALF;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  lds_char* const L = (lds_char*)lds;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;     // lane half
  const int col = lane & 31;   // head within a 32-head tile
  const int hbase = blockIdx.z * C::HEADS;
  const int head = hbase + wave * 32 + col;  // head whose scores this lane owns
  // (query row, split) of this workgroup; the row's splits fill partial
  // slots slot0 .. slot0 + n_split - 1
  int bq, split, slot0;
  if (plan) {
    const BalWork bw = balanced_work(kv_lens, rows, n_q, slots, blockIdx.x,
                                     lane);
    if (bw.row < 0) return;  // no work left (whole workgroup, no barrier yet)
    bq = __builtin_amdgcn_readfirstlane(bw.row);
    split = __builtin_amdgcn_readfirstlane(bw.split);
    n_split = __builtin_amdgcn_readfirstlane(bw.count);
    slot0 = __builtin_amdgcn_readfirstlane(bw.slot0);
    if (split == 0 && blockIdx.z == 0 && threadIdx.x == 0)
      plan[bq] = make_int2(slot0, n_split);
  } else {
    bq = blockIdx.x;   // b * n_q + i
    split = blockIdx.y;
    slot0 = bq * n_split;
  }
  const int b = bq / n_q;
  const int qi = bq - b * n_q;

  // Query slice: lane holds Q[head][16ks + 8g .. +7] for every k-step.  Its
  // address needs neither kv_lens nor the block table, so the loads go out
  // first and travel while those two dependent scalar loads return.
  bf16x8 qreg[KSTEPS];
  {
    const bf16x8* const qp =
        (const bf16x8*)(q + ((size_t)bq * n_h + head) * ROW) + g;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qreg[ks] = qp[2 * ks];
  }

  const int kv = kv_lens[b];
  const int visible = kv - n_q + qi + 1;  // keys 0 .. P
  const int nblk = (visible + BS - 1) / BS;
  // Split j covers blocks [j nblk / n_split, (j + 1) nblk / n_split).
  const int blk0 = (int)((long)split * nblk / n_split);
  const int blk1 = (int)((long)(split + 1) * nblk / n_split);
  const size_t row_base = ((size_t)slot0 + split) * n_h;

  if (blk0 >= blk1) {
    // No visible key (an empty split, or kv_len < n_q): weight zero in the
    // combine.  With one split there are no partials; the row's output is
    // written as zeros with lse = -inf instead.
    if (n_split == 1) {
      float* dst = o_final + ((size_t)bq * n_h + head) * DC;
      for (int c = 4 * g; c < DC; c += 8) *(f32x4*)(dst + c) = (f32x4){0, 0, 0, 0};
      if (g == 0 && lse_final) lse_final[(size_t)bq * n_h + head] = -INFINITY;
    } else if (g == 0) {
      m_part[row_base + head] = -INFINITY;
      l_part[row_base + head] = 0.0f;
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the query loads
    return;
  }
  const int tok0 = blk0 * BS;
  const int n_half = (min(blk1 * BS, visible) - tok0 + HT - 1) / HT;

  const int32_t* bt = block_table + (size_t)b * max_blocks;
  const uint32_t lds0 = lds_u32(lds);
  // The copies of half j from cache block `bid`.
  auto half_copy = [&](int j, int bid) __attribute__((always_inline)) {
    const int ts = tok0 + HT * j;
    return HalfCopy<NW, NTC>(cache + (size_t)bid * BLOCK_BYTES, j & 1,
                        lds0 + (j & (NBUF - 1)) * HALF_BYTES,
                        min(HT, visible - ts), wave, lane);
  };
  auto block_of = [&](int j) __attribute__((always_inline)) {
    return bt[(tok0 + HT * j) / BS];
  };
  auto issue = [&](int j) __attribute__((always_inline)) {
    const HalfCopy<NW, NTC> hc = half_copy(j, block_of(j));
    CopyAll<0, PER>::run(hc, wave);
  };

  f32x16 o[MTW][NW];
  float m_ref = -INFINITY;  // per owned head, log2 units
  float l_run = 0.0f;
  bool pass_ovf = false;    // a score exceeded m_ref + REF_SLACK this pass

  // Per-lane LDS byte offsets; every read is a buffer base plus one of these
  // plus an immediate.
  //  Scores, k-step ks: token t = col, chunk c = 2 ks + g, group (ks / 4,
  //  col / 8), c % 8 = 2 (ks % 4) + g:  a_s[ks % 4] + 4096 (ks / 4).
  int a_s[4];
  {
    const int t8 = col & 7;
    const int par = 2 * ((col >> 3) & 1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a_s[j] = (col >> 3) * 1024 + t8 * 128 +
               16 * ((2 * j + g) ^ swz(t8) ^ par);
  }
  //  Values, k-step kk (16 tokens), read h in {0,1}, latent tile mt of the
  //  wave (global tile MTW w + mt): the 16-lane group q16 supplies rows
  //  t = 16 kk + 8 h + vt (vt = 4 (q16 / 2) + s16 / 4) and the 4 bf16 at
  //  chunk c = 4 (MTW w + mt) + vc (vc = 2 (q16 % 2) + (s16 % 4) / 2), byte
  //  8 (s16 % 2).  After the transposing read, lane L holds latent column
  //  L % 32 of the tile for tokens 16 kk + 8 h + 4 (L / 32) + 0..3, i.e. MFMA
  //  k slot 8 g + e <-> token 16 kk + 8 (e / 4) + 4 g + e % 4, the order of
  //  the score accumulator rows.  Group (c / 8, t / 8):
  //  a_v[mt % 2] + 4096 (mt / 2) + 2048 kk, then for h = 1 the chunk parity
  //  term (byte offset ^ 32) and + 1024.
  int a_v[2];
  {
    const int q16 = lane >> 4, s16 = lane & 15;
    const int vt = 4 * (q16 >> 1) + (s16 >> 2);
    const int vc = 2 * (q16 & 1) + ((s16 & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      a_v[e] = vt * 128 + 16 * ((4 * e + vc) ^ swz(vt)) + 8 * (s16 & 1) +
               4096 * (MTW / 2) * wave;
  }
  //  P of a half: head-major rows of 64 bytes, chunk 2 kk + g holding k slots
  //  8 g .. 8 g + 7 of k-step kk (bf16), at position (2 kk + g) ^ ((h / 4) % 4)
  //  so that 16 consecutive heads hit 16 distinct 16-byte bank groups.
  //  Head 32 nt + col: a_p[kk] + 2048 nt.
  int a_p[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    a_p[kk] = 64 * col + 16 * ((2 * kk + g) ^ ((col >> 2) & 3));
  int* const flags = (int*)(lds + C::P_OFF);

  // Scores of half j: two interleaved accumulation chains (even / odd k
  // steps), so consecutive MFMAs never wait on each other's results.
  auto s_phase = [&](int j, auto hook) __attribute__((always_inline)) {
    const lds_char* kb = L + (j & (NBUF - 1)) * HALF_BYTES;
    const lds_char* sp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sp[i] = kb + a_s[i];
    auto frag = [&](int ks) __attribute__((always_inline)) {
      return *(const lds_bf16x8*)(sp[ks & 3] + 4096 * (ks >> 2));
    };
    bf16x8 af[SDEPTH];
#pragma unroll
    for (int i = 0; i < SDEPTH; ++i) af[i] = frag(i);
    f32x16 sa = mfma_v_first(af[0], qreg[0]);
    af[0] = frag(SDEPTH);
    hook(0);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 sb = mfma_v_first(af[1], qreg[1]);
    af[1] = frag(SDEPTH + 1);
    hook(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 2; ks < KSTEPS; ++ks) {
      mfma_v_acc((ks & 1) ? sb : sa, af[ks % SDEPTH], qreg[ks]);
      if (ks + SDEPTH < KSTEPS) af[ks % SDEPTH] = frag(ks + SDEPTH);
      hook(ks);
      __builtin_amdgcn_sched_barrier(0);  // keep the ring depth as written
    }
    mfma_v_drain(sb);  // sa's last MFMA is one MFMA further back
    return sa + sb;
  };

  // Softmax of one half tile, split in steps so that it can be spread over
  // the value MFMAs (scores s are raw dot products; scale_log2 > 0 turns
  // them into log2 units, so the maximum can be taken before scaling):
  //   step r = 0..15  : running max of the raw scores
  //   step 16         : per-head max over both lane halves, scaled;
  //                     reference update
  //   step 17..24     : P = 2^(s scale - m_ref) for a pair, bf16 pack, row sum
  struct Half {
    f32x16 s;
    float tmax;
    uint32_t pw[8];
  };
  auto softmax_step = [&](Half& H, int step) __attribute__((always_inline)) {
    if (step < 16) {
      const int r = step;
      H.tmax = r == 0 ? H.s[0] : fmaxf(H.tmax, H.s[r]);
    } else if (step == 16) {
      const float t = fmaxf(H.tmax, lane_xor32(H.tmax, g)) * scale_log2;
      if (m_ref == -INFINITY) m_ref = t;  // first half tile of the split
      const bool ovf = t > m_ref + REF_SLACK;
      m_ref = ovf ? t : m_ref;            // raised reference, next pass
      pass_ovf |= ovf;
    } else if (step < 25) {
      const int e = step - 17;
      const float p0 =
          __builtin_amdgcn_exp2f(__builtin_fmaf(H.s[2 * e], scale_log2, -m_ref));
      const float p1 = __builtin_amdgcn_exp2f(
          __builtin_fmaf(H.s[2 * e + 1], scale_log2, -m_ref));
      const bf16x2 pb = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
      H.pw[e] = __builtin_bit_cast(uint32_t, pb);
      // The sum uses the same bf16 weights as the value product.
      l_run = __builtin_amdgcn_fdot2_f32_bf16(
          pb, __builtin_bit_cast(bf16x2, 0x3F803F80u), l_run, false);
      // Materialise here, between the MFMAs this step is spread over,
      // instead of being sunk towards its use.
      asm volatile("" : "+v"(H.pw[e]), "+v"(l_run));
    }
  };
  // Keys at or past `lim` (only in the last half tile of a sequence) get
  // score -inf, hence weight 0.  Accumulator row r of lane half g is token
  // 8 (r / 4) + 4 g + r % 4.
  auto mask = [&](Half& H, int lim) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 8 * (r >> 2) + 4 * g + (r & 3);
      H.s[r] = t < lim ? H.s[r] : -INFINITY;
    }
  };
  // P of half j (already in k-slot order: pw[4 kk .. 4 kk + 3] are k slots
  // 8 g .. 8 g + 7 of k-step kk) to the P buffer of j.
  auto store_p = [&](int j, const Half& H) __attribute__((always_inline)) {
    lds_char* pb = L + C::P_OFF + (j & 1) * C::PBYTES + 2048 * wave;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      *(lds_u32x4*)(pb + a_p[kk]) = (u32x4){H.pw[4 * kk], H.pw[4 * kk + 1],
                                            H.pw[4 * kk + 2], H.pw[4 * kk + 3]};
  };

  // Step j, one instruction stream: the scores of half j+1 (36 MFMAs on the
  // keys in buffer (j+1) % 4) and the values of half j (32 MFMAs,
  // O^T[tile mt][head tile nt] += V^T(mt, kk) P(nt, kk), value MFMA
  // i = NW (MTW kk + mt) + nt).  Part A (16 groups): group g issues the score
  // MFMAs (36 g / 16) .. (36 (g+1) / 16) - 1 and value MFMA g, so the key
  // reads of the score MFMAs and the value/P reads share the LDS evenly and
  // neither kind of MFMA waits for a whole phase of reads.  Part B: value
  // MFMAs 16 .. 31, with the softmax of half j+1 spread over them.  The
  // copies of half j+3 go with the groups of part A.  Scores of the step
  // after the last half are computed on stale buffer contents and fully
  // masked by the caller's lim (0 there).
  auto step = [&](int j, Half& H, int lim, const HalfCopy<NW, NTC>& hc,
                  bool copying) __attribute__((always_inline)) {
    constexpr int AR = C::AR;
    constexpr int NPV = 2 * MTW * NW;  // value MFMAs per half: 32
    constexpr int NG = NPV / 2;        // groups of part A (kk = 0)
    static_assert(NPV == 32, "value MFMAs per half");
    // keys of half j+1
    const lds_char* kb = L + ((j + 1) & (NBUF - 1)) * HALF_BYTES;
    const lds_char* sp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sp[i] = kb + a_s[i];
    auto frag = [&](int ks) __attribute__((always_inline)) {
      return *(const lds_bf16x8*)(sp[ks & 3] + 4096 * (ks >> 2));
    };
    // values and P of half j
    const int vb = (j & (NBUF - 1)) * HALF_BYTES;
    const lds_char* pb = L + C::P_OFF + (j & 1) * C::PBYTES;
    const int vp0 = vb + a_v[0];
    const int vp1 = vb + a_v[1];
    auto vfrag = [&](int p) __attribute__((always_inline)) {
      const int kk = p / MTW, mt = p % MTW;
      // Bit 5 of every other term is 0, so ^ 32 flips the chunk parity.
      const int off = ((mt & 1) ? vp1 : vp0) + 4096 * (mt >> 1) + 2048 * kk;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(L + off));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(L + ((off ^ 32) + 1024)));
      const s16x8 lohi =
          __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, lohi);
    };
    auto pfrag = [&](int kk, int nt) __attribute__((always_inline)) {
      return *(const lds_bf16x8*)(pb + a_p[kk] + 2048 * nt);
    };
    bf16x8 pf[NW];
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) pf[nt] = pfrag(0, nt);
    bf16x8 vf[AR];
#pragma unroll
    for (int p = 0; p < AR; ++p) vf[p] = vfrag(p);
    bf16x8 af[SDEPTH];
#pragma unroll
    for (int i = 0; i < SDEPTH; ++i) af[i] = frag(i);

    f32x16 sa, sb;
    auto s_mfma = [&](int ks) __attribute__((always_inline)) {
      if (ks == 0)
        sa = mfma_v_first(af[0], qreg[0]);
      else if (ks == 1)
        sb = mfma_v_first(af[1], qreg[1]);
      else
        mfma_v_acc((ks & 1) ? sb : sa, af[ks % SDEPTH], qreg[ks]);
      if (ks + SDEPTH < KSTEPS) af[ks % SDEPTH] = frag(ks + SDEPTH);
      __builtin_amdgcn_sched_barrier(0);  // keep the ring depth as written
    };
    auto v_mfma = [&](int i) __attribute__((always_inline)) {
      const int p = i / NW, nt = i % NW, mt = p % MTW;
      o[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[p % AR], pf[nt],
                                                          o[mt][nt], 0, 0, 0);
      // P of kk = 1 replaces that of kk = 0 after its last use.
      if (p == MTW - 1) pf[nt] = pfrag(1, nt);
      if (nt == NW - 1 && p + AR < 2 * MTW) vf[p % AR] = vfrag(p + AR);
      __builtin_amdgcn_sched_barrier(0);
    };

    // Part A
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int ks = (KSTEPS * g) / NG; ks < (KSTEPS * (g + 1)) / NG; ++ks)
        s_mfma(ks);
      v_mfma(g);
      copy_group<PER, NG>(hc, wave, g, copying);
    }
    mfma_v_drain(sb);  // sa's last MFMA is one MFMA further back
    H.s = sa + sb;
    if (lim < HT) mask(H, lim);
    // Part B: softmax steps 0..7, 8..15, 16, then one exponent pair each.
#pragma unroll
    for (int i = NG; i < NPV; ++i) {
      v_mfma(i);
      const int k = i - NG;
      if (k == 0) {
#pragma unroll
        for (int st = 0; st < 8; ++st) softmax_step(H, st);
      } else if (k == 1) {
#pragma unroll
        for (int st = 8; st < 16; ++st) softmax_step(H, st);
      } else if (k < 11) {
        softmax_step(H, k + 14);
      }
    }
  };

  // Passes over the split: a second one only after an overflow.  m_ref only
  // rises, and after the first pass every half tile's maximum is at most
  // m_ref + REF_SLACK, so the second pass cannot overflow; the loop stops
  // there regardless.
  // The copies of half 0 of the first pass go out right behind the query
  // loads, before the pass loop (whose header reloads spilled values).
  issue(0);
  for (int pass = 0;; ++pass) {
    // Prologue: the scores and P of half 0 start as soon as its copies and
    // the query slice landed, while halves 1 and 2 are in flight.  The query
    // loads are retired by a wait the compiler sees (a builtin, not asm),
    // issued before the copies of halves 1 and 2: the compiler's own waits
    // for the query registers then never stand for those copies, and inside
    // the loop vmcnt tracks the copies only.
    if (pass > 0) issue(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if (n_half > 1) issue(1);
    if (n_half > 2) issue(2);
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int nt = 0; nt < NW; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mt][nt][r] = 0.0f;
    barrier();  // half 0 visible to every wave
    {
      Half h;
      h.s = s_phase(0, [](int) __attribute__((always_inline)) {});
      const int lim = visible - tok0;
      if (lim < HT) mask(h, lim);
#pragma unroll
      for (int st = 0; st < 25; ++st) softmax_step(h, st);
      store_p(0, h);
    }
    // Half 1 landed before the first step's barrier; half 2 may stay in
    // flight.
    if (n_half > 2)
      wait_vm<PER>();
    else
      wait_vm<0>();
    wait_lgkm0();

    // Step j: entry state (after the barrier) is P of half j and the
    // copies of halves j and j+1 visible, half j+2 in flight, and every
    // wave done with half j-1; so half j+3 goes into j-1's buffer.
    // The last step has no next half: its scores are skipped and a fully
    // masked softmax (lim = 0) leaves m_ref, l and the flags alone (P = 0,
    // maximum -inf), so one body serves every step.
    // The block id of the half copied in step j is loaded one step ahead
    // (a scalar load, complete by the end-of-step lgkm wait).  The copies
    // are spread over the value MFMAs: issued together, the workgroup's 36
    // copies queue at the address unit (16 cycles each per CU) and block
    // the issuing waves; spread out, the queue drains while they compute.
    int bid_next = n_half > 3 ? block_of(3) : 0;
    for (int j = 0; j < n_half; ++j) {
      barrier();
      const bool copying = j + 3 < n_half;
      const HalfCopy<NW, NTC> hc = half_copy(j + 3, bid_next);
      if (j + 4 < n_half) bid_next = block_of(j + 4);
      const bool next = j + 1 < n_half;
      Half h;
      step(j, h, next ? visible - (tok0 + HT * (j + 1)) : 0, hc, copying);
      if (next) store_p(j + 1, h);
      // Half j+2 must have landed by the next barrier; j+3 may stay in
      // flight.
      if (j + 3 < n_half)
        wait_vm<PER>();
      else
        wait_vm<0>();
      wait_lgkm0();
    }

    // Restart the split when any wave saw a score beyond its reference.
    // The flags use the P buffer that the last step did not read (P of
    // half n_half - 1 sits in buffer (n_half - 1) % 2).
    int* fl = flags + (n_half & 1) * (C::PBYTES / 4);
    if (lane == 0) fl[wave] = __builtin_amdgcn_ballot_w64(pass_ovf) != 0;
    wait_lgkm0();
    barrier();
    int any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= fl[w];
    if (!any || pass > 0) break;
    l_run = 0.0f;
    pass_ovf = false;
  }

  // ---- epilogue ----------------------------------------------------------
  // l of every head of the workgroup, through the P buffer the last step
  // read (free after the flag barrier, and apart from the flags).
  l_run += lane_xor32(l_run, g);
  float* lsh = (float*)(lds + C::P_OFF + ((n_half - 1) & 1) * C::PBYTES);
  if (g == 0) lsh[wave * 32 + col] = l_run;
  wait_lgkm0();
  barrier();
  float l_nt[NW];
#pragma unroll
  for (int nt = 0; nt < NW; ++nt) l_nt[nt] = lsh[nt * 32 + col];

  // O^T accumulator (mt, nt), register r: head hbase + 32 nt + col, latent
  // 32 (MTW w + mt) + 8 (r / 4) + 4 g + r % 4.
  if (n_split == 1) {
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
      const float inv = 1.0f / l_nt[nt];
      float* dst = o_final + ((size_t)bq * n_h + hbase + 32 * nt + col) * DC +
                   32 * MTW * wave;
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 v = {o[mt][nt][4 * i] * inv, o[mt][nt][4 * i + 1] * inv,
                     o[mt][nt][4 * i + 2] * inv, o[mt][nt][4 * i + 3] * inv};
          *(f32x4*)(dst + 32 * mt + 8 * i + 4 * g) = v;
        }
    }
    if (g == 0 && lse_final)
      lse_final[(size_t)bq * n_h + head] =
          (m_ref + __log2f(l_run)) * 0.69314718055994531f;
  } else {
    // fp16 partials: row (query row, split, head) of DC elements holding
    // O / (l s), s = 2^e per head with e chosen so that the head's largest
    // |O / l| lands in [2^14, 2^15): any input range fits fp16 (max 65504)
    // and every value keeps 11 significant bits.  The rows' scales follow
    // the fp16 rows in the same buffer.  Per-head maxima cross the waves
    // through the first half-tile buffer: no copy is in flight and every
    // wave is past its last read of it (flag barrier above).  The rows
    // themselves are assembled in LDS (the ring is free) and stored whole:
    // stored straight from the accumulator layout, every instruction would
    // write 32 scattered 16-byte pieces, and the stores then took most of
    // the epilogue.
    uint16_t* const o16 = (uint16_t*)o_part;
    float* const sc_part = (float*)(o16 + (size_t)slots * n_h * DC);
    float* const mx = (float*)lds;  // [NW][HEADS]
    float inv[NW];
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
      inv[nt] = 1.0f / l_nt[nt];  // l >= 1: the maximum key has P = 1
      float a = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) a = fmaxf(a, fabsf(o[mt][nt][r]));
      a = fmaxf(a, lane_xor32(a, g)) * inv[nt];
      if (g == 0) mx[wave * C::HEADS + 32 * nt + col] = a;
    }
    wait_lgkm0();
    barrier();
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
      float hm = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) hm = fmaxf(hm, mx[w * C::HEADS + 32 * nt + col]);
      const int e = hm > 0.0f
                        ? min(max(__builtin_amdgcn_frexp_expf(hm) - 15, -100), 120)
                        : 0;
      const float mul = inv[nt] * __builtin_amdgcn_ldexpf(1.0f, -e);
      // this lane's 4-column pieces into LDS row 32 nt + col
      lds_char* row = L + EPI_OFF + (32 * nt + col) * EPI_STRIDE +
                      2 * 32 * MTW * wave;
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f16x4 h = __builtin_convertvector(
              ((f32x4){o[mt][nt][4 * i], o[mt][nt][4 * i + 1],
                       o[mt][nt][4 * i + 2], o[mt][nt][4 * i + 3]}) * mul,
              f16x4);
          *(lds_u32x2*)(row + 2 * (32 * mt + 8 * i + 4 * g)) =
              __builtin_bit_cast(u32x2, h);
        }
      if (g == 0 && wave == 0)
        sc_part[row_base + hbase + 32 * nt + col] =
            __builtin_amdgcn_ldexpf(1.0f, e);
    }
    wait_lgkm0();
    barrier();
    // Wave w stores rows 32 w .. 32 w + 31, one whole 1 KiB row per
    // instruction (16 bytes per lane), eight rows in flight.
    {
      uint16_t* const dst0 = o16 + (row_base + hbase + 32 * wave) * DC;
      const lds_char* const src0 = L + EPI_OFF + 32 * wave * EPI_STRIDE;
#pragma unroll
      for (int r0 = 0; r0 < 32; r0 += 8) {
        u32x4 v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
          v[r] = *(const lds_u32x4*)(src0 + (r0 + r) * EPI_STRIDE + 16 * lane);
#pragma unroll
        for (int r = 0; r < 8; ++r)
          *(u32x4*)(dst0 + (size_t)(r0 + r) * DC + 8 * lane) = v[r];
      }
    }
    if (g == 0) {
      m_part[row_base + head] = m_ref;
      l_part[row_base + head] = l_run;
    }
  }
}

template <int NW, bool NTC = false>
hipError_t launch_nw(const mla_dims& d, int B, int n_q, const void* q,
                     const void* cache, const int32_t* block_table,
                     int max_blocks, const int32_t* kv_lens, int n_split,
                     const DecodeBalance& bal, float* o_part, float* m_part,
                     float* l_part, float* o_final, float* lse_final,
                     hipStream_t stream) {
  const float scale_log2 =
      (float)(1.4426950408889634 / __builtin_sqrt((double)(d.d_h + d.d_r)));
  constexpr size_t lds = Cfg<NW>::LDS;
  static std::atomic<unsigned long long> lds_set{0};
  {
    const hipError_t e = set_lds_limit_once(
        (const void*)decode_mfma_kernel<NW, NTC>, (int)lds, lds_set);
    if (e != hipSuccess) return e;
  }
  const int rows = B * n_q;
  const int slots = bal.plan ? BAL_SLOTS : rows * n_split;
  const dim3 grid(bal.plan ? BAL_SLOTS : rows, bal.plan ? 1 : n_split,
                  d.n_h / (NW * 32));
  hipLaunchKernelGGL((decode_mfma_kernel<NW, NTC>), grid, dim3(NW * 64), lds,
                     stream,
                     (const uint16_t*)q, (const char*)cache, block_table,
                     max_blocks, kv_lens, n_q, d.n_h, n_split, rows, slots,
                     bal.plan, scale_log2, o_part, m_part, l_part, o_final,
                     lse_final);
  return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_c == DC && d.d_r == DR &&
         d.block_size == BS &&
         (d.n_h % 128 == 0 || d.n_h == 64 || d.n_h == 32);
}

hipError_t launch_decode_mfma(const mla_dims& d, int B, int n_q,
                              const void* q, const void* cache,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* kv_lens, int n_split,
                              const DecodeBalance& balance, float* o_part,
                              float* m_part, float* l_part, float* o_final,
                              float* lse_final, bool cache_nt,
                              hipStream_t stream) {
  if (balance.plan && B * n_q > BAL_SLOTS) return hipErrorInvalidValue;
#define MLA_DECODE_ARGS                                                     \
  d, B, n_q, q, cache, block_table, max_blocks, kv_lens, n_split, balance, \
      o_part, m_part, l_part, o_final, lse_final, stream
  if (d.n_h % 128 == 0) {
    // Small grids (a batch of one or two sequences): two workgroups of 64
    // heads per (query row, split), so that twice the compute units stream
    // the cache and each loads half the queries (B = 1 at 4K context: 32.6
    // -> 27.5 us).  Per-head arithmetic is unchanged, so the results are
    // identical.
    const long wgs = balance.plan ? balance.est_wgs : (long)B * n_q * n_split;
    if (wgs * (d.n_h / 128) <= 128) return launch_nw<2>(MLA_DECODE_ARGS);
    // Cache rows read once per call (see the caller) are copied with
    // non-temporal loads.
    if (cache_nt) return launch_nw<4, true>(MLA_DECODE_ARGS);
    return launch_nw<4>(MLA_DECODE_ARGS);
  }
  if (d.n_h == 64) return launch_nw<2>(MLA_DECODE_ARGS);
  if (d.n_h == 32) return launch_nw<1>(MLA_DECODE_ARGS);
#undef MLA_DECODE_ARGS
  return hipErrorInvalidValue;
}

}  // namespace mla
