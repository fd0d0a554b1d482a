// Split-KV MLA decode on gfx950 matrix cores, latent width 512 + RoPE 64.
//
// What is computed ('MLA：潜在表示压缩与解耦 RoPE', sections 4, 6 and 7;
// 'Latent 压缩', MLA section): for one (sequence b, query i) and every head h,
//   score_s = (q_lat_h . c_KV_s + q_R_h . k_R_s) / sqrt(d_h + d_r)
//   o_lat_h = sum_s softmax(score)_s c_KV_s
// over the key range of one split.  In the latent space every head uses the
// same key (the 576-wide cache row) and the same value (its first 512
// columns), so one workgroup serves all heads and each cache tile crosses
// HBM once.
//
// Work decomposition (one workgroup = NW waves, NW * 32 heads):
//   * wave w owns heads 32w .. 32w+31.  Its query slice Q[32][576] lives in
//     VGPRs as 36 MFMA B-operands; its output O^T[512][32] fp32 is 16
//     32x32 accumulators (the whole accumulation register file).
//   * keys stream in 64-token tiles (one cache block).  A tile is copied
//     HBM -> LDS by direct-to-LDS loads (no VGPR staging) into one of two
//     buffers, so tile k+1 is in flight while tile k is consumed.
//   * LDS tile layout: 16-byte chunk c (of 72 per row) of token t lives in
//     group (c / 8, t / 8) of 64 chunks (1 KiB), at position
//     8 (t % 8) + ((c % 8) ^ swz(t % 8)).  One DMA instruction fills one
//     group, i.e. 8 tokens x 128 contiguous bytes; the XOR makes both read
//     patterns below bank-conflict free.
//   * each tile is processed as two 32-token halves:
//       scores S^T[32 tok][32 heads] = K . Q^T: 36 MFMA 32x32x16 (A = K rows
//       from LDS, B = Q from VGPRs; accumulators in VGPRs);
//       softmax in base 2 against a reference maximum m_ref per head, taken
//       from the split's first half-tile: P = 2^(s - m_ref), rounded to
//       bf16; l and O accumulate with no rescaling, so O is never touched by
//       vector ALU code inside the loop.  Keys far below m_ref underflow to
//       0 as in any softmax; a half-tile whose maximum exceeds m_ref by more
//       than 2^64 (still finite, but beyond the range trusted for P and the
//       sums) makes the workgroup restart the split with a raised m_ref.
//       Real scores never span that range; the restart keeps the result
//       exact for inputs that do;
//       values O^T[512][32] += V^T[512][32 tok] . P^T: 16 x 2 MFMA.  The A
//       operand (V^T) comes straight from the LDS tile through
//       ds_read_b64_tr_b16 transposing loads; P^T is already in the right
//       lanes because the MFMA k-slots are mapped to tokens the way the
//       score accumulator lays them out.
//   * the workgroup writes its unnormalised O, m_ref (log2 units) and l, or
//     the final o_lat and lse when there is one split.

#include "mla_common.hpp"
#include "mla_kernels.hpp"

namespace mla {
namespace {

constexpr int DC = 512;
constexpr int DR = 64;
constexpr int ROW = DC + DR;          // elements per cache row
constexpr int ROWB = ROW * 2;         // bytes per cache row
constexpr int BS = 64;                // tokens per block (= tile)
constexpr int CHUNKS = ROWB / 16;     // 72 sixteen-byte chunks per row
constexpr int TILE_BYTES = BS * ROWB; // 73728
constexpr int GROUPS = CHUNKS / 8 * BS / 8;  // 72 DMA groups per tile
constexpr int KSTEPS = ROW / 16;      // 36 k-steps of the score MFMA
constexpr int MT_LAT = DC / 32;       // 16 latent tiles of the value MFMA
constexpr float REF_SLACK = 64.0f;    // log2 headroom above m_ref

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

// Swizzle of the chunk position inside a row of 8 chunks, keyed by t % 8.
__device__ __forceinline__ int swz(int t8) { return ((2 * t8) & 7) | (t8 >> 2); }

// Score MFMAs with the accumulator pinned to VGPRs.  The output O^T of a
// wave fills all 256 accumulation registers, so the score accumulators must
// live in the other register file; the compiler picks one file for every
// MFMA of a function, so these few are written out.  Hazards the compiler
// cannot see through the asm: the first MFMA of a chain takes a literal 0 as
// accumulator (no VALU write feeds it), back-to-back accumulation into the
// same registers needs no wait states, and mfma_v_drain adds the wait
// states a 32x32x16 result needs before VALU reads it (>= 18).
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

// Tile copies, their waits and the tile barriers are written out: the
// compiler tracks direct-to-LDS loads conservatively and would wait for the
// whole prefetch before every transposing LDS read, serialising copy and
// compute.  None of these statements returns a register, and each is a
// compiler memory barrier ("memory" clobber), so LDS reads stay between the
// waits and barriers they are written between.
//
// dma16: the wave's 64 lanes copy 16 bytes each from sbase + voff (lane's
// offset) to LDS address lds_addr + 16 * lane.  M0 carries the LDS address;
// one wait state separates its write from the load that reads it.
__device__ __forceinline__ void dma16(uint32_t lds_addr, const char* sbase,
                                      uint32_t voff) {
  // Both addresses are wave-uniform; readfirstlane makes that explicit so
  // they can sit in scalar registers.
  // readfirstlane returns a signed int: convert through uint32_t so the
  // low word is zero-extended, not sign-extended, into the 64-bit address.
  const uint64_t b = (uint64_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %1"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "s"((const char*)sb),
        "v"(voff)
      : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() {
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
}
__device__ __forceinline__ void barrier() {
  asm volatile("s_barrier" : : : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Copy one 64-token block into an LDS tile.  Wave `wave` issues groups
// k = wave, wave + NW, ...; group k = (chunk group k / 8, token group k % 8).
// Lane l fetches token 8 (k % 8) + l / 8, chunk 8 (k / 8) + ((l % 8) ^
// swz(l / 8)).  Rows at or past `nvalid` are filled from the last valid row:
// their scores are masked, and finite data keeps 0 * value at zero.
template <int NW>
__device__ __forceinline__ void issue_tile(const char* __restrict__ blk,
                                           char* lds_tile, int nvalid,
                                           int wave, int lane) {
  constexpr int PER_WAVE = GROUPS / NW;
  static_assert(GROUPS % NW == 0, "tile groups must split evenly over waves");
  static_assert(PER_WAVE <= 63, "outstanding loads must fit the vmcnt field");
  const int tl = lane >> 3;
  uint32_t lane_off = tl * ROWB + ((lane & 7) ^ swz(tl)) * 16;
  // Opaque per tile, so the per-copy offsets below are recomputed (one add
  // each) instead of being hoisted into long-lived registers.
  asm volatile("" : "+v"(lane_off));
  const uint32_t lds0 = lds_u32(lds_tile);
  if (nvalid == BS) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int k = j * NW + wave;
      dma16(lds0 + k * 1024, blk,
            lane_off + 8 * (k & 7) * ROWB + (k >> 3) * 128);
    }
  } else {  // the last, partial block of a sequence
    const uint32_t ch = lane_off - tl * ROWB;
#pragma unroll 1
    for (int j = 0; j < PER_WAVE; ++j) {
      const int k = j * NW + wave;
      const int t = min(8 * (k & 7) + tl, nvalid - 1);
      dma16(lds0 + k * 1024, blk, t * ROWB + (k >> 3) * 128 + ch);
    }
  }
}

template <int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(1, 1))) void
decode_mfma_kernel(
    const uint16_t* __restrict__ q, const char* __restrict__ cache,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ kv_lens, int n_q, int n_h, int n_split, float scale_log2, float* __restrict__ o_part,
    float* __restrict__ m_part, float* __restrict__ l_part,
    float* __restrict__ o_final, float* __restrict__ lse_final) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int PER_WAVE = GROUPS / NW;
  typedef __attribute__((address_space(3))) char lds_char;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;     // lane half
  const int col = lane & 31;   // head within the wave
  const int bq = blockIdx.x;   // b * n_q + i
  const int split = blockIdx.y;
  const int head = blockIdx.z * NW * 32 + wave * 32 + col;
  const int b = bq / n_q;
  const int qi = bq - b * n_q;

  const int kv = kv_lens[b];
  const int visible = kv - n_q + qi + 1;  // keys 0 .. P
  const int nblk = (visible + BS - 1) / BS;
  // Split j covers blocks [j nblk / n_split, (j + 1) nblk / n_split).
  const int blk0 = (int)((long)split * nblk / n_split);
  const int blk1 = (int)((long)(split + 1) * nblk / n_split);
  const size_t row_id = ((size_t)bq * n_split + split) * n_h + head;

  if (blk0 >= blk1) {  // empty split: no keys, weight zero in the combine
    if (g == 0) {
      m_part[row_id] = -INFINITY;
      l_part[row_id] = 0.0f;
    }
    return;
  }

  const int32_t* bt = block_table + (size_t)b * max_blocks;
  issue_tile<NW>(cache + (size_t)bt[blk0] * TILE_BYTES, lds,
                 min(BS, visible - blk0 * BS), wave, lane);

  // Query slice: lane holds Q[head][16ks + 8g .. +7] for every k-step.
  bf16x8 qreg[KSTEPS];
  {
    const bf16x8* qp =
        (const bf16x8*)(q + ((size_t)bq * n_h + head) * ROW) + g;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qreg[ks] = qp[2 * ks];
  }
  // The first tile is needed before any compute anyway; waiting for every
  // load here also tells the compiler that no query load is outstanding
  // inside the loop, where vmcnt only tracks the prefetch of the next tile.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  wait_vm<0>();

  f32x16 o[MT_LAT];
#pragma unroll
  for (int i = 0; i < MT_LAT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
  float m_ref = -INFINITY;  // per head, log2 units
  float l_run = 0.0f;
  int* restart_flag = (int*)(lds + 2 * TILE_BYTES);  // [2][NW]

  // Per-lane LDS byte offsets; every read is one of these plus an
  // immediate.  Group (cg, tg) starts at 1024 (8 cg + tg).
  //  Scores, half hf, k-step ks: token t = 32 hf + col, chunk c = 2 ks + g:
  //  cg = ks / 4, tg = 4 hf + col / 8, c % 8 = 2 (ks % 4) + g, so
  //  a_s[ks % 4] + 8192 (ks / 4) + 4096 hf; for ks / 4 >= 4 the first
  //  32 KiB of that offset sits in a_s[4 + ks % 4] so that immediates stay
  //  below 64 KiB.
  int a_s[8];
  {
    const int t8 = col & 7;
    const int base = (col >> 3) * 1024 + t8 * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a_s[j] = base + 16 * ((2 * j + g) ^ swz(t8));
      a_s[4 + j] = a_s[j] + 32768;
    }
  }
  //  Values, half hf, k-step kk (16 tokens), read h in {0,1}, latent tile
  //  mtl: the 16-lane group q16 supplies rows t = 32 hf + 16 kk + 8 h + vt
  //  (vt = 4 (q16 / 2) + s16 / 4) and the 4 bf16 at chunk c = 4 mtl + vc
  //  (vc = 2 (q16 % 2) + (s16 % 4) / 2), byte 8 (s16 % 2).  cg = mtl / 2,
  //  tg = 4 hf + 2 kk + h, c % 8 = 4 (mtl % 2) + vc:
  //  a_v[mtl % 2] + 8192 (mtl / 2) + 1024 (4 hf + 2 kk + h).
  int a_v[2];
  {
    const int q16 = lane >> 4, s16 = lane & 15;
    const int vt = 4 * (q16 >> 1) + (s16 >> 2);
    const int vc = 2 * (q16 & 1) + ((s16 & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      a_v[e] = vt * 128 + 16 * ((4 * e + vc) ^ swz(vt)) + 8 * (s16 & 1);
  }

  int first = blk0;  // first tile of the current pass over the split
  for (int kb = blk0; kb < blk1; ++kb) {
    const int cur_off = ((kb - first) & 1) * TILE_BYTES;
    char* cur = lds + cur_off;
    lds_char* curl = (lds_char*)cur;
    const bool more = kb + 1 < blk1;
    if (more) {
      issue_tile<NW>(cache + (size_t)bt[kb + 1] * TILE_BYTES,
                     lds + (TILE_BYTES - cur_off),
                     min(BS, visible - (kb + 1) * BS), wave, lane);
      wait_vm<PER_WAVE>();  // this tile landed, the next one is in flight
    } else {
      wait_vm<0>();
    }
    barrier();

    bool wave_ovf = false;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // ---- scores S^T = K Q^T for tokens 32 hf .. 32 hf + 31 ----------
      f32x16 s;
      s = mfma_v_first(*(const bf16x8*)(cur + a_s[0] + 4096 * hf), qreg[0]);
#pragma unroll
      for (int ks = 1; ks < KSTEPS; ++ks) {
        const int ka = ks >> 2;  // chunk group 0 .. 8
        const int hi = ka >= 4 ? 4 : 0;
        const bf16x8 a = *(const bf16x8*)(cur + a_s[hi + (ks & 3)] +
                                          8192 * (ka - hi) + 4096 * hf);
        mfma_v_acc(s, a, qreg[ks]);
      }
      mfma_v_drain(s);

      // ---- softmax against m_ref ----------------------------------------
      const int tok0 = kb * BS + 32 * hf;
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = tok0 + 8 * (r >> 2) + 4 * g + (r & 3);
        float v = s[r] * scale_log2;
        v = tok < visible ? v : -INFINITY;
        s[r] = v;
        tmax = fmaxf(tmax, v);
      }
      tmax = fmaxf(tmax, lane_xor32(tmax, g));
      if (m_ref == -INFINITY) m_ref = tmax;  // first half-tile of the split
      const bool ovf = tmax > m_ref + REF_SLACK;
      if (ovf) m_ref = tmax;  // raised reference for the next pass
      wave_ovf |= __builtin_amdgcn_ballot_w64(ovf) != 0;
      if (wave_ovf) continue;

      // P^T as MFMA B operands: k-step kk covers registers 8 kk .. 8 kk + 7.
      bf16x8 pb[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = exp2f(s[8 * kk + 2 * e] - m_ref);
          const float p1 = exp2f(s[8 * kk + 2 * e + 1] - m_ref);
          const uint32_t pk = pack_bf2(p0, p1);
          l_run +=
              __uint_as_float(pk << 16) + __uint_as_float(pk & 0xFFFF0000u);
          w4[e] = pk;
        }
        pb[kk] = __builtin_bit_cast(bf16x8, (u32x4){w4[0], w4[1], w4[2], w4[3]});
      }

      // ---- values O^T += V^T P^T ----------------------------------------
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int mtl = 0; mtl < MT_LAT; ++mtl) {
          const int imm = 8192 * (mtl >> 1) + 1024 * (4 * hf + 2 * kk);
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (s16x4 __attribute__((address_space(3)))*)(
                  curl + a_v[mtl & 1] + imm));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (s16x4 __attribute__((address_space(3)))*)(
                  curl + a_v[mtl & 1] + imm + 1024));
          const s16x8 lohi =
              __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[mtl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, lohi), pb[kk], o[mtl], 0, 0, 0);
        }
      }
    }
    if (lane == 0) restart_flag[(kb & 1) * NW + wave] = wave_ovf;
    // Every read of `cur` (and the flag write) has landed before any wave
    // may refill the buffer.
    wait_lgkm0();
    barrier();

    // Restart the split when any wave saw a score beyond its reference.
    int any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= restart_flag[(kb & 1) * NW + w];
    if (any) {
      wait_vm<0>();  // drain the prefetch
      barrier();
#pragma unroll
      for (int i = 0; i < MT_LAT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
      l_run = 0.0f;
      first = blk0;
      kb = blk0 - 1;
      issue_tile<NW>(cache + (size_t)bt[blk0] * TILE_BYTES, lds,
                     min(BS, visible - blk0 * BS), wave, lane);
    }
  }

  // ---- epilogue ----------------------------------------------------------
  l_run += lane_xor32(l_run, g);
  if (n_split == 1) {
    const float inv = 1.0f / l_run;
    float* dst = o_final + ((size_t)bq * n_h + head) * DC;
#pragma unroll
    for (int mtl = 0; mtl < MT_LAT; ++mtl)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 v = {o[mtl][4 * i] * inv, o[mtl][4 * i + 1] * inv,
                   o[mtl][4 * i + 2] * inv, o[mtl][4 * i + 3] * inv};
        *(f32x4*)(dst + 32 * mtl + 8 * i + 4 * g) = v;
      }
    if (g == 0 && lse_final)
      lse_final[(size_t)bq * n_h + head] =
          (m_ref + __log2f(l_run)) * 0.69314718055994531f;
  } else {
    float* dst = o_part + row_id * DC;
#pragma unroll
    for (int mtl = 0; mtl < MT_LAT; ++mtl)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 v = {o[mtl][4 * i], o[mtl][4 * i + 1], o[mtl][4 * i + 2],
                   o[mtl][4 * i + 3]};
        *(f32x4*)(dst + 32 * mtl + 8 * i + 4 * g) = v;
      }
    if (g == 0) {
      m_part[row_id] = m_ref;
      l_part[row_id] = l_run;
    }
  }
}

template <int NW>
hipError_t launch_nw(const mla_dims& d, int B, int n_q, const void* q,
                     const void* cache, const int32_t* block_table,
                     int max_blocks, const int32_t* kv_lens, int n_split,
                     float* o_part,
                     float* m_part, float* l_part, float* o_final,
                     float* lse_final, hipStream_t stream) {
  const float scale_log2 =
      (float)(1.4426950408889634 / __builtin_sqrt((double)(d.d_h + d.d_r)));
  const size_t lds = 2 * TILE_BYTES + 2 * NW * sizeof(int);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        (const void*)decode_mfma_kernel<NW>,
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid(B * n_q, n_split, d.n_h / (NW * 32));
  hipLaunchKernelGGL(decode_mfma_kernel<NW>, grid, dim3(NW * 64), lds, stream,
                     (const uint16_t*)q, (const char*)cache, block_table,
                     max_blocks, kv_lens, n_q, d.n_h, n_split, scale_log2, o_part, m_part, l_part, o_final,
                     lse_final);
  return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_c == DC && d.d_r == DR &&
         d.block_size == BS && d.n_h % 32 == 0 &&
         (d.n_h % 128 == 0 || d.n_h == 64 || d.n_h == 96);
}

hipError_t launch_decode_mfma(const mla_dims& d, int B, int n_q,
                              const void* q, const void* cache,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* kv_lens, int n_split,
                              float* o_part, float* m_part,
                              float* l_part, float* o_final, float* lse_final,
                              hipStream_t stream) {
#define MLA_DECODE_ARGS                                                    \
  d, B, n_q, q, cache, block_table, max_blocks, kv_lens, n_split, o_part, \
      m_part, l_part, o_final, lse_final, stream
  if (d.n_h % 128 == 0) return launch_nw<4>(MLA_DECODE_ARGS);
  if (d.n_h == 96) return launch_nw<3>(MLA_DECODE_ARGS);
  if (d.n_h == 64) return launch_nw<2>(MLA_DECODE_ARGS);
#undef MLA_DECODE_ARGS
  return hipErrorInvalidValue;
}

}  // namespace mla
