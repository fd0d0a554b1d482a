// Chunked prefill on the non-absorbed (MHA) path, gfx950 matrix cores.
//
// What is computed ('MLA：潜在表示压缩与解耦 RoPE', sections 4 and 7; 'MiniMind
// 学习笔记 10', sections 10 and 12: for many queries per step the explicit
// keys and values cost fewer operations than the absorbed form): for a chunk
// of n_q new tokens of each sequence b, the cached latents are up-projected
// once per head,
//   k_C[t, h] = W_UK_h c_KV[t],  v_C[t, h] = W_UV_h c_KV[t],
// and every query i of the chunk attends over the keys t <= kv_len - n_q + i
// (causal, bottom-right) with
//   score = (q_C[i, h] . k_C[t, h] + q_R[i, h] . k_R[t]) / sqrt(d_h + d_r),
//   o[i, h] = sum_t softmax(score)_t v_C[t, h],
// written in value space (d_v = d_h per head, fp32) with its log-sum-exp.
//
// Kernels:
//   gather_rows_kernel   the sequence's cache rows (paged) -> contiguous rows
//   (up-projection)      one GEMM, rows[:, :d_c] x [W_UK; W_UV]^T -> bf16
//   prefill_mha_kernel   causal flash attention, d_qk = 192, d_v = 128
//   query_mha_kernel     q_C (bf16) and RoPE(q_R) rows of the chunk
//
// prefill_mha_kernel: workgroup = (sequence, head, 128 queries), 4 waves of
// 32 queries.  Keys stream in tiles of 64 by direct-to-LDS copies through
// two-slot rings, one for keys (K_C 16 KiB + k_R 8 KiB per tile) and one for
// values (16 KiB), so that the score MFMAs of tile j + 1 run together with
// the value MFMAs of tile j (80 KiB: two workgroups per CU).  The
// scores are computed transposed, S^T = K Q^T (A = key rows from LDS, B =
// the wave's queries held in VGPRs), so each lane owns one query: its row
// maximum needs one exchange with the lane 32 away, and its probabilities,
// in the token order of the accumulator rows, are directly the B operand of
// O^T += V^T P^T (A = V^T through transposing LDS reads, the value layout of
// the decode kernel).  Online softmax in base 2 against a lazily moved
// reference: O and l are rescaled only when a tile's maximum exceeds the
// reference by more than 2^8 (a branch the whole wave takes or skips), so
// most tiles run no vector code on O; masks are applied only on tiles that
// cross the wave's causal limit.  The 16 query tiles of one (sequence,
// head) read the same keys; the grid maps them to one XCD so that the keys
// they stream together are shared through its L2.
#include "lds_dma.hpp"
#include "mla_common.hpp"
#include "mla_kernels.hpp"

namespace mla {
namespace {

constexpr int PF_QW = 128;          // queries per workgroup (4 waves x 32)
constexpr int PF_KT = 64;           // keys per tile
constexpr int PF_DH = 128;          // d_h = d_v
constexpr int PF_DR = 64;           // d_r
constexpr int PF_KS = (PF_DH + PF_DR) / 16;  // 12 k-steps of the scores
constexpr int PF_KC_BYTES = PF_KT * PF_DH * 2;   // 16 KiB
constexpr int PF_KR_OFF = PF_KC_BYTES;
constexpr int PF_KR_BYTES = PF_KT * PF_DR * 2;   // 8 KiB
constexpr int PF_KSLOT = PF_KR_OFF + PF_KR_BYTES;   // 24 KiB of keys
constexpr int PF_VSLOT = PF_KT * PF_DH * 2;          // 16 KiB of values
constexpr int PF_V_BASE = 2 * PF_KSLOT;
constexpr int PF_LDS = PF_V_BASE + 2 * PF_VSLOT;     // 80 KiB
constexpr float PF_SLACK = 8.0f;    // log2 headroom of P above the reference

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ float lane_xor32f(float x, int g) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                   __float_as_uint(x), false,
                                                   false);
  return __uint_as_float(g ? sw[0] : sw[1]);
}

// Cache rows of token t of sequence b (paged) -> rows[b * kv_cap + t].
__global__ __launch_bounds__(256) void gather_rows_kernel(
    const uint16_t* __restrict__ cache, const int32_t* __restrict__ block_table,
    int max_blocks, int block_size, const int32_t* __restrict__ kv_lens,
    int kv_cap, int width, uint16_t* __restrict__ rows) {
  const int b = blockIdx.y;
  const int kv = min(kv_lens[b], kv_cap);
  const int vec = width / 8;  // 16-byte pieces per row
  for (long i = blockIdx.x * 256L + threadIdx.x; i < (long)kv * vec;
       i += (long)gridDim.x * 256) {
    const int t = (int)(i / vec), c = (int)(i - (long)t * vec);
    const int blk = block_table[(long)b * max_blocks + t / block_size];
    const uint16_t* src =
        cache + ((long)blk * block_size + t % block_size) * width + 8 * c;
    *(uint4*)(rows + ((long)b * kv_cap + t) * width + 8 * c) =
        *(const uint4*)src;
  }
}

__global__ __launch_bounds__(256, 2) void prefill_mha_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rows,
    int ldr, const uint16_t* __restrict__ kv, int ldkv,
    const int32_t* __restrict__ kv_lens, int kv_cap, int n_q, int n_h,
    int h0, int gh, int ntq, int causal, float scale_log2,
    float* __restrict__ o_v, float* __restrict__ lse) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const lds_char* L = (const lds_char*)lds;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;
  const int col = lane & 31;

  // Block id -> work item: each XCD (ids dealt round-robin) takes a
  // contiguous range of (sequence-head major, query tile minor) items.
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int w = xcd * (nwg >> 3) + min(xcd, nwg & 7) + (blockIdx.x >> 3);
  // heads h0 .. h0 + gh - 1 of n_h; kv holds [k_C | v_C] of those heads
  const int bh = w / ntq, qt = w - bh * ntq;
  const int b = bh / gh, hl = bh - b * gh, h = h0 + hl;
  const int kvl = min(kv_lens[b], kv_cap);
  const int i0 = qt * PF_QW;
  auto lim_of = [&](int i) { return causal ? kvl - n_q + i : kvl - 1; };
  // the lane owns query iq (wave's queries i0 + 32 wave + 0..31)
  const int iq = i0 + 32 * wave + col;
  const int lim = lim_of(min(iq, n_q - 1));
  const int lim_wave_min = lim_of(min(i0 + 32 * wave, n_q - 1));
  const int lim_wg_max = lim_of(min(i0 + PF_QW - 1, n_q - 1));
  const int ntiles = (lim_wg_max + PF_KT) / PF_KT;

  // queries: lane holds q[iq][16 ks + 8 g .. + 7] for every k-step
  bf16x8 qreg[PF_KS];
  {
    const uint16_t* qp = q + ((size_t)(b * n_q + min(iq, n_q - 1)) * n_h +
                              h) * (PF_DH + PF_DR) + 8 * g;
#pragma unroll
    for (int ks = 0; ks < PF_KS; ++ks)
      qreg[ks] = *(const bf16x8*)(qp + 16 * ks);
  }

  // ---- copies: keys of tile j into key slot j % 2 (6 per wave), values of
  // tile j into value slot j % 2 (4 per wave) -------------------------------
  const uint32_t l0 = lds_u32(lds);
  const size_t row0 = (size_t)b * kv_cap;
  // rows past the keys repeat the last one (row 0 of an empty sequence)
  auto last_of = [&](int j) { return max(kvl - 1 - j * PF_KT, 0); };
  auto issue_k = [&](int j) __attribute__((always_inline)) {
    const int t0 = j * PF_KT, last = last_of(j);
    const uint32_t st = l0 + (j & 1) * PF_KSLOT;
    const char* kvb = (const char*)(kv + (row0 + t0) * ldkv);
    const char* rb = (const char*)(rows + (row0 + t0) * ldr);
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // K_C: rows 4 i .. 4 i + 3
      const int i = 4 * c + wave;
      const int r = 4 * i + (lane >> 4);
      const int ch = (lane & 15) ^ (r & 15);
      dma16(st + i * 1024, kvb,
            (uint32_t)(min(r, last) * ldkv * 2 + (hl * PF_DH + 8 * ch) * 2));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {  // k_R: rows 8 i .. 8 i + 7
      const int i = 4 * c + wave;
      const int r = 8 * i + (lane >> 3);
      const int ch = (lane & 7) ^ ((r >> 1) & 7);
      dma16(st + PF_KR_OFF + i * 1024, rb,
            (uint32_t)(min(r, last) * ldr * 2 + (ldr - PF_DR + 8 * ch) * 2));
    }
  };
  auto issue_v = [&](int j) __attribute__((always_inline)) {
    const int t0 = j * PF_KT, last = last_of(j);
    const uint32_t st = l0 + PF_V_BASE + (j & 1) * PF_VSLOT;
    const char* kvb = (const char*)(kv + (row0 + t0) * ldkv);
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // V: group (chunk group cg, tokens tg)
      const int k = 4 * c + wave;
      const int cg = k >> 3, tg = k & 7;
      const int t8 = lane >> 3;
      const int ch = (lane & 7) ^ swz(t8) ^ (2 * (tg & 1));
      const int r = 8 * tg + t8;
      dma16(st + 1024 * (8 * cg + tg), kvb,
            (uint32_t)(min(r, last) * ldkv * 2 +
                       (gh * PF_DH + hl * PF_DH + 8 * (8 * cg + ch)) * 2));
    }
  };

  // ---- fragment offsets ---------------------------------------------------
  // V^T (A operand of the value MFMA), dv tile mt, k-step kk (16 tokens):
  // the decode kernel's value reads with a chunk-group stride of 8 KiB.
  int a_v[2];
  {
    const int q16 = lane >> 4, s16 = lane & 15;
    const int vt = 4 * (q16 >> 1) + (s16 >> 2);
    const int vc = 2 * (q16 & 1) + ((s16 & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      a_v[e] = vt * 128 + 16 * ((4 * e + vc) ^ swz(vt)) + 8 * (s16 & 1);
  }

  // S^T = K Q^T of tile j (two 32-token halves) from key slot j % 2.
  // Accumulator register r of lane (col, g), half tt: token
  // 32 tt + 8 (r / 4) + 4 g + r % 4 of the tile, query iq.
  auto scores = [&](int j, f32x16 (&s)[2]) __attribute__((always_inline)) {
    const lds_char* st = L + (j & 1) * PF_KSLOT;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[tt][r] = 0.0f;
      const int t = 32 * tt + col;
#pragma unroll
      for (int ks = 0; ks < PF_KS; ++ks) {
        const lds_char* a =
            ks < 8 ? st + t * 256 + 16 * ((2 * ks + g) ^ (t & 15))
                   : st + PF_KR_OFF + t * 128 +
                         16 * ((2 * (ks - 8) + g) ^ ((t >> 1) & 7));
        s[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *(const lds_bf16x8*)a, qreg[ks], s[tt], 0, 0, 0);
      }
    }
  };
  // O^T += V^T P^T of tile j from value slot j % 2
  f32x16 o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mt][r] = 0.0f;
  auto values = [&](int j, const bf16x8 (&pb)[4]) __attribute__((always_inline)) {
    const lds_char* st = L + PF_V_BASE + (j & 1) * PF_VSLOT;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = a_v[mt & 1] + 8192 * (mt >> 1) + 2048 * kk;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(st + off));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(st + ((off ^ 32) + 1024)));
        const bf16x8 vf = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kk], o[mt], 0,
                                                        0, 0);
      }
  };
  // Softmax of tile j against a lazily moved reference m_run: it moves (and
  // l, O are rescaled by the returned alpha) only when the tile's maximum
  // exceeds it by more than PF_SLACK, so P <= 2^PF_SLACK.  Both lanes of a
  // query agree (same mx); the rescale branch is taken by the whole wave or
  // skipped by it.  Scores stay unscaled; the scale enters the maximum and
  // the exponent's fused multiply-add.  P (bf16) comes out in k-slot order:
  // k-step kk uses half kk / 2, registers 8 (kk % 2) .. 8 (kk % 2) + 7.
  // A tile that does not exist (live false) is masked whole: P = 0 and the
  // state stays as it is.
  float m_run = -INFINITY, l_run = 0.0f;
  auto softmax = [&](int j, bool live, f32x16 (&s)[2], bf16x8 (&pb)[4],
                     float& alpha) __attribute__((always_inline)) -> bool {
    const int t0 = j * PF_KT;
    if (__builtin_expect(t0 + PF_KT - 1 > lim_wave_min || !live, 0)) {
      // token t0 + 32 tt + 8 (r / 4) + 4 g + r % 4 visible iff
      // 32 tt + 8 (r / 4) + r % 4 <= lim - t0 - 4 g
      const int rel = live ? lim - t0 - 4 * g : -1;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * tt + 8 * (r >> 2) + (r & 3) > rel) s[tt][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[tt][r]);
    mx = fmaxf(mx, lane_xor32f(mx, g)) * scale_log2;
    const bool grow = mx > m_run + PF_SLACK;
    const bool any = __builtin_amdgcn_ballot_w64(grow) != 0;
    // no branch here, so that this code shares a block with the value
    // MFMAs that follow it in the loop
    const float m_new = grow ? mx : m_run;
    alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = m_new;
    l_run *= alpha;
    const float nm = -m_run;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(
            s[kk >> 1][8 * (kk & 1) + 2 * e], scale_log2, nm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(
            s[kk >> 1][8 * (kk & 1) + 2 * e + 1], scale_log2, nm));
        const bf16x2 pp = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(
            pp, __builtin_bit_cast(bf16x2, 0x3F803F80u), l_run, false);
        pw[e] = __builtin_bit_cast(uint32_t, pp);
      }
      pb[kk] = __builtin_bit_cast(bf16x8, (u32x4){pw[0], pw[1], pw[2], pw[3]});
    }
    return any;
  };

  // ---- pipeline -----------------------------------------------------------
  // Iteration j: keys of tile j + 1 and values of tile j are in LDS, P of
  // tile j in registers.  The score MFMAs of tile j + 1 and the value MFMAs
  // of tile j are independent, so the softmax of tile j + 1 overlaps the
  // value MFMAs; O is rescaled (rarely) after them.  Copies: keys of tile
  // j + 2 into the key slot tile j used, values of tile j + 1 into the value
  // slot tile j - 1 used; both are free after the iteration's barrier.
  bf16x8 pb[4];
  issue_k(0);
  issue_v(0);
  if (ntiles > 1) issue_k(1);
  // queries and every copy in (a wait the compiler sees, so that it adds
  // none of its own for the queries later, when copies are in flight)
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  barrier();
  {
    f32x16 s[2];
    scores(0, s);
    float a0;
    softmax(0, true, s, pb, a0);  // O is still zero: no rescale
  }
  wait_lgkm0();  // key slot 0 read, before iteration 0 refills it
  // A moved reference (rare) rescales O before the next value MFMAs: O
  // then holds the tiles up to the previous one, all against the old
  // reference.
  bool rescale = false;
  float alpha = 1.0f;
  for (int j = 0; j < ntiles; ++j) {
    wait_vm<0>();  // own copies of keys j + 1, values j landed
    barrier();     // everyone's, and every read of the slots refilled next
    if (rescale) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mt][r] *= alpha;
    }
    if (j + 2 < ntiles) issue_k(j + 2);
    if (j + 1 < ntiles) issue_v(j + 1);
    // The last iteration's scores read a stale key slot and are masked
    // whole, so that every iteration runs the same code: the softmax of
    // tile j + 1 in one block with the value MFMAs of tile j.
    f32x16 s[2];
    scores(j + 1, s);
    bf16x8 pn[4];
    rescale = softmax(j + 1, j + 1 < ntiles, s, pn, alpha);
    values(j, pb);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) pb[kk] = pn[kk];
    wait_lgkm0();  // this iteration's LDS reads done before slots refill
  }

  // ---- output: O^T register r of lane (col, g), dv tile mt: value column
  // 32 mt + 8 (r / 4) + 4 g + r % 4 of query iq.
  const float l_tot = l_run + lane_xor32f(l_run, g);
  if (iq < n_q) {
    const float inv = 1.0f / l_tot;
    float* dst = o_v + ((size_t)(b * n_q + iq) * n_h + h) * PF_DH + 4 * g;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(f32x4*)(dst + 32 * mt + 8 * i) =
            (f32x4){o[mt][4 * i] * inv, o[mt][4 * i + 1] * inv,
                    o[mt][4 * i + 2] * inv, o[mt][4 * i + 3] * inv};
    if (g == 0 && lse)
      lse[(size_t)(b * n_q + iq) * n_h + h] =
          (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

// q_mha[t][h] = [bf16(q_C[t, h]) | bf16(RoPE_pos(q_R[t, h]))] from the
// K-split parts of the query up-projection (q_C of head h at column h d_h,
// q_R of head h at n_h d_h + h d_r).  A thread handles 4 consecutive q_C
// values, or 4 consecutive RoPE pairs (j, j + d_r / 2): 16-byte loads and
// 8-byte stores (d_h % 4 == 0, d_r % 8 == 0, lda % 4 == 0).
__global__ __launch_bounds__(256) void query_mha_kernel(
    const float* __restrict__ parts, int nparts, long part_stride, long lda,
    int n_h, int d_h, int d_r, const int32_t* __restrict__ pos,
    const float* __restrict__ rcos, const float* __restrict__ rsin,
    int max_pos, uint16_t* __restrict__ q_out) {
  const int t = blockIdx.x;
  const int half = d_r / 2;
  const int p = pos[t];
  const bool ok = p >= 0 && p < max_pos;
  const float* src = parts + (size_t)t * lda;
  const int per_head = d_h / 4 + half / 4;
  auto sum4 = [&](long c) {
    f32x4 x = *(const f32x4*)(src + c);
    for (int pp = 1; pp < nparts; ++pp) {
      const f32x4 y = *(const f32x4*)(src + pp * part_stride + c);
      x[0] += y[0]; x[1] += y[1]; x[2] += y[2]; x[3] += y[3];
    }
    return x;
  };
  for (int i = blockIdx.y * 256 + threadIdx.x; i < n_h * per_head;
       i += gridDim.y * 256) {
    const int hh = i / per_head, j = i - hh * per_head;
    uint16_t* dst = q_out + ((size_t)t * n_h + hh) * (d_h + d_r);
    if (j < d_h / 4) {
      const f32x4 x = sum4((long)hh * d_h + 4 * j);
      *(uint2*)(dst + 4 * j) =
          make_uint2(pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]));
    } else {
      const int jj = 4 * (j - d_h / 4);
      const long c0 = (long)n_h * d_h + hh * d_r + jj;
      const f32x4 x1 = sum4(c0), x2 = sum4(c0 + half);
      f32x4 c = {NAN, NAN, NAN, NAN}, sn = {NAN, NAN, NAN, NAN};
      if (ok) {
        c = *(const f32x4*)(rcos + (long)p * half + jj);
        sn = *(const f32x4*)(rsin + (long)p * half + jj);
      }
      f32x4 y1, y2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y1[e] = x1[e] * c[e] - x2[e] * sn[e];
        y2[e] = x1[e] * sn[e] + x2[e] * c[e];
      }
      *(uint2*)(dst + d_h + jj) =
          make_uint2(pack_bf2(y1[0], y1[1]), pack_bf2(y1[2], y1[3]));
      *(uint2*)(dst + d_h + jj + half) =
          make_uint2(pack_bf2(y2[0], y2[1]), pack_bf2(y2[2], y2[3]));
    }
  }
}

}  // namespace

bool prefill_mha_supported(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_h == PF_DH && d.d_r == PF_DR &&
         (d.d_c + d.d_r) % 8 == 0;
}

hipError_t launch_gather_rows(const mla_dims& d, int B, const void* cache,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* kv_lens, int kv_cap, void* rows,
                              hipStream_t stream) {
  const int width = d.d_c + d.d_r;
  const long per_seq = (long)kv_cap * (width / 8);
  const long nx = (per_seq + 255) / 256;
  const dim3 grid((unsigned)(nx < 4096 ? (nx > 0 ? nx : 1) : 4096), B);
  hipLaunchKernelGGL(gather_rows_kernel, grid, dim3(256), 0, stream,
                     (const uint16_t*)cache, block_table, max_blocks,
                     d.block_size, kv_lens, kv_cap, width, (uint16_t*)rows);
  return hipGetLastError();
}

hipError_t launch_prefill_mha(const mla_dims& d, int B, int n_q,
                              const void* q, const void* rows, const void* kv,
                              int h0, int gh, const int32_t* kv_lens,
                              int kv_cap, int causal, float* o_v, float* lse,
                              hipStream_t stream) {
  const float scale_log2 =
      (float)(1.4426950408889634 / __builtin_sqrt((double)(d.d_h + d.d_r)));
  static std::atomic<unsigned long long> lds_set{0};
  {
    const hipError_t e =
        set_lds_limit_once((const void*)prefill_mha_kernel, PF_LDS, lds_set);
    if (e != hipSuccess) return e;
  }
  const int ntq = (n_q + PF_QW - 1) / PF_QW;
  const long nwg = (long)B * gh * ntq;
  hipLaunchKernelGGL(prefill_mha_kernel, dim3((unsigned)nwg), dim3(256),
                     PF_LDS, stream, (const uint16_t*)q,
                     (const uint16_t*)rows, d.d_c + d.d_r,
                     (const uint16_t*)kv, 2 * gh * d.d_h, kv_lens, kv_cap,
                     n_q, d.n_h, h0, gh, ntq, causal, scale_log2, o_v, lse);
  return hipGetLastError();
}

hipError_t launch_query_mha(const mla_dims& d, int T, const float* parts,
                            int nparts, long part_stride, long lda,
                            const int32_t* pos, const float* rope_cos,
                            const float* rope_sin, int max_pos, void* q_out,
                            hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (d.d_h % 4 != 0 || d.d_r % 8 != 0 || lda % 4 != 0 || part_stride % 4)
    return hipErrorInvalidValue;
  const int items = d.n_h * (d.d_h / 4 + d.d_r / 8);
  const dim3 grid(T, (items + 255) / 256);
  hipLaunchKernelGGL(query_mha_kernel, grid, dim3(256), 0, stream, parts,
                     nparts, part_stride, lda, d.n_h, d.d_h, d.d_r, pos,
                     rope_cos, rope_sin, max_pos, (uint16_t*)q_out);
  return hipGetLastError();
}

}  // namespace mla
