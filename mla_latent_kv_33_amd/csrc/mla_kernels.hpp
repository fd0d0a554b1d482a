// Internal launchers shared by the C ABI (mla_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

// ---- split-KV decode ---------------------------------------------------
// Split j of a (sequence, query) whose visible keys span nblk blocks covers
// blocks [j nblk / n_split, (j + 1) nblk / n_split).
// Partials: o_part [slot][n_h][d_c], slot = row n_split + split (or the
// balanced plan's slots, BAL_SLOTS of them) (fp32 unnormalised from the
// SIMT kernel; from the matrix-core kernel fp16 O / (l s) in the first half
// of the same buffer, followed by the per-row scales s as fp32),
// m_part/l_part [slot][n_h] with m in log2 units.  A row with one split
// writes o_final [B*n_q][n_h][d_c] and lse_final (natural log) directly.
bool decode_mfma_supported(const mla_dims& d);
// Balanced splits (matrix-core kernel, at most BAL_SLOTS query rows): the
// kernel reads kv_lens and gives query row r n_r = ceil(nb_r / c) splits of
// its nb_r visible blocks, c the smallest chunk >= BAL_MIN_CHUNK blocks with
// sum_r n_r <= BAL_SLOTS; the splits of row r take consecutive partial
// slots from plan[r] = (first slot, n_r) on, written by the row's split 0.
// A row with one split writes o_final / lse_final directly.
constexpr int BAL_SLOTS = 256;
constexpr int BAL_MIN_CHUNK = 2;
struct DecodeBalance {
  int2* plan = nullptr;  // [B*n_q]; null: uniform n_split per row
  int est_wgs = 0;       // upper bound of the workgroups that get work
};
// n_split: splits per row (uniform mode); with balance.plan the partial
// buffers hold BAL_SLOTS slots instead of B*n_q*n_split.
hipError_t launch_decode_mfma(const mla_dims& d, int B, int n_q,
                              const void* q, const void* cache,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* kv_lens, int n_split,
                              const DecodeBalance& balance, float* o_part,
                              float* m_part, float* l_part, float* o_final,
                              float* lse_final, bool cache_nt,
                              hipStream_t stream);
hipError_t launch_decode_simt(const mla_dims& d, int B, int n_q,
                              const void* q, const void* cache,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* kv_lens, int n_split,
                              float* o_part, float* m_part,
                              float* l_part, float* o_final, float* lse_final,
                              hipStream_t stream);
// o_part: fp32 unnormalised partials (decode_simt_kernel), or with
// f16_parts the scaled fp16 partials of decode_mfma_kernel.  plan (fp16
// partials only): balanced splits, slots partial slots; rows with one split
// are already final and skipped.
hipError_t launch_combine(const mla_dims& d, int rows, int n_split,
                          const float* o_part, bool f16_parts,
                          const float* m_part, const float* l_part,
                          float* o_lat, float* lse, hipStream_t stream,
                          const int2* plan = nullptr, int slots = 0);

// ---- projections of decode steps with at most GV_MAXT tokens (gemv.hip) --
// One wave per group of weight rows, full contraction, no partial results.
// The append takes this path up to GV_MAXT tokens; the query and output
// projections, whose per-token arithmetic is larger, up to GV_QO_MAXT (at 3
// and 4 tokens the weight-streaming GEMMs measured faster).
constexpr int GV_MAXT = 4;
constexpr int GV_QO_MAXT = 2;
bool gemv_supported(const mla_dims& d, int T, int t_max = GV_MAXT);
// c_KV and RoPE(k_R) of T tokens straight into their cache rows.
hipError_t launch_gemv_append(const mla_dims& d, int T, const void* h,
                              const void* w_dkv, const void* w_kr,
                              const int32_t* seq_idx, const int32_t* pos,
                              const float* rope_cos, const float* rope_sin,
                              int max_pos, const int32_t* block_table,
                              int max_blocks, void* cache,
                              hipStream_t stream);
// c_Q -> cq [T][d_cq] as bf16 hi|lo pairs (4 bytes per value), q_C -> qc
// [T][n_h d_h] fp32, then q_out[t][h] = [W_UK_h^T q_C_h | RoPE(q_R)_h] in
// bf16.
hipError_t launch_gemv_query(const mla_dims& d, int T, const void* h,
                             const void* w_dq, const void* w_uq,
                             const void* w_qr, const void* w_uk,
                             const int32_t* pos, const float* rope_cos,
                             const float* rope_sin, int max_pos, float* cq,
                             float* qc, void* q_out, hipStream_t stream);
// The query path from c_Q on (cq as bf16 hi|lo pairs): q_C -> qc, then
// q_out as launch_gemv_query.
hipError_t launch_gemv_query_tail(const mla_dims& d, int T, const void* w_uq,
                                  const void* w_qr, const void* w_uk,
                                  const int32_t* pos, const float* rope_cos,
                                  const float* rope_sin, int max_pos,
                                  const float* cq, float* qc, void* q_out,
                                  hipStream_t stream);
// [W_DQ; W_DKV; W_KR] h in one launch (up to GV_QO_MAXT tokens): c_Q -> cq
// as bf16 hi|lo pairs, and the append's cache rows as launch_gemv_append.
hipError_t launch_gemv_down(const mla_dims& d, int T, const void* h,
                            const void* w_dq, const void* w_dkv,
                            const void* w_kr, const int32_t* seq_idx,
                            const int32_t* pos, const float* rope_cos,
                            const float* rope_sin, int max_pos,
                            const int32_t* block_table, int max_blocks,
                            void* cache, float* cq, hipStream_t stream);
// v [T][n_h d_h] = W_UV_h o_lat_h as bf16 hi|lo pairs (4 bytes per value),
// then u [T][d] bf16 = W_O v.
hipError_t launch_gemv_out(const mla_dims& d, int T, const float* o_lat,
                           const void* w_uv, const void* w_o, float* v,
                           void* u, hipStream_t stream);
// u [T][d] bf16 = W_O v from v as launch_gemv_out writes it.
hipError_t launch_gemv_wo(const mla_dims& d, int T, const float* v,
                          const void* w_o, void* u, hipStream_t stream);
// The split combine of a matrix-core decode of T (1 or 2) query rows with
// n_split >= 2 uniform splits, fused with v = W_UV_h o_lat_h: writes o_lat,
// lse (may be null) and v as launch_gemv_out does.  bf16, d_c = 512,
// d_h = 128.
bool combine_uv_supported(const mla_dims& d, int T);
hipError_t launch_combine_uv(const mla_dims& d, int T, int n_split,
                             const float* o_part, const float* m_part,
                             const float* l_part, const void* w_uv,
                             float* o_lat, float* lse, float* v,
                             hipStream_t stream);

// ---- pre-merged absorption (merged.hip) ---------------------------------
// out [n_h][d_c][d_cq] = W_UK_h^T W_UQ_h per head, in the weight dtype.
hipError_t launch_merge_uq_uk(const mla_dims& d, const void* w_uq,
                              const void* w_uk, void* out,
                              hipStream_t stream);

// ---- MHA-path prefill (prefill_mha.hip) --------------------------------
// Shapes the prefill kernel serves: bf16, d_h = 128 (= d_v), d_r = 64.
bool prefill_mha_supported(const mla_dims& d);
// rows[b * kv_cap + t] = cache row of token t of sequence b (t < kv_lens[b]).
hipError_t launch_gather_rows(const mla_dims& d, int B, const void* cache,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* kv_lens, int kv_cap, void* rows,
                              hipStream_t stream);
// Causal attention of q [B*n_q][n_h][d_h + d_r] over keys [k_C | k_R] and
// values v_C: kv [B*kv_cap][2 n_h d_h] bf16 (k_C of head h at h d_h, v_C at
// n_h d_h + h d_h), k_R the last d_r columns of rows; o_v [B*n_q][n_h][d_h]
// fp32, lse [B*n_q][n_h] (natural log) or null.
hipError_t launch_prefill_mha(const mla_dims& d, int B, int n_q,
                              const void* q, const void* rows, const void* kv,
                              int h0, int gh, const int32_t* kv_lens,
                              int kv_cap, int causal, float* o_v, float* lse,
                              hipStream_t stream);
// q_out[t][h] = [q_C | RoPE(q_R)] (bf16) from the K-split parts of the
// query up-projection (as launch_absorb_fast reads them).
hipError_t launch_query_mha(const mla_dims& d, int T, const float* parts,
                            int nparts, long part_stride, long lda,
                            const int32_t* pos, const float* rope_cos,
                            const float* rope_sin, int max_pos, void* q_out,
                            hipStream_t stream);

// ---- query absorption (absorb.hip) -------------------------------------
// q_lat[t, h, :] = W_UK_h^T (sum of nparts fp32 parts of q_C[t, h, :]) into
// the first d_c columns of q_out's rows (bf16), and RoPE(q_R[t, h, :]) into
// the last d_r, for the shapes accepted by absorb_fast_supported (bf16,
// d_h = 128, d_c % 256 == 0, d_r = 64, T <= 64, at most two parts).
// parts: T rows of stride lda floats, q_C of head h at column h d_h, q_R of
// head h at column n_h d_h + h d_r, part p at parts + p part_stride.
bool absorb_fast_supported(const mla_dims& d, int T, int nparts);
hipError_t launch_absorb_fast(const mla_dims& d, int T, const float* parts,
                              int nparts, long part_stride, long lda,
                              const void* w_uk, const int32_t* pos,
                              const float* rope_cos, const float* rope_sin,
                              int max_pos, void* q_out, hipStream_t stream);

// ---- GEMM C = A . B^T --------------------------------------------------
// A [M][K] (row stride lda, batch stride a_bs), fp32 or the layer dtype.
// B (layer dtype) is either [N][K] ("NT", row stride ldb), optionally in two
// parts - rows n < nb1 from B and rows n >= nb1 from B2 (row n - nb1) - or
// [K][N] ("NN", row stride ldb, no second part).  C is fp32 [M][N] (row
// stride ldc).  Batch index z offsets A, B (and B2) and C by their batch
// strides.  With k_split > 1 the K range is cut into k_split chunks and
// chunk kz writes its own partial product at C + kz * c_ks; the consumer
// sums the parts (deterministic, no atomics).
struct GemmArgs {
  const void* A = nullptr;
  int a_f32 = 0;  // A is fp32 (else the layer dtype)
  long lda = 0, a_bs = 0;
  const void* B = nullptr;
  const void* B2 = nullptr;
  int nb1 = 1 << 30;
  // rows >= nb2 from B3 (LDS-staged kernel only)
  const void* B3 = nullptr;
  int nb2 = 1 << 30;
  int b_nn = 0;  // B stored [K][N]
  long ldb = 0, b_bs = 0;
  float* C = nullptr;
  long ldc = 0, c_bs = 0, c_ks = 0;
  int M = 0, N = 0, K = 0, batch = 1;
  int k_split = 1;
  // < 0: LDS-staged kernel with -ntw tiles per wave; 0: tiled (or big).
  int ntw = 0;
  // LDS-staged kernel: rows in blocks of 32, one workgroup per block (1 or 2)
  int m_split = 1;
  void* c16 = nullptr;  // bf16 output instead of C (tiled kernel, k_split 1)
  // 1: large-tile kernel for many rows (bf16 weights, NT, batch 1, one K
  // chunk)
  int big = 0;
  // Pre-split fp32 activations ("hi|lo" layout): every 8 consecutive values
  // of a row are stored as 8 bf16 hi = bf16(x) followed by 8 bf16
  // lo = bf16(x - hi), 4 bytes per value like fp32.  a_hl: A is in that
  // layout (with a_f32 set; LDS-staged kernel only); c_hl: C is written in
  // it (LDS-staged kernel, one K chunk).
  int a_hl = 0;
  int c_hl = 0;
  // LDS-staged kernel: read the weights with non-temporal loads (weights
  // that are not meant to stay in the Infinity Cache between steps)
  int w_nt = 0;
};
hipError_t launch_gemm(const mla_dims& d, const GemmArgs& g,
                       hipStream_t stream);
// Chooses the kernel shape (k_split <= max_split, ntw) of a GEMM; call after
// M, N, K, batch, a_f32 and b_nn are set.
void gemm_plan(const mla_dims& d, GemmArgs& g, int max_split = 16);

// ---- element-wise kernels ----------------------------------------------
// Inputs given as (pointer, nparts, part_stride) are the sum of nparts fp32
// arrays spaced part_stride floats apart (the K chunks of a GEMM).
// dst[i] = sum of the parts at i, for i < n.
hipError_t launch_reduce_parts(const float* src, int nparts, long part_stride,
                               long n, float* dst, hipStream_t stream);
// The same sum written in the pre-split hi|lo layout of rows of `ld` values
// (ld % 8 == 0, n % ld == 0).
hipError_t launch_reduce_parts_hl(const float* src, int nparts,
                                  long part_stride, long n, int ld, void* dst,
                                  hipStream_t stream);
// The stacked down-projection's K parts, rows [c_Q | c_KV | k_R] of
// d_cq + d_c + d_r floats: c_Q to `cq` in the pre-split hi|lo layout, and
// each token's cache row (RoPE on k_R), in one launch.
hipError_t launch_project_epilogue(const mla_dims& d, int T, const float* acc,
                                   int nparts, long part_stride, void* cq,
                                   const int32_t* seq_idx, const int32_t* pos,
                                   const float* rope_cos,
                                   const float* rope_sin, int max_pos,
                                   const int32_t* block_table, int max_blocks,
                                   void* cache, hipStream_t stream);
// acc [T][d_c + d_r] fp32 -> RoPE on the last d_r columns -> cache rows.
hipError_t launch_append_scatter(const mla_dims& d, int T, const float* acc,
                                 int nparts, long part_stride,
                                 const int32_t* seq_idx, const int32_t* pos,
                                 const float* rope_cos, const float* rope_sin,
                                 int max_pos, const int32_t* block_table,
                                 int max_blocks, void* cache,
                                 hipStream_t stream);
// qr rows of ld_qr floats, the [n_h][d_r] block of token t at
// qr + t * ld_qr -> RoPE -> q_out[t][h][d_c ..] (layer dtype).
// qr: the sum of nparts fp32 parts spaced part_stride floats apart.
// The same with the latent half normalised: c_j = w_j x_j / sqrt(mean(x^2)
// + eps) over the d_c latent values of the row (kv_norm_w: d_c weights in
// the layer dtype).
hipError_t launch_append_norm_scatter(const mla_dims& d, int T,
                                      const float* acc, int nparts,
                                      long part_stride, const void* kv_norm_w,
                                      float eps, const int32_t* seq_idx,
                                      const int32_t* pos,
                                      const float* rope_cos,
                                      const float* rope_sin, int max_pos,
                                      const int32_t* block_table,
                                      int max_blocks, void* cache,
                                      hipStream_t stream);
hipError_t launch_query_rope(const mla_dims& d, int T, const float* qr,
                             int nparts, long part_stride, long ld_qr,
                             const int32_t* pos, const float* rope_cos,
                             const float* rope_sin, int max_pos, void* q_out,
                             hipStream_t stream);
// src fp32 [rows][cols] (row stride lds, parts) -> dst layer dtype (row
// stride ldd).
// grp > 0: source rows in groups of grp, lds apart within a group and
// lds_grp from one group to the next (grp <= 0: one group)
hipError_t launch_convert(const mla_dims& d, int rows, int cols,
                          const float* src, long lds, int nparts,
                          long part_stride, void* dst, long ldd,
                          hipStream_t stream, int grp = 0, long lds_grp = 0);

}  // namespace mla
