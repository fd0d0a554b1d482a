/*
 * mla.h - C ABI of the MI355X (gfx950) MLA decode library, libmla.so.
 *
 * Multi-head Latent Attention decode over a paged latent cache.  Each cached
 * token keeps only its latent c_KV (d_c values) and the RoPE key k_R shared by
 * every head (d_r values), one row of d_c + d_r elements
 * ('MLA：潜在表示压缩与解耦 RoPE', sections 3, 6 and 7).  A decode step is four
 * calls, enqueued in this order on one HIP stream:
 *
 *   mla_append_cache  c_KV = W_DKV h, k_R = RoPE(W_KR h), written to the cache
 *   mla_absorb_q      c_Q = W_DQ h, q_C = W_UQ c_Q, q_R = RoPE(W_QR c_Q),
 *                     q_lat_h = W_UK_h^T q_C_h  -> q = [q_lat | q_R] per head
 *   mla_decode        scores q . row / sqrt(d_h + d_r), softmax, o_lat =
 *                     sum_s a_s c_KV_s (split over the keys, then combined)
 *   mla_out           v_h = W_UV_h o_lat_h, u = W_O [v_0; ...; v_{n_h-1}]
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are device memory unless a parameter says "host".  The caller
 *   allocates and frees every buffer (weights, cache pool, block table,
 *   lengths, outputs, workspace); the library allocates nothing and keeps no
 *   state between calls.  Every call only enqueues work on `stream` and
 *   returns; results are ready once the caller synchronises the stream.
 * - The calls never allocate, clear memory or synchronise, so a caller may
 *   capture a whole step into a HIP graph and replay it (after one eager
 *   call of each entry point in the process, which sets kernel attributes).
 * - Weights are row-major [out, in] (y = W x), in the activation dtype.
 *   Head h owns rows h*d_h .. h*d_h+d_h-1 of W_UQ, W_UK, W_UV and rows
 *   h*d_r .. of W_QR.
 * - Activations, weights and the cache share `dims->dtype`; accumulation is
 *   fp32.  o_lat and lse are always fp32.
 * - Cache pool: `cache[num_blocks][block_size][d_c + d_r]`, each row the
 *   token's c_KV followed by its k_R.  Token at position p of sequence b lives
 *   in row p % block_size of block `block_table[b * max_blocks + p /
 *   block_size]`.  Positions are 0-based.
 * - RoPE tables: `rope_cos/rope_sin[max_pos][d_r / 2]` fp32, entry (p, j) =
 *   cos/sin(p * base^(-2j/d_r)); the pair (x_j, x_{j + d_r/2}) is rotated by
 *   that angle.  mla_rope_tables_host builds them.
 * - Errors are returned, never printed or thrown.  Host-checkable arguments
 *   (null pointers, sizes, dims, workspace) are validated before anything is
 *   enqueued.  Values that live on the device (block ids, lengths, positions,
 *   sequence indices) are trusted: they must be in range, as documented per
 *   call.  MLA_ERR_DEVICE reports a failed launch.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* mla_stream_t; /* a hipStream_t; NULL = default */

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,       /* inconsistent or non-positive sizes */
  MLA_ERR_UNSUPPORTED = 3, /* dims/dtype this build has no kernel for */
  MLA_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  MLA_ERR_RANGE = 5,       /* a host-checkable value out of range */
  MLA_ERR_DEVICE = 6       /* a kernel launch failed */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Layer dimensions.  Bracketed names are the usual hyper-parameter names
 * ('MiniMind 学习笔记 10', section 8).  Requirements: all positive, d_r even,
 * block_size a power of two; for BF16 also d, d_cq, d_c and n_h * d_h
 * multiples of 64 and d_h, d_r multiples of 8 (else MLA_ERR_UNSUPPORTED).  The matrix-core decode kernel
 * takes BF16 with d_c = 512, d_r = 64, block_size 64 and n_h = 32, 64 or a
 * multiple of 128; other dims run on the general (SIMT) decode kernel. */
typedef struct {
  int32_t d;          /* hidden size */
  int32_t n_h;        /* attention heads */
  int32_t d_h;        /* per-head content dim [qk_nope_head_dim = v_head_dim] */
  int32_t d_c;        /* KV latent dim [kv_lora_rank] */
  int32_t d_r;        /* decoupled RoPE dim [qk_rope_head_dim] */
  int32_t d_cq;       /* query latent dim [q_lora_rank] */
  int32_t block_size; /* tokens per cache block */
  int32_t dtype;      /* mla_dtype of activations, weights and cache */
} mla_dims;

/* Human-readable name of a status code (static string). */
const char* mla_status_string(mla_status s);

/* Library version string (static). */
const char* mla_version(void);

/* Host helper: fill host arrays cos_out/sin_out[max_pos][d_r/2] with
 * cos/sin(p * base^(-2j/d_r)), angles computed in double and rounded once to
 * float.  RoPE as used for q_R and k_R ('MLA：潜在表示压缩与解耦 RoPE',
 * sections 5-6; the frequency and half-split pairing are this library's
 * convention).  Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (d_r odd or <= 0,
 * max_pos <= 0, base <= 0). */
mla_status mla_rope_tables_host(int32_t d_r, double base, int32_t max_pos,
                                float* cos_out, float* sin_out);

/* ------------------------------------------------------------------------
 * mla_append_cache - write the latent rows of T new tokens into the cache.
 *
 * For token t (0 <= t < T) with hidden state h[t][d], sequence seq_idx[t]
 * and position pos[t]:  c = W_DKV h  (d_c values), r = RoPE_{pos}(W_KR h)
 * (d_r values), rounded once to the cache dtype and stored as the row of that
 * position ('MLA：潜在表示压缩与解耦 RoPE', sections 3 and 6: only c_KV and k_R
 * are cached).
 *
 *   h            [T][d]                  activation dtype
 *   seq_idx, pos [T] int32 (device)      0 <= seq_idx < num_seqs (trusted),
 *                                        0 <= pos < max_pos and
 *                                        pos / block_size < max_blocks
 *   w_dkv        [d_c][d], w_kr [d_r][d]
 *   rope_cos/sin [max_pos][d_r/2] fp32
 *   block_table  [num_seqs][max_blocks] int32, entries < num_blocks
 *   cache        [num_blocks][block_size][d_c + d_r]
 *   ws           workspace of at least mla_append_workspace_bytes(dims, T)
 * Rows of distinct tokens must not coincide.  T = 0 is a no-op.
 * ---------------------------------------------------------------------- */
size_t mla_append_workspace_bytes(const mla_dims* dims, int32_t T);
mla_status mla_append_cache(const mla_dims* dims, int32_t T, const void* h,
                            const int32_t* seq_idx, const int32_t* pos,
                            const void* w_dkv, const void* w_kr,
                            const float* rope_cos, const float* rope_sin,
                            int32_t max_pos, const int32_t* block_table,
                            int32_t max_blocks, void* cache,
                            int32_t num_blocks, void* ws, size_t ws_bytes,
                            mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_append_cache_rmsnorm - mla_append_cache with the latent normalised.
 *
 * As mla_append_cache, except that the latent half of the row is passed
 * through an RMSNorm with weight kv_norm_w before it is stored, while the
 * RoPE key is not ('MiniMind 学习笔记 10', section 9: kv_norm applies to the
 * latent only, and the normalised latent is what the cache holds):
 *   x = W_DKV h,  c_j = kv_norm_w[j] x_j / sqrt(mean_i(x_i^2) + eps)
 * computed in fp32 and rounded once to the cache dtype.
 *
 *   kv_norm_w  [d_c]  activation dtype (device)
 *   eps        >= 0 (host); a negative or NaN eps is MLA_ERR_SHAPE
 * Every other argument, the workspace size and the error behaviour are those
 * of mla_append_cache.  Decode and the query path are unchanged: they read
 * whatever latent the cache holds.
 * ---------------------------------------------------------------------- */
mla_status mla_append_cache_rmsnorm(
    const mla_dims* dims, int32_t T, const void* h, const int32_t* seq_idx,
    const int32_t* pos, const void* w_dkv, const void* w_kr,
    const void* kv_norm_w, float eps, const float* rope_cos,
    const float* rope_sin, int32_t max_pos, const int32_t* block_table,
    int32_t max_blocks, void* cache, int32_t num_blocks, void* ws,
    size_t ws_bytes, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_absorb_q - query path and absorption of W_UK into the query.
 *
 * c_Q = W_DQ h (kept fp32, not rounded), q_C = W_UQ c_Q, q_R = RoPE_{pos}(W_QR
 * c_Q) per head, q_lat_h = W_UK_h^T q_C_h ('MLA：潜在表示压缩与解耦 RoPE',
 * sections 3, 4 and 6; 'Latent 压缩', MLA section: <q, W_K c> = <W_K^T q, c>).
 * Output q[t][h] = [q_lat_h (d_c) | q_R_h (d_r)], rounded once to the
 * activation dtype.
 *
 *   h      [T][d];  pos [T] int32 (device), 0 <= pos < max_pos (trusted)
 *   w_dq [d_cq][d], w_uq [n_h*d_h][d_cq], w_qr [n_h*d_r][d_cq],
 *   w_uk [n_h*d_h][d_c]
 *   q_out  [T][n_h][d_c + d_r]
 *   ws     at least mla_absorb_workspace_bytes(dims, T)
 * ---------------------------------------------------------------------- */
size_t mla_absorb_workspace_bytes(const mla_dims* dims, int32_t T);
mla_status mla_absorb_q(const mla_dims* dims, int32_t T, const void* h,
                        const int32_t* pos, const void* w_dq,
                        const void* w_uq, const void* w_qr, const void* w_uk,
                        const float* rope_cos, const float* rope_sin,
                        int32_t max_pos, void* q_out, void* ws,
                        size_t ws_bytes, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_append_absorb_q - mla_append_cache and mla_absorb_q on the same tokens
 * in one call.
 *
 * Both calls start from the new tokens' hidden states: the cached latent
 * c_KV = W_DKV h and the RoPE key RoPE(W_KR h) on one side, the query latent
 * c_Q = W_DQ h on the other ('MLA：潜在表示压缩与解耦 RoPE', section 3, joint
 * compression of keys/values and of queries; section 6, the decoupled RoPE
 * key).  With bf16 layers the three weights are streamed as one stacked
 * projection [W_DQ; W_DKV; W_KR] h: for one or two tokens (the matrix-vector
 * path) one launch writes both c_Q and the cache rows; for decode batches
 * of 5 to 64 tokens one weight-streaming GEMM is followed by one epilogue
 * launch that sums its K parts into both.  The query path then continues as
 * in mla_absorb_q.  Other shapes run the two calls' own paths in sequence.
 * The cache rows and q_out equal those of mla_append_cache followed by
 * mla_absorb_q up to the order of the fp32 sums of each projection.
 *
 * Arguments: those of mla_append_cache and mla_absorb_q, with h, pos, the
 * RoPE tables and max_pos shared; ws at least
 * mla_append_absorb_workspace_bytes(dims, T) (at least either call's own
 * size).  Every argument is checked before anything is enqueued; the error
 * codes are those of the two calls.
 * ---------------------------------------------------------------------- */
size_t mla_append_absorb_workspace_bytes(const mla_dims* dims, int32_t T);
mla_status mla_append_absorb_q(
    const mla_dims* dims, int32_t T, const void* h, const int32_t* seq_idx,
    const int32_t* pos, const void* w_dkv, const void* w_kr, const void* w_dq,
    const void* w_uq, const void* w_qr, const void* w_uk,
    const float* rope_cos, const float* rope_sin, int32_t max_pos,
    const int32_t* block_table, int32_t max_blocks, void* cache,
    int32_t num_blocks, void* q_out, void* ws, size_t ws_bytes,
    mla_stream_t stream);

/* ------------------------------------------------------------------------
 * Pre-merged query absorption (a variant the pages allow: W_UQ^T W_UK can
 * be merged ahead of time, 'MLA：潜在表示压缩与解耦 RoPE', section 4; the
 * RoPE part cannot, section 5).
 *
 * mla_merge_uq_uk (once per layer): w_merged [n_h][d_c][d_cq] with
 *   w_merged[h] = W_UK_h^T W_UQ_h (fp32 sums of d_h products, rounded once
 *   to the weight dtype).  w_uq, w_uk as in mla_absorb_q; w_merged is
 *   caller-allocated (n_h d_c d_cq elements).
 * mla_absorb_q_merged: the output of mla_absorb_q, computed as
 *   q_lat_h = w_merged[h] c_Q (c_Q = W_DQ h in fp32) and q_R = RoPE(W_QR
 *   c_Q); one projection onto [w_merged; W_QR] replaces W_UQ and the
 *   per-head absorption.  It streams n_h d_c d_cq merged weights instead of
 *   n_h d_h (d_cq + d_c) (3x at DeepSeek-V2 dims), so the unmerged
 *   mla_absorb_q is the faster form at every batch size measured; this
 *   entry point exists to measure that.  Arguments as mla_absorb_q, with
 *   w_merged in place of w_uq and w_uk; ws at least
 *   mla_absorb_merged_workspace_bytes(dims, T).
 * ---------------------------------------------------------------------- */
mla_status mla_merge_uq_uk(const mla_dims* dims, const void* w_uq,
                           const void* w_uk, void* w_merged,
                           mla_stream_t stream);
size_t mla_absorb_merged_workspace_bytes(const mla_dims* dims, int32_t T);
mla_status mla_absorb_q_merged(const mla_dims* dims, int32_t T, const void* h,
                               const int32_t* pos, const void* w_dq,
                               const void* w_merged, const void* w_qr,
                               const float* rope_cos, const float* rope_sin,
                               int32_t max_pos, void* q_out, void* ws,
                               size_t ws_bytes, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_decode - attention of absorbed queries over the latent cache.
 *
 * Sequence b has kv_lens[b] cached rows (positions 0 .. kv_lens[b]-1) and
 * n_q queries, the last n_q positions: query i sits at position
 * P = kv_lens[b] - n_q + i and sees rows 0..P (causal, bottom-right aligned:
 * 'MiniMind 学习笔记 10', section 12).  Per head h:
 *   score_s = (q_lat_h . c_KV_s + q_R_h . k_R_s) / sqrt(d_h + d_r)
 *   o_lat_h = sum_s softmax(score)_s c_KV_s,   lse_h = log sum_s e^score_s
 * ('MLA：潜在表示压缩与解耦 RoPE', sections 4, 6, 7; 'Latent 压缩', MLA
 * section: decode in the latent is MQA with one shared key/value head).
 * The keys of each (b, query) are cut into n_split chunks whose partial
 * softmax states are merged by a log-sum-exp combine.
 *
 *   q           [B][n_q][n_h][d_c + d_r]
 *   cache, block_table, max_blocks, num_blocks as in mla_append_cache
 *   kv_lens     [B] int32 (device), n_q <= kv_lens[b] <= max_kv_len and
 *               ceil(kv_lens[b] / block_size) <= max_blocks (trusted)
 *   max_kv_len  host upper bound of kv_lens (sizes the split plan)
 *   causal      must be 1 when n_q > 1 (the only defined rule); ignored for
 *               n_q = 1
 *   n_split     key chunks per (b, query); 0 lets the library choose one
 *               count for every row (mla_decode_auto_splits);
 *               MLA_SPLIT_BALANCED gives each query row a count
 *               proportional to its visible keys, planned on the device
 *               from kv_lens (for batches of uneven lengths: at most 256
 *               workgroups, the longest chunk as short as that allows;
 *               used for 2 .. 256 query rows on the bf16 matrix-core path
 *               with d_c = 512, d_r = 64, block_size = 64, otherwise as
 *               0); must not exceed ceil(max_kv_len / block_size)
 *   o_lat       [B][n_q][n_h][d_c] fp32 output
 *   lse         [B][n_q][n_h] fp32 output, may be NULL
 *   ws          at least mla_decode_workspace_bytes(dims, B, n_q,
 *               max_kv_len, n_split).  With balanced splits the call
 *               leaves its plan there for inspection: int32 pairs (first
 *               partial slot, split count) per query row b * n_q + i, at
 *               byte offset W - ceil256(8 B n_q), W = the size
 *               mla_decode_workspace_bytes returns, ceil256 rounding up to
 *               a multiple of 256.  A row's splits take consecutive slots,
 *               rows in order; split j of a row with nb visible blocks
 *               and c splits covers blocks [j nb / c, (j + 1) nb / c).
 * A query row that sees no key (kv_lens[b] < n_q, outside the contract
 * above) gets o_lat = 0 and lse = -inf with one split; never a write
 * through a missing partial buffer.
 * ---------------------------------------------------------------------- */
#define MLA_SPLIT_BALANCED (-1)
size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t B,
                                  int32_t n_q, int32_t max_kv_len,
                                  int32_t n_split);
mla_status mla_decode(const mla_dims* dims, int32_t B, int32_t n_q,
                      const void* q, const void* cache, int32_t num_blocks,
                      const int32_t* block_table, int32_t max_blocks,
                      const int32_t* kv_lens, int32_t max_kv_len,
                      int32_t causal, int32_t n_split, float* o_lat,
                      float* lse, void* ws, size_t ws_bytes,
                      mla_stream_t stream);

/* mla_decode without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, results and errors are those of
 * mla_decode; the partial results live in a file-scope device array of
 * MLA_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends (its device address is taken once per device, at the
 * first call on it).  Requests whose mla_decode_workspace_bytes exceed
 * that size return MLA_ERR_WORKSPACE (the largest: 32768 partial rows
 * (query rows x splits x heads) at d_c = 512, e.g. 64 sequences x 4 splits
 * x 128 heads, or the balanced plan's 256 slots x 128 heads).  The call
 * allocates nothing and clears nothing: every value it reads back from the
 * array it wrote first.  All calls on one GPU share the array, so calls
 * that overlap on one GPU (different streams, or host threads) race: the
 * caller serialises them. */
#define MLA_NOALLOC_SCRATCH_BYTES (65u * 1024u * 1024u)
mla_status mla_decode_noalloc(const mla_dims* dims, int32_t B, int32_t n_q,
                              const void* q, const void* cache,
                              int32_t num_blocks, const int32_t* block_table,
                              int32_t max_blocks, const int32_t* kv_lens,
                              int32_t max_kv_len, int32_t causal,
                              int32_t n_split, float* o_lat, float* lse,
                              mla_stream_t stream);

/* The split count mla_decode uses for n_split = 0 (host only). */
int32_t mla_decode_auto_splits(const mla_dims* dims, int32_t B, int32_t n_q,
                               int32_t max_kv_len);

/* Opt-in check of the device-side values the calls above trust, on HOST
 * copies of them (the caller copies the block table and lengths back, or
 * checks them before uploading).  Every decode step reads all of a
 * sequence's cached tokens through its block table ('MLA：潜在表示压缩与
 * 解耦 RoPE', section 1), so one bad entry sends a kernel outside the pool.
 *
 *   block_table  host [B][max_blocks] int32
 *   kv_lens      host [B] int32
 *   n_q          queries per sequence of the step (1 for a decode step)
 *   max_kv_len   the host bound passed to mla_decode (<= 0: not checked)
 *   bad_seq      host, may be NULL: receives the first offending sequence
 *                (-1 when none)
 * For every sequence b: n_q <= kv_lens[b] (and <= max_kv_len when that is
 * positive), ceil(kv_lens[b] / block_size) <= max_blocks, and the entries
 * block_table[b][0 .. ceil(kv_lens[b] / block_size) - 1] lie in
 * [0, num_blocks).  Returns MLA_OK, MLA_ERR_NULL (a required pointer),
 * MLA_ERR_SHAPE (B, max_blocks, n_q, block_size or num_blocks <= 0) or
 * MLA_ERR_RANGE (a violation).  Reads only; touches no device. */
mla_status mla_validate_block_table(const int32_t* block_table, int32_t B,
                                    int32_t max_blocks, const int32_t* kv_lens,
                                    int32_t n_q, int32_t block_size,
                                    int32_t num_blocks, int32_t max_kv_len,
                                    int32_t* bad_seq);

/* ------------------------------------------------------------------------
 * MHA-path chunked prefill: explicit per-head keys and values.
 *
 * For a chunk of many new tokens per sequence the explicit form costs fewer
 * operations than the absorbed one ('MiniMind 学习笔记 10', sections 10 and
 * 12; 'MLA：潜在表示压缩与解耦 RoPE', section 7: the non-absorbed forward).
 * A prefill step is:
 *   mla_append_cache (the chunk's rows), mla_query_mha, mla_prefill_mha,
 *   mla_out_values.
 *
 * mla_query_mha: q[t][h] = [q_C (d_h) | RoPE_{pos}(q_R) (d_r)] with c_Q =
 *   W_DQ h, q_C = W_UQ c_Q, q_R = W_QR c_Q, rounded once to bf16.  Arguments
 *   as mla_absorb_q (same workspace size, mla_absorb_workspace_bytes), output
 *   q_out [T][n_h][d_h + d_r] bf16.
 *
 * mla_prefill_mha: for sequence b and chunk query i (the chunk's n_q tokens
 *   are the last n_q of the sequence's kv_lens[b] keys), every head h:
 *     k_C[t] = W_UK_h c_KV[t], v_C[t] = W_UV_h c_KV[t] for all cached t,
 *     score_t = (q_C . k_C[t] + q_R . k_R[t]) / sqrt(d_h + d_r),
 *     o[b][i][h] = sum_t softmax(score)_t v_C[t]   (fp32, d_h values)
 *   over keys t <= kv_lens[b] - n_q + i (causal != 0) or all keys; lse as in
 *   mla_decode.  q [B][n_q][n_h][d_h + d_r] bf16 (mla_query_mha), the cache
 *   and block table as in mla_decode, kv_lens[b] >= n_q, max_kv_len >= every
 *   kv_lens[b].  Device-side values are trusted as in mla_decode: block ids
 *   must name blocks of the pool; a kv_lens[b] outside [n_q, max_kv_len]
 *   yields unspecified outputs but no access past the table or workspace
 *   (lengths are clamped to max_kv_len).
 *   ws: mla_prefill_mha_workspace_bytes(dims, B, max_kv_len) bytes: the
 *   gathered rows, max(B max_kv_len, 128) (d_c + d_r) 2 bytes, and the bf16
 *   k_C / v_C of one group of heads at a time, the group being the largest
 *   divisor of n_h whose k_C / v_C fit 768 MiB (at least one head): for 8
 *   sequences of 10240 keys at DeepSeek-V2 dims, 16 heads and 765 MB in
 *   all.  The groups run one after another in the call.
 *   Errors: MLA_ERR_SHAPE for max_kv_len < n_q or max_kv_len > max_blocks
 *   block_size, MLA_ERR_WORKSPACE for a short workspace, MLA_ERR_UNSUPPORTED
 *   unless bf16 with d_h = 128 and d_r = 64.
 *
 * mla_out_values: u = W_O o for o [T][n_h d_h] fp32 (value space, the output
 *   of mla_prefill_mha), u [T][d] in the activation dtype.  Workspace as
 *   mla_out (mla_out_workspace_bytes).
 * ---------------------------------------------------------------------- */
mla_status mla_query_mha(const mla_dims* dims, int32_t T, const void* h,
                         const int32_t* pos, const void* w_dq,
                         const void* w_uq, const void* w_qr,
                         const float* rope_cos, const float* rope_sin,
                         int32_t max_pos, void* q_out, void* ws,
                         size_t ws_bytes, mla_stream_t stream);
size_t mla_prefill_mha_workspace_bytes(const mla_dims* dims, int32_t B,
                                       int32_t max_kv_len);
mla_status mla_prefill_mha(const mla_dims* dims, int32_t B, int32_t n_q,
                           const void* q, const void* cache,
                           int32_t num_blocks, const int32_t* block_table,
                           int32_t max_blocks, const int32_t* kv_lens,
                           int32_t max_kv_len, int32_t causal,
                           const void* w_uk, const void* w_uv, float* o_v,
                           float* lse, void* ws, size_t ws_bytes,
                           mla_stream_t stream);
mla_status mla_out_values(const mla_dims* dims, int32_t T, const float* o_v,
                          const void* w_o, void* u, void* ws, size_t ws_bytes,
                          mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_out - value up-projection after the weighted sum, then W_O.
 *
 * v_h = W_UV_h o_lat_h (kept fp32), u = W_O [v_0; ...; v_{n_h-1}] rounded
 * once to the activation dtype ('MLA：潜在表示压缩与解耦 RoPE', section 4
 * per-head output formula and section 7).
 *
 *   o_lat [T][n_h][d_c] fp32;  w_uv [n_h*d_h][d_c];  w_o [d][n_h*d_h]
 *   u     [T][d]
 *   ws    at least mla_out_workspace_bytes(dims, T)
 * ---------------------------------------------------------------------- */
size_t mla_out_workspace_bytes(const mla_dims* dims, int32_t T);
mla_status mla_out(const mla_dims* dims, int32_t T, const float* o_lat,
                   const void* w_uv, const void* w_o, void* u, void* ws,
                   size_t ws_bytes, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_decode_out - mla_decode followed by mla_out on its rows, in one call.
 *
 * The output projection takes the decode's o_lat as it stands: v_h =
 * W_UV_h o_lat_h, u = W_O v for the T = B n_q query rows ('MLA：潜在表示
 * 压缩与解耦 RoPE', section 4: the values are up-projected after the
 * weighted sum over the latent rows; section 7).  For one or two query
 * rows with split keys on the bf16 matrix-core path (d_c = 512, d_h = 128,
 * uniform splits) the split combine and the W_UV product run as one
 * kernel, whose weight reads overlap the combine's; every other shape runs
 * the two calls' own paths.
 *
 *   arguments of mla_decode, then w_uv, w_o and u of mla_out; o_lat and
 *   lse are written as by mla_decode (lse may be NULL)
 *   ws    at least mla_decode_out_workspace_bytes(dims, B, n_q,
 *         max_kv_len, n_split)
 * Results equal those of the two calls up to the order of fp32 sums.
 * Errors: those of either call, all checked before anything is launched.
 * ---------------------------------------------------------------------- */
size_t mla_decode_out_workspace_bytes(const mla_dims* dims, int32_t B,
                                      int32_t n_q, int32_t max_kv_len,
                                      int32_t n_split);
mla_status mla_decode_out(const mla_dims* dims, int32_t B, int32_t n_q,
                          const void* q, const void* cache,
                          int32_t num_blocks, const int32_t* block_table,
                          int32_t max_blocks, const int32_t* kv_lens,
                          int32_t max_kv_len, int32_t causal, int32_t n_split,
                          const void* w_uv, const void* w_o, float* o_lat,
                          float* lse, void* u, void* ws, size_t ws_bytes,
                          mla_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
