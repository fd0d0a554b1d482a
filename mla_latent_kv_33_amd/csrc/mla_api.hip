// C ABI of libmla.so: argument checks, workspace layout and the launch
// sequence of each step.  Declarations and contracts: include/mla.h.

#include <algorithm>
#include <math.h>
#include <mutex>
#include <string.h>

#include "mla_common.hpp"
#include "mla_kernels.hpp"

using namespace mla;

namespace {

constexpr size_t WS_ALIGN = 256;

inline size_t align_up(size_t x) { return (x + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

// Bump allocator over the caller's workspace.
struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* p) : base((char*)p) {}
  float* take(size_t floats) {
    float* p = (float*)(base + used);
    used += align_up(floats * sizeof(float));
    return p;
  }
};

bool dims_ok(const mla_dims* d) {
  if (!d) return false;
  if (d->d <= 0 || d->n_h <= 0 || d->d_h <= 0 || d->d_c <= 0 || d->d_r <= 0 ||
      d->d_cq <= 0 || d->block_size <= 0)
    return false;
  if (d->d_r % 2) return false;
  if (d->block_size & (d->block_size - 1)) return false;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return false;
  return true;
}

// The bf16 kernels move 8 elements (16 bytes) at a time along every row,
// and the decode-batch projections stream their weights in 64-deep k steps:
// every contraction length of a projection (d, d_cq, d_c, n_h d_h) is a
// multiple of 64.
bool dims_supported(const mla_dims* d) {
  if (d->dtype != MLA_BF16) return true;
  return d->d % 64 == 0 && d->d_cq % 64 == 0 && d->d_c % 64 == 0 &&
         ((long)d->n_h * d->d_h) % 64 == 0 && d->d_h % 8 == 0 &&
         d->d_r % 8 == 0;
}

mla_status dev(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_DEVICE; }

#define MLA_TRY(expr)                          \
  do {                                         \
    hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return MLA_ERR_DEVICE; \
  } while (0)

// ---- GEMM argument builders (shared by sizing and launching) ----
GemmArgs append_gemm(const mla_dims& d, int T) {
  GemmArgs g;
  g.w_nt = 1;  // read once per step, not kept in the Infinity Cache
  g.lda = d.d;
  g.nb1 = d.d_c;
  g.ldb = d.d;
  g.ldc = d.d_c + d.d_r;
  g.c_ks = (long)T * (d.d_c + d.d_r);
  g.M = T;
  g.N = d.d_c + d.d_r;
  g.K = d.d;
  gemm_plan(d, g);
  return g;
}
GemmArgs cq_gemm(const mla_dims& d, int T) {
  GemmArgs g;
  g.w_nt = 1;  // read once per step, not kept in the Infinity Cache
  g.lda = d.d;
  g.ldb = d.d;
  g.ldc = d.d_cq;
  g.c_ks = (long)T * d.d_cq;
  g.M = T;
  g.N = d.d_cq;
  g.K = d.d;
  gemm_plan(d, g);
  return g;
}
GemmArgs qcr_gemm(const mla_dims& d, int T) {
  GemmArgs g;
  // W_UQ / W_QR and W_O keep ordinary loads: together (243.5 MB at
  // DeepSeek-V2 dims) they fit the 256 MB Infinity Cache, and the other
  // streams of a step are non-temporal
  g.a_f32 = 1;
  g.lda = d.d_cq;
  g.nb1 = d.n_h * d.d_h;
  g.ldb = d.d_cq;
  g.ldc = (long)d.n_h * (d.d_h + d.d_r);
  g.c_ks = (long)T * g.ldc;
  g.M = T;
  g.N = d.n_h * (d.d_h + d.d_r);
  g.K = d.d_cq;
  gemm_plan(d, g);
  return g;
}
GemmArgs absorb_gemm(const mla_dims& d, int T) {
  GemmArgs g;
  g.a_f32 = 1;
  g.lda = (long)d.n_h * (d.d_h + d.d_r);
  g.a_bs = d.d_h;
  g.b_nn = 1;
  g.ldb = d.d_c;
  g.b_bs = (long)d.d_h * d.d_c;
  g.ldc = (long)d.n_h * d.d_c;
  g.c_bs = d.d_c;
  g.M = T;
  g.N = d.d_c;
  g.K = d.d_h;
  g.batch = d.n_h;
  g.k_split = 1;
  return g;
}
GemmArgs uv_gemm(const mla_dims& d, int T) {
  GemmArgs g;
  g.w_nt = 1;  // read once per step, not kept in the Infinity Cache
  g.a_f32 = 1;
  g.lda = (long)d.n_h * d.d_c;
  g.a_bs = d.d_c;
  g.ldb = d.d_c;
  g.b_bs = (long)d.d_h * d.d_c;
  g.ldc = (long)d.n_h * d.d_h;
  g.c_bs = d.d_h;
  g.M = T;
  g.N = d.d_h;
  g.K = d.d_c;
  g.batch = d.n_h;
  gemm_plan(d, g, 1);  // its consumer reads one C
  return g;
}
GemmArgs o_gemm(const mla_dims& d, int T) {
  GemmArgs g;
  g.a_f32 = 1;
  g.lda = (long)d.n_h * d.d_h;
  g.ldb = (long)d.n_h * d.d_h;
  g.ldc = d.d;
  g.c_ks = (long)T * d.d;
  g.M = T;
  g.N = d.d;
  g.K = d.n_h * d.d_h;
  gemm_plan(d, g);
  return g;
}

size_t parts_floats(const GemmArgs& g) { return (size_t)g.k_split * g.M * g.N * g.batch; }

int decode_nblk(const mla_dims& d, int max_kv_len) {
  return (max_kv_len + d.block_size - 1) / d.block_size;
}

int auto_splits(const mla_dims& d, int B, int n_q, int max_kv_len) {
  const int nblk = decode_nblk(d, max_kv_len);
  long groups = (long)B * n_q;
  long target;
  if (decode_mfma_supported(d)) {
    groups *= (d.n_h + 127) / 128;
    target = 256;   // one workgroup per CU (LDS-bound occupancy)
  } else {
    groups *= d.n_h;
    target = 1024;
  }
  long s = (target + groups - 1) / groups;
  if (decode_mfma_supported(d)) {
    // Matrix-core kernel: down to one 64-token block per split.  A count of
    // 8 or more is rounded down to a multiple of 8: small grids run two
    // 64-head workgroups per split (launch_decode_mfma), launched rows x
    // splits apart, and a multiple of 8 puts both on the same XCD, whose L2
    // then serves the second read of every cache row (B = 1 at 4K context:
    // 32 splits 28.8 us, 64 splits 26.6 us, 65 splits 28.0 us).
    if (s > nblk) s = nblk;
    if (s >= 8) s = s / 8 * 8;
  } else {
    // SIMT kernel: at least 4 blocks per split.
    const long cap = nblk / 4 > 0 ? nblk / 4 : 1;
    if (s > cap) s = cap;
  }
  if (s < 1) s = 1;
  return (int)s;
}

// MLA_SPLIT_BALANCED on the matrix-core path for 2 .. BAL_SLOTS query rows:
// splits balanced per row by the kernel (DecodeBalance).  Elsewhere it
// means the automatic uniform count: a single row has nothing to balance
// (and the plan would put a kv_lens load ahead of its query loads).  The
// plan costs about 3 us per call on uniform lengths (the same load ahead
// of the query loads), hence opt-in.
bool balanced_mode(const mla_dims& d, int B, int n_q, int n_split) {
  const long rows = (long)B * n_q;
  return n_split == MLA_SPLIT_BALANCED && decode_mfma_supported(d) &&
         rows >= 2 && rows <= BAL_SLOTS;
}

// Effective split count for a requested one (at most one block per split).
int split_count(const mla_dims& d, int max_kv_len, int want) {
  const int nblk = decode_nblk(d, max_kv_len);
  if (want < 1) want = 1;
  return want > nblk ? nblk : want;
}

// The uniform split count of a request (0 and MLA_SPLIT_BALANCED: auto).
int uniform_request(const mla_dims& d, int B, int n_q, int max_kv_len,
                    int n_split) {
  return split_count(d, max_kv_len,
                     n_split > 0 ? n_split : auto_splits(d, B, n_q, max_kv_len));
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "null pointer argument";
    case MLA_ERR_SHAPE: return "inconsistent or invalid sizes";
    case MLA_ERR_UNSUPPORTED: return "dims or dtype not supported";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_RANGE: return "argument out of range";
    case MLA_ERR_DEVICE: return "device launch failed";
  }
  return "unknown status";
}

const char* mla_version(void) { return "mla-gfx950 0.1"; }

mla_status mla_rope_tables_host(int32_t d_r, double base, int32_t max_pos,
                                float* cos_out, float* sin_out) {
  if (!cos_out || !sin_out) return MLA_ERR_NULL;
  if (d_r <= 0 || d_r % 2 || max_pos <= 0 || !(base > 0.0)) return MLA_ERR_SHAPE;
  const int half = d_r / 2;
  for (int j = 0; j < half; ++j) {
    const double theta = pow(base, -2.0 * j / (double)d_r);
    for (int p = 0; p < max_pos; ++p) {
      const double a = (double)p * theta;
      cos_out[(size_t)p * half + j] = (float)cos(a);
      sin_out[(size_t)p * half + j] = (float)sin(a);
    }
  }
  return MLA_OK;
}

// ------------------------------------------------------------------ append
size_t mla_append_workspace_bytes(const mla_dims* dims, int32_t T) {
  if (!dims_ok(dims) || T <= 0) return 0;
  return align_up(parts_floats(append_gemm(*dims, T)) * sizeof(float));
}

mla_status mla_append_cache(const mla_dims* dims, int32_t T, const void* h,
                            const int32_t* seq_idx, const int32_t* pos,
                            const void* w_dkv, const void* w_kr,
                            const float* rope_cos, const float* rope_sin,
                            int32_t max_pos, const int32_t* block_table,
                            int32_t max_blocks, void* cache,
                            int32_t num_blocks, void* ws, size_t ws_bytes,
                            mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || T < 0 || max_pos <= 0 || max_blocks <= 0 ||
      num_blocks <= 0)
    return MLA_ERR_SHAPE;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (T == 0) return MLA_OK;
  if (!h || !seq_idx || !pos || !w_dkv || !w_kr || !rope_cos || !rope_sin ||
      !block_table || !cache)
    return MLA_ERR_NULL;
  const mla_dims& d = *dims;
  const size_t need = mla_append_workspace_bytes(dims, T);
  if (!ws || ws_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (gemv_supported(d, T))
    return dev(launch_gemv_append(d, T, h, w_dkv, w_kr, seq_idx, pos,
                                  rope_cos, rope_sin, max_pos, block_table,
                                  max_blocks, cache, s));
  GemmArgs g = append_gemm(d, T);
  g.A = h;
  g.B = w_dkv;
  g.B2 = w_kr;
  g.C = (float*)ws;
  MLA_TRY(launch_gemm(d, g, s));
  MLA_TRY(launch_append_scatter(d, T, g.C, g.k_split, g.c_ks, seq_idx, pos,
                                rope_cos, rope_sin, max_pos, block_table,
                                max_blocks, cache, s));
  return MLA_OK;
}

mla_status mla_append_cache_rmsnorm(
    const mla_dims* dims, int32_t T, const void* h, const int32_t* seq_idx,
    const int32_t* pos, const void* w_dkv, const void* w_kr,
    const void* kv_norm_w, float eps, const float* rope_cos,
    const float* rope_sin, int32_t max_pos, const int32_t* block_table,
    int32_t max_blocks, void* cache, int32_t num_blocks, void* ws,
    size_t ws_bytes, mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || T < 0 || max_pos <= 0 || max_blocks <= 0 ||
      num_blocks <= 0 || !(eps >= 0.0f))
    return MLA_ERR_SHAPE;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (T == 0) return MLA_OK;
  if (!h || !seq_idx || !pos || !w_dkv || !w_kr || !kv_norm_w || !rope_cos ||
      !rope_sin || !block_table || !cache)
    return MLA_ERR_NULL;
  const mla_dims& d = *dims;
  const size_t need = mla_append_workspace_bytes(dims, T);
  if (!ws || ws_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  // The norm needs each whole c_KV row, which the matrix-vector append (two
  // rows per wave) never holds: every T takes the GEMM and the normalising
  // scatter.
  GemmArgs g = append_gemm(d, T);
  g.A = h;
  g.B = w_dkv;
  g.B2 = w_kr;
  g.C = (float*)ws;
  MLA_TRY(launch_gemm(d, g, s));
  MLA_TRY(launch_append_norm_scatter(d, T, g.C, g.k_split, g.c_ks, kv_norm_w,
                                     eps, seq_idx, pos, rope_cos, rope_sin,
                                     max_pos, block_table, max_blocks, cache,
                                     s));
  return MLA_OK;
}

// ------------------------------------------------------------------ absorb
extern "C++" {  // helpers below keep C++ linkage
namespace {
struct AbsorbWs {
  float *cq_parts, *cq, *qcr_parts, *qcr;
  size_t bytes;
};
AbsorbWs absorb_layout(const mla_dims& d, int T, void* base) {
  Carve c(base);
  AbsorbWs w;
  const GemmArgs g1 = cq_gemm(d, T), g2 = qcr_gemm(d, T);
  w.cq_parts = c.take(parts_floats(g1));
  w.cq = g1.k_split > 1 ? c.take((size_t)T * d.d_cq) : w.cq_parts;
  w.qcr_parts = c.take(parts_floats(g2));
  w.qcr = g2.k_split > 1 ? c.take((size_t)T * g2.N) : w.qcr_parts;
  w.bytes = c.used;
  return w;
}
}  // namespace
}  // extern "C++"

extern "C++" {  // helpers below keep C++ linkage
namespace {
// The query path from c_Q on (fp32, or pre-split hi|lo when cq_hl): q_C and
// q_R = W_UQ c_Q, W_QR c_Q, then RoPE(q_R) and q_lat_h = W_UK_h^T q_C_h into
// the query rows.
mla_status query_from_cq(const mla_dims& d, int T, const float* cq,
                         bool cq_hl, float* qcr_parts, float* qcr,
                         const int32_t* pos, const void* w_uq,
                         const void* w_qr, const void* w_uk,
                         const float* rope_cos, const float* rope_sin,
                         int max_pos, void* q_out, hipStream_t s) {
  GemmArgs g2 = qcr_gemm(d, T);
  g2.A = cq;
  g2.a_hl = cq_hl;
  g2.B = w_uq;
  g2.B2 = w_qr;
  g2.C = qcr_parts;
  MLA_TRY(launch_gemm(d, g2, s));
  // Decode batches: one kernel reads the K-split parts of q_C / q_R and
  // writes both halves of every query row.
  if (absorb_fast_supported(d, T, g2.k_split))
    return dev(launch_absorb_fast(d, T, qcr_parts, g2.k_split, g2.c_ks,
                                  g2.ldc, w_uk, pos, rope_cos, rope_sin,
                                  max_pos, q_out, s));
  if (g2.k_split > 1)
    MLA_TRY(launch_reduce_parts(qcr_parts, g2.k_split, g2.c_ks,
                                (long)T * g2.N, qcr, s));

  MLA_TRY(launch_query_rope(d, T, qcr + (long)d.n_h * d.d_h, 1, 0, g2.ldc,
                            pos, rope_cos, rope_sin, max_pos, q_out, s));

  // q_lat_h = W_UK_h^T q_C_h straight into the first d_c columns of each
  // head's q row (rounded to bf16 by the GEMM for bf16 layers).
  GemmArgs g3 = absorb_gemm(d, T);
  g3.A = qcr;
  g3.B = w_uk;
  g3.ldc = (long)d.n_h * (d.d_c + d.d_r);
  g3.c_bs = d.d_c + d.d_r;
  if (d.dtype == MLA_BF16)
    g3.c16 = q_out;
  else
    g3.C = (float*)q_out;
  MLA_TRY(launch_gemm(d, g3, s));
  return MLA_OK;
}
}  // namespace
}  // extern "C++"

size_t mla_absorb_workspace_bytes(const mla_dims* dims, int32_t T) {
  if (!dims_ok(dims) || T <= 0) return 0;
  return absorb_layout(*dims, T, nullptr).bytes;
}

mla_status mla_absorb_q(const mla_dims* dims, int32_t T, const void* h,
                        const int32_t* pos, const void* w_dq,
                        const void* w_uq, const void* w_qr, const void* w_uk,
                        const float* rope_cos, const float* rope_sin,
                        int32_t max_pos, void* q_out, void* ws,
                        size_t ws_bytes, mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || T < 0 || max_pos <= 0) return MLA_ERR_SHAPE;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (T == 0) return MLA_OK;
  if (!h || !pos || !w_dq || !w_uq || !w_qr || !w_uk || !rope_cos ||
      !rope_sin || !q_out)
    return MLA_ERR_NULL;
  const mla_dims& d = *dims;
  if (!ws) return MLA_ERR_WORKSPACE;
  const AbsorbWs w = absorb_layout(d, T, ws);
  if (ws_bytes < w.bytes) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (gemv_supported(d, T, GV_QO_MAXT)) {
    // c_Q (bf16 hi|lo pairs, 4 bytes per value) and q_C (fp32) at the start
    // of the workspace (the layout above holds at least
    // T (d_cq + n_h (d_h + d_r)) floats)
    float* cq = (float*)ws;
    float* qc = cq + (size_t)T * d.d_cq;
    return dev(launch_gemv_query(d, T, h, w_dq, w_uq, w_qr, w_uk, pos,
                                 rope_cos, rope_sin, max_pos, cq, qc, q_out,
                                 s));
  }

  GemmArgs g1 = cq_gemm(d, T);
  const GemmArgs g2 = qcr_gemm(d, T);
  // c_Q goes to the weight-streaming kernel of the next GEMM pre-split
  // (hi|lo), written by the reduce of the K parts or by the GEMM itself
  const bool cq_hl = g2.ntw < 0 && (g1.k_split > 1 || g1.ntw < 0);
  g1.A = h;
  g1.B = w_dq;
  g1.C = w.cq_parts;
  g1.c_hl = cq_hl && g1.k_split == 1;
  MLA_TRY(launch_gemm(d, g1, s));
  if (g1.k_split > 1) {
    if (cq_hl)
      MLA_TRY(launch_reduce_parts_hl(w.cq_parts, g1.k_split, g1.c_ks,
                                     (long)T * d.d_cq, d.d_cq, w.cq, s));
    else
      MLA_TRY(launch_reduce_parts(w.cq_parts, g1.k_split, g1.c_ks,
                                  (long)T * d.d_cq, w.cq, s));
  }
  return query_from_cq(d, T, w.cq, cq_hl, w.qcr_parts, w.qcr, pos, w_uq,
                       w_qr, w_uk, rope_cos, rope_sin, max_pos, q_out, s);
}


// ---------------------------------------- append and query in one call
extern "C++" {  // helpers below keep C++ linkage
namespace {
// [W_DQ; W_DKV; W_KR] h: the three down-projections of the new tokens
// stacked as one weight of d_cq + d_c + d_r rows.
GemmArgs down_gemm(const mla_dims& d, int T) {
  GemmArgs g;
  g.w_nt = 1;  // read once per step, not kept in the Infinity Cache
  g.lda = d.d;
  g.ldb = d.d;
  g.nb1 = d.d_cq;
  g.nb2 = d.d_cq + d.d_c;
  g.ldc = d.d_cq + d.d_c + d.d_r;
  g.c_ks = (long)T * g.ldc;
  g.M = T;
  g.N = (int)g.ldc;
  g.K = d.d;
  gemm_plan(d, g);
  return g;
}
// The stacked form serves bf16 decode batches past the matrix-vector token
// counts: one weight-streaming projection with K parts (summed by the
// shared epilogue), feeding a W_UQ / W_QR projection that takes c_Q
// pre-split.
bool stacked_down(const mla_dims& d, int T) {
  if (d.dtype != MLA_BF16 || gemv_supported(d, T) ||
      gemv_supported(d, T, GV_QO_MAXT))
    return false;
  const GemmArgs g = down_gemm(d, T), g2 = qcr_gemm(d, T);
  return g.ntw < 0 && g.k_split > 1 && g2.ntw < 0 && d.d_cq % 8 == 0;
}
struct StackedWs {
  float *parts, *cq, *qcr_parts, *qcr;
  size_t bytes;
};
StackedWs stacked_layout(const mla_dims& d, int T, void* base) {
  Carve c(base);
  StackedWs w;
  const GemmArgs g = down_gemm(d, T), g2 = qcr_gemm(d, T);
  w.parts = c.take(parts_floats(g));
  w.cq = c.take((size_t)T * d.d_cq);  // hi|lo pairs, 4 bytes per value
  w.qcr_parts = c.take(parts_floats(g2));
  w.qcr = g2.k_split > 1 ? c.take((size_t)T * g2.N) : w.qcr_parts;
  w.bytes = c.used;
  return w;
}
}  // namespace
}  // extern "C++"

size_t mla_append_absorb_workspace_bytes(const mla_dims* dims, int32_t T) {
  if (!dims_ok(dims) || T <= 0) return 0;
  size_t n = mla_append_workspace_bytes(dims, T);
  const size_t a = mla_absorb_workspace_bytes(dims, T);
  if (a > n) n = a;
  if (dims_supported(dims) && stacked_down(*dims, T)) {
    const size_t f = stacked_layout(*dims, T, nullptr).bytes;
    if (f > n) n = f;
  }
  return n;
}

mla_status mla_append_absorb_q(
    const mla_dims* dims, int32_t T, const void* h, const int32_t* seq_idx,
    const int32_t* pos, const void* w_dkv, const void* w_kr, const void* w_dq,
    const void* w_uq, const void* w_qr, const void* w_uk,
    const float* rope_cos, const float* rope_sin, int32_t max_pos,
    const int32_t* block_table, int32_t max_blocks, void* cache,
    int32_t num_blocks, void* q_out, void* ws, size_t ws_bytes,
    mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || T < 0 || max_pos <= 0 || max_blocks <= 0 ||
      num_blocks <= 0)
    return MLA_ERR_SHAPE;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (T == 0) return MLA_OK;
  if (!h || !seq_idx || !pos || !w_dkv || !w_kr || !w_dq || !w_uq || !w_qr ||
      !w_uk || !rope_cos || !rope_sin || !block_table || !cache || !q_out)
    return MLA_ERR_NULL;
  if (!ws || ws_bytes < mla_append_absorb_workspace_bytes(dims, T))
    return MLA_ERR_WORKSPACE;
  const mla_dims& d = *dims;
  hipStream_t s = (hipStream_t)stream;
  if (d.dtype == MLA_BF16 && gemv_supported(d, T, GV_QO_MAXT) &&
      d.d_cq % 2 == 0) {
    // one or two tokens: the three down-projections as one matrix-vector
    // launch, then the query path's own (c_Q and q_C at the start of the
    // workspace, as in mla_absorb_q)
    float* cq = (float*)ws;
    float* qc = cq + (size_t)T * d.d_cq;
    MLA_TRY(launch_gemv_down(d, T, h, w_dq, w_dkv, w_kr, seq_idx, pos,
                             rope_cos, rope_sin, max_pos, block_table,
                             max_blocks, cache, cq, s));
    return dev(launch_gemv_query_tail(d, T, w_uq, w_qr, w_uk, pos, rope_cos,
                                      rope_sin, max_pos, cq, qc, q_out, s));
  }
  if (!stacked_down(d, T)) {
    // the two calls' own paths, one after the other on the stream (the
    // workspace is free again once the append's kernels have run)
    const mla_status st = mla_append_cache(
        dims, T, h, seq_idx, pos, w_dkv, w_kr, rope_cos, rope_sin, max_pos,
        block_table, max_blocks, cache, num_blocks, ws, ws_bytes, stream);
    if (st != MLA_OK) return st;
    return mla_absorb_q(dims, T, h, pos, w_dq, w_uq, w_qr, w_uk, rope_cos,
                        rope_sin, max_pos, q_out, ws, ws_bytes, stream);
  }
  const StackedWs w = stacked_layout(d, T, ws);
  GemmArgs g = down_gemm(d, T);
  g.A = h;
  g.B = w_dq;
  g.B2 = w_dkv;
  g.B3 = w_kr;
  g.C = w.parts;
  MLA_TRY(launch_gemm(d, g, s));
  MLA_TRY(launch_project_epilogue(d, T, w.parts, g.k_split, g.c_ks, w.cq,
                                  seq_idx, pos, rope_cos, rope_sin, max_pos,
                                  block_table, max_blocks, cache, s));
  return query_from_cq(d, T, w.cq, true, w.qcr_parts, w.qcr, pos, w_uq, w_qr,
                       w_uk, rope_cos, rope_sin, max_pos, q_out, s);
}

// ------------------------------------------------- pre-merged absorption
extern "C++" {  // helpers below keep C++ linkage
namespace {
GemmArgs merged_gemm(const mla_dims& d, int T) {
  GemmArgs g;
  g.a_f32 = 1;
  g.lda = d.d_cq;
  g.nb1 = d.n_h * d.d_c;
  g.ldb = d.d_cq;
  g.ldc = (long)d.n_h * (d.d_c + d.d_r);
  g.c_ks = (long)T * g.ldc;
  g.M = T;
  g.N = d.n_h * (d.d_c + d.d_r);
  g.K = d.d_cq;
  gemm_plan(d, g);
  return g;
}
struct MergedWs {
  float *cq_parts, *cq, *parts;
  size_t bytes;
};
MergedWs merged_layout(const mla_dims& d, int T, void* base) {
  Carve c(base);
  MergedWs w;
  const GemmArgs g1 = cq_gemm(d, T), g2 = merged_gemm(d, T);
  w.cq_parts = c.take(parts_floats(g1));
  w.cq = g1.k_split > 1 ? c.take((size_t)T * d.d_cq) : w.cq_parts;
  w.parts = c.take(parts_floats(g2));
  w.bytes = c.used;
  return w;
}
}  // namespace
}  // extern "C++"

mla_status mla_merge_uq_uk(const mla_dims* dims, const void* w_uq,
                           const void* w_uk, void* w_merged,
                           mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims)) return MLA_ERR_SHAPE;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (!w_uq || !w_uk || !w_merged) return MLA_ERR_NULL;
  return dev(launch_merge_uq_uk(*dims, w_uq, w_uk, w_merged,
                                (hipStream_t)stream));
}

size_t mla_absorb_merged_workspace_bytes(const mla_dims* dims, int32_t T) {
  if (!dims_ok(dims) || T <= 0) return 0;
  return merged_layout(*dims, T, nullptr).bytes;
}

mla_status mla_absorb_q_merged(const mla_dims* dims, int32_t T, const void* h,
                               const int32_t* pos, const void* w_dq,
                               const void* w_merged, const void* w_qr,
                               const float* rope_cos, const float* rope_sin,
                               int32_t max_pos, void* q_out, void* ws,
                               size_t ws_bytes, mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || T < 0 || max_pos <= 0) return MLA_ERR_SHAPE;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (T == 0) return MLA_OK;
  if (!h || !pos || !w_dq || !w_merged || !w_qr || !rope_cos || !rope_sin ||
      !q_out)
    return MLA_ERR_NULL;
  const mla_dims& d = *dims;
  if (!ws) return MLA_ERR_WORKSPACE;
  const MergedWs w = merged_layout(d, T, ws);
  if (ws_bytes < w.bytes) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  // c_Q = W_DQ h (fp32)
  GemmArgs g1 = cq_gemm(d, T);
  g1.A = h;
  g1.B = w_dq;
  g1.C = w.cq_parts;
  MLA_TRY(launch_gemm(d, g1, s));
  if (g1.k_split > 1)
    MLA_TRY(launch_reduce_parts(w.cq_parts, g1.k_split, g1.c_ks,
                                (long)T * d.d_cq, w.cq, s));
  // [q_lat of every head | q_R before RoPE] = c_Q [M_0; ...; W_QR]^T
  GemmArgs g2 = merged_gemm(d, T);
  g2.A = w.cq;
  g2.B = w_merged;
  g2.B2 = w_qr;
  g2.C = w.parts;
  MLA_TRY(launch_gemm(d, g2, s));
  // q_lat rows (t, h) of d_c values into the first d_c columns of the query
  // rows (source: token t's GEMM row, head h's d_c columns), then RoPE(q_R)
  // into the last d_r
  MLA_TRY(launch_convert(d, T * d.n_h, d.d_c, w.parts, d.d_c, g2.k_split,
                         g2.c_ks, q_out, d.d_c + d.d_r, s, d.n_h, g2.ldc));
  MLA_TRY(launch_query_rope(d, T, w.parts + (long)d.n_h * d.d_c, g2.k_split,
                            g2.c_ks, g2.ldc, pos, rope_cos, rope_sin, max_pos,
                            q_out, s));
  return MLA_OK;
}

// ------------------------------------------------------------------ decode
int32_t mla_decode_auto_splits(const mla_dims* dims, int32_t B, int32_t n_q,
                               int32_t max_kv_len) {
  if (!dims_ok(dims) || B <= 0 || n_q <= 0 || max_kv_len <= 0) return 1;
  return split_count(*dims, max_kv_len, auto_splits(*dims, B, n_q, max_kv_len));
}

size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t B, int32_t n_q,
                                  int32_t max_kv_len, int32_t n_split) {
  if (!dims_ok(dims) || B <= 0 || n_q <= 0 || max_kv_len <= 0 ||
      n_split < MLA_SPLIT_BALANCED)
    return 0;
  const mla_dims& d = *dims;
  if (balanced_mode(d, B, n_q, n_split)) {
    const size_t rows = (size_t)BAL_SLOTS * d.n_h;
    return align_up(rows * d.d_c * sizeof(float)) +
           2 * align_up(rows * sizeof(float)) +
           align_up((size_t)B * n_q * sizeof(int2));
  }
  const int ns = uniform_request(d, B, n_q, max_kv_len, n_split);
  if (ns <= 1) return 0;
  const size_t rows = (size_t)B * n_q * ns * d.n_h;
  return align_up(rows * d.d_c * sizeof(float)) + 2 * align_up(rows * sizeof(float));
}

}  // extern "C"

namespace {
// One query per sequence reads each cache row once per call: beyond a
// quarter of the 256 MB Infinity Cache the rows are copied with
// non-temporal loads, so that they do not push out the weights it holds
// between steps (B = 64 at 8K context, 604 MB of rows: 293-294 -> 287-288
// us per step together with the weights' policy, same box).  Causal chunks
// (n_q > 1) reread every row for each query and keep ordinary loads.
bool decode_cache_nt(const mla_dims& d, int B, int n_q, int max_kv_len) {
  return n_q == 1 &&
         (double)B * max_kv_len * (d.d_c + d.d_r) * 2.0 > 64.0 * 1048576;
}
}  // namespace

extern "C" {

mla_status mla_decode(const mla_dims* dims, int32_t B, int32_t n_q,
                      const void* q, const void* cache, int32_t num_blocks,
                      const int32_t* block_table, int32_t max_blocks,
                      const int32_t* kv_lens, int32_t max_kv_len,
                      int32_t causal, int32_t n_split, float* o_lat,
                      float* lse, void* ws, size_t ws_bytes,
                      mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || B <= 0 || n_q <= 0 || max_kv_len <= 0 ||
      num_blocks <= 0 || max_blocks <= 0 || n_split < MLA_SPLIT_BALANCED)
    return MLA_ERR_SHAPE;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (!q || !cache || !block_table || !kv_lens || !o_lat) return MLA_ERR_NULL;
  const mla_dims& d = *dims;
  if (n_q > max_kv_len) return MLA_ERR_SHAPE;
  if (n_q > 1 && causal != 1) return MLA_ERR_UNSUPPORTED;
  const int nblk = decode_nblk(d, max_kv_len);
  if (nblk > max_blocks) return MLA_ERR_RANGE;
  if (n_split > nblk) return MLA_ERR_RANGE;
  const size_t need = mla_decode_workspace_bytes(dims, B, n_q, max_kv_len, n_split);
  if (need && (!ws || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool mfma = decode_mfma_supported(d);
  const int rows = B * n_q;
  const bool cache_nt = decode_cache_nt(d, B, n_q, max_kv_len);
  if (balanced_mode(d, B, n_q, n_split)) {
    Carve c(ws);
    const size_t prow = (size_t)BAL_SLOTS * d.n_h;
    float* o_part = c.take(prow * d.d_c);
    float* m_part = c.take(prow);
    float* l_part = c.take(prow);
    DecodeBalance bal;
    bal.plan = (int2*)c.take(2 * (size_t)rows);
    const long per_row = (nblk + BAL_MIN_CHUNK - 1) / BAL_MIN_CHUNK;
    bal.est_wgs = (int)std::min((long)BAL_SLOTS, (long)rows * per_row);
    MLA_TRY(launch_decode_mfma(d, B, n_q, q, cache, block_table, max_blocks,
                               kv_lens, 1, bal, o_part, m_part, l_part, o_lat,
                               lse, cache_nt, s));
    MLA_TRY(launch_combine(d, rows, 1, o_part, true, m_part, l_part, o_lat,
                           lse, s, bal.plan, BAL_SLOTS));
    return MLA_OK;
  }
  const int ns = uniform_request(d, B, n_q, max_kv_len, n_split);
  float *o_part = nullptr, *m_part = nullptr, *l_part = nullptr;
  if (ns > 1) {
    Carve c(ws);
    const size_t prow = (size_t)rows * ns * d.n_h;
    o_part = c.take(prow * d.d_c);
    m_part = c.take(prow);
    l_part = c.take(prow);
  }
  if (mfma)
    MLA_TRY(launch_decode_mfma(d, B, n_q, q, cache, block_table, max_blocks,
                               kv_lens, ns, DecodeBalance(), o_part, m_part,
                               l_part, o_lat, lse, cache_nt, s));
  else
    MLA_TRY(launch_decode_simt(d, B, n_q, q, cache, block_table, max_blocks,
                               kv_lens, ns, o_part, m_part, l_part, o_lat,
                               lse, s));
  if (ns > 1)
    MLA_TRY(launch_combine(d, rows, ns, o_part, mfma, m_part, l_part, o_lat,
                           lse, s));
  return MLA_OK;
}

size_t mla_decode_out_workspace_bytes(const mla_dims* dims, int32_t B,
                                      int32_t n_q, int32_t max_kv_len,
                                      int32_t n_split) {
  if (!dims_ok(dims) || B <= 0 || n_q <= 0 || max_kv_len <= 0 ||
      n_split < MLA_SPLIT_BALANCED || (int64_t)B * n_q > INT32_MAX)
    return 0;
  return align_up(mla_decode_workspace_bytes(dims, B, n_q, max_kv_len,
                                             n_split)) +
         mla_out_workspace_bytes(dims, B * n_q);
}

mla_status mla_decode_out(const mla_dims* dims, int32_t B, int32_t n_q,
                          const void* q, const void* cache,
                          int32_t num_blocks, const int32_t* block_table,
                          int32_t max_blocks, const int32_t* kv_lens,
                          int32_t max_kv_len, int32_t causal, int32_t n_split,
                          const void* w_uv, const void* w_o, float* o_lat,
                          float* lse, void* u, void* ws, size_t ws_bytes,
                          mla_stream_t stream) {
  // every check of both calls before anything is launched
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || B <= 0 || n_q <= 0 || max_kv_len <= 0 ||
      num_blocks <= 0 || max_blocks <= 0 || n_split < MLA_SPLIT_BALANCED ||
      (int64_t)B * n_q > INT32_MAX)
    return MLA_ERR_SHAPE;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (!q || !cache || !block_table || !kv_lens || !o_lat || !w_uv || !w_o ||
      !u)
    return MLA_ERR_NULL;
  const mla_dims& d = *dims;
  if (n_q > max_kv_len) return MLA_ERR_SHAPE;
  if (n_q > 1 && causal != 1) return MLA_ERR_UNSUPPORTED;
  const int nblk = decode_nblk(d, max_kv_len);
  if (nblk > max_blocks || n_split > nblk) return MLA_ERR_RANGE;
  const size_t dec_bytes =
      align_up(mla_decode_workspace_bytes(dims, B, n_q, max_kv_len, n_split));
  const size_t need =
      mla_decode_out_workspace_bytes(dims, B, n_q, max_kv_len, n_split);
  if (!ws || ws_bytes < need) return MLA_ERR_WORKSPACE;
  void* ws_out = (char*)ws + dec_bytes;
  const int T = B * n_q;
  hipStream_t s = (hipStream_t)stream;
  const int ns = balanced_mode(d, B, n_q, n_split)
                     ? 0
                     : uniform_request(d, B, n_q, max_kv_len, n_split);
  if (ns > 1 && decode_mfma_supported(d) &&
      gemv_supported(d, T, GV_QO_MAXT) && combine_uv_supported(d, T)) {
    // decode, then the split combine fused with W_UV, then W_O
    Carve c(ws);
    const size_t prow = (size_t)T * ns * d.n_h;
    float* o_part = c.take(prow * d.d_c);
    float* m_part = c.take(prow);
    float* l_part = c.take(prow);
    MLA_TRY(launch_decode_mfma(d, B, n_q, q, cache, block_table, max_blocks,
                               kv_lens, ns, DecodeBalance(), o_part, m_part,
                               l_part, o_lat, lse,
                               decode_cache_nt(d, B, n_q, max_kv_len), s));
    float* v = (float*)ws_out;
    MLA_TRY(launch_combine_uv(d, T, ns, o_part, m_part, l_part, w_uv, o_lat,
                              lse, v, s));
    return dev(launch_gemv_wo(d, T, v, w_o, u, s));
  }
  const mla_status st =
      mla_decode(dims, B, n_q, q, cache, num_blocks, block_table, max_blocks,
                 kv_lens, max_kv_len, causal, n_split, o_lat, lse, ws,
                 dec_bytes, stream);
  if (st != MLA_OK) return st;
  return mla_out(dims, T, o_lat, w_uv, w_o, u, ws_out, ws_bytes - dec_bytes,
                 stream);
}

mla_status mla_validate_block_table(const int32_t* block_table, int32_t B,
                                    int32_t max_blocks, const int32_t* kv_lens,
                                    int32_t n_q, int32_t block_size,
                                    int32_t num_blocks, int32_t max_kv_len,
                                    int32_t* bad_seq) {
  if (bad_seq) *bad_seq = -1;
  if (!block_table || !kv_lens) return MLA_ERR_NULL;
  if (B <= 0 || max_blocks <= 0 || n_q <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return MLA_ERR_SHAPE;
  for (int32_t b = 0; b < B; ++b) {
    const long kv = kv_lens[b];
    bool ok = kv >= n_q && (max_kv_len <= 0 || kv <= max_kv_len);
    const long need = (kv + block_size - 1) / block_size;
    ok = ok && need <= max_blocks;
    const int32_t* row = block_table + (size_t)b * max_blocks;
    for (long k = 0; ok && k < need; ++k)
      ok = row[k] >= 0 && row[k] < num_blocks;
    if (!ok) {
      if (bad_seq) *bad_seq = b;
      return MLA_ERR_RANGE;
    }
  }
  return MLA_OK;
}

// ------------------------------------------------- decode, no allocation
// The workspace of mla_decode_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  In host code its name is only a
// stand-in; the device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address reaches
// kernels.
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

// Device address of this device's `scratch`, or null on failure.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
    return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess)
      return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}
}  // namespace

mla_status mla_decode_noalloc(const mla_dims* dims, int32_t B, int32_t n_q,
                              const void* q, const void* cache,
                              int32_t num_blocks, const int32_t* block_table,
                              int32_t max_blocks, const int32_t* kv_lens,
                              int32_t max_kv_len, int32_t causal,
                              int32_t n_split, float* o_lat, float* lse,
                              mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || B <= 0 || n_q <= 0 || max_kv_len <= 0 ||
      num_blocks <= 0 || max_blocks <= 0 || n_split < MLA_SPLIT_BALANCED)
    return MLA_ERR_SHAPE;
  const size_t need =
      mla_decode_workspace_bytes(dims, B, n_q, max_kv_len, n_split);
  if (need > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need) {
    ws = scratch_address();
    if (!ws) return MLA_ERR_DEVICE;
  }
  // Every partial, maximum, sum and plan entry the decode reads is written
  // by the same call first, so nothing in `scratch` needs clearing.
  return mla_decode(dims, B, n_q, q, cache, num_blocks, block_table,
                    max_blocks, kv_lens, max_kv_len, causal, n_split, o_lat,
                    lse, ws, need ? (size_t)MLA_NOALLOC_SCRATCH_BYTES : 0,
                    stream);
}

// --------------------------------------------------------------------- out
namespace {
struct OutWs {
  float *v, *u_parts;
  size_t bytes;
};
OutWs out_layout(const mla_dims& d, int T, void* base) {
  Carve c(base);
  OutWs w;
  w.v = c.take(parts_floats(uv_gemm(d, T)));
  w.u_parts = c.take(parts_floats(o_gemm(d, T)));
  w.bytes = c.used;
  return w;
}
}  // namespace

// ------------------------------------------------------------ MHA prefill
mla_status mla_query_mha(const mla_dims* dims, int32_t T, const void* h,
                         const int32_t* pos, const void* w_dq,
                         const void* w_uq, const void* w_qr,
                         const float* rope_cos, const float* rope_sin,
                         int32_t max_pos, void* q_out, void* ws,
                         size_t ws_bytes, mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || T < 0 || max_pos <= 0) return MLA_ERR_SHAPE;
  if (!dims_supported(dims) || !prefill_mha_supported(*dims))
    return MLA_ERR_UNSUPPORTED;
  if (T == 0) return MLA_OK;
  if (!h || !pos || !w_dq || !w_uq || !w_qr || !rope_cos || !rope_sin ||
      !q_out)
    return MLA_ERR_NULL;
  const mla_dims& d = *dims;
  if (!ws) return MLA_ERR_WORKSPACE;
  const AbsorbWs w = absorb_layout(d, T, ws);
  if (ws_bytes < w.bytes) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  GemmArgs g1 = cq_gemm(d, T);
  g1.A = h;
  g1.B = w_dq;
  g1.C = w.cq_parts;
  MLA_TRY(launch_gemm(d, g1, s));
  if (g1.k_split > 1)
    MLA_TRY(launch_reduce_parts(w.cq_parts, g1.k_split, g1.c_ks,
                                (long)T * d.d_cq, w.cq, s));
  GemmArgs g2 = qcr_gemm(d, T);
  g2.A = w.cq;
  g2.B = w_uq;
  g2.B2 = w_qr;
  g2.C = w.qcr_parts;
  MLA_TRY(launch_gemm(d, g2, s));
  MLA_TRY(launch_query_mha(d, T, w.qcr_parts, g2.k_split, g2.c_ks, g2.ldc,
                           pos, rope_cos, rope_sin, max_pos, q_out, s));
  return MLA_OK;
}

namespace {
struct PrefillWs {
  uint16_t *rows, *kv;
  int group;  // heads whose k_C / v_C are materialised at a time
  size_t bytes;
};
// Rows of the gathered latents and of [k_C | v_C]: B kv_cap, at least 128
// (the up-projection GEMM's bf16 output needs more than 64 rows).
long prefill_rows(int B, int kv_cap) {
  return std::max((long)B * kv_cap, 128L);
}
// The explicit keys and values are materialised for one group of heads at
// a time: the largest divisor of n_h whose [k_C | v_C] rows fit
// PREFILL_KV_BUDGET bytes (at least one head).  The heads are independent,
// so the groups run one after another with no merge.
constexpr size_t PREFILL_KV_BUDGET = 768ull << 20;
int prefill_group(const mla_dims& d, long R) {
  const size_t per_head = (size_t)R * 2 * d.d_h * 2;
  int best = 1;
  for (int gsz = 1; gsz <= d.n_h; ++gsz)
    if (d.n_h % gsz == 0 && (size_t)gsz * per_head <= PREFILL_KV_BUDGET)
      best = gsz;
  return best;
}
PrefillWs prefill_layout(const mla_dims& d, int B, int kv_cap, void* base) {
  PrefillWs w;
  char* p = (char*)base;
  const long R = prefill_rows(B, kv_cap);
  w.group = prefill_group(d, R);
  const size_t rows_b = align_up((size_t)R * (d.d_c + d.d_r) * 2);
  const size_t kv_b = align_up((size_t)R * 2 * w.group * d.d_h * 2);
  w.rows = (uint16_t*)p;
  w.kv = (uint16_t*)(p ? p + rows_b : nullptr);
  w.bytes = rows_b + kv_b;
  return w;
}
}  // namespace

size_t mla_prefill_mha_workspace_bytes(const mla_dims* dims, int32_t B,
                                       int32_t max_kv_len) {
  if (!dims_ok(dims) || B <= 0 || max_kv_len <= 0) return 0;
  return prefill_layout(*dims, B, max_kv_len, nullptr).bytes;
}

mla_status mla_prefill_mha(const mla_dims* dims, int32_t B, int32_t n_q,
                           const void* q, const void* cache,
                           int32_t num_blocks, const int32_t* block_table,
                           int32_t max_blocks, const int32_t* kv_lens,
                           int32_t max_kv_len, int32_t causal,
                           const void* w_uk, const void* w_uv, float* o_v,
                           float* lse, void* ws, size_t ws_bytes,
                           mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || B < 0 || n_q < 0 || num_blocks <= 0 ||
      max_blocks <= 0 || max_kv_len < n_q || max_kv_len <= 0 ||
      (long)max_kv_len > (long)max_blocks * dims->block_size)
    return MLA_ERR_SHAPE;
  if (!dims_supported(dims) || !prefill_mha_supported(*dims))
    return MLA_ERR_UNSUPPORTED;
  if (B == 0 || n_q == 0) return MLA_OK;
  if (!q || !cache || !block_table || !kv_lens || !w_uk || !w_uv || !o_v)
    return MLA_ERR_NULL;
  const mla_dims& d = *dims;
  if (!ws) return MLA_ERR_WORKSPACE;
  const PrefillWs w = prefill_layout(d, B, max_kv_len, ws);
  if (ws_bytes < w.bytes) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  MLA_TRY(launch_gather_rows(d, B, cache, block_table, max_blocks, kv_lens,
                             max_kv_len, w.rows, s));
  // Per group of heads: [k_C | v_C] of every gathered row (one GEMM), then
  // the attention of those heads.
  for (int h0 = 0; h0 < d.n_h; h0 += w.group) {
    GemmArgs g;
    g.A = w.rows;
    g.lda = d.d_c + d.d_r;
    g.B = (const uint16_t*)w_uk + (size_t)h0 * d.d_h * d.d_c;
    g.B2 = (const uint16_t*)w_uv + (size_t)h0 * d.d_h * d.d_c;
    g.nb1 = w.group * d.d_h;
    g.ldb = d.d_c;
    g.M = (int)prefill_rows(B, max_kv_len);
    g.N = 2 * w.group * d.d_h;
    g.K = d.d_c;
    g.ldc = g.N;
    gemm_plan(d, g);
    if (g.k_split != 1 || g.ntw != 0) return MLA_ERR_UNSUPPORTED;
    g.c16 = w.kv;
    MLA_TRY(launch_gemm(d, g, s));
    MLA_TRY(launch_prefill_mha(d, B, n_q, q, w.rows, w.kv, h0, w.group,
                               kv_lens, max_kv_len, causal ? 1 : 0, o_v, lse,
                               s));
  }
  return MLA_OK;
}

mla_status mla_out_values(const mla_dims* dims, int32_t T, const float* o_v,
                          const void* w_o, void* u, void* ws, size_t ws_bytes,
                          mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || T < 0) return MLA_ERR_SHAPE;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (T == 0) return MLA_OK;
  if (!o_v || !w_o || !u) return MLA_ERR_NULL;
  const mla_dims& d = *dims;
  if (!ws) return MLA_ERR_WORKSPACE;
  const OutWs w = out_layout(d, T, ws);
  if (ws_bytes < w.bytes) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  GemmArgs g2 = o_gemm(d, T);
  g2.A = o_v;
  g2.B = w_o;
  g2.C = w.u_parts;
  MLA_TRY(launch_gemm(d, g2, s));
  MLA_TRY(launch_convert(d, T, d.d, w.u_parts, d.d, g2.k_split, g2.c_ks, u,
                         d.d, s));
  return MLA_OK;
}

size_t mla_out_workspace_bytes(const mla_dims* dims, int32_t T) {
  if (!dims_ok(dims) || T <= 0) return 0;
  return out_layout(*dims, T, nullptr).bytes;
}

mla_status mla_out(const mla_dims* dims, int32_t T, const float* o_lat,
                   const void* w_uv, const void* w_o, void* u, void* ws,
                   size_t ws_bytes, mla_stream_t stream) {
  if (!dims) return MLA_ERR_NULL;
  if (!dims_ok(dims) || T < 0) return MLA_ERR_SHAPE;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (T == 0) return MLA_OK;
  if (!o_lat || !w_uv || !w_o || !u) return MLA_ERR_NULL;
  const mla_dims& d = *dims;
  if (!ws) return MLA_ERR_WORKSPACE;
  const OutWs w = out_layout(d, T, ws);
  if (ws_bytes < w.bytes) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  // v as bf16 hi|lo pairs (the layout holds T n_h d_h floats)
  if (gemv_supported(d, T, GV_QO_MAXT))
    return dev(launch_gemv_out(d, T, o_lat, w_uv, w_o, (float*)ws, u, s));
  GemmArgs g1 = uv_gemm(d, T);
  GemmArgs g2 = o_gemm(d, T);
  // v goes to the weight-streaming kernel of W_O pre-split (hi|lo), written
  // so by the per-head GEMM
  const bool v_hl = g1.ntw < 0 && g1.k_split == 1 && g2.ntw < 0;
  g1.A = o_lat;
  g1.B = w_uv;
  g1.C = w.v;
  g1.c_hl = v_hl;
  MLA_TRY(launch_gemm(d, g1, s));
  g2.A = w.v;
  g2.a_hl = v_hl;
  g2.B = w_o;
  g2.C = w.u_parts;
  MLA_TRY(launch_gemm(d, g2, s));
  MLA_TRY(launch_convert(d, T, d.d, w.u_parts, d.d, g2.k_split, g2.c_ks, u,
                         d.d, s));
  return MLA_OK;
}

}  // extern "C"
