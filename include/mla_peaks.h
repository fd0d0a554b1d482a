/*
 * mla_peaks.h - machine-rate kernels of libmla.so (measurement only).
 *
 * These entry points compute nothing of the MLA layer.  They measure what
 * the GPU they run on reaches on a plain HBM read stream and on a loop of
 * bf16 matrix-core operations, so that a kernel's rate can be stated both
 * against the datasheet peaks and against these measured ones.  The
 * decode path reads its whole latent cache every step and is bounded by
 * HBM bandwidth and matrix-core rate together ('MLA：潜在表示压缩与解耦
 * RoPE', section 1: the KV cache, read in full at every decode step, is
 * the bottleneck), which is why both rates are measured.
 *
 * Conventions are those of mla.h: device pointers, caller-owned buffers,
 * asynchronous on `stream`, status codes returned and nothing printed.
 */
#ifndef MLA_PEAKS_H
#define MLA_PEAKS_H

#include "mla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` of `buf` once, 16 bytes per lane per load: `workgroups`
 * workgroups of 256 threads each stream their own contiguous chunk of
 * bytes / workgroups.  `sink` (device, >= 4 * workgroups bytes) receives at
 * most one word per workgroup (to keep the loads live); its contents are
 * meaningless.  Rate = bytes / elapsed time.  Use a buffer well above the
 * 256 MB Infinity Cache so that the reads come from HBM.
 * MLA_ERR_NULL, MLA_ERR_SHAPE (bytes not a positive multiple of
 * 16 * workgroups, workgroups <= 0), MLA_ERR_DEVICE. */
mla_status mla_peak_stream_read(const void* buf, size_t bytes, void* sink,
                                int32_t workgroups, mla_stream_t stream);

/* Bytes of `sink` that mla_peak_mfma_loop writes (one float per thread);
 * 0 for workgroups <= 0. */
size_t mla_peak_mfma_sink_bytes(int32_t workgroups);

/* Floating-point operations one mla_peak_mfma_loop launch performs. */
double mla_peak_mfma_flops(int32_t workgroups, int32_t iters);

/* `workgroups` workgroups of 4 waves each run `iters` iterations of 8
 * independent v_mfma_f32_32x32x16_bf16 on register operands (hashed,
 * non-zero bf16 values) and write one float per thread to `sink`
 * (mla_peak_mfma_sink_bytes).  Rate = mla_peak_mfma_flops / elapsed time.
 * MLA_ERR_NULL, MLA_ERR_SHAPE (workgroups or iters <= 0), MLA_ERR_DEVICE. */
mla_status mla_peak_mfma_loop(int32_t workgroups, int32_t iters, void* sink,
                              mla_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PEAKS_H */
