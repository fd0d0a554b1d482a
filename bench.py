"""Benchmark of one MLA decode step on one MI355X.

A step is one pass of the whole hot path over one batch: append the 64 new
tokens' latents to the paged cache, build their absorbed queries, split-KV
decode over the 8192 + 1 cached rows of every sequence (plus the combine),
and the output projection.  Workload: B = 64 sequences, context 8192 each,
one query token per sequence, DeepSeek-V2 dimensions, bf16, 64-token blocks
under a random-permutation block table; synthetic seeded inputs, resident in
HBM before timing starts.

Prints one JSON line (see the keys below).  `--gpus N` with N > 1 exits: this
build measures one GPU.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MLA decode queries/sec + latent-cache GB/s & MFMA util vs peak "
          "(B=64,S=8K)")
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
DECODE_KERNEL = "decode_mfma_kernel"
PREFILL_KERNEL = "prefill_mha_kernel"
PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_b64_ctx8k_pmc.json")
KERNEL_SOURCES = [os.path.join(ROOT, "mla_latent_kv_33_amd", "csrc", f)
                  for f in ("decode_mfma.hip", "decode_simt.hip")]


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Clocks ramp up over the first few tens of milliseconds of sustained
    # load (about 60 steps here); the warmup covers that ramp so that the
    # timed steps see the steady state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="b64_ctx8k")
    ap.add_argument("--path", choices=("absorbed", "mha"), default="absorbed",
                    help="attention form of the step: absorbed queries over "
                         "the latent cache (mla_absorb_q, mla_decode, "
                         "mla_out), or explicit per-head keys and values for "
                         "chunked prefill (mla_query_mha, mla_prefill_mha, "
                         "mla_out_values)")
    ap.add_argument("--cpu-sample", type=int, default=24,
                    help="sequences of the workload the CPU oracle times")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timed-events", choices=("decode", "all"),
                    default="decode",
                    help="timing events recorded inside the timed steps: "
                         "around the decode call only (default), or around "
                         "every stage.  A timed event makes the stream drain "
                         "before the next launch, so each one costs a few "
                         "microseconds of idle GPU; the per-stage split is "
                         "taken from separate untimed steps by default.")
    ap.add_argument("--event-every", type=int, default=8,
                    help="with --timed-events decode: record the pair of "
                         "events around the decode call in every N-th timed "
                         "step (the decode duration is their average)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for "
                         "scaling HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain copy of 1 GiB, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "launches": 3}))


def cpu_baseline(wl, sample):
    """Time the CPU fp64 oracle (non-absorbed MLA) on `sample` sequences of
    the workload; queries/s scaled from the sample."""
    import numpy as np
    from mla_latent_kv_33_amd import workloads as W
    from oracle import mla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 0) for i in threadpool_info()] or
                    [os.cpu_count()])
    except Exception:   # threadpoolctl missing: report the visible CPUs
        cores = os.cpu_count()
    d = wl.dims
    w = {k: v.astype(np.float64) for k, v in
         W.make_weights(d, wl.dtype, wl.seed).items()}
    total = 0.0
    for b in range(sample):
        rows = W.latent_rows(d, wl.dtype, wl.seed, b, 0, wl.ctx[b]).astype(
            np.float64)
        h_new = W.hidden_states(d, wl.dtype, wl.seed, b, wl.ctx[b], wl.n_q)
        t0 = time.perf_counter()
        orc.decode_step(w, d.n_h, W.ROPE_BASE, h_new, rows[:, :d.d_c],
                        rows[:, d.d_c:])
        total += time.perf_counter() - t0
    return {"value": sample * wl.n_q / total, "unit": "queries/s",
            "cores": int(cores), "kind": "oracle",
            "sample": f"{sample} of {wl.batch} sequences (context "
                      f"{wl.ctx[0]} + {wl.n_q} query), full non-absorbed "
                      f"layer step per sequence, fp64 numpy; {total:.1f} s"}


def workload_text(wl, mha):
    d = wl.dims
    dims = (f"DeepSeek-V2 dims (d {d.d}, n_h {d.n_h}, d_h {d.d_h}, d_c "
            f"{d.d_c}, d_r {d.d_r}, d_c' {d.d_cq})")
    ctx = (f"context {wl.ctx[0]}" if len(set(wl.ctx)) == 1 else
           f"contexts {min(wl.ctx)}..{max(wl.ctx)}")
    kind = ("MLA chunked-prefill step on the explicit-key (MHA) path"
            if mha else "MLA decode step" if wl.n_q == 1 else
            "MLA chunked-prefill step on the absorbed path")
    return (f"{kind}, B={wl.batch}, {ctx} + {wl.n_q} new token(s) per "
            f"sequence (causal), {dims}, paged latent cache of 64-token "
            f"blocks, {'random-permutation' if wl.permuted else 'linear'} "
            "block table")


def stored_traffic(bytes_per_launch_alg):
    """HBM traffic of the decode kernel from the committed counter summary,
    if it was taken on the current kernel source."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    s = json.load(open(PMC_SUMMARY))
    if s.get("kernel_source_hash") != kernel_source_hash():
        return None
    return s.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not "
              "supported by this build (one process, one MI355X).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    import numpy as np
    from mla_latent_kv_33_amd import binding as B
    from mla_latent_kv_33_amd import flow
    from mla_latent_kv_33_amd import workloads as W

    B.lib()   # fail loudly if the library is not built
    wl = W.workload(args.workload)
    d = wl.dims
    torch.cuda.set_device(0)
    layer = flow.make_layer(wl)
    st = flow.prepare(wl, layer)
    stream = torch.cuda.current_stream()
    # 0: the library's automatic splits (balanced per sequence for up to
    # 256 query rows on the matrix-core path)
    n_split = wl.n_split
    mha = args.path == "mha"
    # allocates outputs and workspaces once
    out = flow.run_prefill_mha(st) if mha else flow.run_step(st)
    torch.cuda.synchronize()

    names = (("append", "query", "prefill", "out") if mha else
             ("append", "absorb", "decode", "out"))

    def new_events(n):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
                for _ in range(n)]

    def attention():
        if mha:
            layer.prefill_mha(out.q, st.cache, st.table, st.kv_lens,
                              st.max_kv_len, o_v=out.o_v, lse=out.lse)
        else:
            layer.decode(out.q, st.cache, st.table, st.kv_lens,
                         st.max_kv_len, n_split=n_split, o_lat=out.o_lat,
                         lse=out.lse)

    def step(e=None, which="all"):
        """One pass of the hot path; e[k] recorded before stage k and after
        the last stage, all of them ("all") or only around decode."""
        rec_all = e is not None and which == "all"
        rec_dec = e is not None
        if rec_all: e[0].record(stream)
        layer.append(st.h_new, st.seq_idx, st.pos, st.table, st.cache)
        if rec_all: e[1].record(stream)
        if mha:
            layer.query_mha(st.h_new, st.pos,
                            q_out=out.q.view(-1, d.n_h, d.d_h + d.d_r))
        else:
            layer.absorb(st.h_new, st.pos,
                         q_out=out.q.view(-1, d.n_h, d.d_c + d.d_r))
        if rec_dec: e[2].record(stream)
        attention()
        if rec_dec: e[3].record(stream)
        if mha:
            layer.out_values(out.o_v.view(-1, d.n_h * d.d_h), u=out.u)
        else:
            layer.out(out.o_lat.view(-1, d.n_h, d.d_c), u=out.u)
        if rec_all: e[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = new_events(args.steps)
    every = 1 if args.timed_events == "all" else max(1, args.event_every)
    sampled = [i for i in range(args.steps) if i % every == 0]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i] if i % every == 0 else None, args.timed_events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # attention stage (decode kernel + split combine, or the MHA prefill
    # call) inside the timed steps
    t_dec_ms = float(np.mean([ev[i][2].elapsed_time(ev[i][3])
                              for i in sampled]))
    if args.timed_events == "all":
        ev_st, n_st = ev, args.steps
    else:
        # per-stage split from separate, untimed steps with every event,
        # queued behind a few plain steps so that the GPU never waits for
        # the host inside them
        n_st = min(args.steps, 20)
        ev_st = new_events(n_st)
        for _ in range(10):
            step()
        for i in range(n_st):
            step(ev_st[i], "all")
        torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([ev_st[i][k].elapsed_time(ev_st[i][k + 1])
                                  for i in range(n_st)]))
                for k, n in enumerate(names)}
    # The attention stage alone, outside the step, medians of 10 calls each:
    # right after writing a 512 MiB scratch buffer, right after reading one
    # (either evicts L2 and the 256 MB Infinity Cache, so the cache rows come
    # from HBM; the write also leaves dirty lines that are written back while
    # the attention runs), and back to back.
    scratch = torch.ones(512 << 18, dtype=torch.int32, device="cuda")
    kinds = ("write", "read", "repeated")
    ev_fl = {k: [(torch.cuda.Event(enable_timing=True),
                  torch.cuda.Event(enable_timing=True)) for _ in range(10)]
             for k in kinds}
    sink = []
    for k in kinds:
        for r in range(10):
            if k == "write":
                scratch.fill_(r + 1)
            elif k == "read":
                sink.append(scratch.amax())
            ev_fl[k][r][0].record(stream)
            attention()
            ev_fl[k][r][1].record(stream)
    torch.cuda.synchronize()
    del scratch, sink
    att_us = {k: float(np.median([a.elapsed_time(b) for a, b in ev_fl[k]]))
              * 1e3 for k in kinds}
    ms_per_step = wall * 1e3 / args.steps
    queries = wl.batch * wl.n_q
    kv = wl.kv_lens
    # (query, key) pairs the causal attention visits: query i of a chunk of
    # n_q sees ctx + i + 1 keys
    pairs = float(sum(wl.n_q * c + wl.n_q * (wl.n_q + 1) // 2
                      for c in wl.ctx))
    cache_bytes = float(kv.sum()) * (d.d_c + d.d_r) * 2
    if mha:
        # gathered rows written and read, [k_C | v_C] written and read once,
        # queries read, fp32 values written
        kv_rows = float(wl.batch * st.max_kv_len)
        kv_el = 2 * d.n_h * d.d_h
        alg_bytes = (cache_bytes + 2 * kv_rows * (d.d_c + d.d_r) * 2 +
                     kv_rows * kv_el * 2 * 2 +
                     queries * d.n_h * (d.d_h + d.d_r) * 2 +
                     queries * d.n_h * d.d_h * 4)
        flops = (d.n_h * pairs * (2 * (d.d_h + d.d_r) + 2 * d.d_h) +
                 2.0 * kv_rows * kv_el * d.d_c)
    else:
        q_bytes = queries * d.n_h * (d.d_c + d.d_r) * 2
        olat_bytes = queries * d.n_h * d.d_c * 4
        alg_bytes = cache_bytes + q_bytes + olat_bytes
        flops = d.n_h * pairs * (2 * (d.d_c + d.d_r) + 2 * d.d_c)
    t_dec = t_dec_ms * 1e-3
    achieved = alg_bytes / t_dec / 1e9
    tflops = flops / t_dec / 1e12
    # the bound is the roof the stage is closer to
    mfma_bound = tflops / BF16_PEAK_TFLOPS > achieved / HBM_PEAK_GBPS
    traffic = None if (mha or wl.name != "b64_ctx8k") else \
        stored_traffic(alg_bytes)
    stage_kernel = ("mla_prefill_mha: gather_rows_kernel + gemm_big_kernel "
                    "(k_C, v_C up-projection) + " + PREFILL_KERNEL if mha else
                    "mla_decode: " + DECODE_KERNEL + " + combine_rows_kernel")
    result = {
        "metric": METRIC,
        "value": queries / (ms_per_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) hidden states and latent cache "
                "rows, N(0,1/fan_in) weights)",
        "config": {
            "workload": workload_text(wl, mha),
            "batch": wl.batch, "context": wl.ctx[0], "kv_len": int(kv[0]),
            "n_q": wl.n_q,
            "n_split": None if mha else (
                int(n_split) if n_split > 0 else
                "balanced" if n_split == B.MLA_SPLIT_BALANCED else "auto"),
            "block_size": 64, "path": args.path,
        },
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "kernel": stage_kernel,
            "achieved": tflops if mfma_bound else achieved,
            "peak": BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBPS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": (tflops / BF16_PEAK_TFLOPS if mfma_bound
                     else achieved / HBM_PEAK_GBPS),
            "traffic": traffic,
            "alg_bytes_per_launch": alg_bytes,
            "flops_per_launch": flops,
            "hbm_GBps": achieved,
            "hbm_frac": achieved / HBM_PEAK_GBPS,
            "mfma_tflops": tflops,
            "mfma_frac": tflops / BF16_PEAK_TFLOPS,
            "decode_us": t_dec * 1e6,
        },
        "decode_queries_per_s": queries / t_dec,
        "latent_cache_GBps": cache_bytes / t_dec / 1e9,
        "decode_timing": f"HIP events around the mla_decode call in "
                         f"{len(sampled)} of the {args.steps} timed steps "
                         f"(every {every})",
        "attention_alone_us": {
            "after_512MiB_write": att_us["write"],
            "after_512MiB_read": att_us["read"],
            "repeated": att_us["repeated"],
            "cache_GBps_after_read_flush":
                cache_bytes / att_us["read"] / 1e3,
            "how": "the attention stage called on its own, outside the "
                   "step: median of 10 calls each right after writing, or "
                   "after reading, a 512 MiB scratch buffer (L2 and "
                   "Infinity Cache evicted; the write also leaves dirty "
                   "lines to write back), and of 10 calls back to back"},
        "stage_us": {k: v * 1e3 for k, v in stage_ms.items()},
        "stage_us_from": ("the timed steps" if args.timed_events == "all"
                          else f"{n_st} untimed steps with an event around "
                               "every stage"),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample)
    if mha or wl.name != "b64_ctx8k":
        result["note"] = ("not the headline configuration: a measurement of "
                          "another workload or attention path")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
