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
import dataclasses
import gc
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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="b64_ctx8k")
    ap.add_argument("--path", choices=("absorbed", "mha"), default="absorbed",
                    help="attention form of the step: absorbed queries over "
                         "the latent cache (mla_absorb_q, mla_decode, "
                         "mla_out), or explicit per-head keys and values for "
                         "chunked prefill (mla_query_mha, mla_prefill_mha, "
                         "mla_out_values)")
    ap.add_argument("--batch", type=int, default=0,
                    help="with --context: sequences of the uniform workload "
                         "(default: the named workload's batch)")
    ap.add_argument("--context", type=int, default=0,
                    help="uniform prior context for every sequence instead "
                         "of the named workload's lengths (a sweep over it "
                         "separates the decode's per-key cost from its fixed "
                         "per-launch cost); the line is then marked as not "
                         "the headline configuration")
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
    ap.add_argument("--event-every", type=int, default=2,
                    help="with --timed-events decode: record the pair of "
                         "events around the decode call in every N-th timed "
                         "step (the decode duration is their median)")
    # The GPU's power management runs the start of a sustained load in a
    # transient (the decode kernel first runs at ~155 us, slows to ~190-200
    # us, then settles near ~160 us).  Untimed steps for this long come
    # before the warmup steps, so that the timed steps see the sustained
    # state whatever W is (see the settle loop below).
    ap.add_argument("--settle-ms", type=float, default=1500.0,
                    help="untimed steps for at least this long (wall clock) "
                         "before the warmup steps")
    ap.add_argument("--streams", type=int, choices=(1, 2), default=1,
                    help="2: the append runs on a second stream, concurrent "
                         "with the query path (both read only h; the decode "
                         "waits for both); 1: the four calls on one stream")
    ap.add_argument("--query", choices=("absorbed", "merged"),
                    default="absorbed",
                    help="absorbed path only: the query projection as "
                         "mla_absorb_q (W_UQ, then W_UK_h^T per head) or "
                         "mla_absorb_q_merged (one projection onto the "
                         "pre-merged W_UK_h^T W_UQ_h, built once)")
    ap.add_argument("--project", choices=("stacked", "separate"),
                    default="stacked",
                    help="absorbed path, --query absorbed: the append and "
                         "the query projection as one mla_append_absorb_q "
                         "call (the down-projections W_DQ, W_DKV, W_KR of h "
                         "stacked into one weight stream) or as "
                         "mla_append_cache followed by mla_absorb_q")
    ap.add_argument("--out-call", choices=("auto", "fused", "separate"),
                    default="auto",
                    help="the decode and the output projection as one "
                         "mla_decode_out call (fused; its event pair then "
                         "brackets both) or as mla_decode followed by "
                         "mla_out; auto: fused for one or two query rows, "
                         "where the library merges the split combine into "
                         "the W_UV kernel")
    ap.add_argument("--unbound", action="store_true",
                    help="check and marshal every library call's arguments "
                         "on every step (by default the step's calls are "
                         "bound once: binding.BoundCall)")
    ap.add_argument("--graph", action="store_true",
                    help="timed steps replay HIP graphs (captured once after "
                         "the warmup: append + query, attention, output) "
                         "instead of launching each kernel from the host; "
                         "for small batches, where the host's launch calls "
                         "take longer than the GPU work")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured HBM-read and matrix-core rates")
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


def measure_peaks(B, torch, stream):
    """Measured machine rates on this machine, in the power state the step
    leaves: a plain read of a 1 GiB buffer (4x the Infinity Cache), and a
    loop of independent bf16 32x32x16 MFMAs (include/mla_peaks.h).  Medians
    of 10 launches each."""
    import numpy as np
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    buf.random_(0, 255)
    wgs_read = 512
    sink = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    mf_wgs, mf_iters = 512, 2048
    mf_sink = torch.empty(B.lib().mla_peak_mfma_sink_bytes(mf_wgs),
                          dtype=torch.uint8, device="cuda")
    times = {"read": [], "mfma": []}
    nbytes = flops = 0
    for r in range(12):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        nbytes = B.mla_peak_stream_read(buf, sink, wgs_read)
        e1.record(stream)
        flops = B.mla_peak_mfma_loop(mf_wgs, mf_iters, mf_sink)
        e2.record(stream)
        torch.cuda.synchronize()
        if r >= 2:
            times["read"].append(e0.elapsed_time(e1) * 1e-3)
            times["mfma"].append(e1.elapsed_time(e2) * 1e-3)
    t_read = float(np.median(times["read"]))
    t_mfma = float(np.median(times["mfma"]))
    del buf, sink, mf_sink
    return {
        "hbm_read_GBps": nbytes / t_read / 1e9,
        "mfma_bf16_TFLOPs": flops / t_mfma / 1e12,
        "how": "mla_peak_stream_read over a 1 GiB buffer (16-byte loads, "
               f"{wgs_read} workgroups, a contiguous 2 MiB chunk each) and "
               f"mla_peak_mfma_loop ({mf_wgs} "
               f"workgroups x 4 waves x {mf_iters} x 8 independent "
               "32x32x16 bf16 MFMAs); medians of 10 launches after 2, timed "
               "with HIP events right after the timed steps"}


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
    if args.context > 0 or args.batch > 0:
        if args.context <= 0:
            raise SystemExit("--batch needs --context")
        nb = args.batch if args.batch > 0 else wl.batch
        wl = dataclasses.replace(
            wl, name=f"{wl.name}@B{nb}xctx{args.context}", batch=nb,
            ctx=(args.context,) * nb,
            n_split=0 if wl.n_split < 0 else wl.n_split)
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

    # one call for the append and the query path (stacked projections)
    stacked = (not mha and args.query == "absorbed" and
               args.project == "stacked" and args.streams == 1)
    names = (("append", "query", "prefill", "out") if mha else
             ("append", "absorb", "decode", "out"))

    def new_events(n):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
                for _ in range(n)]

    bound = None   # the step's library calls, bound once (set below)

    def attention(alone=False):
        if bound is not None and not (alone and fuse_out):
            bound.attention()
        elif mha:
            layer.prefill_mha(out.q, st.cache, st.table, st.kv_lens,
                              st.max_kv_len, o_v=out.o_v, lse=out.lse)
        else:
            layer.decode(out.q, st.cache, st.table, st.kv_lens,
                         st.max_kv_len, n_split=n_split, o_lat=out.o_lat,
                         lse=out.lse)

    # The append and the query path both read only h: with two streams the
    # append runs on a side stream (default priority), forked from and
    # joined to the main stream by events, so its small kernels fill the
    # gaps of the query path's chain.
    side = torch.cuda.Stream() if args.streams == 2 else None
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    merged = merged_ws = None
    if args.query == "merged" and not mha:
        import ctypes
        merged = torch.empty((d.n_h, d.d_c, d.d_cq), dtype=torch.bfloat16,
                             device="cuda")
        B.mla_merge_uq_uk(layer.cdims, layer.w["w_uq"], layer.w["w_uk"],
                          merged)
        merged_ws = torch.empty(
            B.lib().mla_absorb_merged_workspace_bytes(
                ctypes.byref(layer.cdims), st.h_new.shape[0]),
            dtype=torch.uint8, device="cuda")

    # The default path issues its library calls bound (binding.BoundCall):
    # the tensor checks and the marshalling of the arguments run once here
    # instead of on every step.  At B = 1 they took as long as the GPU's
    # step (about 85 us per step on the host).
    # (not under --graph: a bound call keeps the stream it was bound on,
    # while capture runs on a capture stream)
    # One or two query rows: the decode and the output projection as one
    # mla_decode_out call, which fuses the split combine with W_UV.
    fuse_out = (not mha and merged is None and side is None and
                not args.unbound and not args.graph and
                (args.out_call == "fused" or
                 (args.out_call == "auto" and wl.batch * wl.n_q <= 2)))
    if (not mha and merged is None and side is None and not args.unbound
            and not args.graph):
        bound = flow.bind_step(st, out, n_split, stacked=(
            args.project == "stacked"), fuse_out=fuse_out)

    def query_path():
        if merged is not None:
            B.mla_absorb_q_merged(layer.cdims, st.h_new, st.pos,
                                  layer.w["w_dq"], merged, layer.w["w_qr"],
                                  layer.rope_cos, layer.rope_sin,
                                  out.q.view(-1, d.n_h, d.d_c + d.d_r),
                                  ws=merged_ws)
        elif mha:
            layer.query_mha(st.h_new, st.pos,
                            q_out=out.q.view(-1, d.n_h, d.d_h + d.d_r))
        else:
            layer.absorb(st.h_new, st.pos,
                         q_out=out.q.view(-1, d.n_h, d.d_c + d.d_r))

    def step(e=None, which="all"):
        """One pass of the hot path; e[k] recorded before stage k and after
        the last stage, all of them ("all", one stream) or only around
        decode."""
        rec_all = e is not None and which == "all"
        rec_dec = e is not None
        if side is not None and not rec_all:
            fork.record(stream)
            side.wait_event(fork)
            layer.append(st.h_new, st.seq_idx, st.pos, st.table, st.cache,
                         stream=side)
            join.record(side)
            query_path()
            stream.wait_event(join)
        elif bound is not None:
            # stacked: one call (e[0] and e[1] around it; the absorb stage
            # is empty); separate: the append, then the query path
            if rec_all: e[0].record(stream)
            bound.pre[0]()
            if rec_all: e[1].record(stream)
            for c in bound.pre[1:]:
                c()
        elif stacked:
            # e[0] and e[1] together: the append stage is part of the call
            if rec_all:
                e[0].record(stream)
                e[1].record(stream)
            layer.append_absorb(st.h_new, st.seq_idx, st.pos, st.table,
                                st.cache,
                                q_out=out.q.view(-1, d.n_h, d.d_c + d.d_r))
        else:
            if rec_all: e[0].record(stream)
            layer.append(st.h_new, st.seq_idx, st.pos, st.table, st.cache)
            if rec_all: e[1].record(stream)
            query_path()
        if rec_dec: e[2].record(stream)
        attention()
        if rec_dec: e[3].record(stream)
        if bound is not None:
            bound.out()
        elif mha:
            layer.out_values(out.o_v.view(-1, d.n_h * d.d_h), u=out.u)
        else:
            layer.out(out.o_lat.view(-1, d.n_h, d.d_c), u=out.u)
        if rec_all: e[4].record(stream)

    # The timed steps' events, and the one garbage collection, come before
    # the untimed steps, so that the GPU does not sit idle between the last
    # warmup step and the first timed one.
    ev = new_events(args.steps)
    every = 1 if args.timed_events == "all" else max(1, args.event_every)
    sampled = [i for i in range(args.steps) if i % every == 0]
    # No garbage collection from here to the end of the timed region: the
    # first bench process on a freshly started box once spent 34.6 ms of its
    # first timed step in a full collection over the workload's host arrays
    # (B = 64 with varying contexts: 408 us per step against 229 us for the
    # next process).
    gc.collect()
    gc.disable()

    # settle phase (untimed), then the W warmup steps
    t_settle = time.perf_counter()
    settle_steps = 0
    # Long groups between synchronisations: the transient comes with
    # continuous load, and with a synchronisation every 8 steps (2 ms of
    # work) it had not run its course when the timed steps began.
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(64):
            step()
        settle_steps += 64
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graphs = None
    if args.graph:
        if args.streams != 1 or args.timed_events != "decode":
            sys.exit("--graph needs one stream and --timed-events decode")

        def out_stage():
            if mha:
                layer.out_values(out.o_v.view(-1, d.n_h * d.d_h), u=out.u)
            else:
                layer.out(out.o_lat.view(-1, d.n_h, d.d_c), u=out.u)

        def pre_stage():
            if stacked:
                layer.append_absorb(
                    st.h_new, st.seq_idx, st.pos, st.table, st.cache,
                    q_out=out.q.view(-1, d.n_h, d.d_c + d.d_r))
                return
            layer.append(st.h_new, st.seq_idx, st.pos, st.table, st.cache)
            query_path()

        # every call is capture-safe (no allocation, memset or
        # synchronisation inside); three graphs so that the timed steps can
        # still bracket the attention stage with events
        graphs = []
        for fn in (pre_stage, attention, out_stage):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            graphs.append(g)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            for g in graphs:
                g.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs is not None:
        for i in range(args.steps):
            graphs[0].replay()
            if i % every == 0: ev[i][2].record(stream)
            graphs[1].replay()
            if i % every == 0: ev[i][3].record(stream)
            graphs[2].replay()
    else:
        for i in range(args.steps):
            step(ev[i] if i % every == 0 else None, args.timed_events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    # attention stage (decode kernel + split combine, or the MHA prefill
    # call) inside the timed steps
    dec_samples = [ev[i][2].elapsed_time(ev[i][3]) for i in sampled]
    t_dec_ms = float(np.median(dec_samples))
    peaks = None if args.no_peaks else measure_peaks(B, torch, stream)
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
    if stacked:
        stage_ms = {"append+absorb": stage_ms["append"] + stage_ms["absorb"],
                    "decode": stage_ms["decode"], "out": stage_ms["out"]}
    if fuse_out:
        # the out stage is empty: mla_decode_out ran it
        stage_ms = {("decode+out" if k == "decode" else k): v
                    for k, v in stage_ms.items() if k != "out"}
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
            attention(alone=True)
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
        if fuse_out:
            # mla_decode_out: the output projection's weights read and u
            # written, and its products
            nv = d.n_h * d.d_h
            alg_bytes += (nv * d.d_c + d.d * nv) * 2 + queries * d.d * 2
            flops += 2.0 * queries * (nv * d.d_c + d.d * nv)
    t_dec = t_dec_ms * 1e-3
    achieved = alg_bytes / t_dec / 1e9
    tflops = flops / t_dec / 1e12
    # the bound is the roof the stage is closer to
    mfma_bound = tflops / BF16_PEAK_TFLOPS > achieved / HBM_PEAK_GBPS
    traffic = None if (mha or wl.name != "b64_ctx8k") else \
        stored_traffic(alg_bytes)
    stage_kernel = ("mla_prefill_mha: gather_rows_kernel + gemm_big_kernel "
                    "(k_C, v_C up-projection) + " + PREFILL_KERNEL if mha else
                    "mla_decode_out: " + DECODE_KERNEL + " + combine_uv_kernel"
                    " (split combine and W_UV) + gemv_plain_kernel (W_O)"
                    if fuse_out else
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
            "decode_us_min_max": [min(dec_samples) * 1e3,
                                  max(dec_samples) * 1e3],
        },
        "decode_queries_per_s": queries / t_dec,
        "latent_cache_GBps": cache_bytes / t_dec / 1e9,
        "decode_timing": f"median of HIP events around the attention "
                         f"call in {len(sampled)} of the {args.steps} timed "
                         f"steps (every {every})",
        "settle": f"{settle_steps} untimed steps ({args.settle_ms:.0f} ms) "
                  "before the warmup steps: the GPU's power management runs "
                  "the first tens of ms of sustained load in a transient",
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
                               "every stage (one stream)"),
        "streams": ("append on a second stream, concurrent with the query "
                    "path" if side is not None else "one stream"),
        "query": args.query,
        "calls": ("bound once (binding.BoundCall)" if bound is not None
                  else "arguments checked on every call"),
        "out_call": ("mla_decode_out (decode, then the combine fused with "
                     "W_UV, then W_O); decode_us covers all of it"
                     if fuse_out else "mla_decode, then mla_out"),
        "projections": ("one mla_append_absorb_q call (W_DQ, W_DKV, W_KR "
                        "stacked)" if stacked else
                        "mla_append_cache, then the query call"),
        "launch": ("timed steps replay three HIP graphs (append + query, "
                   "attention, output) captured after the warmup"
                   if graphs is not None else "eager launches from the host"),
        "kernel_source_hash": kernel_source_hash(),
    }
    if peaks is not None:
        result["peaks_measured"] = peaks
        rf = result["roofline"]
        rf["hbm_frac_achievable"] = achieved / peaks["hbm_read_GBps"]
        rf["mfma_frac_achievable"] = tflops / peaks["mfma_bf16_TFLOPs"]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample)
    if mha or wl.name != "b64_ctx8k" or merged is not None:
        result["note"] = ("not the headline configuration: a measurement of "
                          "another workload, attention path or query form")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
