"""GPU parity of the HIP path (through the C ABI) against the CPU fp64
oracle, on the named synthetic workloads and their edge cases.

Bars: bf16 inputs rel-Frobenius <= 5e-3 and max-abs <= 2e-2; fp32 inputs
1e-5 for both.  Large workloads are checked on sampled sequences / queries
that the oracle computes one by one.
"""
import dataclasses

import numpy as np
import pytest
import torch

from mla_latent_kv_33_amd import flow
from mla_latent_kv_33_amd import workloads as W
from oracle import mla_oracle as orc
from tests.gpu_common import assert_close, check_all_sequences_latent, \
    context_latents, log, oracle_sequence

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.manual_seed(0)
    yield
    torch.cuda.synchronize()


_layers = {}


def layer_for(wl):
    key = (wl.dims, wl.dtype, wl.seed, int(wl.kv_lens.max()))
    if key not in _layers:
        _layers.clear()
        torch.cuda.empty_cache()
        weights = W.make_weights(wl.dims, wl.dtype, wl.seed)
        _layers[key] = (flow.make_layer(wl, weights), weights)
    return _layers[key]


def check_sequence(wl, out, ref, b, q_rows=None, full=True, heads=None):
    d = wl.dims
    rows = np.arange(wl.n_q) if q_rows is None else np.asarray(q_rows)
    o_lat = out.o_lat[b, rows].cpu().numpy()
    lse = out.lse[b, rows].cpu().numpy()
    q = out.q[b, rows].float().cpu().numpy()
    u = out.u.view(wl.batch, wl.n_q, d.d)[b, rows].float().cpu().numpy()
    # q, o_lat and lse of every head against the absorbed-form oracle;
    # lse also against the non-absorbed oracle on the heads it computed.
    assert_close(f"seq{b} q", q, ref["q"], wl.dtype)
    assert_close(f"seq{b} o_lat", o_lat, ref["o_lat"], wl.dtype)
    assert_close(f"seq{b} lse", lse, ref["lse_lat"], wl.dtype)
    sel = slice(None) if heads is None else list(heads)
    assert_close(f"seq{b} lse (non-absorbed)", lse[:, sel],
                 ref["lse"][:, sel], wl.dtype)
    if full:
        assert_close(f"seq{b} u", u, ref["u"] if "u" in ref else ref["u_lat"],
                     wl.dtype)


def check_new_rows(wl, st, ref, b):
    d = wl.dims
    got = flow.gather_rows(st, b, wl.ctx[b], wl.n_q)
    exp = np.concatenate([ref["c_kv"], ref["k_r"]], axis=1)
    assert got.shape == (wl.n_q, d.d_c + d.d_r)
    assert_close(f"seq{b} appended rows", got, exp, wl.dtype)


# ------------------------------------------------------------ tiny, fp32

def test_tiny_full_path():
    wl = W.workload("tiny")
    log(f"case {wl.name}: B={wl.batch} ctx={wl.ctx} fp32")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st)
    torch.cuda.synchronize()
    ref = oracle_sequence(wl, w, 0)
    check_new_rows(wl, st, ref, 0)
    # the context rows written by the context append
    c_kv, k_r = context_latents(wl, w, 0)
    got = flow.gather_rows(st, 0, 0, wl.ctx[0])
    assert_close("context rows", got, np.concatenate([c_kv, k_r], 1), "f32")
    check_sequence(wl, out, ref, 0)
    assert_close("o (non-absorbed heads)",
                 orc.head_values(out.o_lat[0].cpu().numpy(), w["w_uv"],
                                 wl.dims.d_h), ref["o"], "f32")


@pytest.mark.parametrize("n_split", [1, 2, 3, 5])
def test_tiny_splits(n_split):
    wl = dataclasses.replace(W.workload("tiny"), ctx=(300,))  # 5 blocks
    log(f"case tiny ctx=300 n_split={n_split}")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st, n_split=n_split)
    torch.cuda.synchronize()
    check_sequence(wl, out, oracle_sequence(wl, w, 0), 0)


@pytest.mark.parametrize("n_q,n_split", [(5, 1), (7, 2)])
def test_tiny_causal_chunk(n_q, n_split):
    wl = dataclasses.replace(W.workload("tiny"), n_q=n_q, ctx=(100,),
                             name="tiny_chunk")
    log(f"case tiny causal n_q={n_q} n_split={n_split}")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st, n_split=n_split)
    torch.cuda.synchronize()
    ref = oracle_sequence(wl, w, 0)
    check_new_rows(wl, st, ref, 0)
    check_sequence(wl, out, ref, 0)


def test_tiny_batched_ragged():
    """Several sequences of different (ragged) lengths, permuted table."""
    wl = dataclasses.replace(W.workload("tiny"), batch=4,
                             ctx=(1, 63, 64, 130), permuted=True,
                             name="tiny_ragged")
    log("case tiny ragged batch")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st, n_split=3)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        ref = oracle_sequence(wl, w, b)
        check_new_rows(wl, st, ref, b)
        check_sequence(wl, out, ref, b)


# ------------------------------------------------- DeepSeek-V2 dims, bf16

def test_b1_ctx4k():
    wl = W.workload("b1_ctx4k")
    log(f"case {wl.name}: B=1 ctx=4096 bf16")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st)
    torch.cuda.synchronize()
    ref = oracle_sequence(wl, w, 0)
    check_new_rows(wl, st, ref, 0)
    c_kv, k_r = context_latents(wl, w, 0)
    got = flow.gather_rows(st, 0, 0, wl.ctx[0])
    assert_close("context rows", got, np.concatenate([c_kv, k_r], 1), "bf16")
    check_sequence(wl, out, ref, 0)


@pytest.mark.parametrize("ctx,n_q", [((300, 1000), 1),
                                     ((64, 129, 2000), 1),
                                     ((1, 50, 700, 1500), 1),
                                     ((900,), 4)])
def test_ds_few_tokens(ctx, n_q):
    """DeepSeek-V2 dims with 2 to 4 new tokens per step (several sequences
    of one token, or one sequence with a causal 4-token chunk): the append
    takes the matrix-vector path at every count, the query and output
    projections at 2 tokens (the weight-streaming GEMMs at 3 and 4).  Every
    sequence, query, head and appended row against the oracle."""
    base = W.workload("b1_ctx4k")
    wl = dataclasses.replace(base, name=f"ds_few{len(ctx)}x{n_q}",
                             batch=len(ctx), ctx=ctx, n_q=n_q, seed=13,
                             permuted=True)
    log(f"case DeepSeek-V2 dims, {len(ctx) * n_q} tokens: ctx={ctx} "
        f"n_q={n_q}")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        ref = oracle_sequence(wl, w, b)
        check_new_rows(wl, st, ref, b)
        check_sequence(wl, out, ref, b)


def assert_reordered(name, a, b):
    """a and b computed from the same products summed in another fp32
    order, then rounded to bf16: every element within one bf16 step of the
    larger magnitude, plus 2^-10 of the array's RMS (values that cancel to
    near zero carry the sums' absolute error, not a relative one), and
    rel-Frobenius <= 1e-3."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    rms = float(np.sqrt(np.mean(b * b)))
    bound = np.exp2(-7.0) * np.maximum(np.abs(a), np.abs(b)) + rms / 1024
    excess = np.abs(a - b) - bound
    at = np.unravel_index(int(np.argmax(excess)), a.shape)
    worst = float(excess[at])
    rel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
    assert worst <= 0.0 and rel <= 1e-3, \
        (f"{name}: excess over bound {worst:.3g} at {at} ({a[at]:.6g} vs "
         f"{b[at]:.6g}, rms {rms:.3g}), rel-Frobenius {rel:.3g}")


@pytest.mark.parametrize("batch,n_q", [(64, 1), (8, 1), (2, 16), (1, 1),
                                       (2, 1)])
def test_stacked_projections(batch, n_q):
    """mla_append_absorb_q (at these token counts one weight stream for
    W_DQ, W_DKV and W_KR: a matrix-vector launch for 1 and 2 tokens, a GEMM
    and one epilogue for c_Q and the cache rows beyond) against
    mla_append_cache + mla_absorb_q on the same inputs: the
    appended rows and the queries differ only by the order of fp32 sums
    (about one bf16 step), and the stacked step matches the oracle."""
    base = W.workload("b1_ctx4k")
    rng = np.random.default_rng(1000 * batch + n_q)
    ctx = tuple(int(x) for x in rng.integers(64, 700, size=batch))
    wl = dataclasses.replace(base, name=f"stacked{batch}x{n_q}", batch=batch,
                             ctx=ctx, n_q=n_q, seed=21, permuted=True)
    log(f"case DeepSeek-V2 dims, {batch * n_q} tokens, stacked vs separate")
    layer, w = layer_for(wl)
    st_s = flow.prepare(wl, layer)
    out_s = flow.run_step(st_s, stacked=True)
    st_p = flow.prepare(wl, layer)
    out_p = flow.run_step(st_p, stacked=False)
    torch.cuda.synchronize()
    q_s = out_s.q.float().cpu().numpy()
    q_p = out_p.q.float().cpu().numpy()
    assert np.isfinite(q_s).all()
    assert_reordered("q", q_s, q_p)
    rows_s = np.stack([flow.gather_rows(st_s, b, wl.ctx[b], n_q)
                       for b in range(batch)])
    rows_p = np.stack([flow.gather_rows(st_p, b, wl.ctx[b], n_q)
                       for b in range(batch)])
    assert_reordered("appended rows", rows_s, rows_p)
    for b in sorted({0, batch - 1}):
        ref = oracle_sequence(wl, w, b)
        check_new_rows(wl, st_s, ref, b)
        check_sequence(wl, out_s, ref, b)


@pytest.mark.parametrize("batch,n_q,n_split", [(1, 1, 0), (2, 1, 0),
                                               (1, 2, 0), (1, 1, 5),
                                               (1, 1, 1), (4, 1, 0)])
def test_decode_out(batch, n_q, n_split):
    """mla_decode_out against mla_decode + mla_out on the same queries and
    cache.  With one or two query rows and split keys the split combine and
    W_UV run as one kernel (5 uniform splits leave one of its four split
    groups empty); with one split, or four rows, the call takes the two
    calls' own paths.  o_lat and lse differ from the separate calls only by
    the order of fp32 sums, u by that and its bf16 rounding; the fused step
    matches the oracle on every sequence."""
    base = W.workload("b1_ctx4k")
    rng = np.random.default_rng(500 + 10 * batch + n_q)
    ctx = tuple(int(x) for x in rng.integers(300, 3000, size=batch))
    wl = dataclasses.replace(base, name=f"decout{batch}x{n_q}", batch=batch,
                             ctx=ctx, n_q=n_q, seed=23, permuted=True)
    d = wl.dims
    log(f"case DeepSeek-V2 dims, mla_decode_out: ctx={ctx} n_q={n_q} "
        f"n_split={n_split}")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st, n_split=n_split, fuse_out=True)
    o_lat2, lse2 = layer.decode(out.q, st.cache, st.table, st.kv_lens,
                                st.max_kv_len, n_split=n_split)
    u2 = layer.out(o_lat2.view(-1, d.n_h, d.d_c))
    torch.cuda.synchronize()
    for name, a, b in (("o_lat", out.o_lat, o_lat2), ("lse", out.lse, lse2)):
        a = a.cpu().numpy().astype(np.float64)
        b = b.cpu().numpy().astype(np.float64)
        assert np.isfinite(a).all(), name
        rel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
        worst = float(np.max(np.abs(a - b)) / np.max(np.abs(b)))
        assert rel <= 1e-5 and worst <= 1e-5, (name, rel, worst)
    assert_reordered("u", out.u.float().cpu().numpy(),
                     u2.float().cpu().numpy())
    for b in range(batch):
        check_sequence(wl, out, oracle_sequence(wl, w, b), b)


def test_b64_var():
    wl = W.workload("b64_var")
    log(f"case {wl.name}: B=64 ctx U[1024,8192] permuted table bf16")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st)
    torch.cuda.synchronize()
    ctx = np.asarray(wl.ctx)
    picks = sorted({int(ctx.argmin()), int(ctx.argmax()), 17, 42})
    for b in picks:
        ref = oracle_sequence(wl, w, b)
        check_new_rows(wl, st, ref, b)
        check_sequence(wl, out, ref, b)
    check_all_sequences_latent(wl, w, out)


def test_b64_ctx8k_headline():
    wl = W.workload("b64_ctx8k")
    log(f"case {wl.name}: B=64 ctx=8192 (+1) bf16, auto splits")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st)
    torch.cuda.synchronize()
    for b in (0, 63):
        ref = oracle_sequence(wl, w, b)
        check_new_rows(wl, st, ref, b)
        check_sequence(wl, out, ref, b)
    check_all_sequences_latent(wl, w, out)


def test_b4_ctx128k_64_splits():
    wl = W.workload("b4_ctx128k")
    log(f"case {wl.name}: B=4 ctx=131072 (+1) bf16, 64 splits")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st, n_split=64)
    torch.cuda.synchronize()
    heads = [0, 77, 127]
    for b in (0, 3):
        ref = oracle_sequence(wl, w, b, heads=heads)
        check_new_rows(wl, st, ref, b)
        check_sequence(wl, out, ref, b, heads=heads)
        # non-absorbed per-head outputs for the sampled heads
        o_h = orc.head_values(out.o_lat[b].cpu().numpy(), w["w_uv"],
                              wl.dims.d_h)
        assert_close(f"seq{b} o heads {heads}", o_h[:, heads],
                     ref["o"][:, heads], "bf16")
    check_all_sequences_latent(wl, w, out)


@pytest.mark.parametrize("n_q", [30, 50])
def test_ds_ragged_chunk_all_queries(n_q):
    """DeepSeek-V2 dims on the absorbed path with a ragged causal chunk: 3
    sequences (contexts 0, 150, 333) receive n_q new tokens each, so every
    projection runs on T = 3 n_q rows with a partial last row tile (T = 90:
    the tiled kernel throughout; T = 150: the large-tile kernel for W_DKV,
    W_DQ, W_UQ / W_QR and W_O, the tiled kernel for the per-head absorption
    and W_UV), and the decode runs n_q causal queries per sequence, the
    first one over a single key.  Every query, head and appended row against
    the oracle."""
    base = W.workload("b8_prefill")
    wl = dataclasses.replace(base, name=f"ds_ragged_chunk{n_q}", batch=3,
                             ctx=(0, 150, 333), n_q=n_q, seed=9,
                             permuted=True)
    log(f"case DeepSeek-V2 dims, ragged chunk: ctx={wl.ctx} n_q={n_q}")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        ref = oracle_sequence(wl, w, b)
        check_new_rows(wl, st, ref, b)
        check_sequence(wl, out, ref, b)


def test_b8_chunked_prefill_causal():
    wl = W.workload("b8_prefill")
    log(f"case {wl.name}: B=8 ctx=8192 + chunk 2048 causal bf16")
    layer, w = layer_for(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st)
    torch.cuda.synchronize()
    rows = [0, 1, 1023, 2047]
    for b in (0, 5):
        ref = oracle_sequence(wl, w, b, q_rows=rows)
        check_sequence(wl, out, ref, b, q_rows=rows)
    # every 64th query row (and the last) of every sequence, absorbed form
    check_all_sequences_latent(wl, w, out,
                               q_rows=list(range(0, wl.n_q, 64)) + [2047])
    # every appended row of one sequence
    c_kv, k_r = orc.kv_latent(st.h_new_np[2 * wl.n_q:3 * wl.n_q],
                              wl.ctx[2] + np.arange(wl.n_q), w["w_dkv"],
                              w["w_kr"], W.ROPE_BASE)
    got = flow.gather_rows(st, 2, wl.ctx[2], wl.n_q)
    assert_close("seq2 chunk rows", got, np.concatenate([c_kv, k_r], 1),
                 "bf16")


@pytest.mark.parametrize("name,T", [("b1_ctx4k", 1), ("b1_ctx4k", 64),
                                    ("b1_ctx4k", 150), ("tiny", 5)])
def test_premerged_absorption(name, T):
    """The pre-merged query path (M_h = W_UK_h^T W_UQ_h built once, then
    q_lat_h = M_h c_Q) against the oracle's absorbed query on T tokens (a
    single token, a decode batch, a prefill-size chunk; bf16 DeepSeek-V2
    dims, and the fp32 tiny dims), and against the unmerged mla_absorb_q."""
    from mla_latent_kv_33_amd import binding as B
    # a context long enough for the RoPE tables to cover the positions below
    ctx = 4096 if name == "b1_ctx4k" else 64
    wl = dataclasses.replace(W.workload(name), batch=1, ctx=(ctx,),
                             n_q=T, seed=21)
    d = wl.dims
    layer, w = layer_for(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    merged = torch.empty((d.n_h, d.d_c, d.d_cq), dtype=tdt, device="cuda")
    B.mla_merge_uq_uk(layer.cdims, layer.w["w_uq"], layer.w["w_uk"], merged)
    h_np = W.hidden_states(d, wl.dtype, wl.seed, 0, 0, T)
    pos_np = np.arange(T) * 37 % (ctx - 1)
    h = torch.from_numpy(h_np.astype(np.float32)).to(tdt).cuda()
    pos = torch.from_numpy(pos_np.astype(np.int32)).cuda()
    q_m = torch.empty((T, d.n_h, d.d_c + d.d_r), dtype=tdt, device="cuda")
    B.mla_absorb_q_merged(layer.cdims, h, pos, layer.w["w_dq"], merged,
                          layer.w["w_qr"], layer.rope_cos, layer.rope_sin,
                          q_m)
    q_u = layer.absorb(h, pos)
    torch.cuda.synchronize()
    q_c, q_r = orc.query(h_np, pos_np, w["w_dq"], w["w_uq"], w["w_qr"],
                         d.n_h, W.ROPE_BASE)
    ref = orc.absorb_query(q_c, q_r, w["w_uk"])
    assert_close(f"T={T} merged q", q_m.float().cpu().numpy(), ref, wl.dtype)
    assert_close(f"T={T} unmerged q", q_u.float().cpu().numpy(), ref, wl.dtype)
    # the RoPE columns come from the same W_QR projection in both forms
    assert_close(f"T={T} merged vs unmerged q_R",
                 q_m[..., d.d_c:].float().cpu().numpy(),
                 q_u[..., d.d_c:].float().cpu().numpy(), wl.dtype)
