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
from tests.gpu_common import assert_close, context_latents, log, \
    oracle_sequence

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
    # every appended row of one sequence
    c_kv, k_r = orc.kv_latent(st.h_new_np[2 * wl.n_q:3 * wl.n_q],
                              wl.ctx[2] + np.arange(wl.n_q), w["w_dkv"],
                              w["w_kr"], W.ROPE_BASE)
    got = flow.gather_rows(st, 2, wl.ctx[2], wl.n_q)
    assert_close("seq2 chunk rows", got, np.concatenate([c_kv, k_r], 1),
                 "bf16")
