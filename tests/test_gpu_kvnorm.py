"""The latent RMSNorm variant of the cache write, mla_append_cache_rmsnorm
('MiniMind 学习笔记 10', section 9: kv_norm on the latent only): cached rows
against the oracle's normalised latents, every row at its block-table slot,
and a whole decode step over a normalised cache."""
import numpy as np
import pytest
import torch

from mla_latent_kv_33_amd import binding as B
from mla_latent_kv_33_amd import workloads as W
from mla_latent_kv_33_amd.layer import MlaLayer, to_device
from oracle import mla_oracle as orc
from tests.gpu_common import assert_close, log

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def _norm_weight(d_c, dtype, seed):
    g = np.random.default_rng(seed).normal(1.0, 0.2, d_c).astype(np.float32)
    return W.round_bf16(g) if dtype == "bf16" else g


def _append_norm(layer, h, seq, pos, table, cache, g_dev):
    T = h.shape[0]
    ws = layer.workspace("append", B.mla_append_workspace_bytes(layer.cdims, T))
    B.mla_append_cache_rmsnorm(layer.cdims, h, seq, pos, layer.w["w_dkv"],
                               layer.w["w_kr"], g_dev, EPS, layer.rope_cos,
                               layer.rope_sin, table, cache, ws=ws)


@pytest.mark.parametrize("dtype,chunk", [("bf16", 0), ("f32", 0),
                                         ("bf16", 3)])
def test_append_rmsnorm_rows(dtype, chunk):
    """chunk > 0: the rows are appended in calls of `chunk` tokens (the
    token counts a decode step appends)."""
    dims = W.DEEPSEEK_V2 if dtype == "bf16" else W.TINY
    w = W.make_weights(dims, dtype, 31)
    layer = MlaLayer(dims, dtype, w, 4096)
    g = _norm_weight(dims.d_c, dtype, 32)
    lens = np.array([1, 64, 65, 130, 17])      # partial and whole blocks
    table_np, nb = W.block_table(lens, True, 33)
    cache = layer.new_cache(nb)
    cache.fill_(float("nan"))
    table = torch.from_numpy(table_np).cuda()
    T = int(lens.sum())
    h = np.concatenate([W.hidden_states(dims, dtype, 34, b, 0, n)
                        for b, n in enumerate(lens)])
    seq = np.repeat(np.arange(len(lens)), lens).astype(np.int32)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    perm = np.random.default_rng(35).permutation(T)
    step = chunk if chunk else T
    for i in range(0, T, step):
        sel = perm[i:i + step]
        _append_norm(layer, to_device(h[sel], dtype),
                     torch.from_numpy(seq[sel]).cuda(),
                     torch.from_numpy(pos[sel]).cuda(), table, cache,
                     to_device(g, dtype))
    torch.cuda.synchronize()
    host = cache.float().cpu().numpy()
    c_ref, r_ref = orc.kv_latent(h, pos, w["w_dkv"], w["w_kr"], W.ROPE_BASE,
                                 kv_norm=(g, EPS))
    got = np.stack([host[table_np[s_, p // 64], p % 64]
                    for s_, p in zip(seq, pos)])
    assert_close("normalised latents", got[:, :dims.d_c], c_ref, dtype)
    assert_close("RoPE keys", got[:, dims.d_c:], r_ref, dtype)
    # unit weight would give rows of RMS 1: check the weight really applies
    rms = np.sqrt(np.mean((got[:, :dims.d_c] / g) ** 2, axis=1))
    np.testing.assert_allclose(rms, 1.0, rtol=2e-2 if dtype == "bf16" else 1e-5)
    owned = np.zeros(host.shape[:2], bool)
    for s_, p in zip(seq, pos):
        owned[table_np[s_, p // 64], p % 64] = True
    assert np.isnan(host[~owned]).all()
    log(f"  {T} rows ({dtype}, calls of {step} tokens)")


def test_decode_step_over_normalised_cache():
    """Context and new token written with the normalising append, then
    absorb, decode and out: u and o_lat against the oracle step with
    kv_norm."""
    dims = W.DEEPSEEK_V2
    w = W.make_weights(dims, "bf16", 41)
    layer = MlaLayer(dims, "bf16", w, 4096)
    g = _norm_weight(dims.d_c, "bf16", 42)
    ctx = 300
    lens = np.array([ctx + 1])
    table_np, nb = W.block_table(lens, True, 43)
    cache = layer.new_cache(nb)
    table = torch.from_numpy(table_np).cuda()
    h_all = W.hidden_states(dims, "bf16", 44, 0, 0, ctx + 1)
    pos = np.arange(ctx + 1, dtype=np.int32)
    seq = np.zeros(ctx + 1, np.int32)
    # the context in one call, the new token in a call of its own
    for lo, hi in ((0, ctx), (ctx, ctx + 1)):
        _append_norm(layer, to_device(h_all[lo:hi], "bf16"),
                     torch.from_numpy(seq[lo:hi]).cuda(),
                     torch.from_numpy(pos[lo:hi]).cuda(), table, cache,
                     to_device(g, "bf16"))
    h_new = h_all[ctx:]
    q = layer.absorb(to_device(h_new, "bf16"),
                     torch.from_numpy(pos[ctx:]).cuda())
    kv = torch.tensor([ctx + 1], dtype=torch.int32, device="cuda")
    o_lat, _ = layer.decode(q.view(1, 1, dims.n_h, dims.d_c + dims.d_r),
                            cache, table, kv, ctx + 1)
    u = layer.out(o_lat.view(1, dims.n_h, dims.d_c))
    torch.cuda.synchronize()
    c_ctx, r_ctx = orc.kv_latent(h_all[:ctx], pos[:ctx], w["w_dkv"],
                                 w["w_kr"], W.ROPE_BASE, kv_norm=(g, EPS))
    wd = {k: v.astype(np.float64) for k, v in w.items()}
    ref = orc.decode_step(wd, dims.n_h, W.ROPE_BASE, h_new, c_ctx, r_ctx,
                          kv_norm=(g, EPS))
    assert_close("u", u.float().cpu().numpy(), ref["u"], "bf16")
    log("  decode step over a normalised cache")
