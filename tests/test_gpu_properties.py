"""Properties of the HIP path that hold at any size: bit-exact cache
indexing, split-count and block-table invariance, determinism, the
causal/decode consistency of a chunk, and degenerate sizes."""
import dataclasses

import numpy as np
import pytest
import torch

from mla_latent_kv_33_amd import binding as B
from mla_latent_kv_33_amd import flow
from mla_latent_kv_33_amd import workloads as W
from mla_latent_kv_33_amd.layer import MlaLayer, to_device
from oracle import mla_oracle as orc
from tests.gpu_common import assert_close, log, oracle_sequence

pytestmark = pytest.mark.gpu
DS = W.DEEPSEEK_V2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


_cache = {}


def ds_layer(seed=2):
    if seed not in _cache:
        _cache.clear()
        w = W.make_weights(DS, "bf16", seed)
        _cache[seed] = (MlaLayer(DS, "bf16", w, 20000), w)
    return _cache[seed]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cache_indexing_bit_exact(dtype):
    """Integer-valued inputs make every product and sum exact, so each
    cached c_KV row and the k_R of position-0 tokens must equal the oracle
    bit for bit; every row must sit at its block-table slot."""
    dims = DS if dtype == "bf16" else W.TINY
    rng = np.random.default_rng(123)
    w = {k: np.zeros(s, np.float32) for k, s in W.weight_shapes(dims).items()}
    for k in ("w_dkv", "w_kr"):
        o, i = w[k].shape
        for r in range(o):   # 8 entries of +-1 per row
            cols = rng.choice(i, 8, replace=False)
            w[k][r, cols] = rng.choice([-1.0, 1.0], 8)
    layer = MlaLayer(dims, dtype, w, 4096)
    lens = np.array([1, 64, 65, 200, 130])
    table_np, nb = W.block_table(lens, True, 9)
    cache = layer.new_cache(nb)
    cache.fill_(float("nan"))
    table = torch.from_numpy(table_np).cuda()
    T = int(lens.sum())
    h = rng.integers(-3, 4, size=(T, dims.d)).astype(np.float32)
    seq = np.repeat(np.arange(len(lens)), lens).astype(np.int32)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    perm = rng.permutation(T)    # token order does not matter
    layer.append(to_device(h[perm], dtype), torch.from_numpy(seq[perm]).cuda(),
                 torch.from_numpy(pos[perm]).cuda(), table, cache)
    torch.cuda.synchronize()
    host = cache.float().cpu().numpy()
    c_kv, k_r = orc.kv_latent(h, pos, w["w_dkv"], w["w_kr"], W.ROPE_BASE)
    for t in range(T):
        b, p = seq[t], pos[t]
        row = host[table_np[b, p // 64], p % 64]
        np.testing.assert_array_equal(row[:dims.d_c], c_kv[t])
        if p == 0:
            np.testing.assert_array_equal(row[dims.d_c:], k_r[t])
        else:
            np.testing.assert_allclose(row[dims.d_c:], k_r[t], rtol=1e-2,
                                       atol=1e-2 * (1 + np.abs(k_r[t]).max()))
    # slots no token owns stay untouched (NaN)
    owned = np.zeros(host.shape[:2], bool)
    for b, n in enumerate(lens):
        for p in range(n):
            owned[table_np[b, p // 64], p % 64] = True
    assert np.isnan(host[~owned]).all()
    log(f"  {T} rows bit-exact ({dtype})")


def _decode_once(layer, q, cache, table, kv, max_kv, n_split):
    o, lse = layer.decode(q, cache, table, kv, max_kv, n_split=n_split)
    torch.cuda.synchronize()
    return o.clone(), lse.clone()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_count_invariance_and_determinism(dtype):
    """Any split count gives the same result: exactly up to fp32 rounding for
    fp32 layers; for bf16 layers the weights P are rounded to bf16 against
    each split's own reference maximum, so splits agree to that rounding.
    A fixed split count is bitwise deterministic.  n_split = -1 is the
    balanced plan (on bf16 layers: 1 .. 33 splits per row from the device
    kv_lens; on fp32 layers the automatic count)."""
    # bf16: each P carries up to 2^-9 relative rounding, so o agrees to
    # ~1e-3 and l (hence lse) to ~2^-9 / sqrt(keys) relative.
    if dtype == "bf16":
        layer, _ = ds_layer()
        dims, tol, lse_tol = DS, (3e-3, 2e-2), (1e-4, 4e-3)
    else:
        dims, tol, lse_tol = W.TINY, (2e-6, 1e-5), (1e-6, 2e-5)
        layer = MlaLayer(dims, "f32", W.make_weights(dims, "f32", 1), 5000)
    width = dims.d_c + dims.d_r
    rng = np.random.default_rng(5)
    lens = np.array([4097, 1000, 64, 1, 3333])
    table_np, nb = W.block_table(lens, True, 11)
    cache = layer.new_cache(nb)
    cache.copy_(to_device(rng.standard_normal((nb, 64, width)).astype(
        np.float32), dtype))
    table = torch.from_numpy(table_np).cuda()
    kv = torch.from_numpy(lens.astype(np.int32)).cuda()
    q = to_device(0.5 * rng.standard_normal((5, 1, dims.n_h, width)).astype(
        np.float32), dtype)
    base, base_lse = _decode_once(layer, q, cache, table, kv, 4097, 1)
    for ns in (2, 7, 16, 65, B.MLA_SPLIT_BALANCED):
        o, lse = _decode_once(layer, q, cache, table, kv, 4097, ns)
        assert_close(f"n_split={ns} vs 1", o.cpu().numpy(),
                     base.cpu().numpy(), "f32", tol=tol)
        assert_close(f"lse n_split={ns}", lse.cpu().numpy(),
                     base_lse.cpu().numpy(), "f32", tol=lse_tol)
        o2, lse2 = _decode_once(layer, q, cache, table, kv, 4097, ns)
        assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_block_table_permutation_invariance():
    """The same rows under a different physical block order give bitwise
    the same output."""
    layer, _ = ds_layer()
    rng = np.random.default_rng(6)
    lens = np.array([700, 2000])
    rows = [rng.standard_normal((n, 576)).astype(np.float32) for n in lens]
    q = to_device(0.5 * rng.standard_normal((2, 1, 128, 576)).astype(
        np.float32), "bf16")
    kv = torch.from_numpy(lens.astype(np.int32)).cuda()
    outs = []
    for permuted in (False, True):
        table_np, nb = W.block_table(lens, permuted, 21)
        img = np.zeros((nb, 64, 576), np.float32)
        for b in range(2):
            flow.scatter_rows_host(img, table_np, b, 0, rows[b], 64)
        cache = to_device(img, "bf16")
        outs.append(_decode_once(layer, q, cache,
                                 torch.from_numpy(table_np).cuda(), kv, 2000,
                                 3))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_chunk_last_row_equals_decode():
    """In a causal chunk the last query sees the whole cache, the first only
    the context and itself: they equal plain decodes at those lengths."""
    layer, w = ds_layer()
    rng = np.random.default_rng(7)
    ctx, n_q = 1000, 77
    kvl = ctx + n_q
    table_np, nb = W.block_table(np.array([kvl]), False, 1)
    img = np.zeros((nb, 64, 576), np.float32)
    flow.scatter_rows_host(img, table_np, 0, 0,
                           rng.standard_normal((kvl, 576)).astype(np.float32),
                           64)
    cache = to_device(img, "bf16")
    table = torch.from_numpy(table_np).cuda()
    q = to_device(0.5 * rng.standard_normal((1, n_q, 128, 576)).astype(
        np.float32), "bf16")
    o, lse = _decode_once(layer, q, cache, table,
                          torch.tensor([kvl], dtype=torch.int32).cuda(), kvl,
                          1)
    o_last, _ = _decode_once(layer, q[:, -1:].contiguous(), cache, table,
                             torch.tensor([kvl], dtype=torch.int32).cuda(),
                             kvl, 1)
    o_first, _ = _decode_once(layer, q[:, :1].contiguous(), cache, table,
                              torch.tensor([ctx + 1], dtype=torch.int32).cuda(),
                              kvl, 1)
    assert torch.equal(o[:, -1], o_last[:, 0])
    assert torch.equal(o[:, 0], o_first[:, 0])


@pytest.mark.parametrize("ctx,n_q", [((3000, 700), 90), ((5000, 300), 128)])
def test_balanced_causal_chunk(ctx, n_q):
    """Balanced splits over the query rows of causal chunks (rows of one
    sequence see different key counts, two sequences of different lengths):
    the same result as one split per row, to the bf16 rounding of P against
    each split's reference, on every row; checked against the oracle's
    latent attention on sampled rows.  2 x 128 = 256 rows is the plan's
    maximum, where every row gets exactly one split."""
    layer, w = ds_layer()
    rng = np.random.default_rng(12)
    lens = np.array(ctx) + n_q
    table_np, nb = W.block_table(lens, True, 13)
    img = np.zeros((nb, 64, 576), np.float32)
    rows_h = []
    for b, kvl in enumerate(lens):
        r = rng.standard_normal((kvl, 576)).astype(np.float32)
        flow.scatter_rows_host(img, table_np, b, 0, r, 64)
        rows_h.append(r)
    cache = to_device(img, "bf16")
    table = torch.from_numpy(table_np).cuda()
    kv = torch.from_numpy(lens.astype(np.int32)).cuda()
    q = to_device(0.5 * rng.standard_normal((2, n_q, 128, 576)).astype(
        np.float32), "bf16")
    o1, l1 = _decode_once(layer, q, cache, table, kv, int(lens.max()), 1)
    ob, lb = _decode_once(layer, q, cache, table, kv, int(lens.max()),
                          B.MLA_SPLIT_BALANCED)
    ob2, lb2 = _decode_once(layer, q, cache, table, kv, int(lens.max()),
                            B.MLA_SPLIT_BALANCED)
    assert torch.equal(ob, ob2) and torch.equal(lb, lb2)
    if 2 * n_q == 256:
        # the plan's 256 slots, one per row: every row is one split, written
        # directly, with the arithmetic of n_split = 1
        assert torch.equal(ob, o1) and torch.equal(lb, l1)
    assert_close("balanced vs one split", ob.cpu().numpy(), o1.cpu().numpy(),
                 "f32", tol=(3e-3, 2e-2))
    assert_close("balanced lse vs one split", lb.cpu().numpy(),
                 l1.cpu().numpy(), "f32", tol=(1e-4, 4e-3))
    qh = q.float().cpu().numpy()
    for b in (0, 1):
        rows = W.round_bf16(rows_h[b]).astype(np.float64)
        sel = [0, 45, n_q - 1]
        pos = lens[b] - n_q + np.array(sel)
        o_ref, lse_ref = orc.latent_attention(qh[b, sel], pos, rows, 512, 128)
        assert_close(f"seq{b} balanced o_lat", ob[b, sel].cpu().numpy(),
                     o_ref, "bf16")
        assert_close(f"seq{b} balanced lse", lb[b, sel].cpu().numpy(),
                     lse_ref, "bf16")


def test_single_key_and_zero_tokens():
    """kv_len = 1 (the softmax weight is 1: o_lat is the row itself) and
    T = 0 calls (no-ops)."""
    layer, _ = ds_layer()
    rng = np.random.default_rng(8)
    row = rng.standard_normal(576).astype(np.float32)
    img = np.zeros((1, 64, 576), np.float32)
    img[0, 0] = row
    cache = to_device(img, "bf16")
    q = to_device(rng.standard_normal((1, 1, 128, 576)).astype(np.float32),
                  "bf16")
    o, lse = _decode_once(layer, q, cache,
                          torch.zeros((1, 1), dtype=torch.int32).cuda(),
                          torch.ones(1, dtype=torch.int32).cuda(), 1, 0)
    rowq = W.round_bf16(row)
    np.testing.assert_array_equal(o[0, 0].cpu().numpy(),
                                  np.tile(rowq[:512], (128, 1)))
    s = (q[0, 0].float().cpu().numpy().astype(np.float64) @ rowq) / np.sqrt(192)
    assert_close("lse single key", lse[0, 0].cpu().numpy(), s, "f32",
                 tol=(1e-5, 1e-4))
    empty = torch.empty((0, DS.d), dtype=torch.bfloat16, device="cuda")
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    layer.append(empty, e32, e32, torch.zeros((1, 1), dtype=torch.int32,
                                              device="cuda"), cache)
    B.mla_out(layer.cdims, torch.empty((0, 128, 512), device="cuda"),
              layer.w["w_uv"], layer.w["w_o"],
              torch.empty((0, DS.d), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()


@pytest.mark.parametrize("n_h", [16, 32, 64])
def test_head_counts_end_to_end(n_h):
    """n_h = 32 and 64 run the matrix-core kernel with one and two waves per
    workgroup; n_h = 16 (which it does not take) runs the general kernels.
    Each meets the bf16 bar end to end, with ragged lengths that end inside
    a half block and splits."""
    dims = dataclasses.replace(DS, n_h=n_h)
    wl = W.Workload(f"ds_h{n_h}", dims, "bf16", 2, (300, 1000), 1, 12, True)
    w = W.make_weights(dims, "bf16", wl.seed)
    layer = flow.make_layer(wl, w)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st, n_split=3)
    torch.cuda.synchronize()
    for b in range(2):
        ref = oracle_sequence(wl, w, b)
        assert_close(f"h{n_h} seq{b} u",
                     out.u.view(2, 1, dims.d)[b].float().cpu().numpy(),
                     ref["u"], "bf16")
        assert_close(f"h{n_h} seq{b} o_lat", out.o_lat[b].cpu().numpy(),
                     ref["o_lat"], "bf16")


@pytest.mark.parametrize("n_split", [1, 3])
def test_score_jump_restart(n_split):
    """Keys whose scores jump far above the first keys' maximum (more than
    2^64 in weight) make the matrix-core kernel redo a split with a raised
    reference maximum; the result still matches the softmax definition.
    Two jumps, the second above the first, also exercise a second raise
    within one pass."""
    layer, _ = ds_layer()
    rng = np.random.default_rng(31)
    kvl = 700
    rows = 0.1 * rng.standard_normal((kvl, 576)).astype(np.float32)
    rows[100] = 5.0      # score ~ 5 * sum(q) / sqrt(192): about 90 in log2
    rows[450] = 12.0     # above the first jump by more than 64 in log2
    rows = W.round_bf16(rows)
    q = (0.5 * rng.standard_normal((1, 1, 128, 576)) + 0.3).astype(np.float32)
    q = W.round_bf16(q)
    table_np, nb = W.block_table(np.array([kvl]), True, 3)
    img = np.zeros((nb, 64, 576), np.float32)
    flow.scatter_rows_host(img, table_np, 0, 0, rows, 64)
    o, lse = _decode_once(layer, to_device(q, "bf16"), to_device(img, "bf16"),
                          torch.from_numpy(table_np).cuda(),
                          torch.tensor([kvl], dtype=torch.int32).cuda(), kvl,
                          n_split)
    ref_o, ref_lse = orc.latent_attention(q[0], [kvl - 1], rows, 512, 128)
    assert_close("o_lat after restart", o[0].cpu().numpy(), ref_o, "bf16")
    assert_close("lse after restart", lse[0].cpu().numpy(), ref_lse, "bf16")


def _host_chunk(nb, slots=256, min_chunk=2):
    """The balanced plan's chunk from its definition: the smallest c >=
    max(min_chunk, ceil(sum nb / slots)) with sum ceil(nb_r / c) <= slots."""
    nb = np.asarray(nb)
    c = max(min_chunk, -(-int(nb.sum()) // slots))
    while int(np.sum(-(-nb // c))) > slots:
        c += 1
    return c


@pytest.mark.parametrize("case", range(5))
def test_balanced_plan_readback(case):
    """The balanced plan the decode writes (read back from its workspace)
    for seeded random batches: each row's splits take consecutive slots in
    row order, at most 256 slots in all, every row's count is ceil(nb / c)
    for the minimal chunk c, so its splits cover its visible blocks exactly
    once with none empty; and the decode equals one split per row."""
    layer, _ = ds_layer()
    rng = np.random.default_rng(100 + case)
    Bsz = int(rng.choice([2, 7, 64, 100, 256]))
    n_q = 1
    hi = int(rng.choice([300, 5000, 20000]))
    lens = rng.integers(1, hi + 1, size=Bsz)
    lens[rng.integers(0, Bsz)] = 1          # a one-key row
    lens[rng.integers(0, Bsz)] = hi         # the longest row
    log(f"case {case}: B={Bsz} lens in [1, {hi}]")
    table_np, nb_total = W.block_table(lens, True, 200 + case)
    cache = torch.randn((nb_total, 64, 576), device="cuda").to(torch.bfloat16)
    table = torch.from_numpy(table_np).cuda()
    kv = torch.from_numpy(lens.astype(np.int32)).cuda()
    q = (0.5 * torch.randn((Bsz, n_q, 128, 576), device="cuda")).to(
        torch.bfloat16)
    max_kv = int(lens.max())
    nbytes = B.mla_decode_workspace_bytes(layer.cdims, Bsz, n_q, max_kv,
                                          B.MLA_SPLIT_BALANCED)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    o = torch.empty((Bsz, n_q, 128, 512), device="cuda")
    lse = torch.empty((Bsz, n_q, 128), device="cuda")
    B.mla_decode(layer.cdims, q, cache, table, kv, max_kv, o, lse,
                 n_split=B.MLA_SPLIT_BALANCED, ws=ws)
    torch.cuda.synchronize()
    rows = Bsz * n_q
    off = nbytes - (-(-8 * rows // 256) * 256)
    plan = ws[off:off + 8 * rows].cpu().numpy().view(np.int32).reshape(rows, 2)
    slot0, count = plan[:, 0], plan[:, 1]
    nb = np.maximum(-(-lens // 64), 1)
    c = _host_chunk(nb)
    np.testing.assert_array_equal(count, -(-nb // c))
    np.testing.assert_array_equal(slot0, np.concatenate([[0],
                                                         np.cumsum(count)[:-1]]))
    assert int(count.sum()) <= 256
    # minimality: one block less per chunk would not fit (or is below the
    # lower bound)
    lo = max(2, -(-int(nb.sum()) // 256))
    assert c == lo or int(np.sum(-(-nb // (c - 1)))) > 256
    # split j of a row covers [j nb / cnt, (j + 1) nb / cnt): contiguous,
    # disjoint, none empty, union = all the row's blocks
    for n, k in zip(nb, count):
        edges = [(j * int(n)) // int(k) for j in range(int(k) + 1)]
        assert edges[0] == 0 and edges[-1] == n
        assert all(b > a for a, b in zip(edges, edges[1:]))
    o1, l1 = _decode_once(layer, q, cache, table, kv, max_kv, 1)
    assert_close("balanced vs one split", o.cpu().numpy(), o1.cpu().numpy(),
                 "f32", tol=(3e-3, 2e-2))
    assert_close("balanced lse vs one split", lse.cpu().numpy(),
                 l1.cpu().numpy(), "f32", tol=(1e-4, 4e-3))


@pytest.mark.parametrize("dims_name", ["ds", "tiny"])
def test_row_without_visible_key(dims_name):
    """A row outside the contract (kv_lens[b] < n_q, no visible key) with one
    split gets o_lat = 0 and lse = -inf; the other rows are unaffected."""
    if dims_name == "ds":
        layer, _ = ds_layer()
        d, dt, tdt = DS, "bf16", torch.bfloat16
    else:
        d, dt, tdt = W.TINY, "f32", torch.float32
        layer = MlaLayer(d, dt, W.make_weights(d, dt, 1), 256)
    row = d.d_c + d.d_r
    rng = np.random.default_rng(31)
    cache = torch.from_numpy(rng.standard_normal((2, 64, row)).astype(
        np.float32)).to(tdt).cuda()
    table = torch.tensor([[0], [1]], dtype=torch.int32, device="cuda")
    kv = torch.tensor([5, 0], dtype=torch.int32, device="cuda")
    q = torch.from_numpy(rng.standard_normal((2, 1, d.n_h, row)).astype(
        np.float32)).to(tdt).cuda()
    o, lse = _decode_once(layer, q, cache, table, kv, 64, 1)
    assert torch.all(o[1] == 0)
    assert torch.all(torch.isneginf(lse[1]))
    assert torch.all(torch.isfinite(o[0])) and torch.all(torch.isfinite(lse[0]))
    rows = cache[0, :5].float().cpu().numpy().astype(np.float64)
    o_ref, l_ref = orc.latent_attention(
        q[0].float().cpu().numpy().astype(np.float64), [4], rows, d.d_c,
        d.d_h)
    assert_close("valid row", o[0].cpu().numpy(), o_ref, dt)
