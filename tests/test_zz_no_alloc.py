"""mla_decode_noalloc (the decode with the library's static scratch array
instead of a caller workspace) against mla_decode, through the C ABI: two
calls in a row, the second with a smaller input, each bitwise equal to
mla_decode on the same inputs (the same kernels run), plus the size limit
and the no-partials case."""
import numpy as np
import pytest
import torch

from mla_latent_kv_33_amd import binding as B
from mla_latent_kv_33_amd import workloads as W

pytestmark = pytest.mark.gpu
DS = W.DEEPSEEK_V2


def _inputs(rng, lens, n_q=1):
    lens = np.asarray(lens)
    table_np, nb = W.block_table(lens, True, int(rng.integers(1 << 30)))
    g = torch.Generator(device="cuda")
    g.manual_seed(int(rng.integers(1 << 30)))
    cache = torch.randn((nb, 64, 576), device="cuda", generator=g).to(
        torch.bfloat16)
    q = (0.5 * torch.randn((len(lens), n_q, 128, 576), device="cuda",
                           generator=g)).to(torch.bfloat16)
    table = torch.from_numpy(table_np).cuda()
    kv = torch.from_numpy(lens.astype(np.int32)).cuda()
    return q, cache, table, kv, int(lens.max())


def _both(dims, q, cache, table, kv, max_kv, n_split):
    Bn, n_q = q.shape[0], q.shape[1]
    o1 = torch.empty((Bn, n_q, 128, 512), device="cuda")
    l1 = torch.empty((Bn, n_q, 128), device="cuda")
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    B.mla_decode(dims, q, cache, table, kv, max_kv, o1, l1, n_split=n_split)
    B.mla_decode_noalloc(dims, q, cache, table, kv, max_kv, o2, l2,
                         n_split=n_split)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def test_noalloc_matches_decode_two_calls():
    assert torch.cuda.is_available()
    dims = B.make_dims(DS, "bf16")
    rng = np.random.default_rng(77)
    # call 1: 64 sequences of 2048 tokens, automatic splits (4 per row:
    # 32768 partial rows, the scratch array's capacity)
    q, cache, table, kv, mx = _inputs(rng, [2048] * 64)
    assert B.mla_decode_auto_splits(dims, 64, 1, mx) == 4
    o1, l1, o2, l2 = _both(dims, q, cache, table, kv, mx, 0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # call 2, smaller: 5 uneven sequences, balanced splits; the array still
    # holds call 1's partials, which this call must not read
    q, cache, table, kv, mx = _inputs(rng, [3000, 17, 1200, 64, 5000])
    o1, l1, o2, l2 = _both(dims, q, cache, table, kv, mx,
                           B.MLA_SPLIT_BALANCED)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # one split: no partials at all
    o1, l1, o2, l2 = _both(dims, q, cache, table, kv, mx, 1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # beyond the array: refused before anything is enqueued
    q, cache, table, kv, mx = _inputs(rng, [2048] * 64)
    need = B.mla_decode_workspace_bytes(dims, 64, 1, mx, 8)
    assert need > 65 * 1024 * 1024
    with pytest.raises(B.MlaError) as ei:
        B.mla_decode_noalloc(dims, q, cache, table, kv, mx,
                             torch.empty((64, 1, 128, 512), device="cuda"),
                             n_split=8)
    assert ei.value.status == 4  # MLA_ERR_WORKSPACE
