"""HIP graph capture of the whole decode step.

No API call allocates, clears memory or synchronises inside, so a caller
can capture a step (append, absorb, decode with the split combine, out)
into a HIP graph.  The graph is replayed several times, with eager work and
synchronisations in between, and every replay must reproduce the eager
step's outputs bit for bit (same kernels, same inputs, no atomics)."""
import dataclasses

import pytest
import torch

from mla_latent_kv_33_amd import flow
from mla_latent_kv_33_amd import workloads as W
from tests.gpu_common import log

pytestmark = pytest.mark.gpu


def _workload(name, n_split):
    if name == "b1_ctx4k":
        # the single-sequence step (1 x 4096 context + 1 token): 64 splits
        # of 64 heads each, the combine for few query rows
        return dataclasses.replace(W.workload("b1_ctx4k"), n_split=n_split)
    # 16 sequences, ragged contexts (partial last blocks), permuted table,
    # library-chosen splits (several per sequence, so the combine runs):
    # one count for all, or balanced per sequence (a plan the decode kernel
    # writes on every replay).
    base = W.workload("b64_ctx8k")
    return dataclasses.replace(
        base, name="graph_b16", batch=16,
        ctx=tuple(700 + 131 * i for i in range(16)), seed=11,
        n_split=n_split)


def _snapshot(st, out):
    return {"q": out.q.clone(), "o_lat": out.o_lat.clone(),
            "lse": out.lse.clone(), "u": out.u.clone(),
            "cache": st.cache.clone()}


@pytest.mark.parametrize("name,n_split", [("graph_b16", 0),
                                          ("graph_b16", -1),
                                          ("b1_ctx4k", 0)])
def test_step_graph_replays_match_eager(name, n_split):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    wl = _workload(name, n_split)
    log(f"case {name} n_split={n_split}")
    layer = flow.make_layer(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st)           # eager: outputs and workspaces
    torch.cuda.synchronize()
    ref = _snapshot(st, out)

    # capture on a side stream after one warm pass there
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        flow.run_step(st, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        flow.run_step(st, out=out)
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work between replays: clobber the outputs, run an eager step
        # into separate buffers
        for k in ("q", "o_lat", "lse", "u"):
            getattr(out, k).fill_(float("nan"))
        other = flow.run_step(st)
        torch.cuda.synchronize()
        assert torch.equal(other.u, ref["u"]), "eager step changed"
        graph.replay()
        torch.cuda.synchronize()
        for k in ("q", "o_lat", "lse", "u"):
            same = torch.equal(getattr(out, k), ref[k])
            log(f"  replay {rep}: {k} {'identical' if same else 'DIFFERS'}")
            assert same, f"replay {rep}: {k} differs from the eager step"
        assert torch.equal(st.cache, ref["cache"]), \
            f"replay {rep}: cache differs from the eager step"


@pytest.mark.parametrize("name,n_split,stacked,fuse_out",
                         [("graph_b16", 0, True, False),
                          ("graph_b16", -1, False, False),
                          ("b1_ctx4k", 0, True, False),
                          ("b1_ctx4k", 0, True, True)])
def test_bound_step_matches_eager(name, n_split, stacked, fuse_out):
    """flow.bind_step (the step's library calls with their arguments
    checked and marshalled once, as bench.py runs them) reproduces the
    eager step bit for bit, call after call (fuse_out: the decode and the
    output projection as one mla_decode_out call)."""
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    wl = _workload(name, n_split)
    log(f"case {name} n_split={n_split} stacked={stacked} "
        f"fuse_out={fuse_out}, bound calls")
    layer = flow.make_layer(wl)
    st = flow.prepare(wl, layer)
    out = flow.run_step(st, stacked=stacked, fuse_out=fuse_out)
    torch.cuda.synchronize()
    ref = _snapshot(st, out)
    step = flow.bind_step(st, out, stacked=stacked, fuse_out=fuse_out)
    assert len(step.pre) == (1 if stacked else 2)
    for rep in range(3):
        for k in ("q", "o_lat", "lse", "u"):
            getattr(out, k).fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        for k in ("q", "o_lat", "lse", "u"):
            assert torch.equal(getattr(out, k), ref[k]), \
                f"bound call {rep}: {k} differs from the eager step"
        assert torch.equal(st.cache, ref["cache"])
