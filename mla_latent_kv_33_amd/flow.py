"""Host orchestration of a decode step for a named synthetic workload:
upload inputs, build the paged cache, run the four library calls.

No attention arithmetic happens here: contexts enter the cache either through
mla_append_cache (from hidden states) or, for workloads whose context is given
as an existing cache, by copying seeded latent rows into their paged slots.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import workloads as W
from .layer import MlaLayer, to_device


@dataclasses.dataclass
class DeviceStep:
    """Device buffers of one step of a workload."""
    wl: W.Workload
    layer: MlaLayer
    cache: torch.Tensor
    table: torch.Tensor          # int32 [B, max_blocks]
    table_np: np.ndarray
    kv_lens: torch.Tensor        # int32 [B]
    max_kv_len: int
    h_new: torch.Tensor          # [B * n_q, d] new tokens, sequence-major
    seq_idx: torch.Tensor        # int32 [B * n_q]
    pos: torch.Tensor            # int32 [B * n_q]
    h_new_np: np.ndarray


def make_layer(wl: W.Workload, weights=None, device="cuda") -> MlaLayer:
    if weights is None:
        weights = W.make_weights(wl.dims, wl.dtype, wl.seed)
    max_pos = int(wl.kv_lens.max())
    return MlaLayer(wl.dims, wl.dtype, weights, max_pos, W.ROPE_BASE,
                    W.BLOCK_SIZE, device)


def scatter_rows_host(cache_np: np.ndarray, table_np: np.ndarray, seq: int,
                      start: int, rows: np.ndarray, block: int):
    """Place rows of positions start.. of sequence `seq` into their paged
    slots of a host cache image [num_blocks, block, width]."""
    pos = start + np.arange(len(rows))
    blk = table_np[seq, pos // block]
    cache_np[blk, pos % block] = rows


def prepare(wl: W.Workload, layer: MlaLayer, device="cuda",
            context: bool = True, ctx_chunk: int = 8192) -> DeviceStep:
    """Allocate the cache for the workload, fill the context, and upload the
    new tokens of the step (positions ctx .. ctx + n_q - 1)."""
    d = wl.dims
    kv = wl.kv_lens
    table_np, num_blocks = W.block_table(kv, wl.permuted, wl.seed)
    cache = layer.new_cache(num_blocks)
    table = torch.from_numpy(table_np).to(device)
    if context:
        if wl.synthetic_context:
            width = d.d_c + d.d_r
            img = np.zeros((num_blocks, W.BLOCK_SIZE, width), np.float32)
            for b, c in enumerate(wl.ctx):
                rows = W.latent_rows(d, wl.dtype, wl.seed, b, 0, c)
                scatter_rows_host(img, table_np, b, 0, rows, W.BLOCK_SIZE)
            cache.copy_(to_device(img, wl.dtype, device))
        else:
            for b, c in enumerate(wl.ctx):
                for s in range(0, c, ctx_chunk):
                    n = min(ctx_chunk, c - s)
                    h = to_device(W.hidden_states(d, wl.dtype, wl.seed, b, s,
                                                  n), wl.dtype, device)
                    seq = torch.full((n,), b, dtype=torch.int32, device=device)
                    pos = torch.arange(s, s + n, dtype=torch.int32,
                                       device=device)
                    layer.append(h, seq, pos, table, cache)
    h_new_np = np.concatenate([
        W.hidden_states(d, wl.dtype, wl.seed, b, c, wl.n_q)
        for b, c in enumerate(wl.ctx)])
    seq_idx = np.repeat(np.arange(wl.batch), wl.n_q).astype(np.int32)
    pos = np.concatenate([c + np.arange(wl.n_q)
                          for c in wl.ctx]).astype(np.int32)
    return DeviceStep(
        wl=wl, layer=layer, cache=cache, table=table, table_np=table_np,
        kv_lens=torch.from_numpy(kv.astype(np.int32)).to(device),
        max_kv_len=int(kv.max()), h_new=to_device(h_new_np, wl.dtype, device),
        seq_idx=torch.from_numpy(seq_idx).to(device),
        pos=torch.from_numpy(pos).to(device), h_new_np=h_new_np)


@dataclasses.dataclass
class StepOut:
    q: torch.Tensor       # [B, n_q, n_h, d_c + d_r]
    o_lat: torch.Tensor   # [B, n_q, n_h, d_c] fp32
    lse: torch.Tensor     # [B, n_q, n_h] fp32
    u: torch.Tensor       # [B * n_q, d]


def run_step(st: DeviceStep, n_split: Optional[int] = None, stream=None,
             out: Optional[StepOut] = None, stacked: bool = True,
             fuse_out: bool = False) -> StepOut:
    """One pass of the hot path: append the new tokens, absorb their
    queries, decode over the cache, project the output.  stacked: the
    append and the query path as one mla_append_absorb_q call (else
    mla_append_cache, then mla_absorb_q).  fuse_out: the decode and the
    output projection as one mla_decode_out call (else mla_decode, then
    mla_out)."""
    wl, L = st.wl, st.layer
    d = wl.dims
    ns = wl.n_split if n_split is None else n_split
    q_out = None if out is None else out.q.view(-1, d.n_h, d.d_c + d.d_r)
    if stacked:
        q = L.append_absorb(st.h_new, st.seq_idx, st.pos, st.table, st.cache,
                            q_out=q_out, stream=stream)
    else:
        L.append(st.h_new, st.seq_idx, st.pos, st.table, st.cache,
                 stream=stream)
        q = L.absorb(st.h_new, st.pos, q_out=q_out, stream=stream)
    q4 = q.view(wl.batch, wl.n_q, d.n_h, d.d_c + d.d_r)
    if fuse_out:
        o_lat, lse, u = L.decode_out(
            q4, st.cache, st.table, st.kv_lens, st.max_kv_len, n_split=ns,
            o_lat=None if out is None else out.o_lat,
            lse=None if out is None else out.lse,
            u=None if out is None else out.u, stream=stream)
        return StepOut(q=q4, o_lat=o_lat, lse=lse, u=u)
    o_lat, lse = L.decode(q4, st.cache, st.table, st.kv_lens, st.max_kv_len,
                          n_split=ns,
                          o_lat=None if out is None else out.o_lat,
                          lse=None if out is None else out.lse, stream=stream)
    u = L.out(o_lat.view(-1, d.n_h, d.d_c), u=None if out is None else out.u,
              stream=stream)
    return StepOut(q=q4, o_lat=o_lat, lse=lse, u=u)


@dataclasses.dataclass
class BoundStep:
    """The library calls of run_step with their arguments checked and
    marshalled once (binding.BoundCall): `pre` (the append and the query
    path: one stacked call, or the two calls), `attention` (mla_decode, or
    mla_decode_out) and `out` (mla_out, or nothing after mla_decode_out),
    on the buffers of the StepOut given to bind_step."""
    pre: list
    attention: object
    out: object

    def __call__(self) -> None:
        for c in self.pre:
            c()
        self.attention()
        self.out()


def _nothing() -> None:
    pass


def bind_step(st: DeviceStep, out: StepOut, n_split: Optional[int] = None,
              stream=None, stacked: bool = True,
              fuse_out: bool = False) -> BoundStep:
    """run_step(st, n_split, stream, out, stacked, fuse_out) as a
    BoundStep: each call again writes into `out` and the same
    workspaces."""
    wl, L = st.wl, st.layer
    d = wl.dims
    ns = wl.n_split if n_split is None else n_split
    q_out = out.q.view(-1, d.n_h, d.d_c + d.d_r)
    if stacked:
        pre = [L.append_absorb(st.h_new, st.seq_idx, st.pos, st.table,
                               st.cache, q_out=q_out, stream=stream,
                               bind=True)]
    else:
        pre = [L.append(st.h_new, st.seq_idx, st.pos, st.table, st.cache,
                        stream=stream, bind=True),
               L.absorb(st.h_new, st.pos, q_out=q_out, stream=stream,
                        bind=True)]
    if fuse_out:
        attention = L.decode_out(out.q, st.cache, st.table, st.kv_lens,
                                 st.max_kv_len, n_split=ns, o_lat=out.o_lat,
                                 lse=out.lse, u=out.u, stream=stream,
                                 bind=True)
        return BoundStep(pre=pre, attention=attention, out=_nothing)
    attention = L.decode(out.q, st.cache, st.table, st.kv_lens,
                         st.max_kv_len, n_split=ns, o_lat=out.o_lat,
                         lse=out.lse, stream=stream, bind=True)
    o = L.out(out.o_lat.view(-1, d.n_h, d.d_c), u=out.u, stream=stream,
              bind=True)
    return BoundStep(pre=pre, attention=attention, out=o)


@dataclasses.dataclass
class PrefillOut:
    q: torch.Tensor       # [B, n_q, n_h, d_h + d_r]
    o_v: torch.Tensor     # [B, n_q, n_h, d_h] fp32
    lse: torch.Tensor     # [B, n_q, n_h] fp32
    u: torch.Tensor       # [B * n_q, d]


def run_prefill_mha(st: DeviceStep, stream=None,
                    out: Optional[PrefillOut] = None,
                    causal: int = 1) -> PrefillOut:
    """The same step on the explicit-key (MHA) path: append the chunk, its
    queries without absorption, attention with per-head keys and values
    up-projected from the cache, output projection."""
    wl, L = st.wl, st.layer
    d = wl.dims
    L.append(st.h_new, st.seq_idx, st.pos, st.table, st.cache, stream=stream)
    q = L.query_mha(st.h_new, st.pos, q_out=None if out is None else
                    out.q.view(-1, d.n_h, d.d_h + d.d_r), stream=stream)
    q4 = q.view(wl.batch, wl.n_q, d.n_h, d.d_h + d.d_r)
    o_v, lse = L.prefill_mha(q4, st.cache, st.table, st.kv_lens,
                             st.max_kv_len,
                             o_v=None if out is None else out.o_v,
                             lse=None if out is None else out.lse,
                             causal=causal, stream=stream)
    u = L.out_values(o_v.view(-1, d.n_h * d.d_h),
                     u=None if out is None else out.u, stream=stream)
    return PrefillOut(q=q4, o_v=o_v, lse=lse, u=u)


def gather_rows(st: DeviceStep, seq: int, start: int, count: int) -> np.ndarray:
    """Cache rows of positions start .. start+count-1 of a sequence, read back
    to the host as float32 (for checks)."""
    pos = start + np.arange(count)
    blk = st.table_np[seq, pos // W.BLOCK_SIZE]
    idx_b = torch.from_numpy(blk.astype(np.int64)).to(st.cache.device)
    idx_r = torch.from_numpy((pos % W.BLOCK_SIZE).astype(np.int64)).to(
        st.cache.device)
    return st.cache[idx_b, idx_r].float().cpu().numpy()
