"""Device-side holder for one MLA layer: weights, RoPE tables, workspaces,
and the four library calls of a decode step.

Only allocation, host-to-device copies and call ordering live here; the
step's arithmetic is the library's.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import binding as B

WEIGHT_NAMES = ("w_dkv", "w_kr", "w_dq", "w_uq", "w_qr", "w_uk", "w_uv",
                "w_o")


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Upload float32 values (already representable in `dtype`)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device).to(torch_dtype(dtype)).contiguous()


class MlaLayer:
    def __init__(self, dims, dtype: str, weights: Dict[str, np.ndarray],
                 max_pos: int, rope_base: float = 10000.0,
                 block_size: int = 64, device="cuda"):
        self.dims = dims
        self.dtype = dtype
        self.device = device
        self.block_size = block_size
        self.cdims = B.make_dims(dims, dtype, block_size)
        self.w = {k: to_device(weights[k], dtype, device) for k in WEIGHT_NAMES}
        cos, sin = B.mla_rope_tables_host(dims.d_r, rope_base, max_pos)
        self.rope_cos = torch.from_numpy(cos).to(device)
        self.rope_sin = torch.from_numpy(sin).to(device)
        self._ws: Dict[str, torch.Tensor] = {}

    # ---- buffers ---------------------------------------------------------
    def new_cache(self, num_blocks: int) -> torch.Tensor:
        d = self.dims
        return torch.empty((num_blocks, self.block_size, d.d_c + d.d_r),
                           dtype=torch_dtype(self.dtype), device=self.device)

    def workspace(self, key: str, nbytes: int) -> Optional[torch.Tensor]:
        """A cached workspace of at least nbytes (None when 0)."""
        if nbytes == 0:
            return None
        ws = self._ws.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws

    # ---- the four steps ----------------------------------------------------
    # bind=True on the calls below: check and marshal the arguments, and
    # return the call as a binding.BoundCall instead of issuing it.
    def append(self, h, seq_idx, pos, block_table, cache, stream=None,
               bind=False):
        T = h.shape[0]
        ws = self.workspace("append",
                            B.mla_append_workspace_bytes(self.cdims, T)) \
            if T else None
        return B.mla_append_cache(self.cdims, h, seq_idx, pos,
                                  self.w["w_dkv"], self.w["w_kr"],
                                  self.rope_cos, self.rope_sin, block_table,
                                  cache, ws=ws, stream=stream, bind=bind)

    def absorb(self, h, pos, q_out=None, stream=None, bind=False):
        d = self.dims
        T = h.shape[0]
        if q_out is None:
            q_out = torch.empty((T, d.n_h, d.d_c + d.d_r),
                                dtype=torch_dtype(self.dtype),
                                device=self.device)
        ws = self.workspace("absorb",
                            B.mla_absorb_workspace_bytes(self.cdims, T))
        call = B.mla_absorb_q(self.cdims, h, pos, self.w["w_dq"],
                              self.w["w_uq"], self.w["w_qr"], self.w["w_uk"],
                              self.rope_cos, self.rope_sin, q_out, ws=ws,
                              stream=stream, bind=bind)
        return call if bind else q_out

    def append_absorb(self, h, seq_idx, pos, block_table, cache, q_out=None,
                      stream=None, bind=False):
        """append and absorb of the same tokens as one library call."""
        d = self.dims
        T = h.shape[0]
        if q_out is None:
            q_out = torch.empty((T, d.n_h, d.d_c + d.d_r),
                                dtype=torch_dtype(self.dtype),
                                device=self.device)
        ws = self.workspace("append_absorb",
                            B.mla_append_absorb_workspace_bytes(self.cdims,
                                                                T)) \
            if T else None
        call = B.mla_append_absorb_q(
            self.cdims, h, seq_idx, pos, self.w["w_dkv"], self.w["w_kr"],
            self.w["w_dq"], self.w["w_uq"], self.w["w_qr"], self.w["w_uk"],
            self.rope_cos, self.rope_sin, block_table, cache, q_out, ws=ws,
            stream=stream, bind=bind)
        return call if bind else q_out

    def decode(self, q, cache, block_table, kv_lens, max_kv_len: int,
               n_split: int = 0, o_lat=None, lse=None, stream=None,
               bind=False):
        d = self.dims
        Bsz, n_q = q.shape[0], q.shape[1]
        if o_lat is None:
            o_lat = torch.empty((Bsz, n_q, d.n_h, d.d_c), dtype=torch.float32,
                                device=self.device)
        if lse is None:
            lse = torch.empty((Bsz, n_q, d.n_h), dtype=torch.float32,
                              device=self.device)
        ws = self.workspace("decode", B.mla_decode_workspace_bytes(
            self.cdims, Bsz, n_q, max_kv_len, n_split))
        call = B.mla_decode(self.cdims, q, cache, block_table, kv_lens,
                            max_kv_len, o_lat, lse, causal=1,
                            n_split=n_split, ws=ws, stream=stream, bind=bind)
        return call if bind else (o_lat, lse)

    def decode_out(self, q, cache, block_table, kv_lens, max_kv_len: int,
                   n_split: int = 0, o_lat=None, lse=None, u=None,
                   stream=None, bind=False):
        """decode, then out on its rows, as one library call."""
        d = self.dims
        Bsz, n_q = q.shape[0], q.shape[1]
        if o_lat is None:
            o_lat = torch.empty((Bsz, n_q, d.n_h, d.d_c), dtype=torch.float32,
                                device=self.device)
        if lse is None:
            lse = torch.empty((Bsz, n_q, d.n_h), dtype=torch.float32,
                              device=self.device)
        if u is None:
            u = torch.empty((Bsz * n_q, d.d), dtype=torch_dtype(self.dtype),
                            device=self.device)
        ws = self.workspace("decode_out", B.mla_decode_out_workspace_bytes(
            self.cdims, Bsz, n_q, max_kv_len, n_split))
        call = B.mla_decode_out(self.cdims, q, cache, block_table, kv_lens,
                                max_kv_len, self.w["w_uv"], self.w["w_o"],
                                o_lat, u, lse=lse, causal=1, n_split=n_split,
                                ws=ws, stream=stream, bind=bind)
        return call if bind else (o_lat, lse, u)

    def out(self, o_lat, u=None, stream=None, bind=False):
        d = self.dims
        T = o_lat.shape[0]
        if u is None:
            u = torch.empty((T, d.d), dtype=torch_dtype(self.dtype),
                            device=self.device)
        ws = self.workspace("out", B.mla_out_workspace_bytes(self.cdims, T))
        call = B.mla_out(self.cdims, o_lat, self.w["w_uv"], self.w["w_o"], u,
                         ws=ws, stream=stream, bind=bind)
        return call if bind else u

    # ---- MHA-path chunked prefill (explicit keys and values) ---------------
    def query_mha(self, h, pos, q_out=None, stream=None):
        d = self.dims
        T = h.shape[0]
        if q_out is None:
            q_out = torch.empty((T, d.n_h, d.d_h + d.d_r),
                                dtype=torch_dtype(self.dtype),
                                device=self.device)
        ws = self.workspace("absorb",
                            B.mla_absorb_workspace_bytes(self.cdims, T))
        B.mla_query_mha(self.cdims, h, pos, self.w["w_dq"], self.w["w_uq"],
                        self.w["w_qr"], self.rope_cos, self.rope_sin, q_out,
                        ws=ws, stream=stream)
        return q_out

    def prefill_mha(self, q, cache, block_table, kv_lens, max_kv_len: int,
                    o_v=None, lse=None, causal: int = 1, stream=None):
        d = self.dims
        Bsz, n_q = q.shape[0], q.shape[1]
        if o_v is None:
            o_v = torch.empty((Bsz, n_q, d.n_h, d.d_h), dtype=torch.float32,
                              device=self.device)
        if lse is None:
            lse = torch.empty((Bsz, n_q, d.n_h), dtype=torch.float32,
                              device=self.device)
        ws = self.workspace("prefill", B.mla_prefill_mha_workspace_bytes(
            self.cdims, Bsz, max_kv_len))
        B.mla_prefill_mha(self.cdims, q, cache, block_table, kv_lens,
                          max_kv_len, self.w["w_uk"], self.w["w_uv"], o_v,
                          lse=lse, causal=causal, ws=ws, stream=stream)
        return o_v, lse

    def out_values(self, o_v, u=None, stream=None):
        d = self.dims
        T = o_v.shape[0]
        if u is None:
            u = torch.empty((T, d.d), dtype=torch_dtype(self.dtype),
                            device=self.device)
        ws = self.workspace("out", B.mla_out_workspace_bytes(self.cdims, T))
        B.mla_out_values(self.cdims, o_v, self.w["w_o"], u, ws=ws,
                         stream=stream)
        return u
