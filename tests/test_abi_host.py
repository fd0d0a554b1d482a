"""Host-side checks of libmla.so: it loads, exports every function that
include/mla.h declares, and rejects bad arguments with status codes before
enqueueing anything (no GPU needed: nothing here launches a kernel)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest
import torch

from mla_latent_kv_33_amd import binding as B
from mla_latent_kv_33_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

OK, NULL, SHAPE, UNSUP, WS, RANGE = 0, 1, 2, 3, 4, 5
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails first


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = B.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTED)


def test_status_strings_and_version():
    for s in range(7):
        assert B.mla_status_string(s)
    assert B.mla_status_string(99) == "unknown status"
    assert B.mla_version().startswith("mla-gfx950")


def test_rope_tables_host():
    """cos/sin(p * base^(-2j/d_r)) rounded once to float32."""
    cos, sin = B.mla_rope_tables_host(8, 10000.0, 300)
    for p in (0, 1, 17, 299):
        for j in range(4):
            a = p * 10000.0 ** (-2.0 * j / 8)
            assert cos[p, j] == np.float32(math.cos(a))
            assert sin[p, j] == np.float32(math.sin(a))
    lib = B.lib()
    buf = np.zeros(8, np.float32)
    assert lib.mla_rope_tables_host(7, 1e4, 1, buf.ctypes.data_as(
        ctypes.c_void_p), buf.ctypes.data_as(ctypes.c_void_p)) == SHAPE
    assert lib.mla_rope_tables_host(8, 1e4, 1, None, None) == NULL
    assert lib.mla_rope_tables_host(8, -1.0, 1, buf.ctypes.data_as(
        ctypes.c_void_p), buf.ctypes.data_as(ctypes.c_void_p)) == SHAPE


def ds_dims(**kw):
    d = B.make_dims(W.DEEPSEEK_V2, "bf16")
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_workspace_sizes():
    d = ds_dims()
    assert B.mla_append_workspace_bytes(d, 64) > 0
    assert B.mla_absorb_workspace_bytes(d, 64) > 0
    assert B.mla_out_workspace_bytes(d, 64) > 0
    assert B.mla_append_workspace_bytes(d, 0) == 0
    # one split needs no workspace; several need partial states
    assert B.mla_decode_workspace_bytes(d, 1, 1, 64, 1) == 0
    # decode batches stream W_O and W_UQ/W_QR with K-split partials (one K
    # chunk per column tile would leave most compute units idle): the
    # workspaces hold several fp32 partial copies of u (64 x 5120) and of
    # q_C/q_R (64 x 24576)
    assert B.mla_out_workspace_bytes(d, 64) >= \
        64 * 128 * 512 * 4 + 2 * 64 * 5120 * 4
    assert B.mla_absorb_workspace_bytes(d, 64) >= 2 * 64 * 24576 * 4
    ns = B.mla_decode_auto_splits(d, 64, 1, 8193)
    assert ns == 4
    assert B.mla_decode_workspace_bytes(d, 64, 1, 8193, 0) >= \
        64 * ns * 128 * (512 + 2) * 4
    assert B.mla_decode_auto_splits(d, 4, 1, 131073) == 64
    assert B.mla_decode_auto_splits(d, 8, 2048, 10240) == 1
    # one sequence: as many splits as keep two 64-token blocks each
    assert B.mla_decode_auto_splits(d, 1, 1, 4097) == 32
    assert B.mla_decode_auto_splits(d, 1, 1, 100) == 1
    # balanced splits: partial slots for 256 workgroups plus the row plan
    bal = B.mla_decode_workspace_bytes(d, 64, 1, 8193, B.MLA_SPLIT_BALANCED)
    assert bal >= 256 * 128 * (512 + 2) * 4 + 64 * 8
    # a single row is not balanced: the automatic count's workspace
    assert B.mla_decode_workspace_bytes(d, 1, 1, 4097, -1) == \
        B.mla_decode_workspace_bytes(d, 1, 1, 4097, 0)
    bad = ds_dims(d_r=63)
    assert B.mla_append_workspace_bytes(bad, 64) == 0


def call_append(dims, T=4, ws=FAKE, ws_bytes=1 << 30, h=FAKE, max_pos=16,
                max_blocks=1, num_blocks=1):
    return B.lib().mla_append_cache(ctypes.byref(dims), T, h, FAKE, FAKE,
                                    FAKE, FAKE, FAKE, FAKE, max_pos, FAKE,
                                    max_blocks, FAKE, num_blocks, ws,
                                    ws_bytes, None)


def test_append_validation():
    d = ds_dims()
    assert B.lib().mla_append_cache(None, 1, *([None] * 7), 16, None, 1,
                                    None, 1, None, 0, None) == NULL
    assert call_append(ds_dims(d_r=63)) == SHAPE
    assert call_append(ds_dims(block_size=48)) == SHAPE
    assert call_append(ds_dims(dtype=7)) == SHAPE
    assert call_append(ds_dims(d=5121)) == UNSUP
    assert call_append(d, T=-1) == SHAPE
    assert call_append(d, T=0) == OK          # no-op
    assert call_append(d, h=None) == NULL
    assert call_append(d, ws=None) == WS
    assert call_append(d, ws_bytes=16) == WS
    assert call_append(d, max_pos=0) == SHAPE


def test_absorb_and_out_validation():
    d = ds_dims()
    lib = B.lib()
    args = [FAKE] * 7
    assert lib.mla_absorb_q(ctypes.byref(d), 4, *args, FAKE, 16, FAKE, None,
                            0, None) == WS
    assert lib.mla_absorb_q(ctypes.byref(d), 4, *args, FAKE, 16, FAKE, FAKE,
                            16, None) == WS
    assert lib.mla_absorb_q(ctypes.byref(d), 4, None, *args[1:], FAKE, 16,
                            FAKE, FAKE, 1 << 30, None) == NULL
    assert lib.mla_out(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                       None) == WS
    assert lib.mla_out(ctypes.byref(d), 4, None, FAKE, FAKE, FAKE, FAKE,
                       1 << 30, None) == NULL
    assert lib.mla_out(ctypes.byref(d), 0, None, None, None, None, None, 0,
                       None) == OK


def call_decode(dims, B_=2, n_q=1, max_kv=100, causal=1, n_split=0,
                max_blocks=2, ws=FAKE, ws_bytes=1 << 30, q=FAKE):
    return B.lib().mla_decode(ctypes.byref(dims), B_, n_q, q, FAKE, 4, FAKE,
                              max_blocks, FAKE, max_kv, causal, n_split, FAKE,
                              None, ws, ws_bytes, None)


def test_decode_validation():
    d = ds_dims()
    assert call_decode(d, q=None) == NULL
    assert call_decode(d, B_=0) == SHAPE
    assert call_decode(d, n_q=0) == SHAPE
    assert call_decode(d, max_kv=0) == SHAPE
    assert call_decode(d, n_q=200, max_kv=100) == SHAPE      # n_q > kv
    assert call_decode(d, n_q=4, causal=0) == UNSUP
    assert call_decode(d, max_blocks=1) == RANGE             # 100 > 64
    assert call_decode(d, n_split=3) == RANGE                # 2 blocks
    assert call_decode(d, n_split=-2) == SHAPE
    assert call_decode(d, n_split=-1, ws=None) == WS          # balanced
    # fp32 layers: balanced means the automatic uniform count (4 splits of
    # 16 blocks here), which needs the workspace as well
    assert call_decode(ds_dims(dtype=B.MLA_F32), n_split=-1, max_kv=1000,
                       max_blocks=16, ws=None) == WS
    assert call_decode(d, n_split=2, ws=None) == WS
    assert call_decode(d, n_split=2, ws_bytes=64) == WS


def test_header_cites_pages_and_names_callers():
    text = open(HEADER).read()
    assert "MLA：潜在表示压缩与解耦 RoPE" in text
    for fn in ("mla_append_cache", "mla_absorb_q", "mla_decode", "mla_out"):
        assert fn in text


def call_rmsnorm(dims, T=4, ws=FAKE, ws_bytes=1 << 30, h=FAKE, eps=1e-6,
                 norm_w=FAKE, max_pos=16, max_blocks=1, num_blocks=1):
    return B.lib().mla_append_cache_rmsnorm(
        ctypes.byref(dims), T, h, FAKE, FAKE, FAKE, FAKE, norm_w, eps, FAKE,
        FAKE, max_pos, FAKE, max_blocks, FAKE, num_blocks, ws, ws_bytes,
        None)


def test_append_rmsnorm_validation():
    d = ds_dims()
    assert call_rmsnorm(ds_dims(d_r=63)) == SHAPE
    assert call_rmsnorm(d, T=-1) == SHAPE
    assert call_rmsnorm(d, eps=-1.0) == SHAPE
    assert call_rmsnorm(d, eps=float("nan")) == SHAPE
    assert call_rmsnorm(d, max_blocks=0) == SHAPE
    assert call_rmsnorm(ds_dims(d=5121)) == UNSUP
    assert call_rmsnorm(d, T=0) == OK          # no-op
    assert call_rmsnorm(d, norm_w=None) == NULL
    assert call_rmsnorm(d, ws=None) == WS
    assert call_rmsnorm(d, ws_bytes=16) == WS


def test_prefill_workspace_bytes():
    d = ds_dims()
    row, kvw = (512 + 64) * 2, 2 * 128 * 128 * 2
    big = B.mla_prefill_mha_workspace_bytes(d, 8, 10240)
    assert big >= 8 * 10240 * (row + kvw)
    assert big < 8 * 10240 * (row + kvw) + 4096
    # at least 128 rows (the up-projection GEMM's bf16 output)
    assert B.mla_prefill_mha_workspace_bytes(d, 1, 37) >= 128 * (row + kvw)
    assert B.mla_prefill_mha_workspace_bytes(d, 0, 37) == 0
    assert B.mla_prefill_mha_workspace_bytes(ds_dims(d_r=63), 1, 37) == 0


def call_prefill(dims, B_=2, n_q=4, max_kv=100, max_blocks=2, num_blocks=4,
                 ws=FAKE, ws_bytes=1 << 12, q=FAKE, w_uv=FAKE, causal=1):
    return B.lib().mla_prefill_mha(
        ctypes.byref(dims), B_, n_q, q, FAKE, num_blocks, FAKE, max_blocks,
        FAKE, max_kv, causal, FAKE, w_uv, FAKE, None, ws, ws_bytes, None)


def test_prefill_mha_validation():
    d = ds_dims()
    lib = B.lib()
    assert lib.mla_prefill_mha(None, 1, 1, *([None] * 2), 1, None, 1, None,
                               1, 1, None, None, None, None, None, 0,
                               None) == NULL
    assert call_prefill(d, B_=-1) == SHAPE
    assert call_prefill(d, n_q=-1) == SHAPE
    assert call_prefill(d, n_q=200, max_kv=100) == SHAPE     # n_q > kv
    assert call_prefill(d, max_kv=0, n_q=0) == SHAPE
    assert call_prefill(d, max_blocks=1) == SHAPE            # 100 > 64
    assert call_prefill(d, num_blocks=0) == SHAPE
    assert call_prefill(ds_dims(dtype=B.MLA_F32)) == UNSUP   # bf16 only
    assert call_prefill(ds_dims(d_h=64)) == UNSUP
    assert call_prefill(d, B_=0) == OK                       # no-op
    assert call_prefill(d, n_q=0) == OK
    assert call_prefill(d, q=None) == NULL
    assert call_prefill(d, w_uv=None) == NULL
    assert call_prefill(d, ws=None) == WS
    assert call_prefill(d, ws_bytes=1 << 12) == WS           # far too small


def test_query_mha_and_out_values_validation():
    d = ds_dims()
    lib = B.lib()
    args = [FAKE] * 6
    # (dims, T, h, pos, w_dq, w_uq, w_qr, cos, sin, max_pos, q, ws, bytes, s)
    assert lib.mla_query_mha(ctypes.byref(d), 4, *args, FAKE, 16, FAKE, None,
                             0, None) == WS
    assert lib.mla_query_mha(ctypes.byref(d), 4, *args, FAKE, 16, FAKE, FAKE,
                             16, None) == WS
    assert lib.mla_query_mha(ctypes.byref(d), 4, None, *args[1:], FAKE, 16,
                             FAKE, FAKE, 1 << 30, None) == NULL
    assert lib.mla_query_mha(ctypes.byref(d), 4, *args, FAKE, 0, FAKE, FAKE,
                             1 << 30, None) == SHAPE          # max_pos
    assert lib.mla_query_mha(ctypes.byref(ds_dims(dtype=B.MLA_F32)), 4,
                             *args, FAKE, 16, FAKE, FAKE, 1 << 30,
                             None) == UNSUP
    assert lib.mla_query_mha(ctypes.byref(d), 0, *([None] * 7), 16, None,
                             None, 0, None) == OK
    assert lib.mla_out_values(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, 16,
                              None) == WS
    assert lib.mla_out_values(ctypes.byref(d), 4, None, FAKE, FAKE, FAKE,
                              1 << 30, None) == NULL
    assert lib.mla_out_values(ctypes.byref(d), -1, FAKE, FAKE, FAKE, FAKE,
                              1 << 30, None) == SHAPE
    assert lib.mla_out_values(ctypes.byref(d), 0, None, None, None, None, 0,
                              None) == OK


def test_binding_rejects_host_and_strided_tensors():
    # every tensor argument of the library is device memory: a host tensor
    # must be refused before any call, not handed to a kernel
    with pytest.raises(ValueError, match="on the GPU"):
        B._ptr(torch.zeros(8))
    assert B._ptr(None) is None
