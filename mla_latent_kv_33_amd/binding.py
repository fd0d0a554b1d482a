"""Thin ctypes binding of libmla.so (include/mla.h).

Every function here only marshals torch tensors into pointers, sizes and the
current HIP stream, and turns status codes into exceptions; all arithmetic
of the decode path runs in the library's HIP kernels.  Functions carry the
C names.  There is no fallback: if the library is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_LIBRARY names another build of the same library (the host
# AddressSanitizer build of the ABI tests); the in-tree libmla.so otherwise.
LIB_PATH = os.environ.get("MLA_LIBRARY") or os.path.join(_HERE, "libmla.so")

MLA_F32 = 0
MLA_BF16 = 1
# n_split of mla_decode: splits proportional to each query row's keys
MLA_SPLIT_BALANCED = -1


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


class MlaDims(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("n_h", ctypes.c_int32),
                ("d_h", ctypes.c_int32), ("d_c", ctypes.c_int32),
                ("d_r", ctypes.c_int32), ("d_cq", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t
_DP = ctypes.POINTER(MlaDims)

_SIGNATURES = {
    "mla_status_string": (ctypes.c_char_p, [_I]),
    "mla_version": (ctypes.c_char_p, []),
    "mla_rope_tables_host": (_I, [_I, ctypes.c_double, _I, _P, _P]),
    "mla_append_workspace_bytes": (_S, [_DP, _I]),
    "mla_append_cache": (_I, [_DP, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I,
                              _P, _I, _P, _S, _P]),
    "mla_append_cache_rmsnorm": (_I, [_DP, _I, _P, _P, _P, _P, _P, _P,
                                      ctypes.c_float, _P, _P, _I, _P, _I, _P,
                                      _I, _P, _S, _P]),
    "mla_absorb_workspace_bytes": (_S, [_DP, _I]),
    "mla_absorb_q": (_I, [_DP, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                          _S, _P]),
    "mla_append_absorb_workspace_bytes": (_S, [_DP, _I]),
    "mla_append_absorb_q": (_I, [_DP, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _P, _P, _I, _P, _I, _P, _I, _P, _P, _S, _P]),
    "mla_merge_uq_uk": (_I, [_DP, _P, _P, _P, _P]),
    "mla_absorb_merged_workspace_bytes": (_S, [_DP, _I]),
    "mla_absorb_q_merged": (_I, [_DP, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P,
                                 _P, _S, _P]),
    "mla_decode_workspace_bytes": (_S, [_DP, _I, _I, _I, _I]),
    "mla_decode_auto_splits": (_I, [_DP, _I, _I, _I]),
    "mla_decode_noalloc": (_I, [_DP, _I, _I, _P, _P, _I, _P, _I, _P, _I, _I,
                                _I, _P, _P, _P]),
    "mla_validate_block_table": (_I, [_P, _I, _I, _P, _I, _I, _I, _I, _P]),
    "mla_decode": (_I, [_DP, _I, _I, _P, _P, _I, _P, _I, _P, _I, _I, _I, _P,
                        _P, _P, _S, _P]),
    "mla_query_mha": (_I, [_DP, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                           _S, _P]),
    "mla_prefill_mha_workspace_bytes": (_S, [_DP, _I, _I]),
    "mla_prefill_mha": (_I, [_DP, _I, _I, _P, _P, _I, _P, _I, _P, _I, _I, _P,
                             _P, _P, _P, _P, _S, _P]),
    "mla_decode_out_workspace_bytes": (_S, [_DP, _I, _I, _I, _I]),
    "mla_decode_out": (_I, [_DP, _I, _I, _P, _P, _I, _P, _I, _P, _I, _I, _I,
                            _P, _P, _P, _P, _P, _P, _S, _P]),
    "mla_out_values": (_I, [_DP, _I, _P, _P, _P, _P, _S, _P]),
    "mla_out_workspace_bytes": (_S, [_DP, _I]),
    "mla_out": (_I, [_DP, _I, _P, _P, _P, _P, _P, _S, _P]),
    # machine-rate kernels (include/mla_peaks.h), measurement only
    "mla_peak_stream_read": (_I, [_P, _S, _P, _I, _P]),
    "mla_peak_mfma_sink_bytes": (_S, [_I]),
    "mla_peak_mfma_flops": (ctypes.c_double, [_I, _I]),
    "mla_peak_mfma_loop": (_I, [_I, _I, _P, _P]),
}
EXPORTED = tuple(_SIGNATURES)


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                "python -m mla_latent_kv_33_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            # a build without one of the functions (an older library named by
            # MLA_LIBRARY) fails at that function's first call; the in-tree
            # build exports all of them (host test)
            if not hasattr(handle, name):
                continue
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def make_dims(dims, dtype: str, block_size: int = 64) -> MlaDims:
    """mla_dims from an object with d, n_h, d_h, d_c, d_r, d_cq."""
    return MlaDims(dims.d, dims.n_h, dims.d_h, dims.d_c, dims.d_r, dims.d_cq,
                   block_size, MLA_BF16 if dtype == "bf16" else MLA_F32)


def _check(fn: str, status: int):
    if status != 0:
        raise MlaError(fn, status, lib().mla_status_string(status).decode())


def _layer_dtype(dims: MlaDims) -> torch.dtype:
    return torch.bfloat16 if dims.dtype == MLA_BF16 else torch.float32


def _spec(t: Optional[torch.Tensor], name: str = "tensor", dtype=None,
          shape=None, numel: Optional[int] = None,
          ndim: Optional[int] = None) -> None:
    """Element type, rank, shape (None entries are free) and element count
    of a tensor argument, as include/mla.h states them."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got "
                         f"{tuple(t.shape)}")
    if shape is not None:
        if t.dim() != len(shape) or any(
                e is not None and e != a for e, a in zip(shape, t.shape)):
            want = tuple("*" if e is None else e for e in shape)
            raise ValueError(f"{name} must have shape {want}, got "
                             f"{tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got "
                         f"{t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor], name: str = "tensor", **spec):
    """Device pointer of a contiguous GPU tensor on the current device.

    Every tensor argument of the library is device memory read or written
    with the element type and extent that include/mla.h states; a host
    pointer, another device's memory, a wrong element type (an int64 index
    tensor read as int32) or a short buffer would reach a kernel.
    """
    if t is None:
        return None
    _spec(t, name, **spec)
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (libmla takes device "
                         "memory)")
    cur = torch.cuda.current_device()
    if t.device.index != cur:
        raise ValueError(f"{name} is on cuda:{t.device.index}; the current "
                         f"device is cuda:{cur}")
    return ctypes.c_void_p(t.data_ptr())


def _ptrs(*args):
    """Pointers of (tensor, name, spec) triples: every element type and
    shape is checked before any device check, so a malformed argument is
    named even when another one sits on the wrong device."""
    for t, name, spec in args:
        _spec(t, name, **spec)
    return [_ptr(t, name) for t, name, _ in args]


def _a(t, name, dtype=None, shape=None, **kw):
    """One argument triple for _ptrs."""
    return (t, name, dict(dtype=dtype, shape=shape, **kw))


_I32 = torch.int32
_F32 = torch.float32


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class BoundCall:
    """One library call whose tensor arguments were checked and whose
    ctypes arguments were built once (bind=True on a wrapper below).
    Calling it issues the same call again with the same pointers, sizes and
    stream, so the tensors must stay alive and in place; the library still
    checks its scalar arguments on every call.  A serving loop (or a timed
    benchmark) that reuses its buffers step after step pays the argument
    checks once instead of on every call."""
    __slots__ = ("name", "fn", "args")

    def __init__(self, name: str, args):
        self.name = name
        self.fn = getattr(lib(), name)
        self.args = tuple(args)

    def __call__(self) -> None:
        status = self.fn(*self.args)
        if status != 0:
            _check(self.name, status)


def _call(name: str, args, bind: bool):
    """Issue a library call, or return it as a BoundCall."""
    if bind:
        return BoundCall(name, args)
    _check(name, getattr(lib(), name)(*args))
    return None


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return ws, 0 if ws is None else ws.numel() * ws.element_size()
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def mla_status_string(status: int) -> str:
    return lib().mla_status_string(status).decode()


def mla_version() -> str:
    return lib().mla_version().decode()


def mla_rope_tables_host(d_r: int, base: float, max_pos: int):
    """Host cos/sin tables [max_pos, d_r/2] (float32 numpy)."""
    cos = np.empty((max_pos, d_r // 2), np.float32)
    sin = np.empty((max_pos, d_r // 2), np.float32)
    _check("mla_rope_tables_host", lib().mla_rope_tables_host(
        d_r, float(base), max_pos, cos.ctypes.data_as(_P),
        sin.ctypes.data_as(_P)))
    return cos, sin


def mla_append_workspace_bytes(dims: MlaDims, T: int) -> int:
    return lib().mla_append_workspace_bytes(ctypes.byref(dims), T)


def mla_absorb_workspace_bytes(dims: MlaDims, T: int) -> int:
    return lib().mla_absorb_workspace_bytes(ctypes.byref(dims), T)


def mla_append_absorb_workspace_bytes(dims: MlaDims, T: int) -> int:
    return lib().mla_append_absorb_workspace_bytes(ctypes.byref(dims), T)


def mla_decode_workspace_bytes(dims: MlaDims, B: int, n_q: int,
                               max_kv_len: int, n_split: int) -> int:
    return lib().mla_decode_workspace_bytes(ctypes.byref(dims), B, n_q,
                                            max_kv_len, n_split)


def mla_decode_auto_splits(dims: MlaDims, B: int, n_q: int,
                           max_kv_len: int) -> int:
    return lib().mla_decode_auto_splits(ctypes.byref(dims), B, n_q,
                                        max_kv_len)


def mla_validate_block_table(block_table, kv_lens, n_q: int,
                             block_size: int, num_blocks: int,
                             max_kv_len: int = 0) -> int:
    """Host check of a block table and lengths (numpy or CPU tensors);
    raises MlaError (status MLA_ERR_RANGE) naming the first bad sequence."""
    table = np.ascontiguousarray(np.asarray(block_table), dtype=np.int32)
    lens = np.ascontiguousarray(np.asarray(kv_lens), dtype=np.int32)
    if table.ndim != 2 or lens.ndim != 1 or table.shape[0] < lens.shape[0]:
        raise ValueError("block_table must be [B, max_blocks] and kv_lens [B]")
    bad = ctypes.c_int32(-1)
    st = lib().mla_validate_block_table(
        table.ctypes.data_as(_P), lens.shape[0], table.shape[1],
        lens.ctypes.data_as(_P), n_q, block_size, num_blocks, max_kv_len,
        ctypes.byref(bad))
    if st != 0:
        raise MlaError("mla_validate_block_table", st,
                       f"{mla_status_string(st)}; sequence {bad.value}")
    return 0


def mla_out_workspace_bytes(dims: MlaDims, T: int) -> int:
    return lib().mla_out_workspace_bytes(ctypes.byref(dims), T)


def _append_args(dims, h, seq_idx, pos, w_dkv, w_kr, rope_cos, rope_sin,
                 block_table, cache):
    """Argument triples of the append (include/mla.h layouts)."""
    lt = _layer_dtype(dims)
    T = h.shape[0]
    return [_a(h, "h", lt, (T, dims.d)),
            _a(seq_idx, "seq_idx", _I32, (T,)),
            _a(pos, "pos", _I32, (T,)),
            _a(w_dkv, "w_dkv", lt, (dims.d_c, dims.d)),
            _a(w_kr, "w_kr", lt, (dims.d_r, dims.d)),
            _a(rope_cos, "rope_cos", _F32, (None, dims.d_r // 2)),
            _a(rope_sin, "rope_sin", _F32, tuple(rope_cos.shape)),
            _a(block_table, "block_table", _I32, ndim=2),
            _a(cache, "cache", lt,
               (None, dims.block_size, dims.d_c + dims.d_r))]


def _query_args(dims, h, pos, w_dq, w_uq, w_qr, rope_cos, rope_sin):
    """Argument triples of the query path (include/mla.h layouts)."""
    lt = _layer_dtype(dims)
    T = h.shape[0]
    return [_a(h, "h", lt, (T, dims.d)),
            _a(pos, "pos", _I32, (T,)),
            _a(w_dq, "w_dq", lt, (dims.d_cq, dims.d)),
            _a(w_uq, "w_uq", lt, (dims.n_h * dims.d_h, dims.d_cq)),
            _a(w_qr, "w_qr", lt, (dims.n_h * dims.d_r, dims.d_cq)),
            _a(rope_cos, "rope_cos", _F32, (None, dims.d_r // 2)),
            _a(rope_sin, "rope_sin", _F32, tuple(rope_cos.shape))]


def _attention_args(dims, q, cache, block_table, kv_lens, qwidth):
    """Argument triples of q, cache, block_table and kv_lens."""
    lt = _layer_dtype(dims)
    B, n_q = q.shape[0], q.shape[1]
    if block_table.dim() == 2 and block_table.shape[0] < B:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for "
                         f"{B} sequences")
    return [_a(q, "q", lt, (B, n_q, dims.n_h, qwidth)),
            _a(cache, "cache", lt,
               (None, dims.block_size, dims.d_c + dims.d_r)),
            _a(block_table, "block_table", _I32, ndim=2),
            _a(kv_lens, "kv_lens", _I32, (B,))]


def mla_append_cache(dims: MlaDims, h, seq_idx, pos, w_dkv, w_kr, rope_cos,
                     rope_sin, block_table, cache, ws=None, stream=None,
                     bind: bool = False):
    """c_KV = W_DKV h and k_R = RoPE(W_KR h) for T = h.shape[0] tokens,
    written into the paged cache (see include/mla.h)."""
    T = h.shape[0]
    p = _ptrs(*_append_args(dims, h, seq_idx, pos, w_dkv, w_kr, rope_cos,
                            rope_sin, block_table, cache))
    ws, wsb = _workspace(mla_append_workspace_bytes(dims, T) if T else 0,
                         h.device, ws)
    return _call("mla_append_cache", (
        ctypes.byref(dims), T, *p[:7], rope_cos.shape[0], p[7],
        block_table.shape[1], p[8], cache.shape[0], _ptr(ws, "ws"), wsb,
        _stream(stream)), bind)


def mla_append_cache_rmsnorm(dims: MlaDims, h, seq_idx, pos, w_dkv, w_kr,
                             kv_norm_w, eps: float, rope_cos, rope_sin,
                             block_table, cache, ws=None, stream=None):
    """mla_append_cache with the latent RMS-normalised (weight kv_norm_w,
    epsilon eps) before it is cached (see include/mla.h)."""
    T = h.shape[0]
    p = _ptrs(*_append_args(dims, h, seq_idx, pos, w_dkv, w_kr, rope_cos,
                            rope_sin, block_table, cache),
              _a(kv_norm_w, "kv_norm_w", _layer_dtype(dims), (dims.d_c,)))
    ws, wsb = _workspace(mla_append_workspace_bytes(dims, T) if T else 0,
                         h.device, ws)
    _check("mla_append_cache_rmsnorm", lib().mla_append_cache_rmsnorm(
        ctypes.byref(dims), T, *p[:5], p[9], float(eps), p[5], p[6],
        rope_cos.shape[0], p[7], block_table.shape[1], p[8], cache.shape[0],
        _ptr(ws, "ws"), wsb, _stream(stream)))


def mla_absorb_q(dims: MlaDims, h, pos, w_dq, w_uq, w_qr, w_uk, rope_cos,
                 rope_sin, q_out, ws=None, stream=None, bind: bool = False):
    """q_out[t, h] = [W_UK_h^T q_C | RoPE(W_QR c_Q)_h] (see include/mla.h)."""
    T = h.shape[0]
    lt = _layer_dtype(dims)
    p = _ptrs(*_query_args(dims, h, pos, w_dq, w_uq, w_qr, rope_cos,
                           rope_sin),
              _a(w_uk, "w_uk", lt, (dims.n_h * dims.d_h, dims.d_c)),
              _a(q_out, "q_out", lt,
                 numel=T * dims.n_h * (dims.d_c + dims.d_r)))
    ws, wsb = _workspace(mla_absorb_workspace_bytes(dims, T) if T else 0,
                         h.device, ws)
    return _call("mla_absorb_q", (
        ctypes.byref(dims), T, *p[:5], p[7], p[5], p[6], rope_cos.shape[0],
        p[8], _ptr(ws, "ws"), wsb, _stream(stream)), bind)


def mla_append_absorb_q(dims: MlaDims, h, seq_idx, pos, w_dkv, w_kr, w_dq,
                        w_uq, w_qr, w_uk, rope_cos, rope_sin, block_table,
                        cache, q_out, ws=None, stream=None,
                        bind: bool = False):
    """mla_append_cache and mla_absorb_q on the same tokens in one call (see
    include/mla.h)."""
    T = h.shape[0]
    lt = _layer_dtype(dims)
    p = _ptrs(*_append_args(dims, h, seq_idx, pos, w_dkv, w_kr, rope_cos,
                            rope_sin, block_table, cache),
              _a(w_dq, "w_dq", lt, (dims.d_cq, dims.d)),
              _a(w_uq, "w_uq", lt, (dims.n_h * dims.d_h, dims.d_cq)),
              _a(w_qr, "w_qr", lt, (dims.n_h * dims.d_r, dims.d_cq)),
              _a(w_uk, "w_uk", lt, (dims.n_h * dims.d_h, dims.d_c)),
              _a(q_out, "q_out", lt,
                 numel=T * dims.n_h * (dims.d_c + dims.d_r)))
    ws, wsb = _workspace(mla_append_absorb_workspace_bytes(dims, T) if T
                         else 0, h.device, ws)
    # p: h seq_idx pos w_dkv w_kr cos sin table cache w_dq w_uq w_qr w_uk q
    return _call("mla_append_absorb_q", (
        ctypes.byref(dims), T, *p[:5], p[9], p[10], p[11], p[12], p[5], p[6],
        rope_cos.shape[0], p[7], block_table.shape[1], p[8], cache.shape[0],
        p[13], _ptr(ws, "ws"), wsb, _stream(stream)), bind)


def mla_merge_uq_uk(dims: MlaDims, w_uq, w_uk, w_merged, stream=None):
    """w_merged [n_h, d_c, d_cq] = W_UK_h^T W_UQ_h per head."""
    lt = _layer_dtype(dims)
    p = _ptrs(_a(w_uq, "w_uq", lt, (dims.n_h * dims.d_h, dims.d_cq)),
              _a(w_uk, "w_uk", lt, (dims.n_h * dims.d_h, dims.d_c)),
              _a(w_merged, "w_merged", lt, (dims.n_h, dims.d_c, dims.d_cq)))
    _check("mla_merge_uq_uk", lib().mla_merge_uq_uk(
        ctypes.byref(dims), *p, _stream(stream)))


def mla_absorb_q_merged(dims: MlaDims, h, pos, w_dq, w_merged, w_qr,
                        rope_cos, rope_sin, q_out, ws=None, stream=None):
    """The output of mla_absorb_q through the pre-merged W_UK_h^T W_UQ_h."""
    T = h.shape[0]
    lt = _layer_dtype(dims)
    a = _query_args(dims, h, pos, w_dq, w_qr.new_empty((0,)), w_qr, rope_cos,
                    rope_sin)
    a[3] = _a(w_merged, "w_merged", lt, (dims.n_h, dims.d_c, dims.d_cq))
    p = _ptrs(*a, _a(q_out, "q_out", lt,
                     numel=T * dims.n_h * (dims.d_c + dims.d_r)))
    ws, wsb = _workspace(
        lib().mla_absorb_merged_workspace_bytes(ctypes.byref(dims), T)
        if T else 0, h.device, ws)
    _check("mla_absorb_q_merged", lib().mla_absorb_q_merged(
        ctypes.byref(dims), T, *p[:7], rope_cos.shape[0], p[7],
        _ptr(ws, "ws"), wsb, _stream(stream)))


def mla_decode(dims: MlaDims, q, cache, block_table, kv_lens, max_kv_len: int,
               o_lat, lse=None, causal: int = 1, n_split: int = 0, ws=None,
               stream=None, bind: bool = False):
    """Latent attention of q [B, n_q, n_h, d_c + d_r] over the cache
    (see include/mla.h); writes o_lat [B, n_q, n_h, d_c] fp32 and lse."""
    B, n_q = q.shape[0], q.shape[1]
    p = _ptrs(*_attention_args(dims, q, cache, block_table, kv_lens,
                               dims.d_c + dims.d_r),
              _a(o_lat, "o_lat", _F32,
                 numel=B * n_q * dims.n_h * dims.d_c),
              _a(lse, "lse", _F32, numel=B * n_q * dims.n_h))
    ws, wsb = _workspace(
        mla_decode_workspace_bytes(dims, B, n_q, max_kv_len, n_split),
        q.device, ws)
    return _call("mla_decode", (
        ctypes.byref(dims), B, n_q, p[0], p[1], cache.shape[0], p[2],
        block_table.shape[1], p[3], max_kv_len, causal, n_split, p[4], p[5],
        _ptr(ws, "ws"), wsb, _stream(stream)), bind)


def mla_decode_out_workspace_bytes(dims: MlaDims, B: int, n_q: int,
                                   max_kv_len: int, n_split: int) -> int:
    return lib().mla_decode_out_workspace_bytes(ctypes.byref(dims), B, n_q,
                                                max_kv_len, n_split)


def mla_decode_out(dims: MlaDims, q, cache, block_table, kv_lens,
                   max_kv_len: int, w_uv, w_o, o_lat, u, lse=None,
                   causal: int = 1, n_split: int = 0, ws=None, stream=None,
                   bind: bool = False):
    """mla_decode, then mla_out on its B * n_q rows, in one call (see
    include/mla.h): writes o_lat, lse and u [B * n_q, d]."""
    B, n_q = q.shape[0], q.shape[1]
    lt = _layer_dtype(dims)
    p = _ptrs(*_attention_args(dims, q, cache, block_table, kv_lens,
                               dims.d_c + dims.d_r),
              _a(w_uv, "w_uv", lt, (dims.n_h * dims.d_h, dims.d_c)),
              _a(w_o, "w_o", lt, (dims.d, dims.n_h * dims.d_h)),
              _a(o_lat, "o_lat", _F32,
                 numel=B * n_q * dims.n_h * dims.d_c),
              _a(lse, "lse", _F32, numel=B * n_q * dims.n_h),
              _a(u, "u", lt, numel=B * n_q * dims.d))
    ws, wsb = _workspace(
        mla_decode_out_workspace_bytes(dims, B, n_q, max_kv_len, n_split),
        q.device, ws)
    return _call("mla_decode_out", (
        ctypes.byref(dims), B, n_q, p[0], p[1], cache.shape[0], p[2],
        block_table.shape[1], p[3], max_kv_len, causal, n_split, p[4], p[5],
        p[6], p[7], p[8], _ptr(ws, "ws"), wsb, _stream(stream)), bind)


def mla_decode_noalloc(dims: MlaDims, q, cache, block_table, kv_lens,
                       max_kv_len: int, o_lat, lse=None, causal: int = 1,
                       n_split: int = 0, stream=None):
    """mla_decode with the library's static scratch array instead of a
    workspace (see include/mla.h); allocates nothing."""
    B, n_q = q.shape[0], q.shape[1]
    p = _ptrs(*_attention_args(dims, q, cache, block_table, kv_lens,
                               dims.d_c + dims.d_r),
              _a(o_lat, "o_lat", _F32,
                 numel=B * n_q * dims.n_h * dims.d_c),
              _a(lse, "lse", _F32, numel=B * n_q * dims.n_h))
    _check("mla_decode_noalloc", lib().mla_decode_noalloc(
        ctypes.byref(dims), B, n_q, p[0], p[1], cache.shape[0], p[2],
        block_table.shape[1], p[3], max_kv_len, causal, n_split, p[4], p[5],
        _stream(stream)))


def mla_out(dims: MlaDims, o_lat, w_uv, w_o, u, ws=None, stream=None,
            bind: bool = False):
    """u = W_O [W_UV_h o_lat_h]_h for T = o_lat.shape[0] rows."""
    T = o_lat.shape[0]
    lt = _layer_dtype(dims)
    p = _ptrs(_a(o_lat, "o_lat", _F32, numel=T * dims.n_h * dims.d_c),
              _a(w_uv, "w_uv", lt, (dims.n_h * dims.d_h, dims.d_c)),
              _a(w_o, "w_o", lt, (dims.d, dims.n_h * dims.d_h)),
              _a(u, "u", lt, numel=T * dims.d))
    ws, wsb = _workspace(mla_out_workspace_bytes(dims, T) if T else 0,
                         o_lat.device, ws)
    return _call("mla_out", (
        ctypes.byref(dims), T, *p, _ptr(ws, "ws"), wsb, _stream(stream)),
        bind)


def mla_query_mha(dims: MlaDims, h, pos, w_dq, w_uq, w_qr, rope_cos, rope_sin,
                  q_out, ws=None, stream=None):
    """q_out[t, h] = [q_C | RoPE(q_R)] without absorption (see include/mla.h)."""
    T = h.shape[0]
    p = _ptrs(*_query_args(dims, h, pos, w_dq, w_uq, w_qr, rope_cos,
                           rope_sin),
              _a(q_out, "q_out", _layer_dtype(dims),
                 numel=T * dims.n_h * (dims.d_h + dims.d_r)))
    ws, wsb = _workspace(mla_absorb_workspace_bytes(dims, T) if T else 0,
                         h.device, ws)
    _check("mla_query_mha", lib().mla_query_mha(
        ctypes.byref(dims), T, *p[:7], rope_cos.shape[0], p[7],
        _ptr(ws, "ws"), wsb, _stream(stream)))


def mla_prefill_mha_workspace_bytes(dims: MlaDims, B: int,
                                    max_kv_len: int) -> int:
    return lib().mla_prefill_mha_workspace_bytes(ctypes.byref(dims), B,
                                                 max_kv_len)


def mla_prefill_mha(dims: MlaDims, q, cache, block_table, kv_lens,
                    max_kv_len: int, w_uk, w_uv, o_v, lse=None,
                    causal: int = 1, ws=None, stream=None):
    """Explicit-key attention of the chunk q [B, n_q, n_h, d_h + d_r] over
    the cache (see include/mla.h); writes o_v [B, n_q, n_h, d_h] fp32."""
    B, n_q = q.shape[0], q.shape[1]
    lt = _layer_dtype(dims)
    p = _ptrs(*_attention_args(dims, q, cache, block_table, kv_lens,
                               dims.d_h + dims.d_r),
              _a(w_uk, "w_uk", lt, (dims.n_h * dims.d_h, dims.d_c)),
              _a(w_uv, "w_uv", lt, (dims.n_h * dims.d_h, dims.d_c)),
              _a(o_v, "o_v", _F32, numel=B * n_q * dims.n_h * dims.d_h),
              _a(lse, "lse", _F32, numel=B * n_q * dims.n_h))
    ws, wsb = _workspace(mla_prefill_mha_workspace_bytes(dims, B, max_kv_len),
                         q.device, ws)
    _check("mla_prefill_mha", lib().mla_prefill_mha(
        ctypes.byref(dims), B, n_q, p[0], p[1], cache.shape[0], p[2],
        block_table.shape[1], p[3], max_kv_len, causal, *p[4:],
        _ptr(ws, "ws"), wsb, _stream(stream)))


def mla_out_values(dims: MlaDims, o_v, w_o, u, ws=None, stream=None):
    """u = W_O o for value-space o [T, n_h * d_h] fp32."""
    T = o_v.shape[0]
    lt = _layer_dtype(dims)
    p = _ptrs(_a(o_v, "o_v", _F32, numel=T * dims.n_h * dims.d_h),
              _a(w_o, "w_o", lt, (dims.d, dims.n_h * dims.d_h)),
              _a(u, "u", lt, numel=T * dims.d))
    ws, wsb = _workspace(mla_out_workspace_bytes(dims, T) if T else 0,
                         o_v.device, ws)
    _check("mla_out_values", lib().mla_out_values(
        ctypes.byref(dims), T, *p, _ptr(ws, "ws"), wsb, _stream(stream)))


def mla_peak_stream_read(buf, sink, workgroups: int, stream=None):
    """One read of the whole device buffer `buf` (include/mla_peaks.h)."""
    nbytes = buf.numel() * buf.element_size()
    _check("mla_peak_stream_read", lib().mla_peak_stream_read(
        _ptr(buf, "buf"), nbytes, _ptr(sink, "sink"), workgroups,
        _stream(stream)))
    return nbytes


def mla_peak_mfma_loop(workgroups: int, iters: int, sink, stream=None):
    """One launch of the matrix-core loop; returns its flop count."""
    _spec(sink, "sink", numel=None)
    if sink.numel() * sink.element_size() < \
            lib().mla_peak_mfma_sink_bytes(workgroups):
        raise ValueError("sink is smaller than mla_peak_mfma_sink_bytes")
    _check("mla_peak_mfma_loop", lib().mla_peak_mfma_loop(
        workgroups, iters, _ptr(sink, "sink"), _stream(stream)))
    return lib().mla_peak_mfma_flops(workgroups, iters)
