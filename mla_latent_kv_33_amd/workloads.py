"""Seeded synthetic inputs for MLA decode: dimensions, weights, hidden states,
context lengths and paged block tables.

This module only draws and lays out inputs.  It holds none of the attention
arithmetic: no projection, no RoPE, no softmax.  Both the CPU oracle (through
the tests and the benchmark) and the HIP path consume what it produces, so it
is deliberately free of anything either side computes.

Shapes follow the DeepSeek-V2 dimensions given on the page "MLA: latent
compression and decoupled RoPE" (section 8, DeepSeek-V2 dimensions):
d = 5120, n_h = 128, d_h = 128, d_c = 512, d_c' = 1536, d_r = 64.
Weights are stored like a PyTorch Linear, ``[out, in]`` row-major, and drawn
i.i.d. N(0, 1) / sqrt(fan_in) with fan_in the input width; hidden states are
i.i.d. N(0, 1).  For bf16 workloads every weight and hidden state is rounded
once (round-to-nearest-even) before either side sees it, so input quantisation
is never counted as kernel error.

Random streams are keyed, not sequential, so any chunk can be regenerated on
its own: weights use ``default_rng([seed, 0])``, context lengths
``default_rng([seed, 1])``, hidden states of sequence ``b``,
chunk ``k`` (4096 tokens) ``default_rng([seed, 2, b, k])``, and synthetic
latent-cache rows ``default_rng([seed, 3, b, k])``; the block-table
permutation ``default_rng([seed, 4])``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

BLOCK_SIZE = 64          # tokens per paged cache block
ROPE_BASE = 10000.0      # RoPE frequency base on the d_r rotary dims
HIDDEN_CHUNK = 4096      # tokens per hidden-state draw


@dataclasses.dataclass(frozen=True)
class Dims:
    """Layer dimensions.  Names in brackets are the hyper-parameter names used
    by public MLA configs (kv_lora_rank etc.)."""
    d: int        # hidden size
    n_h: int      # attention heads
    d_h: int      # per-head content dim [qk_nope_head_dim = v_head_dim]
    d_c: int      # KV latent dim [kv_lora_rank]
    d_r: int      # decoupled RoPE dim [qk_rope_head_dim]
    d_cq: int     # query latent dim [q_lora_rank]

    @property
    def row(self) -> int:
        """Elements of one latent-cache row: c_KV then k_R."""
        return self.d_c + self.d_r


TINY = Dims(d=64, n_h=4, d_h=16, d_c=32, d_r=8, d_cq=48)
DEEPSEEK_V2 = Dims(d=5120, n_h=128, d_h=128, d_c=512, d_r=64, d_cq=1536)

WEIGHT_ORDER = ("w_dkv", "w_kr", "w_dq", "w_uq", "w_qr", "w_uk", "w_uv", "w_o")


def weight_shapes(dims: Dims) -> Dict[str, tuple]:
    """``[out, in]`` shape of every projection."""
    return {
        "w_dkv": (dims.d_c, dims.d),
        "w_kr": (dims.d_r, dims.d),
        "w_dq": (dims.d_cq, dims.d),
        "w_uq": (dims.n_h * dims.d_h, dims.d_cq),
        "w_qr": (dims.n_h * dims.d_r, dims.d_cq),
        "w_uk": (dims.n_h * dims.d_h, dims.d_c),
        "w_uv": (dims.n_h * dims.d_h, dims.d_c),
        "w_o": (dims.d, dims.n_h * dims.d_h),
    }


# --------------------------------------------------------------------------
# bf16 storage helpers (bit patterns only)
# --------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return the
    16-bit patterns as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
               >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bf16-rounded values of ``x``."""
    return bf16_to_f32(bf16_bits(x))


def quantise(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values as the device will hold them (float32 container)."""
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------

def make_weights(dims: Dims, dtype: str, seed: int) -> Dict[str, np.ndarray]:
    """All eight projections, float32 containers, bf16-rounded for bf16."""
    rng = np.random.default_rng([seed, 0])
    out = {}
    for name in WEIGHT_ORDER:
        shape = weight_shapes(dims)[name]
        w = rng.standard_normal(shape, dtype=np.float32)
        w *= np.float32(1.0 / np.sqrt(shape[1]))
        out[name] = quantise(w, dtype)
    return out


def hidden_states(dims: Dims, dtype: str, seed: int, seq: int, start: int,
                  count: int) -> np.ndarray:
    """Hidden states ``[count, d]`` of tokens ``start .. start+count-1`` of
    sequence ``seq``.  Token t's value does not depend on how the range is
    cut, because each 4096-token chunk has its own stream."""
    rows = []
    t = start
    end = start + count
    while t < end:
        k = t // HIDDEN_CHUNK
        lo = k * HIDDEN_CHUNK
        chunk = np.random.default_rng([seed, 2, seq, k]).standard_normal(
            (HIDDEN_CHUNK, dims.d), dtype=np.float32)
        take_hi = min(end, lo + HIDDEN_CHUNK)
        rows.append(chunk[t - lo:take_hi - lo])
        t = take_hi
    if not rows:
        return np.zeros((0, dims.d), np.float32)
    return quantise(np.concatenate(rows, axis=0), dtype)


def latent_rows(dims: Dims, dtype: str, seed: int, seq: int, start: int,
                count: int) -> np.ndarray:
    """Synthetic latent-cache rows ``[count, d_c + d_r]`` (i.i.d. N(0, 1),
    the distribution a cache written from N(0,1) hidden states with
    1/sqrt(fan_in) weights has).  Used where a long context is given as an
    existing cache rather than rebuilt from hidden states."""
    rows = []
    t = start
    end = start + count
    while t < end:
        k = t // HIDDEN_CHUNK
        lo = k * HIDDEN_CHUNK
        chunk = np.random.default_rng([seed, 3, seq, k]).standard_normal(
            (HIDDEN_CHUNK, dims.row), dtype=np.float32)
        take_hi = min(end, lo + HIDDEN_CHUNK)
        rows.append(chunk[t - lo:take_hi - lo])
        t = take_hi
    if not rows:
        return np.zeros((0, dims.row), np.float32)
    return quantise(np.concatenate(rows, axis=0), dtype)


def context_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence context lengths drawn uniformly from ``[lo, hi]``."""
    rng = np.random.default_rng([seed, 1])
    return rng.integers(lo, hi + 1, size=batch).astype(np.int64)


def block_table(kv_lens: np.ndarray, permuted: bool, seed: int,
                block: int = BLOCK_SIZE, max_blocks: Optional[int] = None):
    """Paged block table.

    Sequence ``b`` needs ``ceil(kv_lens[b] / block)`` blocks.  Blocks are
    numbered sequence-major; with ``permuted`` the physical ids are a random
    permutation of ``0 .. total-1`` drawn from ``default_rng([seed, 4])``.
    Unused table slots hold -1.

    Returns ``(table int32 [B, max_blocks], num_blocks)``.
    """
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    need = (kv_lens + block - 1) // block
    total = int(need.sum())
    if max_blocks is None:
        max_blocks = int(need.max()) if len(need) else 0
    ids = np.arange(total, dtype=np.int64)
    if permuted:
        ids = np.random.default_rng([seed, 4]).permutation(total)
    table = np.full((len(kv_lens), max_blocks), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = ids[off:off + n]
        off += n
    return table, total


# --------------------------------------------------------------------------
# named workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode (or chunked-prefill) step.

    Sequence ``b`` holds ``ctx[b]`` cached tokens (positions 0..ctx-1) and
    receives ``n_q`` new tokens at positions ctx .. ctx+n_q-1, which are
    appended to the cache first; the new tokens are then the queries and
    attend causally, so every sequence ends with kv_len = ctx + n_q.
    """
    name: str
    dims: Dims
    dtype: str            # "f32" or "bf16"
    batch: int
    ctx: tuple            # per-sequence cached prior tokens
    n_q: int              # new tokens (queries) per sequence
    seed: int
    permuted: bool        # random-permutation block table
    # split-KV chunks per sequence: 0 = one count chosen by the library,
    # -1 = balanced per sequence (uneven lengths), else that count
    n_split: int = 0
    synthetic_context: bool = False   # context given as cache rows

    @property
    def kv_lens(self) -> np.ndarray:
        return np.asarray(self.ctx, dtype=np.int64) + self.n_q


def _var_ctx(seed):
    return tuple(int(x) for x in context_lengths(seed, 64, 1024, 8192))


def workload(name: str) -> Workload:
    """The named workloads used by tests and the benchmark."""
    if name == "tiny":
        return Workload("tiny", TINY, "f32", 1, (64,), 1, 1, False)
    if name == "b1_ctx4k":
        return Workload("b1_ctx4k", DEEPSEEK_V2, "bf16", 1, (4096,), 1, 2, False)
    if name == "b64_var":
        return Workload("b64_var", DEEPSEEK_V2, "bf16", 64, _var_ctx(3), 1, 3,
                        True, n_split=-1)
    if name == "b64_ctx8k":
        return Workload("b64_ctx8k", DEEPSEEK_V2, "bf16", 64, (8192,) * 64, 1,
                        6, True, synthetic_context=True)
    if name == "b4_ctx128k":
        return Workload("b4_ctx128k", DEEPSEEK_V2, "bf16", 4, (131072,) * 4, 1,
                        4, False, n_split=64, synthetic_context=True)
    if name == "b8_prefill":
        return Workload("b8_prefill", DEEPSEEK_V2, "bf16", 8, (8192,) * 8,
                        2048, 5, False)
    raise KeyError(name)


WORKLOADS = ("tiny", "b1_ctx4k", "b64_var", "b64_ctx8k", "b4_ctx128k",
             "b8_prefill")
