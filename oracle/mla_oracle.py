"""Plain CPU fp64 oracle for one MLA attention layer over a latent KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this module imports nothing from the product path.  Inputs are arrays; it does
not read any device buffer.

Everything is float64 numpy with no intermediate rounding and no blocking,
fusion or reordering beyond what the pages write.  Pages cited:

* [Latent]   "Latent 压缩" (zdszero.github.io/latent.html), section
  "MLA: latent 作为可缓存的 KV 表示" under "两个典型应用".
* [MLA]      "MLA：潜在表示压缩与解耦 RoPE"
  (lizn-zn.github.io/scholia-log/architecture/MLA/), sections 1-9.
* [MiniMind] "MiniMind 学习笔记 10：Multi-Latent Attention，从 KV Cache 压缩到
  MiniMind 改造思路" (p-chao.com), sections 2-12.

Convention (column vectors, [MLA] sections 3-7): every weight is stored
``[out, in]``, so ``y = W x`` is ``x @ W.T`` on row-major token batches.
Head ``h`` owns rows ``h*d_h .. (h+1)*d_h - 1`` of W_UQ, W_UK and W_UV, and
rows ``h*d_r ..`` of W_QR.

Readings where the pages are silent (each listed in the design notes):

* RoPE: frequencies theta_j = base**(-2j/d_r), j < d_r/2, applied to the pairs
  (x_j, x_{j + d_r/2}) ("half split").  The pages only write RoPE(.) and
  R_t; the pairing is our reading.  Angles are p * theta_j in float64.
* Positions are 0-based.  A query at position P sees exactly the keys at
  positions 0..P ([MiniMind] section 12, causal mask with a cache: the new
  queries see the whole history, the mask covers the last columns).
* Score scale 1/sqrt(d_h + d_r) ([MLA] sections "A Attention" and 7; the
  naive path of [MiniMind] section 10 divides by sqrt(qk_head_dim) with
  qk_head_dim = nope + rope, the same number).
* No normalisation of the latent on the main path (the [MiniMind] kv_norm
  is not on the [MLA] path).  The optional ``kv_norm`` of ``kv_latent``
  follows [MiniMind] section 9 (kv_norm = RMSNorm of the latent only, the
  RoPE key untouched); the page names RMSNorm without writing it out, so its
  formula is the usual one: w * x / sqrt(mean(x^2) + eps) over the latent.

Pins (tests/test_oracle_pins.py): absorbed == non-absorbed, value deferral,
softmax rows sum to one with exact zeros on masked keys, cache width
d_c + d_r and the pages' printed cache counts, the rank bound of the stacked
[K_C V_C], the RoPE relative-position identity and R_0 = I, agreement with
torch's scaled_dot_product_attention on CPU in float64 (MQA form and MHA
form), latent-basis invariance, RMSNorm closed forms (hand-computed values,
unit RMS with unit weight, scale invariance, k_R untouched), a scalar brute-force evaluation of the whole
layer on tiny inputs, and closed forms (one key, equal keys).  The RoPE pair
convention is a reading: the pins hold for either convention, so the pairing
itself is parity unpinned.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# cache arithmetic
# --------------------------------------------------------------------------

def mla_cache_elements(d_c: int, d_r: int) -> int:
    """Elements cached per token per layer by MLA: the latent c_KV plus the
    shared RoPE key k_R ([MLA] sections 2 and 6, table row MLA)."""
    return d_c + d_r


def mha_cache_elements(n_h: int, d_h: int) -> int:
    """Elements cached per token per layer by MHA: K and V of every head
    ([MLA] section 1 formula; [MLA] section 2 table row MHA)."""
    return 2 * n_h * d_h


def gqa_cache_elements(groups: int, d_h: int) -> int:
    """Elements cached per token per layer by GQA with ``groups`` KV heads
    ([MLA] section 2 table; [MiniMind] section 2)."""
    return 2 * groups * d_h


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def rope_frequencies(d_r: int, base: float) -> np.ndarray:
    """theta_j = base ** (-2 j / d_r), j = 0 .. d_r/2 - 1 (reading)."""
    j = np.arange(d_r // 2, dtype=F64)
    return np.power(F64(base), -2.0 * j / F64(d_r))


def apply_rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """R_p x over the last axis (length d_r): each pair (x_j, x_{j+d_r/2}) is
    rotated by the angle p * theta_j.  ``pos`` broadcasts against
    ``x.shape[:-1]``.  [MLA] sections 5-6 (R_t, RoPE(.)), reading for the
    pairing and frequencies."""
    x = np.asarray(x, dtype=F64)
    d_r = x.shape[-1]
    half = d_r // 2
    ang = np.asarray(pos, dtype=F64)[..., None] * rope_frequencies(d_r, base)
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


# --------------------------------------------------------------------------
# projections ([MLA] sections 3, 6, 7)
# --------------------------------------------------------------------------

def rms_norm(x, weight, eps):
    """RMSNorm over the last axis: ``weight * x / sqrt(mean(x^2) + eps)``
    (the kv_norm of [MiniMind] section 9; formula as read in the header)."""
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(weight, F64) * (x / np.sqrt(ms + float(eps)))


def kv_latent(h, pos, w_dkv, w_kr, base, kv_norm=None):
    """What goes into the cache for tokens with hidden states ``h [T, d]`` at
    positions ``pos [T]``: c_KV = W_DKV h ([MLA] section 3) and the shared
    RoPE key k_R = RoPE(W_KR h) ([MLA] section 6).  With ``kv_norm =
    (weight [d_c], eps)`` the latent is RMS-normalised before it is cached
    and k_R is not ([MiniMind] section 9).  Returns
    ``(c_kv [T, d_c], k_r [T, d_r])``."""
    h = np.asarray(h, dtype=F64)
    c_kv = h @ np.asarray(w_dkv, F64).T
    if kv_norm is not None:
        c_kv = rms_norm(c_kv, kv_norm[0], kv_norm[1])
    k_r = apply_rope(h @ np.asarray(w_kr, F64).T, np.asarray(pos), base)
    return c_kv, k_r


def query(h, pos, w_dq, w_uq, w_qr, n_h, base):
    """Query path ([MLA] sections 3 and 6): c_Q = W_DQ h (not cached),
    q_C = W_UQ c_Q per head, q_R = RoPE(W_QR c_Q) per head with every head
    rotated by the token's position.  Returns ``(q_c [T, n_h, d_h],
    q_r [T, n_h, d_r])``."""
    h = np.asarray(h, dtype=F64)
    T = h.shape[0]
    c_q = h @ np.asarray(w_dq, F64).T
    q_c = (c_q @ np.asarray(w_uq, F64).T).reshape(T, n_h, -1)
    q_r = (c_q @ np.asarray(w_qr, F64).T).reshape(T, n_h, -1)
    q_r = apply_rope(q_r, np.asarray(pos)[:, None], base)
    return q_c, q_r


def explicit_kv(c_kv, w_uk, w_uv, head, d_h):
    """Non-absorbed up-projection of the latent for one head:
    k_C = W_UK_h c_KV and v_C = W_UV_h c_KV ([MLA] section 3; [MiniMind]
    section 10, naive version).  Returns ``(k_c [S, d_h], v_c [S, d_h])``."""
    c_kv = np.asarray(c_kv, F64)
    rows = slice(head * d_h, (head + 1) * d_h)
    k_c = c_kv @ np.asarray(w_uk, F64)[rows].T
    v_c = c_kv @ np.asarray(w_uv, F64)[rows].T
    return k_c, v_c


def visibility(q_pos, kv_len):
    """``[n_q, kv_len]`` mask: query at position P sees keys 0..P."""
    return np.arange(kv_len)[None, :] <= np.asarray(q_pos)[:, None]


def _softmax_rows(s, visible):
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.where(visible, np.exp(s - m), 0.0)
    l = e.sum(axis=-1, keepdims=True)
    return e / l, (m + np.log(l))[..., 0]


def attention(q_c, q_r, q_pos, c_kv, k_r, w_uk, w_uv, heads=None,
              return_weights=False):
    """Non-absorbed multi-head attention over the latent cache
    ([MLA] section 7; [MiniMind] section 10 naive form).

    For each head h: k = [W_UK_h c_KV ; k_R] (k_R shared by every head),
    q = [q_C ; q_R], a = softmax(q.k / sqrt(d_h + d_r)) over the visible
    keys, o_h = sum_s a_s W_UV_h c_KV_s.

    ``q_c [n_q, n_h, d_h]``, ``q_r [n_q, n_h, d_r]``, ``q_pos [n_q]``,
    ``c_kv [S, d_c]``, ``k_r [S, d_r]``; ``heads`` restricts the heads
    computed (others stay zero).  Returns ``o [n_q, n_h, d_h]``,
    ``lse [n_q, n_h]`` (natural log of the softmax denominator including
    the max) and, if asked, the weights ``a [n_q, n_h, S]``.
    """
    q_c = np.asarray(q_c, F64)
    q_r = np.asarray(q_r, F64)
    k_r = np.asarray(k_r, F64)
    n_q, n_h, d_h = q_c.shape
    d_r = q_r.shape[-1]
    S = c_kv.shape[0]
    scale = 1.0 / math.sqrt(d_h + d_r)
    vis = visibility(q_pos, S)
    o = np.zeros((n_q, n_h, d_h))
    lse = np.zeros((n_q, n_h))
    weights = np.zeros((n_q, n_h, S)) if return_weights else None
    for h in (range(n_h) if heads is None else heads):
        k_c, v_c = explicit_kv(c_kv, w_uk, w_uv, h, d_h)
        k = np.concatenate([k_c, k_r], axis=1)
        q = np.concatenate([q_c[:, h], q_r[:, h]], axis=1)
        a, lse[:, h] = _softmax_rows((q @ k.T) * scale, vis)
        o[:, h] = a @ v_c
        if return_weights:
            weights[:, h] = a
    if return_weights:
        return o, lse, weights
    return o, lse


def output(o, w_o):
    """u = W_O o with o the concatenation of the heads' outputs
    ([MLA] section 7)."""
    o = np.asarray(o, F64)
    return o.reshape(o.shape[0], -1) @ np.asarray(w_o, F64).T


# --------------------------------------------------------------------------
# absorbed forms ([Latent] MLA section; [MLA] section 4; [MiniMind] 10)
# --------------------------------------------------------------------------

def absorb_query(q_c, q_r, w_uk):
    """Absorbed query: q_lat_h = W_UK_h^T q_C_h in the d_c latent, followed by
    the head's RoPE query, giving ``[n_q, n_h, d_c + d_r]``.  The identity
    <q, W_K c> = <W_K^T q, c> ([Latent] MLA section; [MLA] section 4)."""
    q_c = np.asarray(q_c, F64)
    n_q, n_h, d_h = q_c.shape
    w_uk = np.asarray(w_uk, F64)
    lat = np.stack([q_c[:, h] @ w_uk[h * d_h:(h + 1) * d_h]
                    for h in range(n_h)], axis=1)
    return np.concatenate([lat, np.asarray(q_r, F64)], axis=-1)


def latent_attention(q, q_pos, rows, d_c, d_h, heads=None):
    """Attention in the latent space (decode as MQA, [Latent] MLA section):
    one shared key per token, the cache row [c_KV ; k_R], and one shared
    value, c_KV.  score = q . row / sqrt(d_h + d_r); o_lat = sum_s a_s c_s.

    ``q [n_q, n_h, d_c + d_r]``, ``rows [S, d_c + d_r]``.  Returns
    ``o_lat [n_q, n_h, d_c]`` and ``lse [n_q, n_h]``."""
    q = np.asarray(q, F64)
    rows = np.asarray(rows, F64)
    n_q, n_h, width = q.shape
    d_r = width - d_c
    scale = 1.0 / math.sqrt(d_h + d_r)
    vis = visibility(q_pos, rows.shape[0])
    o_lat = np.zeros((n_q, n_h, d_c))
    lse = np.zeros((n_q, n_h))
    for h in (range(n_h) if heads is None else heads):
        a, lse[:, h] = _softmax_rows((q[:, h] @ rows.T) * scale, vis)
        o_lat[:, h] = a @ rows[:, :d_c]
    return o_lat, lse


def deferred_output(o_lat, w_uv, w_o, d_h):
    """u = sum_h W_O_h W_UV_h o_lat_h: the value up-projection applied after
    the weighted sum ([MLA] section 4 per-head output formula; [Latent]
    value-deferral identity)."""
    return output(head_values(o_lat, w_uv, d_h), w_o)


def head_values(o_lat, w_uv, d_h):
    """v_h = W_UV_h o_lat_h for every head: ``[n_q, n_h, d_h]``."""
    o_lat = np.asarray(o_lat, F64)
    n_h = o_lat.shape[1]
    w_uv = np.asarray(w_uv, F64)
    return np.stack([o_lat[:, h] @ w_uv[h * d_h:(h + 1) * d_h].T
                     for h in range(n_h)], axis=1)


# --------------------------------------------------------------------------
# one decode / chunked-prefill step of a sequence
# --------------------------------------------------------------------------

def decode_step(w, n_h, base, h_new, ctx_c_kv, ctx_k_r, heads=None,
                q_rows=None, kv_norm=None):
    """One step for one sequence, non-absorbed ([MLA] section 7).

    The sequence already holds ``ctx`` tokens whose latents are
    ``ctx_c_kv [ctx, d_c]`` / ``ctx_k_r [ctx, d_r]``; ``h_new [n_q, d]`` are
    the new tokens at positions ctx .. ctx+n_q-1.  Their latents are appended
    (kv_latent), then each new token attends causally over all ctx + n_q
    keys.  ``q_rows`` restricts which of the new tokens are evaluated as
    queries (all by default); ``heads`` restricts the heads.  ``kv_norm``
    (weight, eps) normalises the new tokens' latents as kv_latent does; the
    context latents are taken as given.

    Returns a dict with c_kv / k_r of the new tokens, q_c, q_r, o, lse and u
    (u only when every head is computed).
    """
    h_new = np.asarray(h_new, F64)
    n_new = h_new.shape[0]
    ctx = ctx_c_kv.shape[0]
    pos = ctx + np.arange(n_new)
    c_new, kr_new = kv_latent(h_new, pos, w["w_dkv"], w["w_kr"], base,
                              kv_norm=kv_norm)
    c_all = np.concatenate([np.asarray(ctx_c_kv, F64), c_new], axis=0)
    kr_all = np.concatenate([np.asarray(ctx_k_r, F64), kr_new], axis=0)
    sel = np.arange(n_new) if q_rows is None else np.asarray(q_rows)
    q_c, q_r = query(h_new[sel], pos[sel], w["w_dq"], w["w_uq"], w["w_qr"],
                     n_h, base)
    o, lse = attention(q_c, q_r, pos[sel], c_all, kr_all, w["w_uk"],
                       w["w_uv"], heads=heads)
    out = dict(c_kv=c_new, k_r=kr_new, q_c=q_c, q_r=q_r, o=o, lse=lse,
               q_pos=pos[sel])
    if heads is None:
        out["u"] = output(o, w["w_o"])
    return out
