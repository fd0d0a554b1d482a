"""Planted mistakes in the oracle (on the CPU) must fail a pin.

Each case swaps one oracle function for a version carrying a plausible
mistake (wrong sign, dropped term, wrong scale, wrong head, off-by-one mask)
and checks that the independent scalar evaluation of the layer no longer
agrees.  This shows the pins can see such mistakes; the real oracle is
untouched outside each test.
"""
import math

import numpy as np
import pytest

from oracle import mla_oracle as orc
from tests.test_oracle_pins import BASE, brute_force_layer, tiny_case

DIMS = dict(d=6, n_h=2, d_h=3, d_c=4, d_r=4, d_cq=5)


def _agrees():
    w, h_ctx, h_new, c_ctx, kr_ctx = tiny_case(seed=21, ctx=5, n_q=3,
                                               dims=DIMS)
    ref = orc.decode_step(w, DIMS["n_h"], BASE, h_new, c_ctx, kr_ctx)
    u, o, lse, _, _ = brute_force_layer(
        {k: v.tolist() for k, v in w.items()}, h_ctx, h_new, DIMS["n_h"],
        DIMS["d_h"], DIMS["d_c"], DIMS["d_r"], BASE)
    return (np.allclose(ref["u"], u, rtol=1e-9, atol=1e-12)
            and np.allclose(ref["lse"], lse, rtol=1e-9, atol=1e-12))


def test_unmutated_agrees():
    assert _agrees()


def _rope_sign(x, pos, base):
    x = np.asarray(x, float)
    half = x.shape[-1] // 2
    ang = np.asarray(pos, float)[..., None] * orc.rope_frequencies(
        x.shape[-1], base)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * np.cos(ang) + x2 * np.sin(ang),
                           -x1 * np.sin(ang) + x2 * np.cos(ang)], axis=-1)


def _rope_interleaved(x, pos, base):
    x = np.asarray(x, float)
    ang = np.asarray(pos, float)[..., None] * orc.rope_frequencies(
        x.shape[-1], base)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * np.cos(ang) - x2 * np.sin(ang)
    out[..., 1::2] = x1 * np.sin(ang) + x2 * np.cos(ang)
    return out


def _explicit_kv_wrong_head(c_kv, w_uk, w_uv, head, d_h):
    n_h = w_uk.shape[0] // d_h
    return _real_explicit_kv(c_kv, w_uk, w_uv, (head + 1) % n_h, d_h)


def _explicit_kv_swapped(c_kv, w_uk, w_uv, head, d_h):
    k, v = _real_explicit_kv(c_kv, w_uk, w_uv, head, d_h)
    return v, k


def _visibility_strict(q_pos, kv_len):
    return np.arange(kv_len)[None, :] < np.asarray(q_pos)[:, None] + \
        (np.arange(len(np.atleast_1d(q_pos)))[:, None] == 0)


def _kv_latent_unrotated(h, pos, w_dkv, w_kr, base, kv_norm=None):
    h = np.asarray(h, float)
    return h @ np.asarray(w_dkv).T, h @ np.asarray(w_kr).T


_real_explicit_kv = orc.explicit_kv
_real_attention = orc.attention


def _attention_no_rope_term(q_c, q_r, q_pos, c_kv, k_r, w_uk, w_uv,
                            heads=None, return_weights=False):
    return _real_attention(q_c, np.zeros_like(q_r), q_pos, c_kv, k_r, w_uk,
                           w_uv, heads, return_weights)


def _attention_wrong_scale(q_c, q_r, q_pos, c_kv, k_r, w_uk, w_uv,
                           heads=None, return_weights=False):
    f = math.sqrt((q_c.shape[-1] + q_r.shape[-1]) / q_c.shape[-1])
    return _real_attention(np.asarray(q_c) * f, np.asarray(q_r) * f, q_pos,
                           c_kv, k_r, w_uk, w_uv, heads, return_weights)


MUTATIONS = {
    "rope_sign": ("apply_rope", _rope_sign),
    "rope_interleaved_pairs": ("apply_rope", _rope_interleaved),
    "wrong_head_rows": ("explicit_kv", _explicit_kv_wrong_head),
    "k_v_swapped": ("explicit_kv", _explicit_kv_swapped),
    "mask_off_by_one": ("visibility", _visibility_strict),
    "k_r_not_rotated": ("kv_latent", _kv_latent_unrotated),
    "dropped_rope_term": ("attention", _attention_no_rope_term),
    "scale_sqrt_dh": ("attention", _attention_wrong_scale),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(orc, attr, fn)
    assert not _agrees(), name


# ---- latent RMSNorm: each planted mistake fails one of its pins ----------

def _norm_mean_not_rms(x, weight, eps):        # divides by the mean square
    x = np.asarray(x, float)
    return np.asarray(weight, float) * x / (np.mean(x * x, axis=-1,
                                                    keepdims=True) + eps)


def _norm_sum_not_mean(x, weight, eps):        # sum instead of mean
    x = np.asarray(x, float)
    return np.asarray(weight, float) * x / np.sqrt(
        np.sum(x * x, axis=-1, keepdims=True) + eps)


def _norm_weight_reversed(x, weight, eps):     # weight applied back to front
    x = np.asarray(x, float)
    return np.asarray(weight, float)[::-1] * x / np.sqrt(
        np.mean(x * x, axis=-1, keepdims=True) + eps)


def _norm_eps_outside(x, weight, eps):         # eps added after the root
    x = np.asarray(x, float)
    return np.asarray(weight, float) * x / (np.sqrt(
        np.mean(x * x, axis=-1, keepdims=True)) + eps)


@pytest.mark.parametrize("bad", [_norm_mean_not_rms, _norm_sum_not_mean,
                                 _norm_weight_reversed, _norm_eps_outside])
def test_rms_norm_mutation_fails_a_pin(monkeypatch, bad):
    from tests import test_oracle_pins as pins
    monkeypatch.setattr(orc, "rms_norm", bad)
    failed = 0
    for pin in (pins.test_rms_norm_closed_forms, pins.test_rms_norm_properties):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"{bad.__name__} passes every RMSNorm pin"
