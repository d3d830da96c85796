"""Planted mistakes in the oracle (CPU only): each must fail the brute-force pin.

Each mutant replaces one step of ``oracle.dit_oracle`` by a plausible wrong
version (a dropped term, a wrong sign, a wrong index or operand order) for
the duration of one test; the pin must then report a disagreement.
"""
import numpy as np
import pytest

import datagen
from oracle import bruteforce
from oracle import dit_oracle as O

_ATTN = O.gated_gqa_attention  # the unmutated step, for mutants built on it


def _norm_eps_outside(x, w, shift, scale, eps):
    x = np.asarray(x, np.float64)
    w = np.zeros(x.shape[-1]) if w is None else w
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * (1 + w) * (1 + scale) + shift


def _norm_gain_not_centred(x, w, shift, scale, eps):
    x = np.asarray(x, np.float64)
    w = np.zeros(x.shape[-1]) if w is None else w
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w * (1 + scale) + shift


def _norm_scale_not_offset(x, w, shift, scale, eps):
    x = np.asarray(x, np.float64)
    w = np.zeros(x.shape[-1]) if w is None else w
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * (1 + w) * scale + shift


def _attn_interleaved_groups(q, k, v, g):
    lq, H, d = q.shape
    Hk = k.shape[1]
    out = np.empty((lq, H, d))
    for h in range(H):
        j = h % Hk  # wrong: interleaved instead of contiguous groups
        s = q[:, h] @ k[:, j].T / np.sqrt(d)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        out[:, h] = (p @ v[:, j]) / (1 + np.exp(-g[:, h]))
    return out.reshape(lq, H * d)


def _attn_no_scale(q, k, v, g):
    return _ATTN(q * np.sqrt(q.shape[-1]), k, v, g)


def _attn_gate_missing(q, k, v, g):
    return _ATTN(q, k, v, np.full_like(np.asarray(g, float), 60.0))


def _attn_transposed_scores(q, k, v, g):
    lq, H, d = q.shape
    Hk = k.shape[1]
    out = np.empty((lq, H, d))
    for h in range(H):
        j = h // (H // Hk)
        s = (q[:, h] @ k[:, j].T / np.sqrt(d)).T  # softmax over the query axis
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        out[:, h] = (p @ v[:, j]) / (1 + np.exp(-g[:, h]))
    return out.reshape(lq, H * d)


def _resid_sign(x, gate, y):
    return np.asarray(x, float) - np.asarray(gate, float) * np.asarray(y, float)


def _swiglu_roles_swapped(h, w_13, w_2, ffn):
    h, w_13 = np.asarray(h, float), np.asarray(w_13, float)
    a, b = h @ w_13[ffn:].T, h @ w_13[:ffn].T
    return (a / (1 + np.exp(-a)) * b) @ np.asarray(w_2, float).T


def _split_order(mod_b, bias):
    v = np.asarray(mod_b, float) + np.asarray(bias, float)
    return v[1], v[0], v[2], v[3], v[4], v[5]  # shift and scale swapped


MUTANTS = {
    "eps outside sqrt": ("modulated_rmsnorm", _norm_eps_outside),
    "gain w instead of 1+w": ("modulated_rmsnorm", _norm_gain_not_centred),
    "scale instead of 1+scale": ("modulated_rmsnorm", _norm_scale_not_offset),
    "interleaved GQA groups": ("gated_gqa_attention", _attn_interleaved_groups),
    "no 1/sqrt(d)": ("gated_gqa_attention", _attn_no_scale),
    "gate dropped": ("gated_gqa_attention", _attn_gate_missing),
    "softmax over queries": ("gated_gqa_attention", _attn_transposed_scores),
    "residual sign": ("gated_residual", _resid_sign),
    "SwiGLU roles swapped": ("swiglu_mlp", _swiglu_roles_swapped),
    "modulation order": ("split_modulation", _split_order),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    cfg = datagen.Config("tiny", batch=1, n_image=5, n_text=0, hidden=8, n_heads=4, n_kv_heads=2,
                         head_dim=2, ffn=8, dtype="f32", seed=21, w_std=0.5, out_std=0.5, mod_std=1.0)
    x = datagen.activations(cfg)
    w = datagen.block_weights(cfg)
    mod = datagen.block_mod(cfg, strong=True)
    bf = np.array(bruteforce.block(x, mod, w, 4, 2, 2, 8, cfg.eps))
    oc = O.OracleConfig.of(cfg)
    good = O.block_forward(x, mod, w, oc)
    assert np.max(np.abs(good - bf)) <= 1e-12 * np.max(np.abs(bf))
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    bad = O.block_forward(x, mod, w, oc)
    # the pin tolerates 1e-12 relative; every mutant must exceed it by a wide margin
    assert np.max(np.abs(bad - bf)) > 1e-9 * np.max(np.abs(bf)), name


# ------------------------------------------------------------------ attention prologue mutants
_ROPE = O.apply_rope
_ANGLES = O.rope_angles
_POS = O.rope_positions
_QKN = O.qk_rmsnorm


def _rope_negative_turn(x, ang):
    return _ROPE(x, -np.asarray(ang))


def _rope_half_split_pairs(x, ang):  # pairs (j, j + d/2) instead of adjacent dimensions
    x = np.asarray(x, float)
    h = x.shape[-1] // 2
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    out = np.empty_like(x)
    out[..., :h] = x[..., :h] * c - x[..., h:] * s
    out[..., h:] = x[..., :h] * s + x[..., h:] * c
    return out


def _angles_axes_reversed(pos, axes, theta):
    return _ANGLES(np.asarray(pos)[:, ::-1], axes[::-1], theta)


def _angles_freq_without_2(pos, axes, theta):
    pos = np.asarray(pos, float)
    cols = [pos[:, a:a + 1] * (theta ** (-np.arange(da // 2) / da))[None, :] for a, da in enumerate(axes)]
    return np.concatenate(cols, axis=1)


def _positions_text_continue(seq_len, grid_h, grid_w):
    pos = _POS(seq_len, grid_h, grid_w)
    l = np.arange(grid_h * grid_w, seq_len)
    pos[grid_h * grid_w:, 1] = l // grid_w  # text tokens continue the raster instead of sitting at 0
    pos[grid_h * grid_w:, 2] = l % grid_w
    return pos


def _positions_grid_transposed(seq_len, grid_h, grid_w):
    pos = _POS(seq_len, grid_h, grid_w)
    l = np.arange(grid_h * grid_w)
    pos[:grid_h * grid_w, 1] = l % grid_h
    pos[:grid_h * grid_w, 2] = l // grid_h
    return pos


def _qkn_gain_not_centred(x, w, eps):
    return _QKN(x, None, eps) * (0.0 if w is None else np.asarray(w, float))


def _qkn_eps_outside(x, w, eps):
    x = np.asarray(x, float)
    w = np.zeros(x.shape[-1]) if w is None else np.asarray(w, float)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + 0.3) * (1 + w)


PRO_MUTANTS = {
    "rope turns the other way": ("apply_rope", _rope_negative_turn),
    "rope pairs half-split": ("apply_rope", _rope_half_split_pairs),
    "rope axes reversed": ("rope_angles", _angles_axes_reversed),
    "rope frequency exponent": ("rope_angles", _angles_freq_without_2),
    "text tokens not at zero": ("rope_positions", _positions_text_continue),
    "grid transposed": ("rope_positions", _positions_grid_transposed),
    "qk gain w instead of 1+w": ("qk_rmsnorm", _qkn_gain_not_centred),
    "qk eps outside sqrt": ("qk_rmsnorm", _qkn_eps_outside),
}


@pytest.mark.parametrize("name", sorted(PRO_MUTANTS))
def test_planted_prologue_mistake_is_caught(name, monkeypatch):
    cfg = datagen.Config("tiny-pro", batch=1, n_image=6, n_text=2, hidden=24, n_heads=2, n_kv_heads=1,
                         head_dim=12, ffn=16, dtype="f32", seed=23, w_std=0.5, out_std=0.5, mod_std=1.0,
                         grid_h=2, grid_w=3)
    x = datagen.activations(cfg)
    w = datagen.qk_norm_weights(cfg, datagen.block_weights(cfg))
    mod = datagen.block_mod(cfg, strong=True)
    kw = dict(qk_norm=True, rope=True, grid_h=2, grid_w=3, axes=(2, 4, 6), theta=10.0)
    bf = np.array(bruteforce.block(x, mod, w, 2, 1, 12, 16, cfg.eps, prologue=kw))
    oc = O.OracleConfig.of(cfg)
    pro = O.Prologue(**kw)
    good = O.block_forward(x, mod, w, oc, pro)
    assert np.max(np.abs(good - bf)) <= 1e-12 * np.max(np.abs(bf))
    attr, fn = PRO_MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    bad = O.block_forward(x, mod, w, oc, pro)
    assert np.max(np.abs(bad - bf)) > 1e-9 * np.max(np.abs(bf)), name
