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
