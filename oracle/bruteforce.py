"""Scalar-loop brute force of the DiT block -- TEST INFRASTRUCTURE ONLY.

An independent second statement of the same readings as ``dit_oracle``
(page "Krea 2 技术报告", section 架构): pure Python floats, explicit
loops, the ``math`` module, no numpy in the arithmetic.  It is only fast
enough for tiny shapes (D <= 16, L <= 8) and exists to pin the vectorised
oracle: a transposed operand, a wrong head group, a dropped term or a
wrong sign in either shows up as a disagreement.
"""
from __future__ import annotations

import math


def _rows(a):
    return [[float(v) for v in row] for row in a]


def _vec(a):
    return [float(v) for v in a]


def _prologue_row(vec, gain, pos, qk_norm, rope, axes, theta, eps):
    """One head vector of one token: zero-centred RMSNorm, then the pairs
    (2j, 2j+1) turned by pos[axis] * theta^(-2i/d_axis)."""
    d = len(vec)
    v = list(vec)
    if qk_norm:
        ss = 0.0
        for c in range(d):
            ss += v[c] * v[c]
        inv = 1.0 / math.sqrt(ss / d + eps)
        v = [v[c] * inv * (1.0 + (gain[c] if gain is not None else 0.0)) for c in range(d)]
    if rope:
        out = list(v)
        j = 0
        for a, da in enumerate(axes):
            for i in range(da // 2):
                ang = pos[a] * theta ** (-(2.0 * i) / da)
                c0, c1 = v[2 * j], v[2 * j + 1]
                out[2 * j] = c0 * math.cos(ang) - c1 * math.sin(ang)
                out[2 * j + 1] = c0 * math.sin(ang) + c1 * math.cos(ang)
                j += 1
        v = out
    return v


def block(x, mod, wts, n_heads, n_kv_heads, head_dim, ffn, eps, prologue=None):
    """x: nested lists [B][L][D]; mod [B][6][D]; wts has the same fields as
    ``datagen.BlockWeights``.  prologue: None, or a dict with keys qk_norm,
    rope, grid_h, grid_w, axes, theta (QKNorm and 3D axial RoPE on Q and K;
    image tokens first in raster order, text tokens at position 0).
    Returns nested lists [B][L][D]."""
    w_qkvg = _rows(wts.w_qkvg)
    w_o = _rows(wts.w_o)
    w_13 = _rows(wts.w_13)
    w_2 = _rows(wts.w_2)
    bias = _rows(wts.mod_bias)
    n1 = _vec(wts.norm1_w)
    n2 = _vec(wts.norm2_w)
    out = []
    for b in range(len(x)):
        xs = _rows(x[b])
        L, D = len(xs), len(xs[0])
        m = [[float(mod[b][i][c]) + bias[i][c] for c in range(D)] for i in range(6)]

        def norm(row, gain, shift, scale):
            ss = 0.0
            for c in range(D):
                ss += row[c] * row[c]
            inv = 1.0 / math.sqrt(ss / D + eps)
            return [row[c] * inv * (1.0 + gain[c]) * (1.0 + scale[c]) + shift[c] for c in range(D)]

        def lin(row, w):  # y_o = sum_i row_i * w[o][i]
            res = []
            for o in range(len(w)):
                acc = 0.0
                wr = w[o]
                for i in range(len(row)):
                    acc += row[i] * wr[i]
                res.append(acc)
            return res

        h1 = [norm(xs[t], n1, m[0], m[1]) for t in range(L)]
        z = [lin(h1[t], w_qkvg) for t in range(L)]
        H, Hk, d = n_heads, n_kv_heads, head_dim
        if prologue is not None:
            gq = getattr(wts, "q_norm_w", None)
            gk = getattr(wts, "k_norm_w", None)
            gq = None if gq is None else _vec(gq)
            gk = None if gk is None else _vec(gk)
            gw = prologue["grid_w"]
            n_img = prologue["grid_h"] * gw
            for t in range(L):
                pos = (0, t // gw, t % gw) if t < n_img else (0, 0, 0)
                for hh in range(H + Hk):  # query heads, then key heads
                    lo = hh * d
                    z[t][lo:lo + d] = _prologue_row(z[t][lo:lo + d], gq if hh < H else gk, pos,
                                                    prologue["qk_norm"], prologue["rope"], prologue["axes"],
                                                    prologue["theta"], eps)
        og = [[0.0] * (H * d) for _ in range(L)]
        for h in range(H):
            j = (h * Hk) // H  # contiguous groups of H/Hk query heads
            for t in range(L):
                q = z[t][h * d:(h + 1) * d]
                scores = []
                for u in range(L):
                    kk = z[u][H * d + j * d:H * d + (j + 1) * d]
                    s = 0.0
                    for c in range(d):
                        s += q[c] * kk[c]
                    scores.append(s / math.sqrt(d))
                mx = max(scores)
                e = [math.exp(s - mx) for s in scores]
                tot = sum(e)
                for c in range(d):
                    o = 0.0
                    for u in range(L):
                        o += e[u] / tot * z[u][(H + Hk) * d + j * d + c]
                    gl = z[t][(H + 2 * Hk) * d + h * d + c]
                    og[t][h * d + c] = o * (1.0 / (1.0 + math.exp(-gl)))
        x1 = []
        for t in range(L):
            a = lin(og[t], w_o)
            x1.append([xs[t][c] + m[2][c] * a[c] for c in range(D)])
        res = []
        for t in range(L):
            h2 = norm(x1[t], n2, m[3], m[4])
            up = lin(h2, w_13)
            u = []
            for f in range(ffn):
                g1 = up[f]
                u.append(g1 / (1.0 + math.exp(-g1)) * up[ffn + f])
            mm = lin(u, w_2)
            res.append([x1[t][c] + m[5][c] * mm[c] for c in range(D)])
        out.append(res)
    return out


def time_embedding(t, dim=256):
    half = dim // 2
    res = []
    for tv in t:
        row_c, row_s = [], []
        for i in range(half):
            f = 10000.0 ** (-i / half)
            row_c.append(math.cos(1000.0 * float(tv) * f))
            row_s.append(math.sin(1000.0 * float(tv) * f))
        res.append(row_c + row_s)
    return res
