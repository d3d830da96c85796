"""Plain float64 oracle of the Krea 2 single-stream DiT block forward.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may use it and
for the parity status of each function).  Everything is computed in numpy
float64 from float64 copies of the inputs; nothing is rounded, blocked,
fused or reordered beyond the definitions written out below.  Matrix
products use ``np.matmul`` (BLAS dgemm) as a library primitive.

Sources.  The pages are web pages about Krea 2.  The block is described on
the page "Krea 2 技术报告" (a Chinese translation of the Krea 2 technical
report), section 架构 (architecture):

* 架构 › Transformer块 -- SwiGLU MLP with 4x expansion replaces the GeLU
  MLP; grouped-query attention (GQA, the report's reference 45) with the
  sigmoid-gated attention of "Gated Attention for LLMs" (reference 47);
  single-stream block = one set of attention and MLP weights shared by
  text and image tokens, run over the joint sequence.
* 架构 › 时间步条件化 -- AdaLN-style timestep conditioning is kept, but
  the per-block MLPs that produce shift/scale/gate are replaced by a
  per-block tunable bias; sinusoidal time embeddings are named.
* 架构 › 残差设计 -- standard residual connections.
* 架构 › 归一化 -- all norms are RMSNorm (the report's reference 51),
  zero-centred, with weight decay on the learnable parameters.

The page "Krea 2: Laporan teknis model gambar open-weight 12B" (section
"Pemilihan arsitektur dan ablation") lists the same final choices.

Readings where the pages leave a step open (each is also a test):

* Modulation vector per block: mod = m[b] + bias_block, split in the order
  shift1, scale1, gate1, shift2, scale2, gate2.
* Zero-centred RMSNorm: gain (1 + w) with w stored around zero (w = 0 is
  the identity gain; weight decay pulls the gain towards 1).  Not a mean
  subtraction: that would be the LayerNorm the report replaced.
* Modulated norm: h = rmsnorm(x) * (1 + w) * (1 + scale) + shift, eps
  inside the square root.
* Gated residual: x + gate * branch (zero gates give the identity block).
* Gated attention: softmax attention per query head, then an elementwise
  sigmoid gate over the H*d output channels, computed from the same
  normalised input as Q/K/V, applied before the output projection.
* Softmax scale 1/sqrt(head_dim); query head h reads KV head
  h // (H / Hkv) (contiguous groups); no mask, no positional terms.
* No linear biases; SwiGLU: silu(h W1^T) * (h W3^T), then W2.
* Timestep map (a reading: the pages do not give the map; its arithmetic is
  pinned): e = [cos(1000 t f_i), sin(1000 t f_i)],
  f_i = 10000^(-i/(n/2)), m = W_t2 silu(W_t1 e), bias-free, shared by all
  blocks.

Optional attention prologue (``Prologue``; off in the block the benchmark
measures, which has no positional terms).  Page "Krea 2 技术报告", 架构 ›
归一化: RMSNorm is also the QKNorm; 架构 › 位置编码: 3D axial RoPE with the
head dimensions assigned to frame, height and width, RoPE indices of text
tokens set to zero (the Indonesian and Korean pages list the same).
Readings where the pages are silent:

* QKNorm: zero-centred RMSNorm over head_dim of every query and key head,
  x / sqrt(mean(x^2) + eps) * (1 + w), one gain vector w [head_dim] per
  block for queries and one for keys, shared by the heads; applied to the
  projections before RoPE, not to V or the gate.
* RoPE: head_dim split into (frame, height, width) = axes (32, 48, 48 at
  head_dim 128), each even; rotation pairs are adjacent dimensions
  (2j, 2j+1); pair i of an axis with d_a dimensions turns by
  pos_a * theta^(-2i/d_a), theta = 10000; image token l (raster order on
  the grid_h x grid_w latent grid) has position (0, l // grid_w,
  l % grid_w), text tokens (0, 0, 0).  The split, the pairing and the base
  are readings (the pages do not give them); the rotation's arithmetic is
  pinned.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Iterable, Sequence

import numpy as np

F64 = np.float64


@dataclasses.dataclass(frozen=True)
class OracleConfig:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    eps: float = 1e-6

    @classmethod
    def of(cls, cfg) -> "OracleConfig":
        """Take the model dimensions from any object that carries them."""
        return cls(cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.eps)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


# ------------------------------------------------------------------ timestep
def time_embedding(t, dim: int = 256, t_scale: float = 1000.0, max_period: float = 10000.0) -> np.ndarray:
    """Sinusoidal embedding [B, dim]: cos of the scaled time at dim/2
    geometric frequencies, then sin at the same frequencies (page
    "Krea 2 技术报告", 架构 › 时间步条件化 names sinusoidal time embeddings;
    width, scale and frequency ladder are this build's reading)."""
    t = _f64(t).reshape(-1)
    half = dim // 2
    freqs = max_period ** (-np.arange(half, dtype=F64) / half)
    arg = t_scale * t[:, None] * freqs[None, :]
    return np.concatenate([np.cos(arg), np.sin(arg)], axis=1)


def timestep_modulation(t, w_t1, w_t2, hidden: int) -> np.ndarray:
    """m = W_t2 silu(W_t1 e(t)), reshaped to [B, 6, D].  The shared map from
    t to the modulation vector is a reading (the pages do not give it);
    its arithmetic is pinned by scalar loops."""
    w_t1, w_t2 = _f64(w_t1), _f64(w_t2)
    e = time_embedding(t, dim=w_t1.shape[1])
    z = e @ w_t1.T
    m = silu(z) @ w_t2.T
    return m.reshape(-1, 6, hidden)


def split_modulation(mod_b, bias) -> tuple:
    """Per-block modulation of one sample: m[b] + block bias, split into
    shift1, scale1, gate1, shift2, scale2, gate2 (page "Krea 2 技术报告",
    架构 › 时间步条件化: per-block tunable bias instead of per-block MLP)."""
    v = _f64(mod_b) + _f64(bias)
    return tuple(v[i] for i in range(6))


# ------------------------------------------------------------------ steps
def modulated_rmsnorm(x, w, shift, scale, eps: float) -> np.ndarray:
    """Zero-centred RMSNorm with adaLN shift/scale over the last axis:
    x / sqrt(mean(x^2) + eps) * (1 + w) * (1 + scale) + shift
    (page "Krea 2 技术报告", 架构 › 归一化 and 架构 › 时间步条件化)."""
    x = _f64(x)
    w = np.zeros(x.shape[-1]) if w is None else _f64(w)
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / rms * (1.0 + w) * (1.0 + _f64(scale)) + _f64(shift)


def qkvg_projection(h, w_qkvg, oc: OracleConfig):
    """Z = h W_qkvg^T, split by columns into Q [.., H, d], K [.., Hkv, d],
    V [.., Hkv, d], G [.., H, d] (row blocks of W_qkvg: Q | K | V | G)."""
    z = _f64(h) @ _f64(w_qkvg).T
    H, Hk, d = oc.n_heads, oc.n_kv_heads, oc.head_dim
    lead = z.shape[:-1]
    q = z[..., : H * d].reshape(*lead, H, d)
    k = z[..., H * d : (H + Hk) * d].reshape(*lead, Hk, d)
    v = z[..., (H + Hk) * d : (H + 2 * Hk) * d].reshape(*lead, Hk, d)
    g = z[..., (H + 2 * Hk) * d :].reshape(*lead, H, d)
    return q, k, v, g


def gated_gqa_attention(q, k, v, g) -> np.ndarray:
    """One sample.  q, g: [Lq, H, d]; k, v: [Lk, Hkv, d].  Returns [Lq, H*d].

    For query head h with KV head j = h // (H/Hkv):
    O_h = softmax(Q_h K_j^T / sqrt(d)) V_j  (max-subtracted softmax over
    all keys, no mask, no positions), then O_h * sigmoid(G_h)
    (page "Krea 2 技术报告", 架构 › Transformer块: GQA with a sigmoid
    output gate).
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    lq, H, d = q.shape
    Hk = k.shape[1]
    group = H // Hk
    out = np.empty((lq, H, d))
    for h in range(H):
        j = h // group
        s = (q[:, h, :] @ k[:, j, :].T) / np.sqrt(d)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = (p @ v[:, j, :]) * sigmoid(g[:, h, :])
    return out.reshape(lq, H * d)


def swiglu_mlp(h, w_13, w_2, ffn: int) -> np.ndarray:
    """silu(h W1^T) * (h W3^T), then W2 (page "Krea 2 技术报告",
    架构 › Transformer块: SwiGLU, the report's reference 44).  W_13 holds
    W1 in its first ffn rows and W3 in the next ffn rows."""
    u = swiglu_hidden(h, w_13, ffn)
    return u @ _f64(w_2).T


def swiglu_hidden(h, w_13, ffn: int) -> np.ndarray:
    w_13 = _f64(w_13)
    a = _f64(h) @ w_13[:ffn].T
    b = _f64(h) @ w_13[ffn:].T
    return silu(a) * b


def gated_residual(x, gate, y) -> np.ndarray:
    """x + gate * y (page "Krea 2 技术报告", 架构 › 残差设计: standard
    residual; the adaLN gate scales the branch)."""
    return _f64(x) + _f64(gate) * _f64(y)


# ------------------------------------------------------------------ prologue
@dataclasses.dataclass(frozen=True)
class Prologue:
    """QKNorm and 3D axial RoPE in front of the attention (see the module
    docstring for the readings)."""

    qk_norm: bool = True
    rope: bool = True
    grid_h: int = 0
    grid_w: int = 0
    axes: tuple = (32, 48, 48)
    theta: float = 10000.0


def qk_rmsnorm(x, w, eps: float) -> np.ndarray:
    """Zero-centred RMSNorm over the last axis (head_dim):
    x / sqrt(mean(x^2) + eps) * (1 + w) (page "Krea 2 技术报告", 架构 ›
    归一化: RMSNorm as the QKNorm, zero-centred gain)."""
    x = _f64(x)
    w = np.zeros(x.shape[-1]) if w is None else _f64(w)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * (1.0 + w)


def rope_positions(seq_len: int, grid_h: int, grid_w: int) -> np.ndarray:
    """[L, 3] (frame, height, width) index of every token: image tokens
    first, in raster order on the grid_h x grid_w latent grid, frame 0;
    text tokens all zero (page "Krea 2 技术报告", 架构 › 位置编码)."""
    pos = np.zeros((seq_len, 3), dtype=np.int64)
    n_img = min(seq_len, grid_h * grid_w)
    l = np.arange(n_img)
    pos[:n_img, 1] = l // grid_w
    pos[:n_img, 2] = l % grid_w
    return pos


def rope_angles(pos, axes, theta: float) -> np.ndarray:
    """[L, sum(axes)/2] rotation angle of every dimension pair: the pairs of
    axis a (d_a dimensions, in the order frame, height, width) turn by
    pos[:, a] * theta^(-2i/d_a), i < d_a/2."""
    pos = np.asarray(pos, dtype=F64)
    cols = []
    for a, da in enumerate(axes):
        freq = theta ** (-np.arange(0, da, 2, dtype=F64) / da)
        cols.append(pos[:, a:a + 1] * freq[None, :])
    return np.concatenate(cols, axis=1)


def apply_rope(x, ang) -> np.ndarray:
    """Rotate the adjacent pairs (2j, 2j+1) of x [L, heads, d] by ang [L, d/2]."""
    x = _f64(x)
    c, sn = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * sn
    out[..., 1::2] = x0 * sn + x1 * c
    return out


def attention_prologue(q, k, pro: Prologue, wts, eps: float, q_rows=None):
    """QKNorm then RoPE on q [Lq, H, d] (tokens q_rows of the sample, all if
    None) and k [L, Hkv, d] (all tokens)."""
    L, d = k.shape[0], k.shape[-1]
    if pro.qk_norm:
        q = qk_rmsnorm(q, getattr(wts, "q_norm_w", None), eps)
        k = qk_rmsnorm(k, getattr(wts, "k_norm_w", None), eps)
    if pro.rope:
        assert sum(pro.axes) == d and all(a % 2 == 0 for a in pro.axes)
        ang = rope_angles(rope_positions(L, pro.grid_h, pro.grid_w), pro.axes, pro.theta)
        q = apply_rope(q, ang if q_rows is None else ang[q_rows])
        k = apply_rope(k, ang)
    return q, k


# ------------------------------------------------------------------ block
def _sample_forward(x, mod_b, wts, oc: OracleConfig, rows=None, pro: Prologue | None = None):
    """Block forward of one sample x [L, D]; outputs for ``rows`` (all if None)."""
    shift1, scale1, gate1, shift2, scale2, gate2 = split_modulation(mod_b, wts.mod_bias)
    x = _f64(x)
    h1 = modulated_rmsnorm(x, wts.norm1_w, shift1, scale1, oc.eps)
    w_qkvg = _f64(wts.w_qkvg)
    H, Hk, d = oc.n_heads, oc.n_kv_heads, oc.head_dim
    # keys and values need every token; queries and gates only the rows asked for
    kv = h1 @ w_qkvg[H * d : (H + 2 * Hk) * d].T
    k = kv[:, : Hk * d].reshape(-1, Hk, d)
    v = kv[:, Hk * d :].reshape(-1, Hk, d)
    xr = x if rows is None else x[rows]
    hr = h1 if rows is None else h1[rows]
    q = (hr @ w_qkvg[: H * d].T).reshape(-1, H, d)
    g = (hr @ w_qkvg[(H + 2 * Hk) * d :].T).reshape(-1, H, d)
    if pro is not None:
        q, k = attention_prologue(q, k, pro, wts, oc.eps, q_rows=rows)
    og = gated_gqa_attention(q, k, v, g)
    a = og @ _f64(wts.w_o).T
    x1 = gated_residual(xr, gate1, a)
    h2 = modulated_rmsnorm(x1, wts.norm2_w, shift2, scale2, oc.eps)
    mlp = swiglu_mlp(h2, wts.w_13, wts.w_2, oc.ffn)
    return gated_residual(x1, gate2, mlp)


def block_forward(x, mod, wts, oc: OracleConfig, pro: Prologue | None = None) -> np.ndarray:
    """x [B, L, D], mod [B, 6, D] -> [B, L, D]; samples are independent."""
    x = _f64(x)
    return np.stack([_sample_forward(x[b], mod[b], wts, oc, pro=pro) for b in range(x.shape[0])])


def block_forward_rows(x, mod, wts, oc: OracleConfig, b: int, rows: Sequence[int],
                       pro: Prologue | None = None) -> np.ndarray:
    """The same definition evaluated only at query tokens ``rows`` of sample b."""
    return _sample_forward(_f64(x[b]), mod[b], wts, oc, rows=np.asarray(rows), pro=pro)


def stack_forward(x, mod, weights: Iterable | Callable[[int], object], n_blocks: int,
                  oc: OracleConfig, pro: Prologue | None = None) -> np.ndarray:
    """Apply blocks 0..n_blocks-1 in order with one shared modulation m.

    ``weights`` is either a sequence of per-block weights or a function
    block index -> weights, so large stacks can be streamed one block at a
    time."""
    get = weights if callable(weights) else (lambda i, _w=list(weights): _w[i])
    y = _f64(x)
    for i in range(n_blocks):
        y = block_forward(y, mod, get(i), oc, pro)
    return y


# ------------------------------------------------------------------ boundary layers and sampler
# Page "Krea 2 技术报告": 架构 (the DiT over latent tokens of an autoencoder,
# Qwen-Image / FLUX 2 VAE, text features from Qwen3-VL); 训练 › 预训练: the
# model is trained with the standard rectified-flow loss and
# v-parameterization, and training and inference use a shifted sampling
# schedule whose inference shift is kept constant.  Readings where the
# pages are silent (conventions of the boundary layers; their arithmetic is
# pinned):
#
# * latent z [B, C, Hl, Wl]; 2 x 2 patches in raster order, patch vector
#   index c * 4 + dy * 2 + dx; image tokens first, then text tokens;
# * bias-free linear embeddings: image token = W_in p, text token = W_txt f;
# * final layer on the image tokens: zero-centred RMSNorm with adaLN
#   shift/scale (mod_f = W_tf silu(W_t1 e(t)), [B, 2, D]: shift, scale),
#   then v_patch = W_out h, unpatchified to [B, C, Hl, Wl];
# * velocity v = eps - x0 on the path z_t = (1 - t) x0 + t eps, sampled from
#   t = 1 to 0 with Euler steps z <- z + (t_next - t) v(z, t);
# * schedule t_i = s u_i / (1 + (s - 1) u_i), u_i = 1 - i / N, shift s.
def patchify(z) -> np.ndarray:
    """[B, C, Hl, Wl] -> [B, (Hl/2)(Wl/2), 4C]: 2 x 2 patches in raster order,
    vector index c * 4 + dy * 2 + dx."""
    z = _f64(z)
    B, C, Hl, Wl = z.shape
    t = z.reshape(B, C, Hl // 2, 2, Wl // 2, 2)          # b c py dy px dx
    t = t.transpose(0, 2, 4, 1, 3, 5)                    # b py px c dy dx
    return t.reshape(B, (Hl // 2) * (Wl // 2), C * 4)


def unpatchify(p, C: int, Hl: int, Wl: int) -> np.ndarray:
    """Inverse of patchify: [B, (Hl/2)(Wl/2), 4C] -> [B, C, Hl, Wl]."""
    p = _f64(p)
    B = p.shape[0]
    t = p.reshape(B, Hl // 2, Wl // 2, C, 2, 2).transpose(0, 3, 1, 4, 2, 5)
    return t.reshape(B, C, Hl, Wl)


def embed_tokens(z, txt, w_in, w_txt) -> np.ndarray:
    """Joint token sequence [B, n_img + n_txt, D]: W_in applied to the
    patches of z, then W_txt applied to the text features txt [B, n_txt, D_txt]."""
    img = patchify(z) @ _f64(w_in).T
    return np.concatenate([img, _f64(txt) @ _f64(w_txt).T], axis=1)


def final_mod(t, w_t1, w_tf, hidden: int) -> np.ndarray:
    """[B, 2, D] shift and scale of the final norm: W_tf silu(W_t1 e(t))."""
    e = time_embedding(t, dim=_f64(w_t1).shape[1])
    return (silu(e @ _f64(w_t1).T) @ _f64(w_tf).T).reshape(-1, 2, hidden)


def final_layer(x_img, modf, norm_w, w_out, eps: float) -> np.ndarray:
    """v tokens [B, n_img, 4C] = W_out (rmsnorm(x) (1 + w) (1 + scale) + shift)."""
    x_img = _f64(x_img)
    out = []
    for b in range(x_img.shape[0]):
        h = modulated_rmsnorm(x_img[b], norm_w, modf[b, 0], modf[b, 1], eps)
        out.append(h @ _f64(w_out).T)
    return np.stack(out)


def flow_schedule(n_steps: int, shift: float) -> np.ndarray:
    """n_steps + 1 times from 1 to 0: s u / (1 + (s - 1) u), u = 1 - i / n_steps."""
    u = 1.0 - np.arange(n_steps + 1, dtype=F64) / n_steps
    return shift * u / (1.0 + (shift - 1.0) * u)


def euler_sample(z, times, velocity: Callable) -> np.ndarray:
    """z <- z + (t_{i+1} - t_i) velocity(z, t_i) over the schedule."""
    z = _f64(z)
    for i in range(len(times) - 1):
        z = z + (times[i + 1] - times[i]) * velocity(z, times[i])
    return z


def model_velocity(z, t, txt, model, blocks, n_blocks: int, oc: OracleConfig, pro=None) -> np.ndarray:
    """The DiT as a velocity field: embed, the block stack with the shared
    timestep modulation, final layer, unpatchify.  ``model`` carries w_in,
    w_txt, w_t1, w_t2, w_tf, norm_f_w, w_out; t is one time for every sample."""
    B, C, Hl, Wl = np.shape(z)
    tb = np.full(B, t)
    x = embed_tokens(z, txt, model.w_in, model.w_txt)
    mod = timestep_modulation(tb, model.w_t1, model.w_t2, oc.hidden)
    y = stack_forward(x, mod, blocks, n_blocks, oc, pro)
    n_img = (Hl // 2) * (Wl // 2)
    v = final_layer(y[:, :n_img], final_mod(tb, model.w_t1, model.w_tf, oc.hidden), model.norm_f_w,
                    model.w_out, oc.eps)
    return unpatchify(v, C, Hl, Wl)


def guided_velocity(z, t, txt, txt_null, guidance: float, model, blocks, n_blocks: int, oc: OracleConfig,
                    pro=None) -> np.ndarray:
    """Classifier-free guidance (page "Krea 2 技术报告", 训练 › 强化学习: an
    optional control at inference; the guidance of Ho and Salimans cited
    there): v = v_u + g (v_c - v_u), with v_c the velocity under the text
    features txt and v_u under txt_null (the caller's unconditional
    features).  g = 1 is the conditional velocity, g = 0 the unconditional."""
    vc = model_velocity(z, t, txt, model, blocks, n_blocks, oc, pro)
    vu = model_velocity(z, t, txt_null, model, blocks, n_blocks, oc, pro)
    return vu + guidance * (vc - vu)


# ------------------------------------------------------------------ 8-bit projections
# Page "Krea 2 技术报告", 训练 › 预训练 (and the Indonesian / Korean pages):
# 8-bit training ran 15-20 % faster than bf16, with tensor-wise scaling at
# 256 px and row-wise scaling at 512 px.  Here the 8-bit format is OCP FP8
# e4m3 (largest finite 448) with row-wise scales for both operands of a
# projection: a row (one token of A, one output channel of W) is divided by
# s = amax(row) / 448 before rounding to the nearest e4m3 value (ties to
# even).  The scale and the division are float32 operations so that both
# implementations take the same rounding decisions; the product is then
#   C[m, n] = sa[m] sw[n] sum_k qa[m, k] qw[n, k].
FP8_MAX = 448.0


def fp8_e4m3_round(y) -> np.ndarray:
    """Nearest OCP e4m3 (3 mantissa bits, exponent bias 7, subnormal step
    2^-9, largest finite 448) to each value, ties to the even mantissa.
    Inputs must lie within [-464, 464] (they round to at most 448)."""
    y = _f64(y)
    a = np.abs(y)
    assert np.all(a <= 464.0), "outside the e4m3 range"
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex - 1, -6)              # binade; below 2^-6 the subnormal spacing
    step = np.ldexp(1.0, e - 3)             # 3 mantissa bits
    q = np.round(a / step) * step           # numpy rounds halves to even
    return np.sign(y) * q


def quantize_rows_fp8(x):
    """Row-wise FP8 quantisation of x [m, k] (values exact in float32):
    returns (q [m, k] float64 holding e4m3 values, s [m] float32) with
    x ~ q * s.  amax = max |x| per row; s = amax / 448 and the quotient
    x * (448 / amax) in float32; an all-zero row gets s = 1, q = 0."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1)
    zero = amax == 0
    safe = np.where(zero, np.float32(1), amax).astype(np.float32)
    s = np.where(zero, np.float32(1), safe / np.float32(FP8_MAX)).astype(np.float32)
    inv = (np.float32(FP8_MAX) / safe).astype(np.float32)
    y = (x32 * inv[:, None]).astype(np.float32)
    q = fp8_e4m3_round(y)
    q[zero] = 0.0
    return q, s


def quantize_tensor_fp8(x):
    """Tensor-wise FP8 quantisation (the pages' 256 px scheme): one scale for
    all of x, s = amax(x) / 448, the quotient in float32 as in
    quantize_rows_fp8; returned per row (every row the same) so the same
    product serves both schemes."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32)))
    if amax == 0:
        return np.zeros(x32.shape), np.ones(x32.shape[0], dtype=np.float32)
    s = np.float32(amax / np.float32(FP8_MAX))
    inv = np.float32(np.float32(FP8_MAX) / amax)
    q = fp8_e4m3_round((x32 * inv).astype(np.float32))
    return q, np.full(x32.shape[0], s, dtype=np.float32)


def gemm_fp8(qa, sa, qw, sw) -> np.ndarray:
    """C = (qa qw^T) * sa[:, None] * sw[None, :] in float64."""
    return (_f64(qa) @ _f64(qw).T) * _f64(sa)[:, None] * _f64(sw)[None, :]


def swiglu_fp8(qa, sa, qw13, sw13, ffn: int) -> np.ndarray:
    """SiLU(A W1^T) * (A W3^T) with both halves of W13 = [W1; W3] in FP8."""
    c = gemm_fp8(qa, sa, qw13, sw13)
    return silu(c[:, :ffn]) * c[:, ffn:]


def _quant_identity(x):
    """No quantisation: q = x, s = 1 (the composition then equals the exact
    block; used to pin its wiring)."""
    x = _f64(x)
    return x, np.ones(x.shape[0])


def block_forward_fp8(x, mod, wts, oc: OracleConfig, quant: Callable = quantize_rows_fp8) -> np.ndarray:
    """The block with its four projections in 8 bits (page "Krea 2 技术报告",
    训练 › 预训练: 8-bit matrix products with row-wise scaling): every
    product's activation rows and weight rows are quantised with ``quant``
    (row-wise e4m3 by default: one float32 scale per token row and per weight
    row) and multiplied as gemm_fp8 / swiglu_fp8 do; everything else is the
    exact block of _sample_forward.  The activations are quantised from their
    exact values (h1, Og, h2, U of this oracle)."""
    H, Hk, d, F = oc.n_heads, oc.n_kv_heads, oc.head_dim, oc.ffn
    qw = {n: quant(getattr(wts, n)) for n in ("w_qkvg", "w_o", "w_13", "w_2")}

    def prod(a, name):
        qa, sa = quant(a)
        return gemm_fp8(qa, sa, *qw[name])

    out = []
    for b in range(_f64(x).shape[0]):
        xb = _f64(x[b])
        shift1, scale1, gate1, shift2, scale2, gate2 = split_modulation(mod[b], wts.mod_bias)
        h1 = modulated_rmsnorm(xb, wts.norm1_w, shift1, scale1, oc.eps)
        z = prod(h1, "w_qkvg")
        L = z.shape[0]
        q = z[:, : H * d].reshape(L, H, d)
        k = z[:, H * d:(H + Hk) * d].reshape(L, Hk, d)
        v = z[:, (H + Hk) * d:(H + 2 * Hk) * d].reshape(L, Hk, d)
        g = z[:, (H + 2 * Hk) * d:].reshape(L, H, d)
        og = gated_gqa_attention(q, k, v, g)
        x1 = gated_residual(xb, gate1, prod(og, "w_o"))
        h2 = modulated_rmsnorm(x1, wts.norm2_w, shift2, scale2, oc.eps)
        qa, sa = quant(h2)
        u = swiglu_fp8(qa, sa, *qw["w_13"], F)
        out.append(gated_residual(x1, gate2, prod(u, "w_2")))
    return np.stack(out)


def stack_forward_fp8(x, mod, weights: Iterable | Callable[[int], object], n_blocks: int, oc: OracleConfig,
                      quant: Callable = quantize_rows_fp8) -> np.ndarray:
    """The stack of stack_forward with every block the 8-bit block of
    block_forward_fp8 (the residual stream exact between blocks)."""
    get = weights if callable(weights) else (lambda i, _w=list(weights): _w[i])
    y = _f64(x)
    for i in range(n_blocks):
        y = block_forward_fp8(y, mod, get(i), oc, quant)
    return y
