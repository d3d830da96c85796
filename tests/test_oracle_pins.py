"""Pins of the fp64 oracle against things other than itself (CPU only).

* an independent scalar-loop brute force on tiny shapes;
* torch's own float64 CPU routines (rms_norm, linear,
  scaled_dot_product_attention, silu, sigmoid) composed per the readings;
* closed forms and invariants the definitions fix.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import datagen
from oracle import bruteforce
from oracle import dit_oracle as O


def tiny_cfg(batch=1, L=5, hkv=2, seed=7, D=8, H=2, d=4, ffn=8):
    return datagen.Config("tiny", batch=batch, n_image=L, n_text=0, hidden=D, n_heads=H,
                          n_kv_heads=hkv, head_dim=d, ffn=ffn, dtype="f32", seed=seed,
                          w_std=0.5, out_std=0.5, mod_std=1.0)


def inputs(cfg, strong=True):
    x = datagen.activations(cfg)
    w = datagen.block_weights(cfg, 0)
    mod = datagen.block_mod(cfg, strong=strong)
    return x, w, mod


def oc(cfg):
    return O.OracleConfig.of(cfg)


# ------------------------------------------------------------------ brute force
@pytest.mark.parametrize("batch", [1, 2])
@pytest.mark.parametrize("L", [1, 2, 3, 5, 7])
@pytest.mark.parametrize("hkv", [1, 2])
def test_block_matches_bruteforce(batch, L, hkv):
    cfg = tiny_cfg(batch=batch, L=L, hkv=hkv, seed=100 + 10 * L + hkv)
    x, w, mod = inputs(cfg)
    ref = O.block_forward(x, mod, w, oc(cfg))
    bf = np.array(bruteforce.block(x, mod, w, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.eps))
    assert np.max(np.abs(ref - bf)) <= 1e-12 * max(1.0, np.max(np.abs(bf)))
    # the update itself (not just x + small) must agree as well
    dref, dbf = ref - x, bf - x
    assert np.max(np.abs(dref - dbf)) <= 1e-12 * max(1.0, np.max(np.abs(dbf)))
    assert np.max(np.abs(dbf)) > 1e-2  # the block did real work


def test_bruteforce_four_heads_two_groups():
    cfg = tiny_cfg(batch=1, L=4, hkv=2, H=4, D=16, d=4, ffn=12, seed=5)
    x, w, mod = inputs(cfg)
    ref = O.block_forward(x, mod, w, oc(cfg))
    bf = np.array(bruteforce.block(x, mod, w, 4, 2, 4, 12, cfg.eps))
    assert np.max(np.abs(ref - bf)) <= 1e-12 * np.max(np.abs(bf))


def test_time_embedding_matches_bruteforce():
    t = np.array([0.0, 0.25, 0.731, 1.0])
    ref = O.time_embedding(t, 256)
    bf = np.array(bruteforce.time_embedding(t, 256))
    assert np.max(np.abs(ref - bf)) <= 1e-9  # arguments up to 1000 rad


# ------------------------------------------------------------------ torch library routines
def torch_block(x, mod, w, cfg):
    """The block composed of torch float64 CPU library routines."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    X, M = t(x), t(mod)
    bias = t(w.mod_bias)
    H, Hk, d, D, Fn = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden, cfg.ffn
    out = []
    for b in range(X.shape[0]):
        m = M[b] + bias
        xb = X[b]
        h1 = F.rms_norm(xb, (D,), weight=1 + t(w.norm1_w), eps=cfg.eps) * (1 + m[1]) + m[0]
        z = F.linear(h1, t(w.w_qkvg))
        q = z[:, : H * d].reshape(-1, H, d).transpose(0, 1)
        k = z[:, H * d:(H + Hk) * d].reshape(-1, Hk, d).transpose(0, 1)
        v = z[:, (H + Hk) * d:(H + 2 * Hk) * d].reshape(-1, Hk, d).transpose(0, 1)
        g = z[:, (H + 2 * Hk) * d:]
        k = k.repeat_interleave(H // Hk, dim=0)
        v = v.repeat_interleave(H // Hk, dim=0)
        o = F.scaled_dot_product_attention(q[None], k[None], v[None])[0]
        o = o.transpose(0, 1).reshape(-1, H * d) * torch.sigmoid(g)
        x1 = xb + m[2] * F.linear(o, t(w.w_o))
        h2 = F.rms_norm(x1, (D,), weight=1 + t(w.norm2_w), eps=cfg.eps) * (1 + m[4]) + m[3]
        up = F.linear(h2, t(w.w_13))
        u = F.silu(up[:, :Fn]) * up[:, Fn:]
        out.append(x1 + m[5] * F.linear(u, t(w.w_2)))
    return torch.stack(out).numpy()


@pytest.mark.parametrize("name", ["c0"])
@pytest.mark.parametrize("strong", [False, True])
def test_block_matches_torch_routines(name, strong):
    cfg = datagen.get_config(name).replace(batch=2)
    x, w, mod = inputs(cfg, strong=strong)
    ref = O.block_forward(x, mod, w, oc(cfg))
    lib = torch_block(x, mod, w, cfg)
    assert np.max(np.abs(ref - lib)) <= 1e-12 * np.max(np.abs(lib))
    d1, d2 = ref - x, lib - x
    assert np.max(np.abs(d1 - d2)) <= 1e-11 * np.max(np.abs(d2))


def test_attention_matches_sdpa_gqa():
    rng = np.random.default_rng(3)
    L, H, Hk, d = 37, 8, 2, 16
    q, g = rng.standard_normal((L, H, d)), rng.standard_normal((L, H, d))
    k, v = rng.standard_normal((L, Hk, d)), rng.standard_normal((L, Hk, d))
    ref = O.gated_gqa_attention(q, k, v, g).reshape(L, H, d)
    T = lambda a: torch.as_tensor(a).transpose(0, 1)[None]
    o = F.scaled_dot_product_attention(T(q), T(k), T(v), enable_gqa=True)[0].transpose(0, 1)
    lib = o.numpy() * (1 / (1 + np.exp(-g)))
    assert np.max(np.abs(ref - lib)) <= 1e-13


# ------------------------------------------------------------------ closed forms / invariants
def test_one_key_returns_gated_value():
    rng = np.random.default_rng(1)
    q, g = rng.standard_normal((1, 4, 8)), rng.standard_normal((1, 4, 8))
    k, v = rng.standard_normal((1, 2, 8)), rng.standard_normal((1, 2, 8))
    og = O.gated_gqa_attention(q, k, v, g).reshape(1, 4, 8)
    for h in range(4):
        np.testing.assert_allclose(og[0, h], v[0, h // 2] / (1 + np.exp(-g[0, h])), rtol=0, atol=1e-15)


def test_two_keys_weights_are_logistic():
    rng = np.random.default_rng(2)
    d = 16
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((2, 1, d))
    v = rng.standard_normal((2, 1, d))
    g = np.full((1, 1, d), 50.0)  # sigmoid(50) = 1 - 2e-22 -> 1 in fp64
    s = k[:, 0, :] @ q[0, 0] / math.sqrt(d)
    w0 = 1 / (1 + math.exp(-(s[0] - s[1])))
    expect = w0 * v[0, 0] + (1 - w0) * v[1, 0]
    np.testing.assert_allclose(O.gated_gqa_attention(q, k, v, g)[0], expect, rtol=0, atol=1e-14)


def test_identical_keys_give_mean_value():
    rng = np.random.default_rng(4)
    L, d = 9, 8
    q = rng.standard_normal((L, 2, d))
    k = np.repeat(rng.standard_normal((1, 1, d)), L, axis=0)
    v = rng.standard_normal((L, 1, d))
    g = np.full((L, 2, d), 60.0)
    og = O.gated_gqa_attention(q, k, v, g).reshape(L, 2, d)
    np.testing.assert_allclose(og, np.broadcast_to(v.mean(axis=0)[None], (L, 2, d)), atol=1e-14)


def test_gqa_equals_mha_with_replicated_kv():
    cfg = tiny_cfg(batch=2, L=6, hkv=2, H=4, D=16, d=4, ffn=12, seed=9)
    x, w, mod = inputs(cfg)
    ref = O.block_forward(x, mod, w, oc(cfg))
    H, Hk, d = 4, 2, 4
    wq = w.w_qkvg
    q_rows, k_rows = wq[: H * d], wq[H * d:(H + Hk) * d]
    v_rows, g_rows = wq[(H + Hk) * d:(H + 2 * Hk) * d], wq[(H + 2 * Hk) * d:]
    rep = lambda r: np.concatenate([r[(h // (H // Hk)) * d:(h // (H // Hk) + 1) * d] for h in range(H)])
    w_mha = datagen.BlockWeights(np.concatenate([q_rows, rep(k_rows), rep(v_rows), g_rows]),
                                 w.w_o, w.w_13, w.w_2, w.mod_bias, w.norm1_w, w.norm2_w)
    mha = O.block_forward(x, mod, w_mha, oc(cfg.replace(n_kv_heads=4)))
    assert np.max(np.abs(ref - mha)) <= 1e-13 * np.max(np.abs(ref))


def test_group_size_one_is_mha_per_head():
    rng = np.random.default_rng(5)
    L, H, d = 7, 3, 8
    q, k, v, g = (rng.standard_normal((L, H, d)) for _ in range(4))
    og = O.gated_gqa_attention(q, k, v, g).reshape(L, H, d)
    for h in range(H):
        s = q[:, h] @ k[:, h].T / math.sqrt(d)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(og[:, h], (p @ v[:, h]) / (1 + np.exp(-g[:, h])), atol=1e-14)


def test_zero_gates_make_block_identity():
    cfg = datagen.get_config("c0")
    x, w, mod = inputs(cfg)
    mod = mod.copy()
    w.mod_bias = w.mod_bias.copy()
    for i in (2, 5):
        mod[:, i, :] = 0
        w.mod_bias[i] = 0
    np.testing.assert_array_equal(O.block_forward(x, mod, w, oc(cfg)), x.astype(np.float64))


def test_gate_logits_to_minus_inf_zero_the_attention_branch():
    cfg = tiny_cfg(batch=1, L=5, hkv=1, seed=11)
    x, w, mod = inputs(cfg)
    H, Hk, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    w.w_qkvg = w.w_qkvg.copy()
    w.w_qkvg[(H + 2 * Hk) * d:] = 0
    oc_ = oc(cfg)
    # with G = -inf the attention output is exactly zero, so x1 = x
    q, k, v, g = O.qkvg_projection(np.ones((5, cfg.hidden)), w.w_qkvg, oc_)
    with np.errstate(over="ignore"):
        og = O.gated_gqa_attention(q, k, v, np.full_like(g, -1e4))
    assert np.all(og == 0)
    # and gate1 = 0 gives the same x1: compare two blocks that differ only in W_o
    mod2 = mod.copy()
    mod2[:, 2, :] = -w.mod_bias[2]
    w_b = datagen.BlockWeights(w.w_qkvg, w.w_o * 3.0, w.w_13, w.w_2, w.mod_bias, w.norm1_w, w.norm2_w)
    np.testing.assert_array_equal(O.block_forward(x, mod2, w, oc_), O.block_forward(x, mod2, w_b, oc_))


def test_scale_minus_one_gives_shift():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 32))
    shift = rng.standard_normal(32)
    h = O.modulated_rmsnorm(x, rng.standard_normal(32), shift, -np.ones(32), 1e-6)
    np.testing.assert_array_equal(h, np.broadcast_to(shift, h.shape))


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 64)) * 3.0
    z = np.zeros(64)
    h = O.modulated_rmsnorm(x, None, z, z, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(h * h, axis=1)), 1.0, atol=1e-14)
    np.testing.assert_allclose(O.modulated_rmsnorm(5.5 * x, None, z, z, 0.0), h, atol=1e-14)
    # eps sits inside the square root: a zero row stays finite and maps to shift
    shift = rng.standard_normal(64)
    np.testing.assert_array_equal(O.modulated_rmsnorm(np.zeros((1, 64)), None, shift, z, 1e-6)[0], shift)
    # the zero-centred gain: w multiplies as (1 + w)
    w = rng.standard_normal(64)
    np.testing.assert_allclose(O.modulated_rmsnorm(x, w, z, z, 0.0), h * (1 + w), atol=1e-14)
    np.testing.assert_allclose(np.sqrt(np.mean(x[:1] ** 2)) * h[0], x[0], atol=1e-13)


def test_swiglu_zero_w1_is_zero_and_scalar_formula():
    rng = np.random.default_rng(8)
    h = rng.standard_normal((3, 8))
    w13 = rng.standard_normal((10, 8))
    w2 = rng.standard_normal((8, 5))
    z13 = w13.copy()
    z13[:5] = 0
    assert np.all(O.swiglu_mlp(h, z13, w2, 5) == 0)
    u = O.swiglu_hidden(h, w13, 5)
    for r in range(3):
        for f in range(5):
            a = float(h[r] @ w13[f])
            b = float(h[r] @ w13[5 + f])
            assert abs(u[r, f] - a / (1 + math.exp(-a)) * b) <= 1e-13


def test_permutation_equivariance_and_batch_independence():
    cfg = datagen.get_config("c0").replace(batch=2)
    x, w, mod = inputs(cfg, strong=True)
    ref = O.block_forward(x, mod, w, oc(cfg))
    perm = np.random.default_rng(9).permutation(cfg.seq_len)
    per = O.block_forward(x[:, perm], mod, w, oc(cfg))
    assert np.max(np.abs(per - ref[:, perm])) <= 1e-12 * np.max(np.abs(ref))
    one = O.block_forward(x[1:2], mod[1:2], w, oc(cfg))
    np.testing.assert_array_equal(one[0], ref[1])


def test_rows_and_stack_agree_with_block():
    cfg = datagen.get_config("c0").replace(batch=2)
    x, w, mod = inputs(cfg, strong=True)
    ref = O.block_forward(x, mod, w, oc(cfg))
    rows = [0, 17, 63, 64, 79]
    r = O.block_forward_rows(x, mod, w, oc(cfg), 1, rows)
    assert np.max(np.abs(r - ref[1, rows])) <= 1e-13 * np.max(np.abs(ref))
    w1 = datagen.block_weights(cfg, 1)
    two = O.stack_forward(x, mod, [w, w1], 2, oc(cfg))
    np.testing.assert_array_equal(two, O.block_forward(ref, mod, w1, oc(cfg)))


def test_time_embedding_closed_forms():
    e = O.time_embedding([0.0], 256)[0]
    np.testing.assert_array_equal(e, np.r_[np.ones(128), np.zeros(128)])
    # lowest-index frequency is 1 rad per unit of scaled time: t = pi/1000 gives cos = -1
    e = O.time_embedding([math.pi / 1000], 256)[0]
    assert abs(e[0] + 1) < 1e-15 and abs(e[128]) < 1e-15
    # the frequency ladder is geometric down to 10000^(-127/128); at i = 64, f = 1e-2
    t = 0.5 * math.pi / 1000 / 1e-2
    e = O.time_embedding([t], 256)[0]
    assert abs(e[64]) < 1e-12 and abs(e[128 + 64] - 1) < 1e-12
    e = O.time_embedding(np.linspace(0, 1, 11), 256)
    np.testing.assert_allclose(e[:, :128] ** 2 + e[:, 128:] ** 2, 1.0, atol=1e-15)


def test_timestep_modulation_structure():
    rng = np.random.default_rng(10)
    D = 16
    t = np.array([0.3, 0.9])
    w1 = rng.standard_normal((D, 256)) * 0.1
    w2 = rng.standard_normal((6 * D, D)) * 0.1
    m = O.timestep_modulation(t, w1, w2, D)
    assert m.shape == (2, 6, D)
    e = np.array(bruteforce.time_embedding(t, 256))
    z = np.array([[sum(w1[r, c] * e[b, c] for c in range(256)) for r in range(D)] for b in range(2)])
    s = z / (1 + np.exp(-z))
    expect = np.array([[sum(w2[o, r] * s[b, r] for r in range(D)) for o in range(6 * D)] for b in range(2)])
    np.testing.assert_allclose(m.reshape(2, -1), expect, atol=1e-12)
    assert np.all(O.timestep_modulation(t, w1, np.zeros_like(w2), D) == 0)


def test_parameter_count_pins_elementwise_gate():
    """An elementwise sigmoid gate (H*d extra output rows of W_qkvg) gives the
    ~11.7B parameters of the 60-block stack; the 12B model of the page
    "Krea 2: Laporan teknis model gambar open-weight 12B" (title)."""
    c4 = datagen.get_config("c4")
    stack = c4.n_blocks * c4.block_params()
    assert abs(stack - 11.64e9) < 0.01e9
    total = stack + c4.timestep_params()
    assert abs(total - 11.74e9) < 0.01e9
    assert abs(2 * stack / 1e9 - 23.28) < 0.01  # bf16 bytes of the block weights
    # a per-head gate (H outputs instead of H*d) would give ~10.7B: not ~11.7B
    per_head = stack - c4.n_blocks * (c4.n_heads * c4.head_dim - c4.n_heads) * c4.hidden
    assert per_head < 10.8e9
    # SwiGLU width: 2/3 * 4 * D rounded up to a multiple of 256
    assert c4.ffn == int(math.ceil(2 / 3 * 4 * 4096 / 256) * 256)
    assert datagen.get_config("c0").ffn == int(math.ceil(2 / 3 * 4 * 256 / 16) * 16)


# ------------------------------------------------------------------ attention prologue
def prologue_cfg(batch=1, n_image=6, n_text=2, hkv=1, seed=3, gh=2, gw=3):
    return datagen.Config("tiny-pro", batch=batch, n_image=n_image, n_text=n_text, hidden=24, n_heads=2,
                          n_kv_heads=hkv, head_dim=12, ffn=16, dtype="f32", seed=seed, w_std=0.5,
                          out_std=0.5, mod_std=1.0, grid_h=gh, grid_w=gw)


@pytest.mark.parametrize("qk_norm,rope", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("batch,hkv", [(1, 1), (2, 2)])
def test_prologue_matches_bruteforce(qk_norm, rope, batch, hkv):
    """QKNorm + 3D axial RoPE in the block: vectorised oracle = scalar loops,
    text tokens after the image grid, two heads per KV group or one."""
    cfg = prologue_cfg(batch=batch, hkv=hkv, seed=40 + batch + hkv)
    x = datagen.activations(cfg)
    w = datagen.qk_norm_weights(cfg, datagen.block_weights(cfg))
    mod = datagen.block_mod(cfg, strong=True)
    pro = O.Prologue(qk_norm=qk_norm, rope=rope, grid_h=2, grid_w=3, axes=(2, 4, 6), theta=10.0)
    ref = O.block_forward(x, mod, w, oc(cfg), pro)
    bf = np.array(bruteforce.block(x, mod, w, 2, hkv, 12, 16, cfg.eps,
                                   prologue=dict(qk_norm=qk_norm, rope=rope, grid_h=2, grid_w=3,
                                                 axes=(2, 4, 6), theta=10.0)))
    assert np.max(np.abs(ref - bf)) <= 1e-12 * np.max(np.abs(bf))
    assert np.max(np.abs(ref - O.block_forward(x, mod, w, oc(cfg)))) > 1e-3  # the prologue did something


def test_rope_closed_form_one_pair():
    """A unit vector on the first dimension of height pair i = 1 (axes
    (4, 4, 4), theta 100) at height position 3 turns by 3 * 100^(-2/4) = 0.3
    rad into that pair: (cos 0.3, sin 0.3), nothing elsewhere."""
    x = np.zeros((1, 1, 12))
    x[0, 0, 6] = 1.0  # pairs: frame 0,1 | height 2,3 | width 4,5 -> dims 6,7 = height pair i = 1
    ang = O.rope_angles(np.array([[0, 3, 5]]), (4, 4, 4), 100.0)
    y = O.apply_rope(x, ang)[0, 0]
    want = np.zeros(12)
    want[6], want[7] = math.cos(0.3), math.sin(0.3)
    assert np.max(np.abs(y - want)) < 1e-15
    # width pair i = 0 at position 5 turns by 5 rad
    assert abs(ang[0, 4] - 5.0) < 1e-15 and abs(ang[0, 5] - 5.0 * 0.1) < 1e-15
    assert ang[0, 0] == 0.0 and ang[0, 1] == 0.0  # frame axis: position 0


def test_rope_scores_depend_on_position_differences():
    """Along any one axis, <rope(q, p), rope(k, p')> depends only on p - p'
    (the defining property of rotary embeddings); norms are kept."""
    r = np.random.default_rng(5)
    q, k = r.standard_normal((1, 1, 16)), r.standard_normal((1, 1, 16))
    axes = (4, 6, 6)
    for axis in (1, 2):
        def score(pq, pk):
            a = np.zeros((1, 3)); a[0, axis] = pq
            b = np.zeros((1, 3)); b[0, axis] = pk
            return float(np.sum(O.apply_rope(q, O.rope_angles(a, axes, 10000.0)) *
                                O.apply_rope(k, O.rope_angles(b, axes, 10000.0))))
        for pq, pk in ((0, 3), (7, 2), (40, 41)):
            for delta in (1, 5, 23):
                assert abs(score(pq, pk) - score(pq + delta, pk + delta)) < 1e-12
        a = np.zeros((1, 3)); a[0, axis] = 13
        y = O.apply_rope(q, O.rope_angles(a, axes, 10000.0))
        assert abs(np.linalg.norm(y) - np.linalg.norm(q)) < 1e-12
        pairs_in, pairs_out = q[0, 0].reshape(-1, 2), y[0, 0].reshape(-1, 2)
        assert np.allclose(np.linalg.norm(pairs_in, axis=1), np.linalg.norm(pairs_out, axis=1), atol=1e-13)


def test_rope_positions_text_and_origin_unchanged():
    """Image tokens in raster order (row l // grid_w, column l % grid_w), frame
    0; text tokens at (0, 0, 0); the rotation leaves position 0 alone."""
    pos = O.rope_positions(14, 3, 4)
    assert pos[5].tolist() == [0, 1, 1] and pos[11].tolist() == [0, 2, 3]
    assert (pos[12:] == 0).all() and (pos[0] == 0).all() and (pos[:, 0] == 0).all()
    x = np.random.default_rng(1).standard_normal((14, 2, 12))
    y = O.apply_rope(x, O.rope_angles(pos, (4, 4, 4), 10000.0))
    assert np.array_equal(y[12:], x[12:]) and np.array_equal(y[0], x[0])
    assert not np.allclose(y[5], x[5])


def test_qk_norm_is_torch_rms_norm():
    """QKNorm = torch's float64 rms_norm over head_dim with gain 1 + w."""
    r = np.random.default_rng(9)
    x = r.standard_normal((5, 3, 16)) * 3.0
    w = r.standard_normal(16) * 0.1
    got = O.qk_rmsnorm(x, w, 1e-6)
    want = F.rms_norm(torch.from_numpy(x), (16,), weight=torch.from_numpy(1.0 + w), eps=1e-6).numpy()
    assert np.max(np.abs(got - want)) < 1e-13
    unit = O.qk_rmsnorm(x, None, 0.0)
    assert np.allclose(np.sqrt(np.mean(unit ** 2, axis=-1)), 1.0, atol=1e-14)
    assert np.allclose(O.qk_rmsnorm(7.5 * x, w, 0.0), O.qk_rmsnorm(x, w, 0.0), atol=1e-13)


# ------------------------------------------------------------------ boundary layers and sampler
def test_patchify_layout_and_round_trip():
    """Token (py, px) in raster order holds z[c, 2py+dy, 2px+dx] at c*4 + dy*2 + dx;
    unpatchify inverts it."""
    B, C, Hl, Wl = 2, 3, 4, 6
    z = np.arange(B * C * Hl * Wl, dtype=np.float64).reshape(B, C, Hl, Wl)
    p = O.patchify(z)
    assert p.shape == (B, (Hl // 2) * (Wl // 2), 4 * C)
    for b in range(B):
        for py in range(Hl // 2):
            for px in range(Wl // 2):
                for c in range(C):
                    for dy in range(2):
                        for dx in range(2):
                            assert p[b, py * (Wl // 2) + px, c * 4 + dy * 2 + dx] == z[b, c, 2 * py + dy, 2 * px + dx]
    assert np.array_equal(O.unpatchify(p, C, Hl, Wl), z)


def test_flow_schedule_closed_forms():
    t = O.flow_schedule(8, 3.0)
    assert t[0] == 1.0 and t[-1] == 0.0 and np.all(np.diff(t) < 0)
    assert np.allclose(O.flow_schedule(4, 1.0), [1.0, 0.75, 0.5, 0.25, 0.0], atol=0, rtol=0)
    assert abs(O.flow_schedule(2, 3.0)[1] - 0.75) < 1e-15  # s u / (1 + (s-1) u) at u = 1/2: 3/4


def test_euler_integrates_a_straight_path_exactly():
    """For the straight path z_t = (1-t) x0 + t eps the velocity is eps - x0 at
    every point, so the sampler must land on x0 for any schedule (signs and
    step direction pinned)."""
    r = np.random.default_rng(2)
    x0, eps = r.standard_normal((2, 3, 4, 4)), r.standard_normal((2, 3, 4, 4))
    for n, s in ((1, 1.0), (8, 3.0), (28, 6.0)):
        out = O.euler_sample(eps, O.flow_schedule(n, s), lambda z, t: (z - x0) / t)
        assert np.max(np.abs(out - x0)) < 1e-12


def test_embed_and_final_layer_against_torch_and_loops():
    """Embedding = torch linear on patches / text features; the final layer =
    torch rms_norm with the adaLN terms, then linear; scale = -1 gives W_out shift."""
    cfg = datagen.Config("tiny-model", batch=2, n_image=6, n_text=3, hidden=8, n_heads=2, n_kv_heads=1,
                         head_dim=4, ffn=8, dtype="f32", seed=9, w_std=0.5, out_std=0.5, grid_h=2, grid_w=3,
                         latent_ch=2, txt_dim=5, t_dim=8)
    mw = datagen.model_weights(cfg)
    z = datagen.latent_noise(cfg)
    txt = datagen.text_features(cfg)
    x = O.embed_tokens(z, txt, mw.w_in, mw.w_txt)
    pt = torch.from_numpy(O.patchify(z))
    assert np.allclose(x[:, :6], F.linear(pt, torch.from_numpy(mw.w_in).double()).numpy(), atol=1e-13)
    assert np.allclose(x[:, 6:], F.linear(torch.from_numpy(txt).double(), torch.from_numpy(mw.w_txt).double()).numpy(),
                       atol=1e-13)
    modf = O.final_mod(np.array([0.3, 0.8]), mw.w_t1, mw.w_tf, 8)
    v = O.final_layer(x[:, :6], modf, mw.norm_f_w, mw.w_out, 1e-6)
    xt = torch.from_numpy(x[:, :6])
    h = F.rms_norm(xt, (8,), weight=torch.from_numpy(1.0 + mw.norm_f_w).double(), eps=1e-6)
    h = h * (1 + torch.from_numpy(modf[:, 1:2])) + torch.from_numpy(modf[:, 0:1])
    assert np.allclose(v, F.linear(h, torch.from_numpy(mw.w_out).double()).numpy(), atol=1e-12)
    m2 = modf.copy()
    m2[:, 1] = -1.0
    v2 = O.final_layer(x[:, :6], m2, mw.norm_f_w, mw.w_out, 1e-6)
    assert np.allclose(v2, (m2[:, 0] @ mw.w_out.astype(np.float64).T)[:, None, :], atol=1e-13)


def test_model_velocity_with_no_blocks_matches_per_token_loops():
    """With an empty stack the velocity is the boundary layers alone: check
    every latent element against scalar loops (text tokens do not reach the
    output; image token order = patch order)."""
    cfg = datagen.Config("tiny-model", batch=1, n_image=4, n_text=2, hidden=4, n_heads=1, n_kv_heads=1,
                         head_dim=4, ffn=4, dtype="f32", seed=11, w_std=0.5, out_std=0.5, grid_h=2, grid_w=2,
                         latent_ch=1, txt_dim=3, t_dim=4)
    mw = datagen.model_weights(cfg)
    z = datagen.latent_noise(cfg)
    txt = datagen.text_features(cfg)
    oc_ = O.OracleConfig.of(cfg)
    v = O.model_velocity(z, 0.6, txt, mw, [], 0, oc_)
    e = bruteforce.time_embedding([0.6], dim=4)[0]
    zs = [sum(float(mw.w_t1[r][k]) * e[k] for k in range(4)) for r in range(4)]
    zs = [a / (1 + math.exp(-a)) for a in zs]
    fm = [sum(float(mw.w_tf[o][r]) * zs[r] for r in range(4)) for o in range(8)]
    shift, scale = fm[:4], fm[4:]
    for py in range(2):
        for px in range(2):
            patch = [float(z[0, 0, 2 * py + dy, 2 * px + dx]) for dy in range(2) for dx in range(2)]
            tok = [sum(float(mw.w_in[o][i]) * patch[i] for i in range(4)) for o in range(4)]
            rms = math.sqrt(sum(a * a for a in tok) / 4 + cfg.eps)
            h = [tok[c] / rms * (1 + float(mw.norm_f_w[c])) * (1 + scale[c]) + shift[c] for c in range(4)]
            out = [sum(float(mw.w_out[o][c]) * h[c] for c in range(4)) for o in range(4)]
            for dy in range(2):
                for dx in range(2):
                    assert abs(v[0, 0, 2 * py + dy, 2 * px + dx] - out[dy * 2 + dx]) < 1e-12


def test_guided_velocity_special_cases():
    """Classifier-free guidance reduces to the pinned model velocity: g = 1
    gives the conditional velocity, g = 0 the unconditional one (a planted
    swap of the two roles fails here), and when the text cannot reach the
    output (no blocks) every g gives the same velocity."""
    cfg = datagen.Config("tiny-model", batch=2, n_image=6, n_text=3, hidden=8, n_heads=2, n_kv_heads=1,
                         head_dim=4, ffn=8, dtype="f32", seed=13, w_std=0.5, out_std=0.5, grid_h=2, grid_w=3,
                         latent_ch=2, txt_dim=5, t_dim=8)
    mw = datagen.model_weights(cfg)
    blocks = [datagen.block_weights(cfg, i) for i in range(2)]
    z = datagen.latent_noise(cfg)
    txt = datagen.text_features(cfg)
    txt_null = datagen.text_features(cfg.replace(seed=cfg.seed + 1))
    oc_ = O.OracleConfig.of(cfg)
    vc = O.model_velocity(z, 0.4, txt, mw, blocks, 2, oc_)
    vu = O.model_velocity(z, 0.4, txt_null, mw, blocks, 2, oc_)
    assert np.max(np.abs(vc - vu)) > 1e-3  # the text matters through the blocks
    g1 = O.guided_velocity(z, 0.4, txt, txt_null, 1.0, mw, blocks, 2, oc_)
    g0 = O.guided_velocity(z, 0.4, txt, txt_null, 0.0, mw, blocks, 2, oc_)
    assert np.max(np.abs(g1 - vc)) < 1e-12 and np.max(np.abs(g0 - vu)) < 1e-12

    def swapped(g):  # the planted mistake: the roles of the two velocities exchanged
        return vc + g * (vu - vc)
    assert np.max(np.abs(swapped(0.0) - g0)) > 1e-3
    e0 = O.model_velocity(z, 0.4, txt, mw, [], 0, oc_)
    for g in (0.0, 3.5, -1.0):
        assert np.max(np.abs(O.guided_velocity(z, 0.4, txt, txt_null, g, mw, [], 0, oc_) - e0)) < 1e-12


# ------------------------------------------------------------------ 8-bit projections
def _e4m3_values():
    """Every finite OCP e4m3 value, decoded from its bit fields."""
    vals = []
    for v in range(256):
        if (v & 0x7F) == 0x7F:
            continue  # NaN codes
        s, e, m = v >> 7, (v >> 3) & 15, v & 7
        x = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
        vals.append((-x if s else x, v))
    return vals


def test_fp8_round_is_nearest_even_over_all_codes():
    """Against an exhaustive search over the 254 finite codes: nearest value,
    ties to the code with the even mantissa; covers subnormals, ties, the top."""
    vals = _e4m3_values()
    r = np.random.default_rng(4)
    xs = np.concatenate([r.standard_normal(3000) * 50, r.standard_normal(1000) * 0.01,
                         np.array([448.0, -448.0, 447.9, 1.0625, 1.1875, 0.0009765625, 3 * 2.0 ** -10, 0.0, 240.0, 464.0])])
    xs = xs[np.abs(xs) <= 464].astype(np.float32).astype(np.float64)
    got = O.fp8_e4m3_round(xs)
    for x, g in zip(xs, got):
        d = [(abs(v - x), (c & 1), v) for v, c in vals]
        best = min(d)[0]
        cands = [v for (dist, odd, v) in d if dist == best]
        want = [v for (dist, odd, v) in d if dist == best and odd == 0] if len(cands) > 1 else cands
        assert g in want or (g == 0.0 and 0.0 in [abs(w) for w in want]), (x, g, want)


def test_fp8_quantize_rows_properties():
    """Representable values are fixed points; each row's largest |x| lands on
    +-448; dequantised rows are within half a step; zero rows give zeros."""
    r = np.random.default_rng(8)
    x = (r.standard_normal((6, 64)) * np.array([1e-3, 0.5, 3.0, 40.0, 1.0, 7.0])[:, None]).astype(np.float32)
    x[4] = 0.0
    q, s = O.quantize_rows_fp8(x)
    assert s.dtype == np.float32 and s[4] == 1.0 and np.all(q[4] == 0)
    for i in (0, 1, 2, 3, 5):
        j = np.argmax(np.abs(x[i]))
        assert abs(q[i, j]) == 448.0
        y = (x[i] * (np.float32(448.0) / np.max(np.abs(x[i])))).astype(np.float64)
        _, ex = np.frexp(np.maximum(np.abs(y), 2.0 ** -6))
        assert np.all(np.abs(q[i] - y) <= np.ldexp(1.0, ex - 1 - 4) + 1e-12)  # half a step of the binade
    fixed = np.array([v for v, c in _e4m3_values()])
    assert np.array_equal(O.fp8_e4m3_round(fixed), fixed)


def test_fp8_gemm_is_the_scaled_product():
    """gemm_fp8 = decoded operands multiplied in float64 and scaled per row and
    column; with exactly representable operands it equals the plain product."""
    r = np.random.default_rng(12)
    a = O.fp8_e4m3_round(r.integers(-8, 9, (5, 32)).astype(np.float32))
    w = O.fp8_e4m3_round(r.integers(-8, 9, (7, 32)).astype(np.float32))
    sa, sw = np.float32(r.random(5) + 0.5), np.float32(r.random(7) + 0.5)
    c = O.gemm_fp8(a, sa, w, sw)
    for m in range(5):
        for n in range(7):
            assert abs(c[m, n] - sum(float(a[m, k]) * float(w[n, k]) for k in range(32)) * float(sa[m]) * float(sw[n])) < 1e-9
    u = O.swiglu_fp8(a, sa, np.concatenate([w, w]), np.concatenate([sw, sw]), 7)
    assert np.allclose(u, c / (1 + np.exp(-c)) * c)


def test_fp8_tensor_scale_is_row_scale_of_the_whole_tensor():
    """Tensor-wise quantisation = row-wise quantisation of the flattened tensor."""
    r = np.random.default_rng(21)
    x = (r.standard_normal((7, 48)) * np.geomspace(0.01, 9.0, 7)[:, None]).astype(np.float32)
    q, s = O.quantize_tensor_fp8(x)
    qf, sf = O.quantize_rows_fp8(x.reshape(1, -1))
    assert np.array_equal(q, qf.reshape(x.shape)) and np.all(s == sf[0])
    assert np.max(np.abs(q)) == 448.0


def test_fp8_swiglu_roles_against_scalar_loop():
    """swiglu_fp8 with distinct W1 and W3 (and distinct scales) against a
    scalar loop of its definition: u = SiLU(sa sw1 a.w1) * (sa sw3 a.w3),
    W1 the first ffn rows of W13 (the SiLU branch), W3 the next ffn rows
    (the linear branch; page "Krea 2 技术报告", 架构 › Transformer块:
    SwiGLU, the GLU-variants paper's roles).  Swapping the roles must change
    the result, so the pin tells them apart."""
    r = np.random.default_rng(44)
    m, f, k = 4, 5, 32
    a = O.fp8_e4m3_round(r.integers(-12, 13, (m, k)).astype(np.float32) / 4)
    w1 = O.fp8_e4m3_round(r.integers(-12, 13, (f, k)).astype(np.float32) / 8)
    w3 = O.fp8_e4m3_round(r.integers(-12, 13, (f, k)).astype(np.float32) / 8 + 0.5)
    sa = np.float32(r.random(m) + 0.25)
    sw1, sw3 = np.float32(r.random(f) + 0.5), np.float32(r.random(f) + 1.5)
    u = O.swiglu_fp8(a, sa, np.concatenate([w1, w3]), np.concatenate([sw1, sw3]), f)
    for i in range(m):
        for n in range(f):
            z1 = sum(float(a[i, kk]) * float(w1[n, kk]) for kk in range(k)) * float(sa[i]) * float(sw1[n])
            z3 = sum(float(a[i, kk]) * float(w3[n, kk]) for kk in range(k)) * float(sa[i]) * float(sw3[n])
            want = z1 / (1.0 + math.exp(-z1)) * z3
            assert abs(u[i, n] - want) <= 1e-12 * max(1.0, abs(want)), (i, n)
    swapped = O.swiglu_fp8(a, sa, np.concatenate([w3, w1]), np.concatenate([sw3, sw1]), f)
    assert np.max(np.abs(swapped - u)) > 1e-3 * np.max(np.abs(u))


def test_qkvg_projection_slices_against_scalar_loop():
    """qkvg_projection's column slices against the row blocks of W_qkvg
    written out per element: Q head h = rows h d .. h d + d - 1, K head j =
    rows (H + j) d .., V head j = rows (H + Hkv + j) d .., G head h = rows
    (H + 2 Hkv + h) d .. (the block's layout); every row block holds
    different values, so a swapped or shifted slice fails."""
    r = np.random.default_rng(45)
    D, H, Hk, d, L = 6, 4, 2, 3, 5
    oc_ = O.OracleConfig(hidden=D, n_heads=H, n_kv_heads=Hk, head_dim=d, ffn=8)
    w = r.standard_normal(((2 * H + 2 * Hk) * d, D)) + np.arange((2 * H + 2 * Hk) * d)[:, None]
    h = r.standard_normal((L, D))
    q, k, v, g = O.qkvg_projection(h, w, oc_)
    assert q.shape == (L, H, d) and k.shape == (L, Hk, d) and v.shape == (L, Hk, d) and g.shape == (L, H, d)

    def dot(l, row):
        return sum(h[l, c] * w[row, c] for c in range(D))

    for l in range(L):
        for e in range(d):
            for hh in range(H):
                assert abs(q[l, hh, e] - dot(l, hh * d + e)) < 1e-9
                assert abs(g[l, hh, e] - dot(l, (H + 2 * Hk + hh) * d + e)) < 1e-9
            for j in range(Hk):
                assert abs(k[l, j, e] - dot(l, (H + j) * d + e)) < 1e-9
                assert abs(v[l, j, e] - dot(l, (H + Hk + j) * d + e)) < 1e-9


def test_fp8_block_composition_without_quantisation_is_the_block():
    """block_forward_fp8's wiring: with the quantiser replaced by the identity
    (codes = values, scales = 1) it must reproduce block_forward (roles of the
    four products, W1/W3 halves, the residual gates), so only the pinned
    quantiser and products separate the 8-bit block from the exact one."""
    for hkv in (1, 2):
        cfg = tiny_cfg(batch=2, L=5, hkv=hkv, seed=71 + hkv)
        x, w, mod = inputs(cfg)
        ref = O.block_forward(x, mod, w, oc(cfg))
        got = O.block_forward_fp8(x, mod, w, oc(cfg), quant=O._quant_identity)
        assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_fp8_stack_composition_without_quantisation_is_the_stack():
    """stack_forward_fp8 applies its blocks in order with their own weights:
    with the identity quantiser it equals stack_forward (three distinct
    blocks), and with e4m3 each block's quantisation is applied."""
    cfg = tiny_cfg(batch=2, L=5, hkv=2, seed=83)
    x, w0, mod = inputs(cfg)
    blocks = [datagen.block_weights(cfg, i) for i in range(3)]
    ref = O.stack_forward(x, mod, blocks, 3, oc(cfg))
    got = O.stack_forward_fp8(x, mod, blocks, 3, oc(cfg), quant=O._quant_identity)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    swapped = O.stack_forward_fp8(x, mod, blocks[::-1], 3, oc(cfg), quant=O._quant_identity)
    assert np.max(np.abs(swapped - ref)) > 1e-6 * np.max(np.abs(ref))  # the block order matters
    q8 = O.stack_forward_fp8(x, mod, blocks, 3, oc(cfg))
    du = np.max(np.abs((q8 - x) - (ref - x))) / np.max(np.abs(ref - x))
    assert 1e-4 < du < 0.5, du


def test_fp8_block_quantises_every_product():
    """With row-wise e4m3 the 8-bit block differs from the exact block by the
    quantisation error: a few percent of the update, neither zero (the
    quantiser is applied) nor of the update's own size."""
    cfg = tiny_cfg(batch=1, L=6, hkv=1, seed=77)
    x, w, mod = inputs(cfg)
    exact = O.block_forward(x, mod, w, oc(cfg))
    q8 = O.block_forward_fp8(x, mod, w, oc(cfg))
    du = np.max(np.abs((q8 - x) - (exact - x))) / np.max(np.abs(exact - x))
    assert 1e-4 < du < 0.5, du
