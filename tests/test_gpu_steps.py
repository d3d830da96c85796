"""GPU parity of each step kernel against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest

import datagen
from oracle import dit_oracle as O
from tests._parity import assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    from datagen import device
    import diffusion_transformer_image_amd as dit
    dit.lib()
    return torch, device, dit


def small_cfg(name, **kw):
    return datagen.get_config(name).replace(**kw)


# ------------------------------------------------------------------ GEMM
GEMM_CASES = [
    ("f32", 80, 768, 256), ("f32", 80, 256, 688), ("f32", 300, 200, 40), ("f32", 1, 1, 8),
    ("bf16", 16, 16, 32), ("bf16", 1, 1, 8), ("bf16", 80, 768, 264), ("bf16", 513, 1040, 4096),
    ("bf16", 1000, 10240, 4096), ("bf16", 300, 4096, 11008), ("bf16", 257, 4096, 4096),
]


@pytest.mark.parametrize("dt,m,n,k", GEMM_CASES)
def test_gemm(dev, dt, m, n, k):
    torch, device, dit = dev
    print(f"gemm {dt} M={m} N={n} K={k}", flush=True)
    cfg = datagen.get_config("c0" if dt == "f32" else "c1")
    a, w = datagen.gemm_operands(cfg, m, n, k, tag=m + n + k)
    A, W = device.to_device(a, dt), device.to_device(w, dt)
    C = torch.empty((m, n), dtype=A.dtype, device="cuda")
    dit.gemm(A, W, C)
    torch.cuda.synchronize()
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    y = device.to_numpy(C)
    # fp32 accumulation; bf16 output rounding (2^-9 relative) dominates
    assert_parity(y, ref, dt, f"gemm {m}x{n}x{k}", maxabs=1e-5 if dt == "f32" else 8e-3, cos_min=0.99999)


SWIGLU_CASES = [("f32", 80, 688, 256), ("f32", 100, 40, 64), ("bf16", 80, 688, 256),
                ("bf16", 600, 11008, 4096), ("bf16", 300, 200, 128)]


@pytest.mark.parametrize("dt,m,f,k", SWIGLU_CASES)
def test_gemm_swiglu(dev, dt, m, f, k):
    torch, device, dit = dev
    print(f"swiglu {dt} M={m} F={f} K={k}", flush=True)
    cfg = datagen.get_config("c0" if dt == "f32" else "c1")
    a, w = datagen.gemm_operands(cfg, m, 2 * f, k, tag=7 + m + f + k)
    A, W = device.to_device(a, dt), device.to_device(w, dt)
    U = torch.empty((m, f), dtype=A.dtype, device="cuda")
    dit.gemm_swiglu(A, W, U)
    torch.cuda.synchronize()
    ref = O.swiglu_hidden(a, w, f)
    assert_parity(device.to_numpy(U), ref, dt, "swiglu", maxabs=1e-5 if dt == "f32" else 8e-3, cos_min=0.99999)


# ------------------------------------------------------------------ attention
ATTN_CASES = [
    ("c0", 1, 80), ("c0", 2, 1), ("c0", 1, 65), ("c0", 3, 200),
    ("c1", 1, 1), ("c1", 2, 80), ("c1", 2, 512), ("c1", 1, 130), ("c1", 1, 4544), ("c1", 1, 4608),
    ("c1", 2, 4544), ("c1", 2, 4608),  # the 1024 px and 768 x 1344 launch shapes
    ("c1", 1, 100), ("c0", 1, 47),  # the last tile ends inside its second 32-key half
]


@pytest.mark.parametrize("name,B,L", ATTN_CASES)
def test_attention(dev, name, B, L):
    torch, device, dit = dev
    print(f"attention {name} B={B} L={L}", flush=True)
    cfg = small_cfg(name, batch=B, n_image=L, n_text=0)
    z = datagen.qkvg_activations(cfg)
    Z = device.to_device(z, cfg.dtype)
    OG = torch.empty((cfg.tokens, cfg.n_heads * cfg.head_dim), dtype=Z.dtype, device="cuda")
    c = dit.config_of(cfg)
    ws = torch.empty(dit.workspace_size(c), dtype=torch.uint8, device="cuda")
    dit.attention(c, Z, OG, ws)
    torch.cuda.synchronize()
    y = device.to_numpy(OG).reshape(B, L, -1)
    oc = O.OracleConfig.of(cfg)
    zz = z.reshape(B, L, -1)
    rows = np.arange(L) if L <= 600 else np.unique(np.r_[0, 1, 63, 64, 65, L // 2, L - 65, L - 64, L - 2, L - 1,
                                                            np.random.default_rng(L).integers(0, L, 24)])
    for b in range(B):
        H, Hk, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
        zb = zz[b].astype(np.float64)
        q = zb[rows, : H * d].reshape(len(rows), H, d)
        k = zb[:, H * d:(H + Hk) * d].reshape(L, Hk, d)
        v = zb[:, (H + Hk) * d:(H + 2 * Hk) * d].reshape(L, Hk, d)
        g = zb[rows, (H + 2 * Hk) * d:].reshape(len(rows), H, d)
        ref = O.gated_gqa_attention(q, k, v, g)
        assert_parity(y[b, rows], ref, cfg.dtype, f"attention b={b}", maxabs=1e-5 if cfg.dtype == "f32" else 1e-2,
                      cos_min=0.99999)


@pytest.mark.parametrize("name,prescaled", [("c0", False), ("c1", False), ("c1", True)])
@pytest.mark.parametrize("glogit", [-np.inf, -1e4])
def test_attention_gate_to_minus_inf_zeroes_the_branch(dev, name, prescaled, glogit):
    """Gate logits at -inf (or far below zero) make the gated attention
    output exactly zero, whatever the scores (sigmoid(-inf) = 0; page
    "Krea 2 技术报告", 架构 › Transformer块: the sigmoid output gate)."""
    torch, device, dit = dev
    cfg = small_cfg(name, batch=2, n_image=130, n_text=0)
    z = datagen.qkvg_activations(cfg).copy()
    H, Hk, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    z[:, (H + 2 * Hk) * d:] = glogit
    Z = device.to_device(z, cfg.dtype)
    OG = torch.full((cfg.tokens, H * d), 7.0, dtype=Z.dtype, device="cuda")
    c = dit.config_of(cfg)
    ws = torch.empty(dit.workspace_size(c), dtype=torch.uint8, device="cuda")
    dit.attention_ex(c, Z, OG, ws, prescaled)
    torch.cuda.synchronize()
    y = device.to_numpy(OG)
    assert np.all(y == 0.0), np.max(np.abs(y))


def test_attention_one_key_returns_gated_value(dev):
    torch, device, dit = dev
    cfg = small_cfg("c1", batch=3, n_image=1, n_text=0)
    z = datagen.qkvg_activations(cfg)
    Z = device.to_device(z, "bf16")
    OG = torch.empty((3, 4096), dtype=torch.bfloat16, device="cuda")
    c = dit.config_of(cfg)
    dit.attention(c, Z, OG, torch.empty(dit.workspace_size(c), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    H, Hk, d = 32, 8, 128
    v = z[:, (H + Hk) * d:(H + 2 * Hk) * d].reshape(3, Hk, d).astype(np.float64)
    g = z[:, (H + 2 * Hk) * d:].reshape(3, H, d).astype(np.float64)
    expect = np.stack([v[:, h // 4] / (1 + np.exp(-g[:, h])) for h in range(H)], axis=1).reshape(3, -1)
    y = device.to_numpy(OG)
    # only the final bf16 rounding separates the two
    assert np.max(np.abs(y - expect)) <= 2 ** -8 * np.max(np.abs(expect))


def prescale_queries(cfg, z):
    """The query columns multiplied by log2(e)/sqrt(d) in fp32 and rounded
    once to bf16 (what the block path's projection epilogue stores), and the
    queries the oracle must then use: the base-2 scores 2^(q' . k) equal the
    softmax weights of q = q' ln(2) sqrt(d) in natural units with 1/sqrt(d)."""
    d, nq = cfg.head_dim, cfg.n_heads * cfg.head_dim
    zs = z.astype(np.float32).copy()
    sc = np.float32(1.4426950408889634) / np.sqrt(np.float32(d))
    zs[:, :nq] = datagen.bf16_round(zs[:, :nq] * sc)
    q_eff = zs[:, :nq].astype(np.float64) * (np.log(2.0) * np.sqrt(d))
    return zs, q_eff


def _attention_vs_oracle(dev, cfg, z, rows, f32_tol=1e-5, prescaled=False):
    torch, device, dit = dev
    B, L = cfg.batch, cfg.seq_len
    H, Hk, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    q_eff = None
    if prescaled:
        z, q_eff = prescale_queries(cfg, z)
        q_eff = q_eff.reshape(B, L, H * d)
    Z = device.to_device(z, cfg.dtype)
    OG = torch.empty((cfg.tokens, cfg.n_heads * cfg.head_dim), dtype=Z.dtype, device="cuda")
    c = dit.config_of(cfg)
    ws = torch.empty(dit.workspace_size(c), dtype=torch.uint8, device="cuda")
    if prescaled:
        dit.attention_ex(c, Z, OG, ws, True)
    else:
        dit.attention(c, Z, OG, ws)
    torch.cuda.synchronize()
    y = device.to_numpy(OG).reshape(B, L, -1)
    zz = z.reshape(B, L, -1)
    for b in range(B):
        zb = zz[b].astype(np.float64)
        q = (q_eff[b] if prescaled else zb[:, : H * d])[rows].reshape(len(rows), H, d)
        k = zb[:, H * d:(H + Hk) * d].reshape(L, Hk, d)
        v = zb[:, (H + Hk) * d:(H + 2 * Hk) * d].reshape(L, Hk, d)
        g = zb[rows, (H + 2 * Hk) * d:].reshape(len(rows), H, d)
        ref = O.gated_gqa_attention(q, k, v, g)
        assert_parity(y[b, rows], ref, cfg.dtype, f"attention b={b}", maxabs=f32_tol if cfg.dtype == "f32" else 1e-2,
                      cos_min=0.99999)


@pytest.mark.parametrize("name,B,L", [("c0", 1, 200), ("c1", 1, 300), ("c1", 2, 4608)])
def test_attention_rising_reference(dev, name, B, L):
    """Scores that step up by about 30 (natural units) at keys placed in the
    first and in the second 32-key half of several tiles: the running
    softmax reference has to be raised again and again after the first tile
    (queries carry a common component along a fixed direction u, and the key
    component along u steps up at each of those keys)."""
    print(f"attention rising reference {name} B={B} L={L}", flush=True)
    cfg = small_cfg(name, batch=B, n_image=L, n_text=0)
    H, Hk, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    z = datagen.qkvg_activations(cfg).reshape(B, L, -1).astype(np.float64)
    u = np.ones(d) / np.sqrt(d)
    steps = [40, 74, 178] + list(range(300, L, 397))  # second, first, second half, then spread out
    c = np.zeros(L)
    for p in steps:
        if p < L:
            c[p:] += 30.0 * np.sqrt(d) / 2.0  # score step ~ 30 for a query with q.u ~ 2
    for hh in range(H):
        z[:, :, hh * d:(hh + 1) * d] += 2.0 * u
    for j in range(Hk):
        z[:, :, (H + j) * d:(H + j + 1) * d] += c[None, :, None] * u
    z = z.reshape(B * L, -1).astype(np.float32)
    if cfg.dtype != "f32":
        z = datagen.bf16_round(z)
    rows = np.arange(L) if L <= 600 else np.unique(np.r_[0, 1, 63, 64, 65, L // 2, L - 65, L - 64, L - 2, L - 1,
                                                            np.random.default_rng(L).integers(0, L, 24)])
    # scores of a few hundred: fp32 rounding of the dot products alone moves
    # them by ~1e-5, so the fp32 bar is the general 1e-4 one here
    _attention_vs_oracle(dev, cfg, z, rows, f32_tol=1e-4)
    if cfg.dtype == "bf16":  # the block path's kernel: queries pre-scaled, reference from 0
        _attention_vs_oracle(dev, cfg, z, rows, prescaled=True)


@pytest.mark.parametrize("B,L", [(1, 1), (2, 80), (1, 100), (1, 130), (2, 512), (1, 4544), (2, 4608)])
def test_attention_prescaled(dev, B, L):
    """Queries carrying log2(e)/sqrt(d) (the block path's attention): ragged
    tails in either 32-key half, one key, a query block that ends past the
    sequence (48 queries per wave), one and two samples."""
    print(f"attention prescaled B={B} L={L}", flush=True)
    cfg = small_cfg("c1", batch=B, n_image=L, n_text=0)
    rows = np.arange(L) if L <= 600 else np.unique(np.r_[0, 1, 63, 64, 65, L // 2, L - 65, L - 64, L - 2, L - 1,
                                                            np.random.default_rng(L).integers(0, L, 24)])
    _attention_vs_oracle(dev, cfg, datagen.qkvg_activations(cfg), rows, prescaled=True)


def test_attention_prescaled_low_scores(dev):
    """Every score far below zero (about -200 in base-2 units): the
    reference starts at 0, so the first tile must lower it to the row
    maximum or every numerator underflows."""
    cfg = small_cfg("c1", batch=1, n_image=200, n_text=0)
    H, Hk, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    z = datagen.qkvg_activations(cfg).astype(np.float64)
    u = np.ones(d) / np.sqrt(d)
    for hh in range(H):
        z[:, hh * d:(hh + 1) * d] += 2.0 * u
    for j in range(Hk):
        z[:, (H + j) * d:(H + j + 1) * d] -= 100.0 * np.sqrt(d) * u / 2.0
    z = datagen.bf16_round(z.astype(np.float32))
    _attention_vs_oracle(dev, cfg, z, np.arange(cfg.seq_len), prescaled=True)


# ------------------------------------------------------------------ modnorm / residual
@pytest.mark.parametrize("name,x_f32", [("c0", True), ("c1", False), ("c1", True)])
@pytest.mark.parametrize("which", [0, 1])
def test_modnorm(dev, name, x_f32, which):
    torch, device, dit = dev
    cfg = small_cfg(name, batch=3, n_image=37, n_text=0)
    x = datagen.activations(cfg)
    w = datagen.block_weights(cfg)
    mod = datagen.block_mod(cfg, strong=True)
    X = device.to_device(x, "f32" if x_f32 else cfg.dtype)
    Hh = torch.empty((cfg.tokens, cfg.hidden), dtype=torch.float32 if cfg.dtype == "f32" else torch.bfloat16, device="cuda")
    gain = w.norm1_w if which == 0 else w.norm2_w
    dit.modnorm(dit.config_of(cfg), X, Hh, device.to_device(mod, "f32"), device.to_device(w.mod_bias, "f32"),
                device.to_device(gain, "f32"), which)
    torch.cuda.synchronize()
    ref = []
    for b in range(3):
        m = O.split_modulation(mod[b], w.mod_bias)
        ref.append(O.modulated_rmsnorm(x[b], gain, m[3 * which], m[3 * which + 1], cfg.eps))
    ref = np.concatenate(ref)
    y = device.to_numpy(Hh)
    if cfg.dtype == "f32":
        assert_parity(y, ref, "f32", "modnorm", maxabs=2e-6)
    else:
        assert np.max(np.abs(y - ref) / (np.abs(ref) + 1e-3)) <= 2 ** -8 + 1e-5  # bf16 rounding only


@pytest.mark.parametrize("name,xd,od", [("c0", "f32", "f32"), ("c1", "bf16", "bf16"), ("c1", "f32", "f32"),
                                        ("c1", "bf16", "f32"), ("c1", "f32", "bf16")])
@pytest.mark.parametrize("which", [0, 1])
def test_gated_residual(dev, name, xd, od, which):
    torch, device, dit = dev
    cfg = small_cfg(name, batch=2, n_image=41, n_text=0)
    x = datagen.activations(cfg)
    y = datagen.activations(cfg.replace(seed=cfg.seed + 17))
    w = datagen.block_weights(cfg)
    mod = datagen.block_mod(cfg, strong=True)
    X, Y = device.to_device(x, xd), device.to_device(y, cfg.dtype)
    out = torch.empty_like(X, dtype=torch.float32 if od == "f32" else torch.bfloat16)
    dit.gated_residual(dit.config_of(cfg), X, Y, device.to_device(mod, "f32"), device.to_device(w.mod_bias, "f32"),
                       which, out)
    torch.cuda.synchronize()
    gates = [O.split_modulation(mod[b], w.mod_bias)[3 * which + 2] for b in range(2)]
    ref = np.concatenate([O.gated_residual(x[b], gates[b], y[b]) for b in range(2)])
    mag = np.concatenate([np.abs(x[b]) + np.abs(gates[b] * y[b]) for b in range(2)])
    r = device.to_numpy(out).reshape(ref.shape)
    tol = (2 ** -8 if od == "bf16" else 0.0) * np.abs(ref) + 1e-6 * mag
    assert np.all(np.abs(r - ref) <= tol)


# ------------------------------------------------------------------ timestep modulation
@pytest.mark.parametrize("name,batch", [("c0", None), ("c0", 3), ("c3", None), ("c3", 4), ("c3", 5),
                                        ("c1", None), ("c3", 17), ("c0", 70), ("c2", None)])
def test_timestep_mod(dev, name, batch):
    """Both stage-2 kernels: up to 4 samples (hidden vectors in LDS) and more
    (fp32 MFMA over blocks of 16 samples, 64 per pass over W_t2: 5, 8, 17,
    32 and 70 samples cover partial sample blocks and a second pass); the
    workspace is the documented minimum, B * hidden floats."""
    torch, device, dit = dev
    cfg = datagen.get_config(name)
    if batch:
        cfg = cfg.replace(batch=batch)
    t, w1, w2 = datagen.timestep_inputs(cfg)
    c = dit.config_of(cfg)
    M = torch.empty((cfg.batch, 6, cfg.hidden), dtype=torch.float32, device="cuda")
    ws = torch.empty(cfg.batch * cfg.hidden * 4, dtype=torch.uint8, device="cuda")
    dit.timestep_mod(c, device.to_device(t, "f32"), device.to_device(w1, "f32"), device.to_device(w2, "f32"), M, ws)
    torch.cuda.synchronize()
    ref = O.timestep_modulation(t, w1, w2, cfg.hidden)
    assert_parity(device.to_numpy(M), ref, "f32", "timestep modulation", maxabs=2e-5)


@pytest.mark.parametrize("group_m", [1, 3, 64])
@pytest.mark.parametrize("variant", [0, 1])
def test_gemm_tile_grouping(dev, variant, group_m):
    """The L2 grouping width reorders tiles only: ragged M with fewer row
    tiles than one group, and several groups with a partial last one."""
    torch, device, dit = dev
    m, n, k = 1100, 776, 264
    cfg = datagen.get_config("c1")
    a, w = datagen.gemm_operands(cfg, m, n, k, tag=61 + group_m)
    A, W = device.to_device(a, "bf16"), device.to_device(w, "bf16")
    C = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    dit.gemm_variant(variant, A, W, C, group_m=group_m)
    torch.cuda.synchronize()
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    assert_parity(device.to_numpy(C), ref, "bf16", f"variant {variant} group {group_m}", maxabs=8e-3,
                  cos_min=0.99999)


@pytest.mark.parametrize("swiglu", [False, True])
def test_gemm_grouping_changes_order_only(dev, swiglu):
    """The L2 grouping width and the tile height only reorder whole tiles:
    every width gives the same bits (each tile's K loop is the same), on a
    shape with ragged row and column tiles and more tiles than CUs."""
    torch, device, dit = dev
    m, n, k = 4100, 2056 if swiglu else 4104, 192  # 289 tiles of 256 rows, 374 of 192
    print(f"grouping swiglu={swiglu} M={m} N={n} K={k}", flush=True)
    cfg = datagen.get_config("c1")
    a, w = datagen.gemm_operands(cfg, m, 2 * n if swiglu else n, k, tag=307 + int(swiglu))
    A, W = device.to_device(a, "bf16"), device.to_device(w, "bf16")
    outs = {}
    for variant in (0, 1):
        for gm in (1, 2, 3, 8, 64):
            C = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
            dit.gemm_variant(variant, A, W, C, swiglu=swiglu, group_m=gm)
            outs[(variant, gm)] = C
    torch.cuda.synchronize()
    ref = outs[(0, 1)]
    for key, c in outs.items():
        assert torch.equal(c, ref), f"tile height / grouping {key} changed the result"
    exact = O.swiglu_hidden(a, w, n) if swiglu else a.astype(np.float64) @ w.astype(np.float64).T
    assert_parity(device.to_numpy(outs[(0, 2)]), exact, "bf16", "grouping", maxabs=8e-3, cos_min=0.99999)


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("k", [328, 384, 64])
def test_gemm_whole_tile_variants(dev, variant, swiglu, k):
    """Both whole-tile plans (256- and 192-row tiles) on ragged M and N, with
    K ragged against the 64-element stage (328), a whole number of stages
    (384) and a single stage (64)."""
    torch, device, dit = dev
    m, n = 300, 200 if swiglu else 520
    cfg = datagen.get_config("c1")
    a, w = datagen.gemm_operands(cfg, m, 2 * n if swiglu else n, k, tag=97 + variant + k)
    A, W = device.to_device(a, "bf16"), device.to_device(w, "bf16")
    C = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    dit.gemm_variant(variant, A, W, C, swiglu=swiglu)
    torch.cuda.synchronize()
    ref = O.swiglu_hidden(a, w, n) if swiglu else a.astype(np.float64) @ w.astype(np.float64).T
    assert_parity(device.to_numpy(C), ref, "bf16", f"variant {variant}", maxabs=8e-3, cos_min=0.99999)


@pytest.mark.parametrize("swiglu,m,n,k,sk_tiles,segs", [
    (False, 2300, 8200, 192, 0, 1),   # 297 tiles of 3 stages, ragged M
    (True, 2304, 4224, 128, 0, 1),    # 297 SwiGLU tiles of two stages each
    (False, 2304, 8192, 256, 32, 2),  # 256 whole tiles (XCD-remapped), then 64 K segments
    (True, 2100, 4100, 320, 40, 2),   # ragged M and F, segments of 2 and 3 stages
])
def test_gemm_more_tiles_than_cus(dev, swiglu, m, n, k, sk_tiles, segs):
    """More work items than the 256 compute units hold at once: a second
    round of workgroups, with the grouped tile order, the XCD remap of a
    whole number of rounds and a split tail after a full round."""
    torch, device, dit = dev
    print(f"gemm rounds swiglu={swiglu} M={m} N={n} K={k} split {sk_tiles}x{segs}", flush=True)
    cfg = datagen.get_config("c1")
    a, w = datagen.gemm_operands(cfg, m, 2 * n if swiglu else n, k, tag=211 + m + k)
    A, W = device.to_device(a, "bf16"), device.to_device(w, "bf16")
    C = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    if sk_tiles:
        ws = torch.empty(sk_tiles * segs * 65536, dtype=torch.float32, device="cuda")
        dit.gemm_splitk(A, W, C, sk_tiles, segs, ws, swiglu=swiglu)
    elif swiglu:
        dit.gemm_swiglu(A, W, C)
    else:
        dit.gemm(A, W, C)
    torch.cuda.synchronize()
    ref = O.swiglu_hidden(a, w, n) if swiglu else a.astype(np.float64) @ w.astype(np.float64).T
    assert_parity(device.to_numpy(C), ref, "bf16", "more tiles than CUs", maxabs=8e-3, cos_min=0.99999)


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("m,n,k,sk_tiles,segs", [
    (300, 520, 328, 6, 3),     # every tile split, ragged M, N and K (K tail in the last segment)
    (600, 776, 1024, 2, 7),    # only the last two tiles split, uneven segment lengths
    (256, 256, 128, 1, 2),     # one tile, two one-stage segments
    (513, 264, 4096, 3, 8),    # ragged row tile among the split ones, long K
])
def test_gemm_split_tail(dev, m, n, k, sk_tiles, segs, swiglu):
    """K-split tail tiles: fp32 partials summed in segment order by the fixup
    pass, whole tiles as before, SwiGLU applied after the sum."""
    torch, device, dit = dev
    if swiglu:
        n = (n // 2 + 7) // 8 * 8
    tiles = ((m + 255) // 256) * ((n + (127 if swiglu else 255)) // (128 if swiglu else 256))
    sk_tiles = min(sk_tiles, tiles)
    cfg = datagen.get_config("c1")
    a, w = datagen.gemm_operands(cfg, m, 2 * n if swiglu else n, k, tag=171 + segs + k)
    A, W = device.to_device(a, "bf16"), device.to_device(w, "bf16")
    C = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(sk_tiles * segs * 65536, 1), dtype=torch.float32, device="cuda")
    dit.gemm_splitk(A, W, C, sk_tiles, segs, ws, swiglu=swiglu)
    C2 = torch.empty_like(C)
    dit.gemm_splitk(A, W, C2, sk_tiles, segs, ws, swiglu=swiglu)
    torch.cuda.synchronize()
    ref = O.swiglu_hidden(a, w, n) if swiglu else a.astype(np.float64) @ w.astype(np.float64).T
    assert_parity(device.to_numpy(C), ref, "bf16", f"split {sk_tiles}x{segs}", maxabs=8e-3, cos_min=0.99999)
    assert torch.equal(C, C2), "split-K tail is not deterministic"
