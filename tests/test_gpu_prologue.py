"""GPU parity of the attention prologue (QKNorm + 3D axial RoPE, text tokens
at position 0) against the fp64 oracle, as a step and inside the block and
the stack, through the C ABI."""
import numpy as np
import pytest

import datagen
from oracle import dit_oracle as O
from tests._parity import assert_parity, assert_update_parity

pytestmark = pytest.mark.gpu

AXES = {64: (16, 24, 24), 128: (32, 48, 48)}


@pytest.fixture(scope="module")
def dev():
    import torch
    from datagen import device
    import diffusion_transformer_image_amd as dit
    dit.lib()
    return torch, device, dit


def prologues(cfg, qk_norm=True, rope=True):
    kw = dict(qk_norm=qk_norm, rope=rope, grid_h=cfg.grid_h, grid_w=cfg.grid_w, axes=AXES[cfg.head_dim],
              theta=10000.0)
    return kw, O.Prologue(**kw)


@pytest.mark.parametrize("qk_norm,rope", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("dtype,hd", [("bf16", 128), ("f32", 64), ("f32", 128)])
def test_qk_prologue_step(dev, dtype, hd, qk_norm, rope):
    """Q and K heads transformed in place: every element against the oracle
    (one rounding of the output in bf16); V and G bitwise untouched; with
    RoPE alone the text tokens come back bitwise unchanged."""
    torch, device, dit = dev
    H, hkv = (4, 2) if hd == 64 else (4, 1)
    cfg = datagen.Config("pro-step", batch=2, n_image=35, n_text=9, hidden=H * hd, n_heads=H, n_kv_heads=hkv,
                         head_dim=hd, ffn=64, dtype=dtype, seed=61 + hd, grid_h=5, grid_w=7)
    z = datagen.qkvg_activations(cfg, std=1.5)
    w = datagen.qk_norm_weights(cfg, datagen.block_weights(cfg))
    kw, pro = prologues(cfg, qk_norm, rope)
    Z = device.to_device(z, dtype)
    wq, wk = device.to_device(w.q_norm_w, "f32"), device.to_device(w.k_norm_w, "f32")
    dit.qk_prologue(dit.config_of(cfg), dit.make_prologue(**kw), Z, wq, wk)
    torch.cuda.synchronize()
    y = device.to_numpy(Z)
    L, nq, nk = cfg.seq_len, H * hd, hkv * hd
    for b in range(cfg.batch):
        zb = z[b * L:(b + 1) * L].astype(np.float64)
        q, k = O.attention_prologue(zb[:, :nq].reshape(L, H, hd), zb[:, nq:nq + nk].reshape(L, hkv, hd), pro, w,
                                    cfg.eps)
        ref = np.concatenate([q.reshape(L, -1), k.reshape(L, -1)], axis=1)
        got = y[b * L:(b + 1) * L, :nq + nk]
        scale = np.max(np.abs(ref))
        tol = (2.0 ** -8) * np.abs(ref) + 1e-6 * scale if dtype == "bf16" else 2e-6 * scale
        bad = np.abs(got - ref) > tol
        assert not bad.any(), f"{bad.sum()} elements off, max err {np.max(np.abs(got - ref)):.3e}"
        if rope and not qk_norm:
            assert np.array_equal(got[cfg.n_image:], zb[cfg.n_image:, :nq + nk])
    assert np.array_equal(y[:, nq + nk:], z[:, nq + nk:].astype(np.float64))  # V | G untouched


class ProRun:
    def __init__(self, dev, cfg, strong=False, qk_norm=True, rope=True):
        torch, device, dit = dev
        self.torch, self.device, self.dit, self.cfg = torch, device, dit, cfg
        self.x = datagen.activations(cfg)
        self.w = datagen.qk_norm_weights(cfg, datagen.block_weights(cfg))
        self.mod = datagen.block_mod(cfg, strong=strong)
        self.kw, self.pro = prologues(cfg, qk_norm, rope)
        self.c = dit.config_of(cfg)
        self.X = device.to_device(self.x.reshape(cfg.tokens, cfg.hidden), cfg.dtype)
        self.W = device.weights_to_device(self.w, cfg.dtype)
        self.M = device.to_device(self.mod, "f32")
        self.ws = torch.empty(dit.workspace_size(self.c), dtype=torch.uint8, device="cuda")

    def forward(self):
        Y = self.torch.empty_like(self.X)
        self.dit.block_fwd_ex(self.c, self.dit.make_prologue(**self.kw), self.W, self.X, Y, self.M, self.ws)
        self.torch.cuda.synchronize()
        return self.device.to_numpy(Y).reshape(self.cfg.batch, self.cfg.seq_len, self.cfg.hidden)


def check(y, ref, x, dtype, what):
    e, c = assert_parity(y, ref, dtype, what + " output")
    eu, cu = assert_update_parity(y, ref, x, dtype, what + " update")
    print(f"{what}: output {e:.2e}/{c:.7f} update {eu:.2e}/{cu:.7f}")


@pytest.mark.parametrize("strong", [False, True])
def test_block_prologue_c0_full(dev, strong):
    cfg = datagen.get_config("c0")
    r = ProRun(dev, cfg, strong)
    y = r.forward()
    ref = O.block_forward(r.x, r.mod, r.w, O.OracleConfig.of(cfg), r.pro)
    check(y, ref, r.x, "f32", "c0 + prologue")
    plain = O.block_forward(r.x, r.mod, r.w, O.OracleConfig.of(cfg))
    assert np.max(np.abs((ref - r.x) - (plain - r.x))) > 1e-2 * np.max(np.abs(plain - r.x))  # it mattered


def test_block_prologue_small_bf16_full(dev):
    """Every output of a small bf16 block (7 x 10 image grid + 27 text tokens, ragged L)."""
    cfg = datagen.get_config("c1").replace(batch=2, n_image=70, n_text=27, hidden=512, n_heads=4, n_kv_heads=1,
                                            ffn=1368, grid_h=7, grid_w=10)
    for strong in (False, True):
        r = ProRun(dev, cfg, strong)
        y = r.forward()
        ref = O.block_forward(r.x, r.mod, r.w, O.OracleConfig.of(cfg), r.pro)
        check(y, ref, r.x, "bf16", f"small bf16 + prologue strong={strong}")


@pytest.mark.parametrize("qk_norm,rope", [(True, False), (False, True)])
@pytest.mark.parametrize("heads,kv", [(4, 4), (4, 2), (8, 2)])
def test_block_prologue_parts_and_groups(dev, qk_norm, rope, heads, kv):
    """Each half of the prologue alone, at query-head groups of 1, 2 and 4 per
    key head (every attention launch shape that takes the prologue on its
    way in), every output of a small bf16 block with a ragged length."""
    cfg = datagen.get_config("c1").replace(batch=2, n_image=54, n_text=21, hidden=heads * 128, n_heads=heads,
                                            n_kv_heads=kv, ffn=688, grid_h=6, grid_w=9, seed=80 + heads + kv)
    r = ProRun(dev, cfg, strong=True, qk_norm=qk_norm, rope=rope)
    y = r.forward()
    ref = O.block_forward(r.x, r.mod, r.w, O.OracleConfig.of(cfg), r.pro)
    check(y, ref, r.x, "bf16", f"H{heads}/{kv} qk_norm={qk_norm} rope={rope}")


@pytest.mark.parametrize("name", ["c3", "c3b"])
def test_block_prologue_full_size_sampled(dev, name):
    """1024 px (64 x 64 grid) and 768 x 1344 (48 x 84) with the prologue: sampled
    query tokens of both samples, image rows at the grid edges and text rows."""
    cfg = datagen.get_config(name)
    print(f"block {name} + prologue", flush=True)
    r = ProRun(dev, cfg, strong=True)
    y = r.forward()
    oc = O.OracleConfig.of(cfg)
    gw, n_img = cfg.grid_w, cfg.n_image
    for b in range(cfg.batch):
        rows = np.unique(np.r_[0, 1, gw - 1, gw, n_img // 2, n_img - gw, n_img - 1, n_img, n_img + 1,
                               cfg.seq_len - 1, np.random.default_rng(b).integers(0, cfg.seq_len, 6)])
        ref = O.block_forward_rows(r.x, r.mod, r.w, oc, b, rows, r.pro)
        check(y[b, rows], ref, r.x[b, rows].astype(np.float64), "bf16", f"{name}+prologue b={b}")


def test_stack_prologue_small(dev):
    """Four blocks, each with its own QKNorm gains, prologue in every block."""
    torch, device, dit = dev
    cfg = datagen.get_config("c4").replace(batch=2, n_image=48, n_text=20, hidden=256, n_heads=2, n_kv_heads=1,
                                            ffn=688, grid_h=6, grid_w=8)
    x = datagen.activations(cfg)
    mod = datagen.block_mod(cfg, strong=True)
    blocks = [datagen.qk_norm_weights(cfg, datagen.block_weights(cfg, i), i) for i in range(4)]
    kw, pro = prologues(cfg)
    c = dit.config_of(cfg)
    X = device.to_device(x.reshape(cfg.tokens, cfg.hidden), cfg.dtype)
    Y = torch.empty_like(X)
    ws = torch.empty(dit.stack_workspace_size(c), dtype=torch.uint8, device="cuda")
    dit.stack_fwd_ex(c, dit.make_prologue(**kw), [device.weights_to_device(w, cfg.dtype) for w in blocks], X, Y,
                     device.to_device(mod, "f32"), ws)
    torch.cuda.synchronize()
    y = device.to_numpy(Y).reshape(x.shape)
    ref = O.stack_forward(x, mod, blocks, 4, O.OracleConfig.of(cfg), pro)
    check(y, ref, x, "bf16", "stack4 + prologue")
