"""GPU parity of the whole block and stack against the fp64 oracle, plus the
invariants the definitions fix, all through the C ABI."""
import numpy as np
import pytest

import datagen
from oracle import dit_oracle as O
from tests._parity import assert_parity, assert_update_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    from datagen import device
    import diffusion_transformer_image_amd as dit
    dit.lib()
    return torch, device, dit


class Run:
    """Uploads one configuration's inputs and runs the block on the GPU."""

    def __init__(self, dev, cfg, strong=False, block=0):
        torch, device, dit = dev
        self.torch, self.device, self.dit = torch, device, dit
        self.cfg = cfg
        self.x = datagen.activations(cfg)
        self.w = datagen.block_weights(cfg, block)
        self.mod = datagen.block_mod(cfg, strong=strong)
        self.c = dit.config_of(cfg)
        self.X = device.to_device(self.x.reshape(cfg.tokens, cfg.hidden), cfg.dtype)
        self.W = device.weights_to_device(self.w, cfg.dtype)
        self.M = device.to_device(self.mod, "f32")
        self.ws = torch.empty(dit.workspace_size(self.c), dtype=torch.uint8, device="cuda")

    def forward(self, X=None, W=None, M=None):
        torch = self.torch
        X = self.X if X is None else X
        Y = torch.empty_like(X)
        self.dit.block_fwd(self.c, self.W if W is None else W, X, Y, self.M if M is None else M, self.ws)
        torch.cuda.synchronize()
        return self.device.to_numpy(Y).reshape(self.cfg.batch, self.cfg.seq_len, self.cfg.hidden)


def check_block(y, ref, x, dtype, what):
    e, c = assert_parity(y, ref, dtype, what + " output")
    eu, cu = assert_update_parity(y, ref, x, dtype, what + " update")
    print(f"{what}: output {e:.2e}/{c:.7f} update {eu:.2e}/{cu:.7f}")


@pytest.mark.parametrize("strong", [False, True])
def test_block_c0_full(dev, strong):
    cfg = datagen.get_config("c0")
    r = Run(dev, cfg, strong)
    y = r.forward()
    ref = O.block_forward(r.x, r.mod, r.w, O.OracleConfig.of(cfg))
    check_block(y, ref, r.x, "f32", "c0")


def sample_rows(L, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.r_[0, 1, 63, 64, L // 2, L - 65, L - 64, L - 1, rng.integers(0, L, 8)])


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c3b"])
@pytest.mark.parametrize("strong", [False, True])
def test_block_full_size_sampled(dev, name, strong):
    """Full-size block in the launch configuration the benchmark times;
    the oracle evaluates sampled query tokens of the first and last sample."""
    cfg = datagen.get_config(name)
    print(f"block {name} strong={strong}", flush=True)
    r = Run(dev, cfg, strong)
    y = r.forward()
    oc = O.OracleConfig.of(cfg)
    for b in sorted({0, cfg.batch - 1}):
        rows = sample_rows(cfg.seq_len, b + 31 * len(name))
        ref = O.block_forward_rows(r.x, r.mod, r.w, oc, b, rows)
        check_block(y[b, rows], ref, r.x[b, rows].astype(np.float64), "bf16", f"{name} b={b}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c1", "c2", "c3b"])
def test_block_full_size_every_output(dev, name):
    """256 px (B = 32, L = 512), 512 px (B = 8, L = 1280) and 768 x 1344
    (B = 2, L = 4544) in the launch configuration the benchmark times: every
    output and the update of the whole batch against the oracle (the 1024 px
    batch is compared element by element by bench.py's parity report)."""
    import time
    cfg = datagen.get_config(name)
    print(f"block {name} every output", flush=True)
    r = Run(dev, cfg)
    y = r.forward()
    t0 = time.time()
    ref = O.block_forward(r.x, r.mod, r.w, O.OracleConfig.of(cfg))
    print(f"oracle {name}: {time.time() - t0:.1f} s", flush=True)
    check_block(y, ref, r.x, "bf16", f"{name} every output")


def test_block_bf16_small_full_output(dev):
    """Every output of a small bf16 block (d = 128, ragged L) against the oracle."""
    cfg = datagen.get_config("c1").replace(batch=2, n_image=70, n_text=27, hidden=512, n_heads=4,
                                            n_kv_heads=1, ffn=1368)
    for strong in (False, True):
        r = Run(dev, cfg, strong)
        y = r.forward()
        ref = O.block_forward(r.x, r.mod, r.w, O.OracleConfig.of(cfg))
        check_block(y, ref, r.x, "bf16", f"small bf16 strong={strong}")


@pytest.mark.parametrize("base,batch,n_image,n_text,hidden,heads,kv,ffn", [
    ("c0", 5, 1, 0, 256, 4, 2, 688),        # fp32, one token per sample: softmax over one key
    ("c1", 3, 1, 0, 512, 4, 1, 1368),       # bf16, one token per sample
    ("c1", 2, 1, 1, 512, 4, 4, 1368),       # bf16, two tokens, MHA
    ("c1", 1, 60, 10, 8192, 64, 16, 2048),  # bf16 at the widest hidden the norms take (8192)
])
def test_block_degenerate_and_widest_shapes(dev, base, batch, n_image, n_text, hidden, heads, kv, ffn):
    """Every output of blocks at the edges of the supported shapes: a
    sequence of one token (each query attends only to itself, so the
    attention branch is sigma(G) V exactly), of two tokens, and hidden 8192
    (the norms' row of 8192 elements in registers, the residual and second
    norm as two passes)."""
    cfg = datagen.get_config(base).replace(batch=batch, n_image=n_image, n_text=n_text, hidden=hidden,
                                            n_heads=heads, n_kv_heads=kv, ffn=ffn)
    for strong in (False, True):
        r = Run(dev, cfg, strong)
        y = r.forward()
        ref = O.block_forward(r.x, r.mod, r.w, O.OracleConfig.of(cfg))
        check_block(y, ref, r.x, cfg.dtype, f"{base} B={batch} L={cfg.seq_len} D={hidden} strong={strong}")


@pytest.mark.parametrize("batch,n_image,n_text,hidden,heads,kv", [
    (2, 100, 28, 512, 4, 1),     # L = 128: a QKVG column tile holds K and V heads side by side
    (3, 130, 62, 1024, 8, 2),    # L = 192, a ragged last row tile of the projection
    (1, 4032, 64, 1024, 8, 4),   # L = 4096, one sample, 2 query heads per KV head
])
def test_block_bf16_value_heads_from_projection(dev, batch, n_image, n_text, hidden, heads, kv):
    """With L a multiple of 64 the QKVG product writes the value heads
    straight into the attention's transposed V layout (no V^T pass); every
    output of the block against the oracle (the 1024-key case sampled)."""
    cfg = datagen.get_config("c1").replace(batch=batch, n_image=n_image, n_text=n_text, hidden=hidden,
                                            n_heads=heads, n_kv_heads=kv, ffn=1368)
    assert cfg.seq_len % 64 == 0
    r = Run(dev, cfg, strong=True)
    y = r.forward()
    oc = O.OracleConfig.of(cfg)
    if cfg.seq_len <= 256:
        check_block(y, O.block_forward(r.x, r.mod, r.w, oc), r.x, "bf16", f"V^T by projection L={cfg.seq_len}")
    else:
        rows = sample_rows(cfg.seq_len, 3)
        ref = O.block_forward_rows(r.x, r.mod, r.w, oc, 0, rows)
        check_block(y[0, rows], ref, r.x[0, rows].astype(np.float64), "bf16", f"V^T by projection L={cfg.seq_len}")


def test_zero_gates_identity_bitwise(dev):
    for name in ("c0", "c1"):
        cfg = datagen.get_config(name).replace(batch=2, n_image=100, n_text=20)
        r = Run(dev, cfg, strong=True)
        mod = r.mod.copy()
        mod[:, 2] = -r.w.mod_bias[2]
        mod[:, 5] = -r.w.mod_bias[5]
        # m + bias is exactly 0 in fp32 for these rows
        y = r.forward(M=r.device.to_device(mod, "f32"))
        np.testing.assert_array_equal(y, r.x.astype(np.float64))


@pytest.mark.parametrize("name", ["c0", "c1"])
def test_gate_logits_far_below_zero_equal_zero_gate1(dev, name):
    """A block whose gate logits are all far below zero runs its attention
    branch to exactly zero, so it equals, bitwise, the same block with
    gate1 = 0.  The logits are driven there through the block's own
    projection: scale1 = -1 makes h1 = shift1 on every token, and the gate
    rows of W_qkvg are -sign(h1), so every gate logit is -sum|h1|."""
    torch, device, dit = dev
    cfg = datagen.get_config(name).replace(batch=1, n_image=100, n_text=30)
    r = Run(dev, cfg, strong=True)
    H, Hk, d, D = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden
    mod = r.mod.copy()
    mod[0, 1] = -1.0 - r.w.mod_bias[1]  # scale1 = -1 (to within an fp32 ulp)
    shift1 = mod[0, 0].astype(np.float64) + r.w.mod_bias[0]
    wq = r.w.w_qkvg.copy()
    wq[(H + 2 * Hk) * d:] = -np.sign(shift1)[None, :]
    logit = -np.sum(np.abs(datagen.bf16_round(shift1.astype(np.float32)) if cfg.dtype == "bf16" else shift1))
    assert logit < -100.0, logit  # sigmoid underflows to exactly 0 in fp32
    W = dict(r.W)
    W["w_qkvg"] = device.to_device(wq, cfg.dtype)
    ya = r.forward(W=W, M=device.to_device(mod, "f32"))
    mod0 = mod.copy()
    mod0[0, 2] = -r.w.mod_bias[2]  # m + bias = 0 exactly: gate1 = 0
    yb = r.forward(W=W, M=device.to_device(mod0, "f32"))
    np.testing.assert_array_equal(ya, yb)
    # and the x1 = x shortcut is what the oracle computes too
    w = datagen.BlockWeights(wq, r.w.w_o, r.w.w_13, r.w.w_2, r.w.mod_bias, r.w.norm1_w, r.w.norm2_w)
    ref = O.block_forward(r.x, mod0, w, O.OracleConfig.of(cfg))
    check_block(ya, ref, r.x, cfg.dtype, f"{name} gate logits -> -inf")


def test_gqa_equals_mha_with_replicated_kv(dev):
    torch, device, dit = dev
    cfg = datagen.get_config("c1").replace(batch=1, n_image=96, n_text=33, hidden=512, n_heads=4,
                                            n_kv_heads=1, ffn=1368)
    r = Run(dev, cfg, strong=True)
    y = r.forward()
    H, Hk, d = 4, 1, 128
    wq = r.w.w_qkvg
    k_rows, v_rows = wq[H * d:(H + Hk) * d], wq[(H + Hk) * d:(H + 2 * Hk) * d]
    w_mha = np.concatenate([wq[:H * d], np.tile(k_rows, (4, 1)), np.tile(v_rows, (4, 1)), wq[(H + 2 * Hk) * d:]])
    W = dict(r.W)
    W["w_qkvg"] = device.to_device(w_mha, "bf16")
    cm = dit.config_of(cfg.replace(n_kv_heads=4))
    Y = torch.empty_like(r.X)
    ws = torch.empty(dit.workspace_size(cm), dtype=torch.uint8, device="cuda")
    dit.block_fwd(cm, W, r.X, Y, r.M, ws)
    torch.cuda.synchronize()
    ym = device.to_numpy(Y).reshape(y.shape)
    # same arithmetic per head; only kernel instantiations differ
    assert_parity(ym - r.x, y - r.x, "bf16", "GQA vs MHA", maxabs=1e-3, cos_min=0.999999)


def test_permutation_equivariance(dev):
    torch, device, dit = dev
    cfg = datagen.get_config("c0").replace(batch=1)
    r = Run(dev, cfg, strong=True)
    y = r.forward()
    perm = np.random.default_rng(5).permutation(cfg.seq_len)
    Xp = device.to_device(r.x[:, perm].reshape(cfg.tokens, cfg.hidden), "f32")
    yp = r.forward(X=Xp)
    assert np.max(np.abs(yp - y[:, perm])) <= 1e-5 * np.max(np.abs(y))


def test_determinism_bitwise(dev):
    cfg = datagen.get_config("c1").replace(batch=2, n_image=300, n_text=33)
    r = Run(dev, cfg, strong=True)
    np.testing.assert_array_equal(r.forward(), r.forward())


def test_end_to_end_from_timestep(dev):
    """t -> timestep modulation -> block, each side with its own a0."""
    torch, device, dit = dev
    cfg = datagen.get_config("c0").replace(batch=2)
    r = Run(dev, cfg)
    t, w1, w2 = datagen.timestep_inputs(cfg)
    M = torch.empty((2, 6, cfg.hidden), dtype=torch.float32, device="cuda")
    dit.timestep_mod(r.c, device.to_device(t, "f32"), device.to_device(w1, "f32"), device.to_device(w2, "f32"), M, r.ws)
    y = r.forward(M=M)
    oc = O.OracleConfig.of(cfg)
    ref = O.block_forward(r.x, O.timestep_modulation(t, w1, w2, cfg.hidden), r.w, oc)
    check_block(y, ref, r.x, "f32", "t -> block")


# ------------------------------------------------------------------ stack
def run_stack(dev, cfg, blocks_np, x, mod):
    torch, device, dit = dev
    c = dit.config_of(cfg)
    X = device.to_device(x.reshape(cfg.tokens, cfg.hidden), cfg.dtype)
    Y = torch.empty_like(X)
    Ws = [device.weights_to_device(w, cfg.dtype) for w in blocks_np]
    ws = torch.empty(dit.stack_workspace_size(c), dtype=torch.uint8, device="cuda")
    dit.stack_fwd(c, Ws, X, Y, device.to_device(mod, "f32"), ws)
    torch.cuda.synchronize()
    return device.to_numpy(Y).reshape(x.shape)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stack_60_blocks_small(dev, dtype):
    """60 blocks with the stack's weight scaling, every output checked."""
    if dtype == "f32":
        cfg = datagen.get_config("c0").replace(n_blocks=60, out_std=0.02 / np.sqrt(120), batch=2)
    else:
        cfg = datagen.get_config("c4").replace(batch=2, n_image=64, n_text=16, hidden=256, n_heads=2,
                                                n_kv_heads=1, ffn=688)
    x = datagen.activations(cfg)
    mod = datagen.block_mod(cfg, strong=True)
    blocks = [datagen.block_weights(cfg, i) for i in range(60)]
    y = run_stack(dev, cfg, blocks, x, mod)
    ref = O.stack_forward(x, mod, blocks, 60, O.OracleConfig.of(cfg))
    check_block(y, ref, x, dtype, "stack60")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stack_one_block_equals_block(dev, dtype):
    """A one-block stack runs the block's kernels with the caller's input and
    output types (no fp32 stream, no join): the outputs equal the block
    entry point's bit for bit."""
    torch, device, dit = dev
    cfg = datagen.get_config("c1" if dtype == "bf16" else "c0").replace(
        batch=2, n_image=100, n_text=28, hidden=512, n_heads=4, n_kv_heads=1, head_dim=128, ffn=1376,
        dtype=dtype)
    r = Run(dev, cfg, strong=True)
    Yb, Ys = torch.empty_like(r.X), torch.empty_like(r.X)
    dit.block_fwd(r.c, r.W, r.X, Yb, r.M, r.ws)
    ws = torch.empty(dit.stack_workspace_size(r.c), dtype=torch.uint8, device="cuda")
    dit.stack_fwd(r.c, [r.W], r.X, Ys, r.M, ws)
    torch.cuda.synchronize()
    assert torch.equal(Yb, Ys)


def test_stack_full_dims_three_blocks(dev):
    cfg = datagen.get_config("c4").replace(n_image=200, n_text=56)
    x = datagen.activations(cfg)
    mod = datagen.block_mod(cfg, strong=False)
    blocks = [datagen.block_weights(cfg, i) for i in range(3)]
    y = run_stack(dev, cfg, blocks, x, mod)
    ref = O.stack_forward(x, mod, blocks, 3, O.OracleConfig.of(cfg))
    check_block(y, ref, x, "bf16", "stack3")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wide_hidden_unfused_passes(dev, dtype):
    """hidden = 6144: three staged fp32 vectors per sample no longer fit the
    64 KiB LDS window, so the block runs the residual and the second norm as
    two passes and the stack does not join blocks; one block and a stack of
    three, every output against the oracle."""
    cfg = datagen.get_config("c4" if dtype == "bf16" else "c0").replace(
        batch=2, n_image=40, n_text=9, hidden=6144, n_heads=48, n_kv_heads=12, head_dim=128, ffn=512,
        dtype=dtype, n_blocks=3, out_std=0.02 / np.sqrt(6))
    x = datagen.activations(cfg)
    mod = datagen.block_mod(cfg, strong=True)
    blocks = [datagen.block_weights(cfg, i) for i in range(3)]
    oc = O.OracleConfig.of(cfg)
    y1 = run_stack(dev, cfg, blocks[:1], x, mod)
    check_block(y1, O.block_forward(x, mod, blocks[0], oc), x, dtype, "wide block")
    y3 = run_stack(dev, cfg, blocks, x, mod)
    check_block(y3, O.stack_forward(x, mod, blocks, 3, oc), x, dtype, "wide stack3")


@pytest.mark.parametrize("live", [0, 59])
def test_stack_c4_full_size_one_live_block(dev, live):
    """The 60-block stack at its full 1024 px shape: 59 blocks run their full
    compute but have zero gates (exact identity), one block is live, so the
    oracle can evaluate sampled output tokens of that one block."""
    torch, device, dit = dev
    cfg = datagen.get_config("c4")
    print(f"stack c4 live={live}", flush=True)
    x = datagen.activations(cfg)
    mod = datagen.block_mod(cfg)
    w = datagen.block_weights(cfg, 0)
    W = device.weights_to_device(w, "bf16")
    dead_bias = w.mod_bias.copy()
    dead_bias[2] = -mod[0, 2]
    dead_bias[5] = -mod[0, 5]
    Wd = dict(W)
    Wd["mod_bias"] = device.to_device(dead_bias, "f32")
    blocks = [W if i == live else Wd for i in range(60)]
    c = dit.config_of(cfg)
    X = device.to_device(x.reshape(cfg.tokens, cfg.hidden), "bf16")
    Y = torch.empty_like(X)
    ws = torch.empty(dit.stack_workspace_size(c), dtype=torch.uint8, device="cuda")
    dit.stack_fwd(c, blocks, X, Y, device.to_device(mod, "f32"), ws)
    torch.cuda.synchronize()
    y = device.to_numpy(Y).reshape(x.shape)
    rows = sample_rows(cfg.seq_len, 7 + live)
    ref = O.block_forward_rows(x, mod, w, O.OracleConfig.of(cfg), 0, rows)
    check_block(y[0, rows], ref, x[0, rows].astype(np.float64), "bf16", f"c4 live block {live}")


@pytest.mark.timeout(900)
def test_stack_c4_width_60_live_blocks(dev):
    """The 60-block bf16 forward at the stack's full width (hidden 4096, 32 /
    8 heads of 128, SwiGLU 11008, W_o and W_2 ~ N(0, 0.02/sqrt(120))) with
    every block live and its own weights: 4 drawn projection sets, rows
    rolled per block (datagen.rolled_block_weights), each block's own
    modulation bias and norm gains.  One sample of 456 image + 64 text
    tokens (L = 520: eight whole 64-key tiles and a ragged ninth).  Every
    output and the update are checked against the oracle's stack, which
    streams the blocks one at a time; this is the error build-up of the
    fp32 residual stream over 60 live 4096-wide blocks."""
    import time
    torch, device, dit = dev
    cfg = datagen.get_config("c4").replace(n_image=456, n_text=64)
    n_sets, nb = 4, cfg.n_blocks
    assert nb == 60
    t0 = time.time()
    bases = [datagen.block_weights(cfg, s) for s in range(n_sets)]
    print(f"drew {n_sets} sets in {time.time() - t0:.1f} s", flush=True)
    dev_bases = [device.weights_to_device(b, "bf16") for b in bases]
    blocks = []
    for i in range(nb):
        base, k = dev_bases[i % n_sets], i // n_sets
        mb, n1, n2 = datagen.block_small_weights(cfg, i)
        blocks.append({name: torch.roll(base[name], datagen.ROLLS[name] * k, dims=0).contiguous()
                       for name in ("w_qkvg", "w_o", "w_13", "w_2")})
        blocks[-1].update(mod_bias=device.to_device(mb, "f32"), norm1_w=device.to_device(n1, "f32"),
                          norm2_w=device.to_device(n2, "f32"))
    del dev_bases
    x = datagen.activations(cfg)
    mod = datagen.block_mod(cfg)
    c = dit.config_of(cfg)
    X = device.to_device(x.reshape(cfg.tokens, cfg.hidden), "bf16")
    Y = torch.empty_like(X)
    ws = torch.empty(dit.stack_workspace_size(c), dtype=torch.uint8, device="cuda")
    dit.stack_fwd(c, blocks, X, Y, device.to_device(mod, "f32"), ws)
    torch.cuda.synchronize()
    y = device.to_numpy(Y).reshape(x.shape)
    del blocks, ws
    torch.cuda.empty_cache()
    print(f"GPU stack done at {time.time() - t0:.1f} s", flush=True)

    def get(i):
        if i % 10 == 0:
            print(f"oracle block {i} at {time.time() - t0:.1f} s", flush=True)
        return datagen.rolled_block_weights(cfg, i, bases)

    ref = O.stack_forward(x, mod, get, nb, O.OracleConfig.of(cfg))
    check_block(y, ref, x, "bf16", "stack60 full width, 60 live blocks")
