"""The block, the stack, the 8-bit block and the allocation-free timestep
modulation captured in a HIP graph (through torch.cuda.CUDAGraph): nothing
on these paths allocates, frees, clears memory with a memset or
synchronises, so the recorded launches replay as they ran.  Every replay,
with the program's own eager work and a synchronisation between replays and
new inputs copied into the captured buffers, is compared with the eager
result bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest

import datagen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    from datagen import device
    import diffusion_transformer_image_amd as dit
    dit.lib()
    return torch, device, dit


def small(n_image, n_text):
    return datagen.get_config("c1").replace(batch=2, n_image=n_image, n_text=n_text, hidden=512, n_heads=4,
                                            n_kv_heads=1, ffn=1368)


def replay_and_check(torch, graph, run_eager, out, set_inputs, n_inputs=3):
    """For each input set: copy it into the captured buffers, compute the
    eager result, replay the graph (eager work and a sync in between) and
    compare bit for bit."""
    for k in range(n_inputs):
        set_inputs(k)
        torch.cuda.synchronize()
        run_eager()
        torch.cuda.synchronize()
        ref = out.clone()
        out.zero_()
        scratch = torch.randn(1 << 20, device="cuda")  # unrelated eager work between runs
        scratch.mul_(2.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"graph replay {k} differs from the eager run"


@pytest.mark.parametrize("n_image,n_text", [(100, 28), (70, 27)])  # V^T by the projection / by its own pass
def test_block_step_in_a_graph(dev, n_image, n_text):
    torch, device, dit = dev
    cfg = small(n_image, n_text)
    c = dit.config_of(cfg)
    W = device.weights_to_device(datagen.block_weights(cfg), "bf16")
    t, w1, w2 = datagen.timestep_inputs(cfg)
    T, W1, W2 = device.to_device(t, "f32"), device.to_device(w1, "f32"), device.to_device(w2, "f32")
    X = device.to_device(datagen.activations(cfg).reshape(cfg.tokens, cfg.hidden), "bf16")
    Y = torch.empty_like(X)
    M = torch.empty((cfg.batch, 6, cfg.hidden), dtype=torch.float32, device="cuda")
    ws = torch.empty(dit.workspace_size(c), dtype=torch.uint8, device="cuda")

    def step():
        dit.timestep_mod(c, T, W1, W2, M, ws)
        dit.block_fwd(c, W, X, Y, M, ws)
    step()  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rng = np.random.default_rng(5)

    def set_inputs(k):
        X.copy_(torch.from_numpy(rng.standard_normal((cfg.tokens, cfg.hidden)).astype(np.float32)).to(X))
        T.copy_(torch.from_numpy(rng.random(cfg.batch).astype(np.float32)).to(T))
    replay_and_check(torch, g, step, Y, set_inputs)


def test_stack_and_noalloc_timestep_in_a_graph(dev):
    torch, device, dit = dev
    cfg = small(100, 28)
    c = dit.config_of(cfg)
    blocks = [device.weights_to_device(datagen.block_weights(cfg, i), "bf16") for i in range(3)]
    t, w1, w2 = datagen.timestep_inputs(cfg)
    T, W1, W2 = device.to_device(t, "f32"), device.to_device(w1, "f32"), device.to_device(w2, "f32")
    X = device.to_device(datagen.activations(cfg).reshape(cfg.tokens, cfg.hidden), "bf16")
    Y = torch.empty_like(X)
    M = torch.empty((cfg.batch, 6, cfg.hidden), dtype=torch.float32, device="cuda")
    ws = torch.empty(dit.stack_workspace_size(c), dtype=torch.uint8, device="cuda")

    def step():
        dit.timestep_mod_noalloc(c, T, W1, W2, M)
        dit.stack_fwd(c, blocks, X, Y, M, ws)
    step()  # the scratch address is taken here, outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rng = np.random.default_rng(6)

    def set_inputs(k):
        X.copy_(torch.from_numpy(rng.standard_normal((cfg.tokens, cfg.hidden)).astype(np.float32)).to(X))
        T.copy_(torch.from_numpy(rng.random(cfg.batch).astype(np.float32)).to(T))
    replay_and_check(torch, g, step, Y, set_inputs)


def test_fp8_block_in_a_graph(dev):
    torch, device, dit = dev
    cfg = small(100, 28).replace(ffn=1376)  # the 8-bit operands need widths in multiples of 16
    c = dit.config_of(cfg)
    W = device.weights_to_device(datagen.block_weights(cfg), "bf16")
    W8 = {n: W[n] for n in ("mod_bias", "norm1_w", "norm2_w")}
    for name, sname in (("w_qkvg", "s_qkvg"), ("w_o", "s_o"), ("w_13", "s_13"), ("w_2", "s_2")):
        W8[name] = torch.empty(W[name].shape, dtype=torch.uint8, device="cuda")
        W8[sname] = torch.empty(W[name].shape[0], dtype=torch.float32, device="cuda")
        dit.quantize_fp8(W[name], W8[name], W8[sname])
    X = device.to_device(datagen.activations(cfg).reshape(cfg.tokens, cfg.hidden), "bf16")
    Y = torch.empty_like(X)
    M = device.to_device(datagen.block_mod(cfg, strong=True), "f32")
    ws = torch.empty(dit.workspace_size_fp8(c), dtype=torch.uint8, device="cuda")

    def step():
        dit.block_fwd_fp8(c, W8, X, Y, M, ws)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rng = np.random.default_rng(7)

    def set_inputs(k):
        X.copy_(torch.from_numpy(rng.standard_normal((cfg.tokens, cfg.hidden)).astype(np.float32)).to(X))
    replay_and_check(torch, g, step, Y, set_inputs)
