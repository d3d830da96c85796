"""GPU parity of the layers around the stack (patch embedding, text
projection, final norm and projection, unpatchify) and of the
rectified-flow Euler sampler against the fp64 oracle, through the C ABI."""
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


class ModelRun:
    def __init__(self, dev, cfg, n_blocks):
        torch, device, dit = dev
        self.torch, self.device, self.dit, self.cfg = torch, device, dit, cfg
        self.mw = datagen.model_weights(cfg)
        self.blocks = [datagen.block_weights(cfg, i) for i in range(n_blocks)]
        self.z = datagen.latent_noise(cfg)
        self.txt = datagen.text_features(cfg)
        self.c = dit.config_of(cfg)
        self.mc = dit.make_model_config(cfg.latent_ch, cfg.grid_h, cfg.grid_w, cfg.n_text, cfg.txt_dim, cfg.t_dim)
        self.MW = device.model_to_device(self.mw, cfg.dtype)
        self.BW = [device.weights_to_device(w, cfg.dtype) for w in self.blocks]
        self.Z = device.to_device(self.z, "f32")
        self.TXT = device.to_device(self.txt, cfg.dtype)
        self.ws = torch.empty(dit.model_workspace_size(self.c, self.mc), dtype=torch.uint8, device="cuda")
        self.oc = O.OracleConfig.of(cfg)

    def velocity(self, t):
        V = self.torch.empty_like(self.Z)
        self.dit.model_velocity(self.c, self.mc, self.MW, self.BW, self.Z, t, self.TXT, V, self.ws)
        self.torch.cuda.synchronize()
        return self.device.to_numpy(V)

    def ref_velocity(self, t, z=None):
        return O.model_velocity(self.z if z is None else z, t, self.txt, self.mw, self.blocks, len(self.blocks),
                                self.oc)


def tiny_f32():
    return datagen.get_config("c0").replace(n_image=64, n_text=16, grid_h=8, grid_w=8, latent_ch=4, txt_dim=32,
                                            w_std=0.1)


def small_bf16():
    return datagen.get_config("c1").replace(batch=2, n_image=70, n_text=27, hidden=512, n_heads=4, n_kv_heads=1,
                                            ffn=1368, grid_h=7, grid_w=10, latent_ch=16, txt_dim=64, w_std=0.05)


@pytest.mark.parametrize("t", [1.0, 0.37])
def test_velocity_tiny_f32(dev, t):
    r = ModelRun(dev, tiny_f32(), n_blocks=2)
    v = r.velocity(t)
    assert_parity(v, r.ref_velocity(t), "f32", f"velocity t={t}")


def test_velocity_small_bf16(dev):
    r = ModelRun(dev, small_bf16(), n_blocks=2)
    v = r.velocity(0.61)
    e, c = assert_parity(v, r.ref_velocity(0.61), "bf16", "velocity bf16")
    print(f"velocity bf16: {e:.2e} / {c:.7f}")


@pytest.mark.parametrize("n_steps,shift", [(1, 1.0), (3, 3.0)])
def test_sampler_tiny_f32(dev, n_steps, shift):
    """Euler steps on the device against the oracle's sampler over the same
    schedule (the latent state stays fp32 on both sides)."""
    r = ModelRun(dev, tiny_f32(), n_blocks=2)
    Z = r.Z.clone()
    r.dit.sample(r.c, r.mc, r.MW, r.BW, Z, n_steps, shift, r.TXT, r.ws)
    r.torch.cuda.synchronize()
    got = r.device.to_numpy(Z)
    ref = O.euler_sample(r.z, O.flow_schedule(n_steps, shift), lambda z, t: r.ref_velocity(t, z))
    assert_parity(got, ref, "f32", f"sampler {n_steps} steps")
    assert_parity(got - r.z, ref - r.z, "f32", f"sampler {n_steps} steps, change")


def test_sampler_small_bf16(dev):
    r = ModelRun(dev, small_bf16(), n_blocks=1)
    Z = r.Z.clone()
    r.dit.sample(r.c, r.mc, r.MW, r.BW, Z, 2, 3.0, r.TXT, r.ws)
    r.torch.cuda.synchronize()
    got = r.device.to_numpy(Z)
    ref = O.euler_sample(r.z, O.flow_schedule(2, 3.0), lambda z, t: r.ref_velocity(t, z))
    e, c = assert_parity(got - r.z, ref - r.z, "bf16", "sampler bf16 change")
    print(f"sampler bf16 change: {e:.2e} / {c:.7f}")


def run_cfg(r, n_steps, shift, g):
    """dit_sample_cfg on a copy of the run's latent; the unconditional text
    features are another seeded draw of the same shape."""
    txt_null = datagen.text_features(r.cfg.replace(seed=r.cfg.seed + 1))
    ws = r.torch.empty(r.dit.sample_cfg_workspace_size(r.c, r.mc), dtype=r.torch.uint8, device="cuda")
    Z = r.Z.clone()
    r.dit.sample_cfg(r.c, r.mc, r.MW, r.BW, Z, n_steps, shift, g, r.TXT, r.device.to_device(txt_null, r.cfg.dtype),
                     ws)
    r.torch.cuda.synchronize()
    ref = O.euler_sample(r.z, O.flow_schedule(n_steps, shift),
                         lambda z, t: O.guided_velocity(z, t, r.txt, txt_null, g, r.mw, r.blocks, len(r.blocks), r.oc))
    return r.device.to_numpy(Z), ref


@pytest.mark.parametrize("n_steps,g", [(1, 1.0), (2, 3.0), (2, 0.0)])
def test_sampler_cfg_tiny_f32(dev, n_steps, g):
    """Classifier-free guidance (conditional and unconditional halves as one
    batch of 2B) against the oracle's guided Euler steps: g = 1 is the plain
    sampler, g = 0 the unconditional one, g = 3 extrapolates."""
    r = ModelRun(dev, tiny_f32(), n_blocks=2)
    got, ref = run_cfg(r, n_steps, 2.0, g)
    assert_parity(got, ref, "f32", f"guided sampler g={g}")
    assert_parity(got - r.z, ref - r.z, "f32", f"guided sampler g={g}, change")


def test_sampler_cfg_small_bf16(dev):
    """bf16 with g = 4.  The guided velocity g v_c + (1 - g) v_u carries up
    to |g| + |1 - g| = 7 times the error of one bf16 velocity, so the bf16
    bounds scale by that amplification: max-abs <= 7 * 2e-2 max|ref| and
    1 - cos <= 7^2 * 1e-4 (the measurement sits far inside both)."""
    g = 4.0
    amp = abs(g) + abs(1.0 - g)
    r = ModelRun(dev, small_bf16(), n_blocks=1)
    got, ref = run_cfg(r, 2, 3.0, g)
    e, c = assert_parity(got - r.z, ref - r.z, "bf16", "guided sampler bf16 change", maxabs=amp * 2e-2,
                         cos_min=1.0 - amp * amp * 1e-4)
    print(f"guided sampler bf16 change: {e:.2e} / {c:.7f}")


def test_velocity_1024px_one_block(dev):
    """The 1024 px shapes (64 x 64 patch grid of a 16-channel latent, 512 text
    tokens of width 4096, hidden 4096), one block, batch 1: every element of
    the velocity against the oracle."""
    cfg = datagen.get_config("c3").replace(batch=1, w_std=0.02)
    print("velocity 1024 px, 1 block", flush=True)
    r = ModelRun(dev, cfg, n_blocks=1)
    v = r.velocity(0.8)
    e, c = assert_parity(v, r.ref_velocity(0.8), "bf16", "velocity 1024 px")
    print(f"velocity 1024 px: {e:.2e} / {c:.7f}")
