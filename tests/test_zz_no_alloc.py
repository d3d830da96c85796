"""The entry point that allocates nothing (dit_timestep_mod_noalloc) against
the workspace entry point it mirrors (dit_timestep_mod), through the C ABI:
two calls in a row on the library's fixed scratch, the second with fewer
samples, each bitwise equal to the workspace path (same kernels, same
arithmetic) and within the fp32 bound of the oracle's timestep map."""
import numpy as np
import pytest

import datagen
from oracle import dit_oracle as O
from tests._parity import assert_parity

pytestmark = pytest.mark.gpu


def _run_both(torch, device, dit, cfg):
    t, w1, w2 = datagen.timestep_inputs(cfg)
    c = dit.config_of(cfg)
    T, W1, W2 = device.to_device(t, "f32"), device.to_device(w1, "f32"), device.to_device(w2, "f32")
    ref_dev = torch.empty((cfg.batch, 6, cfg.hidden), dtype=torch.float32, device="cuda")
    ws = torch.empty(cfg.batch * cfg.hidden * 4, dtype=torch.uint8, device="cuda")
    dit.timestep_mod(c, T, W1, W2, ref_dev, ws)
    out = torch.full((cfg.batch, 6, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
    dit.timestep_mod_noalloc(c, T, W1, W2, out)
    torch.cuda.synchronize()
    return device.to_numpy(out), device.to_numpy(ref_dev), O.timestep_modulation(t, w1, w2, cfg.hidden)


def test_noalloc_matches_workspace_entry_point_twice():
    import torch
    from datagen import device
    import diffusion_transformer_image_amd as dit
    dit.lib()
    # first call: 32 samples at hidden 4096 (512 KiB of scratch), then 2
    # samples, then a 1-sample fp32 block width: the scratch keeps the
    # previous call's contents, each call overwrites what it reads
    for name, batch in (("c1", 32), ("c3", 2), ("c0", 1)):
        cfg = datagen.get_config(name).replace(batch=batch)
        print(f"noalloc timestep map {name} B={batch}", flush=True)
        y, yref, ref = _run_both(torch, device, dit, cfg)
        np.testing.assert_array_equal(y, yref)
        assert_parity(y, ref, "f32", f"noalloc {name}")


def test_noalloc_rejects_more_than_the_scratch():
    import torch
    from datagen import device
    import diffusion_transformer_image_amd as dit
    cfg = datagen.get_config("c1").replace(batch=129)  # 129 * 4096 * 4 B > 2 MiB
    t, w1, w2 = datagen.timestep_inputs(cfg.replace(batch=1))
    c = dit.config_of(cfg)
    T = torch.zeros(129, dtype=torch.float32, device="cuda")
    out = torch.empty((129, 6, cfg.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(dit.DitError) as ei:
        dit.timestep_mod_noalloc(c, T, device.to_device(w1, "f32"), device.to_device(w2, "f32"), out)
    assert ei.value.name == "DIT_ERR_WORKSPACE"
