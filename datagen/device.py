"""Upload / download of datagen arrays as torch tensors (marshalling only)."""
from __future__ import annotations

import numpy as np
import torch

from . import bf16_bits


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """float32 array -> contiguous device tensor of ``dtype`` ("bf16" or "f32").

    bf16 arrays from datagen are bf16-exact, so the bit patterns are
    transferred unchanged."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        t = torch.from_numpy(bf16_bits(a).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(a)
    else:
        raise ValueError(dtype)
    return t.to(device).contiguous()


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy array (exact for bf16 and fp32)."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def weights_to_device(w, dtype: str, device="cuda") -> dict:
    """datagen.BlockWeights -> dict of device tensors keyed like the C struct."""
    return {
        "w_qkvg": to_device(w.w_qkvg, dtype, device),
        "w_o": to_device(w.w_o, dtype, device),
        "w_13": to_device(w.w_13, dtype, device),
        "w_2": to_device(w.w_2, dtype, device),
        "mod_bias": to_device(w.mod_bias, "f32", device),
        "norm1_w": to_device(w.norm1_w, "f32", device),
        "norm2_w": to_device(w.norm2_w, "f32", device),
        **({"q_norm_w": to_device(w.q_norm_w, "f32", device)} if getattr(w, "q_norm_w", None) is not None else {}),
        **({"k_norm_w": to_device(w.k_norm_w, "f32", device)} if getattr(w, "k_norm_w", None) is not None else {}),
    }


def model_to_device(mw, dtype: str, device="cuda") -> dict:
    """datagen.ModelWeights -> dict of device tensors keyed like dit_model_weights."""
    return {
        "w_in": to_device(mw.w_in, dtype, device),
        "w_txt": to_device(mw.w_txt, dtype, device),
        "w_t1": to_device(mw.w_t1, "f32", device),
        "w_t2": to_device(mw.w_t2, "f32", device),
        "w_tf": to_device(mw.w_tf, "f32", device),
        "norm_f_w": to_device(mw.norm_f_w, "f32", device),
        "w_out": to_device(mw.w_out, dtype, device),
    }
