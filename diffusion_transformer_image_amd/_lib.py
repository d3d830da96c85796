"""ctypes binding of libdit.so (argument marshalling only).

Every function here forwards to the C ABI declared in ``include/dit.h``;
all arithmetic runs in the library's gfx950 kernels.  Torch tensors are used
for device memory and streams only: their ``data_ptr()`` and the current
HIP stream are passed through.  If the library has not been built the first
call raises ``RuntimeError``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Mapping, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdit.so")

DIT_F32, DIT_BF16 = 0, 1
STATUS = {0: "DIT_OK", 1: "DIT_ERR_NULL", 2: "DIT_ERR_SHAPE", 3: "DIT_ERR_UNSUPPORTED",
          4: "DIT_ERR_ALIGN", 5: "DIT_ERR_WORKSPACE", 6: "DIT_ERR_DTYPE", 7: "DIT_ERR_HIP"}
KERNEL_KINDS = {"modnorm": 0, "gemm_qkvg": 1, "attn": 2, "gemm_o": 3, "resid": 4,
                "gemm_w13": 5, "gemm_w2": 6, "tmod": 7, "prologue": 8, "quant": 9}

EXPORTS = (
    "dit_workspace_size", "dit_stack_workspace_size", "dit_block_fwd", "dit_stack_fwd",
    "dit_timestep_mod", "dit_modnorm", "dit_gemm", "dit_gemm_swiglu", "dit_gemm_variant", "dit_attention",
    "dit_gated_residual", "dit_status_str", "dit_last_hip_error", "dit_timer_start",
    "dit_timer_stop", "dit_gemm_splitk", "dit_gemm_plan", "dit_block_fwd_ex", "dit_stack_fwd_ex",
    "dit_qk_prologue", "dit_model_workspace_size", "dit_model_velocity", "dit_sample", "dit_quantize_fp8",
    "dit_gemm_fp8", "dit_quantize_fp8_tensor", "dit_attention_ex", "dit_timestep_mod_noalloc",
    "dit_workspace_size_fp8", "dit_block_fwd_fp8", "dit_sample_cfg_workspace_size", "dit_sample_cfg",
    "dit_stack_workspace_size_fp8", "dit_stack_fwd_fp8",
)


class DitError(RuntimeError):
    def __init__(self, status: int, where: str, hip: int = 0):
        self.status = status
        self.name = STATUS.get(status, str(status))
        msg = f"{where}: {self.name}"
        if status == 7:
            msg += f" (hipError {hip})"
        super().__init__(msg)


class Config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("eps", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class BlockWeights(ctypes.Structure):
    _fields_ = [("w_qkvg", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("w_13", ctypes.c_void_p),
                ("w_2", ctypes.c_void_p), ("mod_bias", ctypes.c_void_p),
                ("norm1_w", ctypes.c_void_p), ("norm2_w", ctypes.c_void_p),
                ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p)]


class BlockWeightsFp8(ctypes.Structure):
    _fields_ = [("w_qkvg", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("w_13", ctypes.c_void_p),
                ("w_2", ctypes.c_void_p), ("s_qkvg", ctypes.c_void_p), ("s_o", ctypes.c_void_p),
                ("s_13", ctypes.c_void_p), ("s_2", ctypes.c_void_p), ("mod_bias", ctypes.c_void_p),
                ("norm1_w", ctypes.c_void_p), ("norm2_w", ctypes.c_void_p)]


class ModelConfig(ctypes.Structure):
    """dit_model_config: latent and text shapes around the stack."""
    _fields_ = [("latent_ch", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("n_text", ctypes.c_int32), ("txt_dim", ctypes.c_int32), ("t_dim", ctypes.c_int32)]


class ModelWeights(ctypes.Structure):
    _fields_ = [("w_in", ctypes.c_void_p), ("w_txt", ctypes.c_void_p), ("w_t1", ctypes.c_void_p),
                ("w_t2", ctypes.c_void_p), ("w_tf", ctypes.c_void_p), ("norm_f_w", ctypes.c_void_p),
                ("w_out", ctypes.c_void_p)]


class Prologue(ctypes.Structure):
    """dit_prologue: QKNorm and 3D axial RoPE on Q and K."""
    _fields_ = [("qk_norm", ctypes.c_int32), ("rope", ctypes.c_int32), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("axes", ctypes.c_int32 * 3), ("theta", ctypes.c_float)]


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m diffusion_transformer_image_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        cfgp = ctypes.POINTER(Config)
        wp = ctypes.POINTER(BlockWeights)
        sig = {
            "dit_workspace_size": (sz, [cfgp]),
            "dit_workspace_size_fp8": (sz, [cfgp]),
            "dit_block_fwd_fp8": (i32, [cfgp, ctypes.POINTER(BlockWeightsFp8), vp, vp, vp, vp, sz, vp]),
            "dit_stack_workspace_size_fp8": (sz, [cfgp]),
            "dit_stack_fwd_fp8": (i32, [cfgp, i32, ctypes.POINTER(BlockWeightsFp8), vp, vp, vp, vp, sz, vp]),
            "dit_stack_workspace_size": (sz, [cfgp]),
            "dit_block_fwd": (i32, [cfgp, wp, vp, vp, vp, vp, sz, vp]),
            "dit_block_fwd_ex": (i32, [cfgp, ctypes.POINTER(Prologue), wp, vp, vp, vp, vp, sz, vp]),
            "dit_stack_fwd_ex": (i32, [cfgp, ctypes.POINTER(Prologue), i32, wp, vp, vp, vp, vp, sz, vp]),
            "dit_qk_prologue": (i32, [cfgp, ctypes.POINTER(Prologue), vp, vp, vp, vp]),
            "dit_model_workspace_size": (sz, [cfgp, ctypes.POINTER(ModelConfig)]),
            "dit_quantize_fp8": (i32, [i32, i32, i32, vp, vp, vp, vp]),
            "dit_quantize_fp8_tensor": (i32, [i32, i32, i32, vp, vp, vp, vp, vp]),
            "dit_gemm_fp8": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
            "dit_model_velocity": (i32, [cfgp, ctypes.POINTER(ModelConfig), ctypes.POINTER(Prologue),
                                         ctypes.POINTER(ModelWeights), i32, wp, vp, ctypes.c_float, vp, vp, vp, sz,
                                         vp]),
            "dit_sample": (i32, [cfgp, ctypes.POINTER(ModelConfig), ctypes.POINTER(Prologue),
                                 ctypes.POINTER(ModelWeights), i32, wp, vp, i32, ctypes.c_float, vp, vp, sz, vp]),
            "dit_sample_cfg_workspace_size": (sz, [cfgp, ctypes.POINTER(ModelConfig)]),
            "dit_sample_cfg": (i32, [cfgp, ctypes.POINTER(ModelConfig), ctypes.POINTER(Prologue),
                                     ctypes.POINTER(ModelWeights), i32, wp, vp, i32, ctypes.c_float, ctypes.c_float,
                                     vp, vp, vp, sz, vp]),
            "dit_stack_fwd": (i32, [cfgp, i32, wp, vp, vp, vp, vp, sz, vp]),
            "dit_timestep_mod": (i32, [cfgp, i32, vp, vp, vp, vp, vp, sz, vp]),
            "dit_timestep_mod_noalloc": (i32, [cfgp, i32, vp, vp, vp, vp, vp]),
            "dit_modnorm": (i32, [cfgp, vp, i32, vp, vp, vp, vp, i32, vp]),
            "dit_gemm": (i32, [i32, i32, i32, i32, vp, vp, vp, vp]),
            "dit_gemm_swiglu": (i32, [i32, i32, i32, i32, vp, vp, vp, vp]),
            "dit_gemm_variant": (i32, [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]),
            "dit_gemm_splitk": (i32, [i32, i32, i32, i32, i32, vp, vp, vp, i32, i32, vp, sz, vp]),
            "dit_gemm_plan": (i32, [i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                    ctypes.POINTER(i32), ctypes.POINTER(sz)]),
            "dit_attention": (i32, [cfgp, vp, vp, vp, sz, vp]),
            "dit_attention_ex": (i32, [cfgp, vp, vp, vp, sz, i32, vp]),
            "dit_gated_residual": (i32, [cfgp, vp, i32, vp, vp, vp, i32, vp, i32, vp]),
            "dit_status_str": (ctypes.c_char_p, [i32]),
            "dit_last_hip_error": (ctypes.c_int, []),
            "dit_timer_start": (i32, [i32, i32]),
            "dit_timer_stop": (i32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _LIB = L
    return _LIB


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DitError(status, where, lib().dit_last_hip_error() if status == 7 else 0)


# ------------------------------------------------------------------ marshalling
def _dtype_code(t) -> int:
    import torch
    if t == torch.bfloat16 or t == "bf16" or t == DIT_BF16:
        return DIT_BF16
    if t == torch.float32 or t == "f32" or t == DIT_F32:
        return DIT_F32
    raise ValueError(f"unsupported dtype {t}")


def _ptr(x) -> int | None:
    """Device address of a tensor (or a raw int address, or None)."""
    if x is None or isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not x.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(batch, seq_len, hidden, n_heads, n_kv_heads, head_dim, ffn, eps=1e-6,
                dtype="bf16") -> Config:
    return Config(batch, seq_len, hidden, n_heads, n_kv_heads, head_dim, ffn, eps,
                  _dtype_code(dtype))


def config_of(c, batch: int | None = None, seq_len: int | None = None) -> Config:
    """Config from any object with the block's dimension attributes."""
    return make_config(batch or c.batch, seq_len or c.seq_len, c.hidden, c.n_heads, c.n_kv_heads,
                       c.head_dim, c.ffn, c.eps, c.dtype)


def make_weights(w: Mapping) -> BlockWeights:
    return BlockWeights(_ptr(w["w_qkvg"]), _ptr(w["w_o"]), _ptr(w["w_13"]), _ptr(w["w_2"]),
                        _ptr(w["mod_bias"]), _ptr(w.get("norm1_w")), _ptr(w.get("norm2_w")),
                        _ptr(w.get("q_norm_w")), _ptr(w.get("k_norm_w")))


def make_prologue(qk_norm: bool = True, rope: bool = True, grid_h: int = 0, grid_w: int = 0,
                  axes=(32, 48, 48), theta: float = 10000.0) -> Prologue:
    return Prologue(int(qk_norm), int(rope), grid_h, grid_w, (ctypes.c_int32 * 3)(*axes), theta)


# ------------------------------------------------------------------ entry points
def workspace_size(cfg: Config) -> int:
    return lib().dit_workspace_size(ctypes.byref(cfg))


def stack_workspace_size(cfg: Config) -> int:
    return lib().dit_stack_workspace_size(ctypes.byref(cfg))


def block_fwd(cfg: Config, w: Mapping, x_in, x_out, mod, ws, stream=None) -> None:
    bw = make_weights(w)
    nbytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().dit_block_fwd(ctypes.byref(cfg), ctypes.byref(bw), _ptr(x_in), _ptr(x_out),
                               _ptr(mod), _ptr(ws), nbytes, _stream(stream)), "dit_block_fwd")


def workspace_size_fp8(cfg: Config) -> int:
    return lib().dit_workspace_size_fp8(ctypes.byref(cfg))


def make_weights_fp8(w: Mapping) -> BlockWeightsFp8:
    return BlockWeightsFp8(*[_ptr(w.get(k)) for k in ("w_qkvg", "w_o", "w_13", "w_2", "s_qkvg", "s_o", "s_13", "s_2",
                                                       "mod_bias", "norm1_w", "norm2_w")])


def block_fwd_fp8(cfg: Config, w: Mapping, x_in, x_out, mod, ws, stream=None) -> None:
    """The 8-bit block: w holds the e4m3 codes (w_qkvg, w_o, w_13, w_2, uint8)
    and their row scales (s_qkvg, s_o, s_13, s_2), plus mod_bias, norm1_w,
    norm2_w as for block_fwd."""
    bw = make_weights_fp8(w)
    nbytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().dit_block_fwd_fp8(ctypes.byref(cfg), ctypes.byref(bw), _ptr(x_in), _ptr(x_out), _ptr(mod),
                                   _ptr(ws), nbytes, _stream(stream)), "dit_block_fwd_fp8")


def stack_workspace_size_fp8(cfg: Config) -> int:
    return lib().dit_stack_workspace_size_fp8(ctypes.byref(cfg))


def stack_fwd_fp8(cfg: Config, blocks: Sequence[Mapping], x_in, x_out, mod, ws, stream=None) -> None:
    """n_blocks 8-bit blocks (each a mapping as for block_fwd_fp8)."""
    arr = (BlockWeightsFp8 * len(blocks))(*[make_weights_fp8(b) for b in blocks])
    nbytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().dit_stack_fwd_fp8(ctypes.byref(cfg), len(blocks), arr, _ptr(x_in), _ptr(x_out), _ptr(mod),
                                   _ptr(ws), nbytes, _stream(stream)), "dit_stack_fwd_fp8")


def block_fwd_ex(cfg: Config, pro: Prologue | None, w: Mapping, x_in, x_out, mod, ws, stream=None) -> None:
    bw = make_weights(w)
    nbytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().dit_block_fwd_ex(ctypes.byref(cfg), None if pro is None else ctypes.byref(pro),
                                  ctypes.byref(bw), _ptr(x_in), _ptr(x_out), _ptr(mod), _ptr(ws), nbytes,
                                  _stream(stream)), "dit_block_fwd_ex")


def stack_fwd_ex(cfg: Config, pro: Prologue | None, blocks: Sequence[Mapping], x_in, x_out, mod, ws,
                 stream=None) -> None:
    arr = (BlockWeights * len(blocks))(*[make_weights(b) for b in blocks])
    nbytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().dit_stack_fwd_ex(ctypes.byref(cfg), None if pro is None else ctypes.byref(pro), len(blocks),
                                  arr, _ptr(x_in), _ptr(x_out), _ptr(mod), _ptr(ws), nbytes, _stream(stream)),
           "dit_stack_fwd_ex")


def qk_prologue(cfg: Config, pro: Prologue, qkvg, q_norm_w=None, k_norm_w=None, stream=None) -> None:
    """QKNorm + RoPE in place on the Q and K heads of qkvg [T, (2H+2Hkv)*d]."""
    _check(lib().dit_qk_prologue(ctypes.byref(cfg), ctypes.byref(pro), _ptr(q_norm_w), _ptr(k_norm_w),
                                 _ptr(qkvg), _stream(stream)), "dit_qk_prologue")


def make_model_config(latent_ch: int, grid_h: int, grid_w: int, n_text: int, txt_dim: int,
                      t_dim: int = 256) -> ModelConfig:
    return ModelConfig(latent_ch, grid_h, grid_w, n_text, txt_dim, t_dim)


def make_model_weights(m: Mapping) -> ModelWeights:
    return ModelWeights(_ptr(m["w_in"]), _ptr(m.get("w_txt")), _ptr(m["w_t1"]), _ptr(m["w_t2"]),
                        _ptr(m["w_tf"]), _ptr(m.get("norm_f_w")), _ptr(m["w_out"]))


def model_workspace_size(cfg: Config, mc: ModelConfig) -> int:
    return lib().dit_model_workspace_size(ctypes.byref(cfg), ctypes.byref(mc))


def model_velocity(cfg: Config, mc: ModelConfig, mw: Mapping, blocks: Sequence[Mapping], z, t: float, txt,
                   v_out, ws, pro: Prologue | None = None, stream=None) -> None:
    arr = (BlockWeights * len(blocks))(*[make_weights(b) for b in blocks])
    m = make_model_weights(mw)
    nbytes = ws.numel() * ws.element_size()
    _check(lib().dit_model_velocity(ctypes.byref(cfg), ctypes.byref(mc), None if pro is None else ctypes.byref(pro),
                                    ctypes.byref(m), len(blocks), arr, _ptr(z), float(t), _ptr(txt), _ptr(v_out),
                                    _ptr(ws), nbytes, _stream(stream)), "dit_model_velocity")


def sample(cfg: Config, mc: ModelConfig, mw: Mapping, blocks: Sequence[Mapping], z, n_steps: int, shift: float, txt,
           ws, pro: Prologue | None = None, stream=None) -> None:
    """n_steps Euler steps of the rectified-flow sampler, z updated in place."""
    arr = (BlockWeights * len(blocks))(*[make_weights(b) for b in blocks])
    m = make_model_weights(mw)
    nbytes = ws.numel() * ws.element_size()
    _check(lib().dit_sample(ctypes.byref(cfg), ctypes.byref(mc), None if pro is None else ctypes.byref(pro),
                            ctypes.byref(m), len(blocks), arr, _ptr(z), n_steps, float(shift), _ptr(txt), _ptr(ws),
                            nbytes, _stream(stream)), "dit_sample")


def sample_cfg_workspace_size(cfg: Config, mc: ModelConfig) -> int:
    return lib().dit_sample_cfg_workspace_size(ctypes.byref(cfg), ctypes.byref(mc))


def sample_cfg(cfg: Config, mc: ModelConfig, mw: Mapping, blocks: Sequence[Mapping], z, n_steps: int, shift: float,
               guidance: float, txt, txt_null, ws, pro: Prologue | None = None, stream=None) -> None:
    """n_steps Euler steps with classifier-free guidance v_u + g (v_c - v_u), z updated in place."""
    arr = (BlockWeights * len(blocks))(*[make_weights(b) for b in blocks])
    m = make_model_weights(mw)
    nbytes = ws.numel() * ws.element_size()
    _check(lib().dit_sample_cfg(ctypes.byref(cfg), ctypes.byref(mc), None if pro is None else ctypes.byref(pro),
                                ctypes.byref(m), len(blocks), arr, _ptr(z), n_steps, float(shift), float(guidance),
                                _ptr(txt), _ptr(txt_null), _ptr(ws), nbytes, _stream(stream)), "dit_sample_cfg")


def stack_fwd(cfg: Config, blocks: Sequence[Mapping], x_in, x_out, mod, ws, stream=None) -> None:
    arr = (BlockWeights * len(blocks))(*[make_weights(b) for b in blocks])
    nbytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().dit_stack_fwd(ctypes.byref(cfg), len(blocks), arr, _ptr(x_in), _ptr(x_out),
                               _ptr(mod), _ptr(ws), nbytes, _stream(stream)), "dit_stack_fwd")


def timestep_mod(cfg: Config, t, w_t1, w_t2, mod_out, ws, t_dim: int = 256, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().dit_timestep_mod(ctypes.byref(cfg), t_dim, _ptr(t), _ptr(w_t1), _ptr(w_t2),
                                  _ptr(mod_out), _ptr(ws), nbytes, _stream(stream)),
           "dit_timestep_mod")


def timestep_mod_noalloc(cfg: Config, t, w_t1, w_t2, mod_out, t_dim: int = 256, stream=None) -> None:
    _check(lib().dit_timestep_mod_noalloc(ctypes.byref(cfg), t_dim, _ptr(t), _ptr(w_t1), _ptr(w_t2),
                                          _ptr(mod_out), _stream(stream)),
           "dit_timestep_mod_noalloc")


def modnorm(cfg: Config, x, h, mod, bias, gain, which: int, stream=None) -> None:
    _check(lib().dit_modnorm(ctypes.byref(cfg), _ptr(x), _dtype_code(x.dtype), _ptr(h), _ptr(mod),
                             _ptr(bias), _ptr(gain), which, _stream(stream)), "dit_modnorm")


def gemm(a, w, c, stream=None) -> None:
    m, k = a.shape
    n = w.shape[0]
    _check(lib().dit_gemm(_dtype_code(a.dtype), m, n, k, _ptr(a), _ptr(w), _ptr(c),
                          _stream(stream)), "dit_gemm")


def gemm_swiglu(a, w13, u, stream=None) -> None:
    m, k = a.shape
    f = w13.shape[0] // 2
    _check(lib().dit_gemm_swiglu(_dtype_code(a.dtype), m, f, k, _ptr(a), _ptr(w13), _ptr(u),
                                 _stream(stream)), "dit_gemm_swiglu")


def gemm_variant(variant: int, a, w, c, swiglu: bool = False, group_m: int = 0, stream=None) -> None:
    m, k = a.shape
    n = w.shape[0] // 2 if swiglu else w.shape[0]
    _check(lib().dit_gemm_variant(_dtype_code(a.dtype), variant, group_m, int(swiglu), m, n, k, _ptr(a),
                                  _ptr(w), _ptr(c), _stream(stream)), "dit_gemm_variant")


def gemm_splitk(a, w, c, sk_tiles: int, segs: int, ws=None, swiglu: bool = False, stream=None) -> None:
    """256 x 256 tiles with the last sk_tiles tiles split into segs K ranges
    (fp32 partials in ws: sk_tiles * segs * 256 * 256 floats)."""
    m, k = a.shape
    n = w.shape[0] // 2 if swiglu else w.shape[0]
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().dit_gemm_splitk(_dtype_code(a.dtype), int(swiglu), m, n, k, _ptr(a), _ptr(w), _ptr(c),
                                 sk_tiles, segs, _ptr(ws), nbytes, _stream(stream)), "dit_gemm_splitk")


def gemm_plan(m: int, n: int, k: int, swiglu: bool = False) -> dict:
    """The tile configuration the block uses for a bf16 product of this shape."""
    v, t, sg, pb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_size_t()
    _check(lib().dit_gemm_plan(m, n, k, int(swiglu), ctypes.byref(v), ctypes.byref(t), ctypes.byref(sg),
                               ctypes.byref(pb)), "dit_gemm_plan")
    return {"variant": v.value, "sk_tiles": t.value, "segs": sg.value, "part_bytes": pb.value}


def quantize_fp8(x, q, scale, stream=None) -> None:
    """Row-wise e4m3 quantisation of x [m, k] (bf16 or fp32) into q (uint8) and scale [m] fp32."""
    m, k = x.shape
    _check(lib().dit_quantize_fp8(_dtype_code(x.dtype), m, k, _ptr(x), _ptr(q), _ptr(scale), _stream(stream)),
           "dit_quantize_fp8")


def quantize_fp8_tensor(x, q, scale, ws, stream=None) -> None:
    """Tensor-wise e4m3 quantisation (one scale for all of x, repeated per row)."""
    m, k = x.shape
    _check(lib().dit_quantize_fp8_tensor(_dtype_code(x.dtype), m, k, _ptr(x), _ptr(q), _ptr(scale), _ptr(ws),
                                         _stream(stream)), "dit_quantize_fp8_tensor")


def gemm_fp8(qa, sa, qw, sw, c, swiglu: bool = False, stream=None) -> None:
    """bf16 C = (qa qw^T) sa sw (or the SwiGLU hidden with qw = [W1; W3])."""
    m, k = qa.shape
    n = qw.shape[0] // 2 if swiglu else qw.shape[0]
    _check(lib().dit_gemm_fp8(int(swiglu), m, n, k, _ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _ptr(c),
                              _stream(stream)), "dit_gemm_fp8")


def attention(cfg: Config, qkvg, og, ws, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().dit_attention(ctypes.byref(cfg), _ptr(qkvg), _ptr(og), _ptr(ws), nbytes, _stream(stream)),
           "dit_attention")


def attention_ex(cfg: Config, qkvg, og, ws, q_prescaled: bool, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().dit_attention_ex(ctypes.byref(cfg), _ptr(qkvg), _ptr(og), _ptr(ws), nbytes, int(q_prescaled),
                                  _stream(stream)), "dit_attention_ex")


def gated_residual(cfg: Config, x, y, mod, bias, which: int, out, stream=None) -> None:
    _check(lib().dit_gated_residual(ctypes.byref(cfg), _ptr(x), _dtype_code(x.dtype), _ptr(y),
                                    _ptr(mod), _ptr(bias), which, _ptr(out),
                                    _dtype_code(out.dtype), _stream(stream)),
           "dit_gated_residual")


def timer_start(kind: str, capacity: int) -> None:
    _check(lib().dit_timer_start(KERNEL_KINDS[kind], capacity), "dit_timer_start")


def timer_stop() -> tuple[float, int]:
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int32(0)
    _check(lib().dit_timer_stop(ctypes.byref(ms), ctypes.byref(n)), "dit_timer_stop")
    return ms.value, n.value
