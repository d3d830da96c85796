"""Seeded synthetic inputs for the single-stream DiT block path.

This module holds shapes, seeds, value distributions and the bf16
quantisation of drawn values -- and nothing of the block's own arithmetic.
Both the fp64 oracle (through the tests) and the HIP path consume the
arrays made here, so the two sides always see bit-identical inputs.

Recipe
------
* Every tensor has its own numpy PCG64 stream:
  ``SeedSequence(config.seed, spawn_key=(block, tensor_id))``.
* Values are drawn as float32 ``standard_normal`` (or ``random`` for t),
  scaled by the tensor's standard deviation in float32, then -- for the
  tensors stored in the model dtype -- rounded to bfloat16 with
  round-to-nearest-even.  The returned float32 arrays hold exactly the
  bf16 values, so upcasting them to float64 gives the oracle the same
  numbers the GPU reads.
* Model-dtype tensors: the activations x and the four projection weight
  matrices.  Always-fp32 tensors: the modulation vector, the per-block
  modulation bias, the two norm gains, the timestep t and the timestep-MLP
  weights.

Shapes follow the 256/512/1024 px stages of the resolution curriculum
described on the page "Krea 2 技术报告" (section 训练 › 预训练): a latent
of (px/16)^2 image tokens followed by the text tokens, one joint sequence.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Config", "CONFIGS", "get_config", "bf16_bits", "bf16_round", "bits_to_f32",
    "BlockWeights", "block_weights", "activations", "block_mod", "timestep_inputs",
    "qkvg_activations", "rng", "qk_norm_weights", "ModelWeights", "model_weights", "latent_noise",
    "text_features", "block_small_weights", "ROLLS", "rolled_block_weights",
]

# tensor ids used in the spawn keys (stable: changing one changes the data)
TID_X, TID_T, TID_WT1, TID_WT2, TID_MOD = 0, 1, 2, 3, 4
TID_WQKVG, TID_WO, TID_W13, TID_W2, TID_MODBIAS, TID_NORM1, TID_NORM2 = 10, 11, 12, 13, 14, 15, 16
TID_QNORM, TID_KNORM = 17, 18
TID_WIN, TID_WTXT, TID_WTF, TID_NORMF, TID_WOUT, TID_Z, TID_TXT = 40, 41, 42, 43, 44, 45, 46
TID_QKVG_ACT = 20
TID_GEMM_A, TID_GEMM_W = 30, 31


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload.  ``seq_len`` = n_image + n_text (image first)."""

    name: str
    batch: int
    n_image: int
    n_text: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    dtype: str  # "f32" or "bf16": dtype of x and of the projection weights
    seed: int
    eps: float = 1e-6
    n_blocks: int = 1
    w_std: float = 0.02  # every weight ~ N(0, w_std)
    out_std: float = 0.02  # W_o and W_2 ~ N(0, out_std)
    mod_std: float = 0.15  # synthetic modulation vector for block-level inputs
    t_dim: int = 256  # sinusoidal timestep-embedding width
    grid_h: int = 0  # latent patch grid of the image tokens (grid_h * grid_w = n_image)
    grid_w: int = 0
    latent_ch: int = 16  # autoencoder latent channels C; 2 x 2 patches -> 4C per token
    txt_dim: int = 4096  # width of the text-encoder features

    @property
    def seq_len(self) -> int:
        return self.n_image + self.n_text

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    @property
    def n_qkvg(self) -> int:
        return (2 * self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    def block_params(self) -> int:
        """Parameters of one block (projections + modulation bias + norm gains)."""
        d, f = self.hidden, self.ffn
        return (self.n_qkvg * d + d * self.n_heads * self.head_dim + 2 * f * d + d * f
                + 6 * d + 2 * d)

    def timestep_params(self) -> int:
        return self.hidden * self.t_dim + 6 * self.hidden * self.hidden


_BIG = dict(hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, ffn=11008, dtype="bf16")

CONFIGS = {
    # tiny fp32 block: 64 image + 16 text tokens
    "c0": Config("c0-tiny-f32", batch=1, n_image=64, n_text=16, hidden=256, n_heads=4,
                 n_kv_heads=2, head_dim=64, ffn=688, dtype="f32", seed=0, mod_std=0.04, grid_h=8, grid_w=8),
    # 256 px stage: 16x16 latent patches + 256 text tokens
    "c1": Config("c1-256px", batch=32, n_image=256, n_text=256, seed=1, grid_h=16, grid_w=16, **_BIG),
    # 512 px stage: 32x32 + 256
    "c2": Config("c2-512px", batch=8, n_image=1024, n_text=256, seed=2, grid_h=32, grid_w=32, **_BIG),
    # 1024 px stage: 64x64 + 512
    "c3": Config("c3-1024px", batch=2, n_image=4096, n_text=512, seed=3, grid_h=64, grid_w=64, **_BIG),
    # non-square 768x1344: 48x84 + 512
    "c3b": Config("c3b-768x1344", batch=2, n_image=4032, n_text=512, seed=1003, grid_h=48, grid_w=84,
                  **_BIG),
    # 60-block stack, one denoising step at 1024 px, batch 1
    "c4": Config("c4-stack60-1024px", batch=1, n_image=4096, n_text=512, seed=4, n_blocks=60,
                 out_std=0.02 / math.sqrt(2 * 60), grid_h=64, grid_w=64, **_BIG),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]


# ---------------------------------------------------------------- bf16 helpers
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    Inputs are finite by construction (normal draws), so NaN handling is
    not needed.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 array holding the nearest bf16 values (ties to even)."""
    return bits_to_f32(bf16_bits(a))


# ---------------------------------------------------------------- generators
def rng(cfg: Config, block: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(cfg.seed, spawn_key=(block, tid))))


def _normal(cfg: Config, block: int, tid: int, shape, std: float, model_dtype: bool) -> np.ndarray:
    a = rng(cfg, block, tid).standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    if model_dtype and cfg.dtype == "bf16":
        a = bf16_round(a)
    return a


@dataclasses.dataclass
class BlockWeights:
    """float32 arrays (bf16-exact for bf16 configs); nn.Linear [out, in] layout."""

    w_qkvg: np.ndarray  # [(2H+2Hkv)*d, D]: rows Q | K | V | G
    w_o: np.ndarray  # [D, H*d]
    w_13: np.ndarray  # [2F, D]: rows W1 (SiLU branch) then W3 (linear branch)
    w_2: np.ndarray  # [D, F]
    mod_bias: np.ndarray  # [6, D] fp32: shift1, scale1, gate1, shift2, scale2, gate2
    norm1_w: np.ndarray  # [D] fp32 zero-centred gain
    norm2_w: np.ndarray  # [D] fp32
    q_norm_w: np.ndarray | None = None  # [head_dim] fp32 zero-centred QKNorm gains (optional prologue)
    k_norm_w: np.ndarray | None = None


def block_weights(cfg: Config, block: int = 0) -> BlockWeights:
    d, f, hd = cfg.hidden, cfg.ffn, cfg.n_heads * cfg.head_dim
    return BlockWeights(
        w_qkvg=_normal(cfg, block, TID_WQKVG, (cfg.n_qkvg, d), cfg.w_std, True),
        w_o=_normal(cfg, block, TID_WO, (d, hd), cfg.out_std, True),
        w_13=_normal(cfg, block, TID_W13, (2 * f, d), cfg.w_std, True),
        w_2=_normal(cfg, block, TID_W2, (d, f), cfg.out_std, True),
        mod_bias=_normal(cfg, block, TID_MODBIAS, (6, d), cfg.w_std, False),
        norm1_w=_normal(cfg, block, TID_NORM1, (d,), cfg.w_std, False),
        norm2_w=_normal(cfg, block, TID_NORM2, (d,), cfg.w_std, False),
    )


def block_small_weights(cfg: Config, block: int):
    """Block ``block``'s modulation bias and two norm gains alone (the same
    streams ``block_weights`` draws them from), without drawing its 194 M
    projection weights."""
    d = cfg.hidden
    return (_normal(cfg, block, TID_MODBIAS, (6, d), cfg.w_std, False),
            _normal(cfg, block, TID_NORM1, (d,), cfg.w_std, False),
            _normal(cfg, block, TID_NORM2, (d,), cfg.w_std, False))


# Row rolls that turn a few drawn projection sets into many distinct blocks:
# block i uses set i % n_sets with the rows of each matrix rolled by
# ROLLS[name] * (i // n_sets) (plain re-arrangement of drawn values, so every
# block of a long full-width stack has its own matrices at the cost of
# drawing n_sets of them).
ROLLS = {"w_qkvg": 37, "w_o": 11, "w_13": 53, "w_2": 29}


def rolled_block_weights(cfg: Config, block: int, bases) -> BlockWeights:
    """Block ``block`` of a stack built from the drawn sets ``bases`` (a list
    of BlockWeights): set block % len(bases), projection rows rolled per
    ROLLS, and block ``block``'s own modulation bias and norm gains."""
    n = len(bases)
    base, k = bases[block % n], block // n
    mod_bias, n1, n2 = block_small_weights(cfg, block)
    return BlockWeights(
        w_qkvg=np.roll(base.w_qkvg, ROLLS["w_qkvg"] * k, axis=0),
        w_o=np.roll(base.w_o, ROLLS["w_o"] * k, axis=0),
        w_13=np.roll(base.w_13, ROLLS["w_13"] * k, axis=0),
        w_2=np.roll(base.w_2, ROLLS["w_2"] * k, axis=0),
        mod_bias=mod_bias, norm1_w=n1, norm2_w=n2)


def qk_norm_weights(cfg: Config, w: BlockWeights, block: int = 0) -> BlockWeights:
    """The same weights with QKNorm gains w_q, w_k [head_dim] ~ N(0, w_std) fp32."""
    return dataclasses.replace(
        w, q_norm_w=_normal(cfg, block, TID_QNORM, (cfg.head_dim,), cfg.w_std, False),
        k_norm_w=_normal(cfg, block, TID_KNORM, (cfg.head_dim,), cfg.w_std, False))


def activations(cfg: Config) -> np.ndarray:
    """x ~ N(0,1), [B, L, D], model dtype."""
    return _normal(cfg, 0, TID_X, (cfg.batch, cfg.seq_len, cfg.hidden), 1.0, True)


def block_mod(cfg: Config, strong: bool = False) -> np.ndarray:
    """Synthetic per-sample modulation vector m, [B, 6, D] fp32.

    Default std matches what the timestep MLP produces with N(0, 0.02)
    weights at this width (about 0.15 at D=4096, 0.04 at D=256);
    ``strong=True`` draws N(0, 1) so the block's update dominates x.
    """
    std = 1.0 if strong else cfg.mod_std
    return _normal(cfg, 0, TID_MOD + (100 if strong else 0), (cfg.batch, 6, cfg.hidden), std, False)


def timestep_inputs(cfg: Config):
    """t ~ U(0,1) per sample, W_t1 [D, t_dim] and W_t2 [6D, D] ~ N(0, w_std), all fp32."""
    t = rng(cfg, 0, TID_T).random(cfg.batch, dtype=np.float32)
    w_t1 = _normal(cfg, 0, TID_WT1, (cfg.hidden, cfg.t_dim), cfg.w_std, False)
    w_t2 = _normal(cfg, 0, TID_WT2, (6 * cfg.hidden, cfg.hidden), cfg.w_std, False)
    return t, w_t1, w_t2


def qkvg_activations(cfg: Config, std: float = 1.0) -> np.ndarray:
    """Direct [T, (2H+2Hkv)*d] Q|K|V|G rows for attention-step tests (gate logits ~ N(0,1))."""
    return _normal(cfg, 0, TID_QKVG_ACT, (cfg.tokens, cfg.n_qkvg), std, True)


def gemm_operands(cfg: Config, m: int, n: int, k: int, tag: int = 0):
    """A [m, k] ~ N(0,1) and W [n, k] ~ N(0, w_std) in the model dtype."""
    a = _normal(cfg, 1000 + tag, TID_GEMM_A, (m, k), 1.0, True)
    w = _normal(cfg, 1000 + tag, TID_GEMM_W, (n, k), cfg.w_std, True)
    return a, w


# ---------------------------------------------------------------- boundary layers and sampler inputs
@dataclasses.dataclass
class ModelWeights:
    """The layers around the block stack (float32 arrays; model-dtype ones bf16-exact)."""

    w_in: np.ndarray  # [D, 4C] patch embedding
    w_txt: np.ndarray  # [D, txt_dim] text-feature projection
    w_t1: np.ndarray  # [D, t_dim] fp32 timestep MLP, first layer
    w_t2: np.ndarray  # [6D, D] fp32 shared block modulation
    w_tf: np.ndarray  # [2D, D] fp32 final-norm shift / scale
    norm_f_w: np.ndarray  # [D] fp32 zero-centred gain of the final norm
    w_out: np.ndarray  # [4C, D] output projection to the patch vector


def model_weights(cfg: Config) -> ModelWeights:
    d, p = cfg.hidden, 4 * cfg.latent_ch
    _, w_t1, w_t2 = timestep_inputs(cfg)
    return ModelWeights(
        w_in=_normal(cfg, 0, TID_WIN, (d, p), cfg.w_std, True),
        w_txt=_normal(cfg, 0, TID_WTXT, (d, cfg.txt_dim), cfg.w_std, True),
        w_t1=w_t1, w_t2=w_t2,
        w_tf=_normal(cfg, 0, TID_WTF, (2 * d, d), cfg.w_std, False),
        norm_f_w=_normal(cfg, 0, TID_NORMF, (d,), cfg.w_std, False),
        w_out=_normal(cfg, 0, TID_WOUT, (p, d), cfg.w_std, True),
    )


def latent_noise(cfg: Config) -> np.ndarray:
    """Starting latent z ~ N(0, 1) [B, C, 2 grid_h, 2 grid_w] fp32."""
    return _normal(cfg, 0, TID_Z, (cfg.batch, cfg.latent_ch, 2 * cfg.grid_h, 2 * cfg.grid_w), 1.0, False)


def text_features(cfg: Config) -> np.ndarray:
    """Text-encoder features ~ N(0, 1) [B, n_text, txt_dim], model dtype."""
    return _normal(cfg, 0, TID_TXT, (cfg.batch, cfg.n_text, cfg.txt_dim), 1.0, True)
