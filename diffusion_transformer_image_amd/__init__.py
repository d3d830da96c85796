"""MI355X (gfx950) forward pass of the Krea 2 single-stream DiT block.

The compute lives in ``libdit.so`` (hand-written HIP kernels behind the C
ABI of ``include/dit.h``); this package is its ctypes binding.  Build the
library with ``python -m diffusion_transformer_image_amd.build``.
"""
from ._lib import (  # noqa: F401
    DIT_BF16,
    DIT_F32,
    EXPORTS,
    KERNEL_KINDS,
    LIB_PATH,
    BlockWeights,
    Prologue,
    Config,
    DitError,
    attention,
    block_fwd,
    block_fwd_ex,
    config_of,
    gated_residual,
    gemm,
    gemm_plan,
    gemm_splitk,
    gemm_swiglu,
    gemm_variant,
    lib,
    make_config,
    make_prologue,
    make_weights,
    modnorm,
    qk_prologue,
    stack_fwd,
    stack_fwd_ex,
    stack_workspace_size,
    timer_start,
    timer_stop,
    timestep_mod,
    workspace_size,
)
