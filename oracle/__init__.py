"""fp64 CPU oracle for the Krea 2 single-stream DiT block -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The HIP library never
links, loads or calls it, and it imports nothing from the HIP side: the two
share only the seeded input generators of ``datagen``, which hold none of
the block's arithmetic.

Parity status (what pins each function; see the tests under
``tests/test_oracle_*.py``):

* ``modulated_rmsnorm``, ``gated_gqa_attention``, ``swiglu_mlp``,
  ``gated_residual``, ``block_forward``, ``block_forward_rows``,
  ``stack_forward``: pinned by an independent scalar-loop brute force
  (``oracle.bruteforce``), by torch's own float64 CPU routines
  (``scaled_dot_product_attention``, ``rms_norm``, ``silu``, ``linear``)
  and by closed forms and invariants (one-key sequence returns the gated
  V, two-key softmax is a logistic, GQA equals MHA with replicated K/V
  heads, zero gates give the identity, scale = -1 gives h = shift,
  permutation equivariance, batch independence).
* ``time_embedding``: pinned by closed forms of the sinusoid at chosen t.
* ``timestep_modulation``: its arithmetic pinned by scalar loops over the
  brute-force embedding (and a zero W_t2 giving zero).  The pages name a
  sinusoidal time embedding and a per-block bias replacing per-block MLPs,
  but do not give the shared map from t to the modulation vector: the
  two-layer bias-free MLP is a reading (the HIP path implements the same
  reading).
* ``qk_rmsnorm``, ``rope_positions``, ``rope_angles``, ``apply_rope``,
  ``attention_prologue`` (the optional QKNorm + 3D axial RoPE): pinned by
  the scalar-loop brute force, by torch's float64 ``rms_norm``, by the
  rotation's closed forms (one pair turned by a known angle, norms kept,
  position 0 and text tokens unchanged, scores depending only on position
  differences along an axis) and by planted mistakes.  The axis split
  (32, 48, 48), the adjacent-pair convention and the base 10000 are
  readings of conventions the pages do not give.
* ``patchify``/``unpatchify``, ``embed_tokens``, ``final_mod``,
  ``final_layer``, ``flow_schedule``, ``euler_sample``,
  ``model_velocity`` (the stack's boundary layers and the rectified-flow
  sampler): pinned by explicit index loops for the patch layout and its
  round trip, by the schedule's closed forms, by exact integration of a
  straight-path velocity field (Euler lands on x0), and by torch routines
  for the norm; the layer conventions (16-channel latent, 2 x 2 patches,
  bias-free embeddings, the final modulation map, the shift form) are
  readings of conventions the pages do not give.
* ``block_forward_fp8``, ``stack_forward_fp8`` (the 8-bit block and stack):
  with the quantiser replaced by the identity they reproduce
  ``block_forward`` / ``stack_forward``; with row-wise e4m3 they depart
  from them by a few percent of the update.
* ``fp8_e4m3_round``, ``quantize_rows_fp8``, ``quantize_tensor_fp8``, ``gemm_fp8``, ``swiglu_fp8``
  (the 8-bit projections): pinned by an exhaustive nearest-value search over
  all finite e4m3 codes (ties to even), fixed points at representable
  values, the row maximum landing on +-448, and float64 products of the
  decoded values; ``swiglu_fp8`` also by a scalar loop with distinct W1 and
  W3 halves and scales (swapping the SiLU and linear roles fails it); e4m3
  with row-wise scales is a reading of the pages' 8-bit training (their
  scaling schemes, not an inference format).
* ``guided_velocity`` (classifier-free guidance): pinned by its special
  cases, which reduce to the pinned ``model_velocity`` (g = 1 the
  conditional, g = 0 the unconditional velocity, text without influence
  makes g irrelevant) and by a planted swap of the two roles; the use of
  caller-given unconditional text features is a reading.
* ``qkvg_projection`` (the column split Q | K | V | G): pinned by a scalar
  loop over every head and channel with a distinct value in every row
  block of W_qkvg.
* The zero-centred gain form ``(1 + w)`` of the RMSNorm is a reading of
  the pages (weight decay on a zero-centred parameter); the arithmetic
  under it is pinned as above.
"""
from .dit_oracle import (  # noqa: F401
    OracleConfig,
    Prologue,
    apply_rope,
    embed_tokens,
    euler_sample,
    fp8_e4m3_round,
    gemm_fp8,
    guided_velocity,
    quantize_rows_fp8,
    quantize_tensor_fp8,
    swiglu_fp8,
    final_layer,
    final_mod,
    flow_schedule,
    model_velocity,
    patchify,
    unpatchify,
    attention_prologue,
    qk_rmsnorm,
    rope_angles,
    rope_positions,
    block_forward,
    block_forward_rows,
    gated_gqa_attention,
    gated_residual,
    modulated_rmsnorm,
    qkvg_projection,
    split_modulation,
    stack_forward,
    stack_forward_fp8,
    swiglu_mlp,
    time_embedding,
    timestep_modulation,
)
