/*
 * dit.h -- C ABI of the MI355X (gfx950) forward pass of the Krea 2
 * single-stream DiT block and of a stack of such blocks.
 *
 * The block (page "Krea 2 技术报告", the Chinese translation of the Krea 2
 * technical report, section 架构 = architecture):
 *   - 架构 › 时间步条件化: AdaLN-style modulation whose shift/scale/gate come
 *     from one shared timestep vector plus a per-block tunable bias;
 *   - 架构 › 归一化: zero-centred RMSNorm as the pre-norm;
 *   - 架构 › Transformer块: grouped-query attention with a sigmoid output gate,
 *     single-stream (one set of weights over the joint text+image sequence),
 *     and a SwiGLU MLP;
 *   - 架构 › 残差设计: standard (here: gated) residual connections.
 * Positional terms and QKNorm are off by default; the *_ex entry points
 * add the pages' attention prologue (QKNorm and 3D axial RoPE, see
 * dit_prologue).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer unless marked (host).
 *   - All matrices are row-major.  Projection weights use the nn.Linear
 *     layout [out_features, in_features]: Y = X * W^T, no bias.
 *   - Activations are [batch, seq_len, hidden] = [T, hidden] with
 *     T = batch * seq_len; within a sample the image tokens come first,
 *     then the text tokens (their order does not change the result).
 *   - `dtype` (DIT_BF16 or DIT_F32) is the element type of x and of the
 *     four projection weights; modulation vectors, the modulation bias,
 *     the norm gains, t and the timestep-MLP weights are always float32.
 *     Arithmetic: bf16 operands with fp32 accumulation, fp32 softmax and
 *     norm statistics; the fp32 path computes everything in fp32.
 *   - Device pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work: results are valid once the stream has been
 *     synchronised.  Nothing is allocated or freed by the library, except
 *     the host-side timing events of dit_timer_*.
 *   - Every argument is checked before anything is enqueued; on a failed
 *     check nothing is launched and a status other than DIT_OK comes back.
 *     No exception or abort crosses the ABI.
 *   - Identical inputs give bitwise identical outputs (no atomics).
 *   - Calls on different streams are independent if each has its own
 *     workspace; one workspace used by two overlapping calls races.
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DIT_OK = 0,
  DIT_ERR_NULL = 1,        /* a required pointer is NULL                       */
  DIT_ERR_SHAPE = 2,       /* inconsistent or non-positive sizes, or aliasing  */
  DIT_ERR_UNSUPPORTED = 3, /* valid but not implemented (e.g. head_dim 96)     */
  DIT_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned          */
  DIT_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required          */
  DIT_ERR_DTYPE = 6,       /* unknown dtype                                    */
  DIT_ERR_HIP = 7          /* a HIP call failed; see dit_last_hip_error()      */
} dit_status;

typedef enum { DIT_F32 = 0, DIT_BF16 = 1 } dit_dtype;

/* Block dimensions.  Requirements: all sizes > 0; hidden == n_heads*head_dim;
 * n_heads % n_kv_heads == 0; n_heads / n_kv_heads in {1, 2, 4} (other
 * group sizes return DIT_ERR_UNSUPPORTED: no attention kernel exists for
 * them); head_dim == 128
 * for bf16, head_dim == 64 or 128 for f32; hidden % 8 == 0, hidden <= 8192;
 * ffn % 8 == 0; eps >= 0. */
typedef struct {
  int32_t batch;      /* B                                                  */
  int32_t seq_len;    /* L: joint image + text tokens per sample            */
  int32_t hidden;     /* D                                                  */
  int32_t n_heads;    /* H query heads (and gate heads)                     */
  int32_t n_kv_heads; /* Hkv key/value heads; query head h reads KV head    */
                      /* h / (H / Hkv) (contiguous groups)                  */
  int32_t head_dim;   /* d                                                  */
  int32_t ffn;        /* F: SwiGLU hidden width                             */
  float eps;          /* RMSNorm epsilon, inside the square root            */
  dit_dtype dtype;    /* element type of x and the projection weights       */
} dit_config;

/* One block's weights (host struct of device pointers).
 * w_qkvg rows: Q (H*d rows, head h = rows h*d..h*d+d-1) | K (Hkv*d) |
 *              V (Hkv*d) | G (H*d, the sigmoid gate logits, elementwise).  */
typedef struct {
  const void *w_qkvg;    /* [(2H + 2Hkv) * d, D]                               */
  const void *w_o;       /* [D, H*d]                                           */
  const void *w_13;      /* [2F, D]: rows 0..F-1 = W1 (through SiLU),           */
                         /*          rows F..2F-1 = W3 (linear branch)          */
  const void *w_2;       /* [D, F]                                             */
  const float *mod_bias; /* [6, D] fp32 per-block bias added to the shared     */
                         /* modulation: shift1, scale1, gate1, shift2,         */
                         /* scale2, gate2                                       */
  const float *norm1_w;  /* [D] fp32 zero-centred gain w (gain = 1 + w);        */
  const float *norm2_w;  /* NULL means w = 0                                    */
  const float *q_norm_w; /* [d] fp32 zero-centred QKNorm gains of the query and */
  const float *k_norm_w; /* key heads (used only with dit_prologue.qk_norm);    */
                         /* NULL means w = 0                                    */
} dit_block_weights;

/* Optional attention prologue (page "Krea 2 技术报告", 架构 › 归一化:
 * RMSNorm also as the QKNorm; 架构 › 位置编码: 3D axial RoPE with the head
 * dimensions assigned to frame, height and width, text tokens at RoPE index
 * zero).  Applied to every query and key head right after the QKVG
 * projection, before attention; V and the gate are untouched:
 *   qk_norm: q = q / sqrt(mean_d(q^2) + eps) * (1 + q_norm_w), k likewise
 *            with k_norm_w;
 *   rope:    the dimension pairs (2j, 2j+1) are rotated,
 *            (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a), where
 *            pair i of axis A (axes[A] dimensions, axes in the order frame,
 *            height, width) has a = pos_A * theta^(-2i / axes[A]).  Image
 *            token l < grid_h * grid_w of a sample (raster order) has
 *            pos = (0, l / grid_w, l % grid_w); every later token (text)
 *            has pos = (0, 0, 0).
 * The axis split, the adjacent-pair convention and theta are this library's
 * readings (the pages do not give them).  Requirements: qk_norm, rope in
 * {0, 1}; with rope: grid_h, grid_w >= 1, grid_h * grid_w <= seq_len, each
 * axes[i] >= 0 and even, axes[0] + axes[1] + axes[2] == head_dim, theta > 0
 * (else DIT_ERR_SHAPE). */
typedef struct {
  int32_t qk_norm;
  int32_t rope;
  int32_t grid_h, grid_w;
  int32_t axes[3];
  float theta;
} dit_prologue;

/* Kernel classes, for the timing hook. */
typedef enum {
  DIT_K_MODNORM = 0,   /* modulated RMSNorm (both norms)       */
  DIT_K_GEMM_QKVG = 1, /* h1 * W_qkvg^T                        */
  DIT_K_ATTN = 2,      /* gated GQA flash attention            */
  DIT_K_GEMM_O = 3,    /* Og * W_o^T                           */
  DIT_K_RESID = 4,     /* gated residual adds (both)           */
  DIT_K_GEMM_W13 = 5,  /* h2 * W_13^T with SwiGLU epilogue     */
  DIT_K_GEMM_W2 = 6,   /* U * W_2^T                            */
  DIT_K_TMOD = 7,      /* timestep embedding + modulation MLP  */
  DIT_K_PROLOGUE = 8,  /* QKNorm + RoPE on Q and K (if enabled) */
  DIT_K_QUANT = 9,     /* row-wise e4m3 quantisation of the activations (8-bit block) */
  DIT_K_COUNT = 10
} dit_kernel_kind;

/* Workspace bytes needed by dit_block_fwd for this configuration
 * (0 if cfg is invalid).  Holds the normalised activations, the Q|K|V|G
 * projection (later reused for the SwiGLU hidden U), the transposed V, the
 * gated attention output, the branch outputs, x1 (fp32) and, for bf16,
 * the fp32 partial tiles of projections whose last round of output tiles
 * is split along K (at most 256 tiles' worth, 64 MiB). */
size_t dit_workspace_size(const dit_config *cfg /* host */);

/* Workspace bytes needed by dit_stack_fwd: the block workspace plus one
 * fp32 [T, D] buffer that carries the residual stream between blocks. */
size_t dit_stack_workspace_size(const dit_config *cfg /* host */);

/* One block forward.
 *   x_in  [T, D] dtype; x_out [T, D] dtype (must not overlap x_in);
 *   mod   [B, 6, D] fp32: the shared modulation vector m of each sample
 *         (m[b] + w->mod_bias gives shift1, scale1, gate1, shift2, scale2,
 *         gate2);
 *   ws    workspace of at least dit_workspace_size(cfg) bytes, not
 *         overlapping any other argument.
 * Computes, per sample b:
 *   h1 = x / sqrt(mean(x^2) + eps) * (1 + norm1_w) * (1 + scale1) + shift1
 *   [Q|K|V|G] = h1 * W_qkvg^T
 *   Og_h = softmax(Q_h K_j^T / sqrt(d)) V_j * sigmoid(G_h),  j = h / (H/Hkv)
 *   x1 = x + gate1 * (Og * W_o^T)
 *   h2 = x1 / sqrt(mean(x1^2) + eps) * (1 + norm2_w) * (1 + scale2) + shift2
 *   x_out = x1 + gate2 * ((SiLU(h2 W1^T) * (h2 W3^T)) * W_2^T)
 * In the bf16 path the intermediates h, QKVG, Og, the branch outputs and
 * U are stored as bf16 between kernels; x1 is kept in fp32, so the
 * residual stream is rounded once, into x_out. */
dit_status dit_block_fwd(const dit_config *cfg /* host */, const dit_block_weights *w /* host */,
                         const void *x_in, void *x_out, const float *mod, void *ws,
                         size_t ws_bytes, void *stream);

/* n_blocks blocks applied in order, all with the same modulation vector
 * mod (one denoising step of the stack).  blocks is a host array of
 * n_blocks weight structs.  The residual stream between blocks is kept in
 * fp32 in the workspace and rounded to dtype once, into x_out.  ws needs
 * dit_stack_workspace_size(cfg) bytes.  n_blocks >= 1. */
dit_status dit_stack_fwd(const dit_config *cfg /* host */, int32_t n_blocks,
                         const dit_block_weights *blocks /* host [n_blocks] */, const void *x_in,
                         void *x_out, const float *mod, void *ws, size_t ws_bytes, void *stream);

/* dit_block_fwd / dit_stack_fwd with the attention prologue `pro` (host;
 * NULL = none, the same as the plain entry points) applied to Q and K
 * after every block's QKVG projection, with that block's q_norm_w and
 * k_norm_w.  Same workspace sizes. */
dit_status dit_block_fwd_ex(const dit_config *cfg /* host */, const dit_prologue *pro /* host */,
                            const dit_block_weights *w /* host */, const void *x_in, void *x_out,
                            const float *mod, void *ws, size_t ws_bytes, void *stream);
dit_status dit_stack_fwd_ex(const dit_config *cfg /* host */, const dit_prologue *pro /* host */,
                            int32_t n_blocks, const dit_block_weights *blocks /* host [n_blocks] */,
                            const void *x_in, void *x_out, const float *mod, void *ws, size_t ws_bytes,
                            void *stream);

/* The prologue as a step: transforms the Q and K column blocks of qkvg
 * [T, (2H+2Hkv)*d] (dtype, as produced by the QKVG projection) in place;
 * V and G are not touched.  q_norm_w, k_norm_w [d] fp32 or NULL. */
dit_status dit_qk_prologue(const dit_config *cfg /* host */, const dit_prologue *pro /* host */,
                           const float *q_norm_w, const float *k_norm_w, void *qkvg, void *stream);

/* ---- The layers around the stack and the sampler (page "Krea 2 技术报告":
 * the DiT runs on autoencoder latent tokens next to text-encoder features;
 * 训练 › 预训练: rectified-flow loss with v-parameterization, a shifted
 * sampling schedule whose inference shift is kept constant).  Readings (the
 * pages do not give them): latent z [B, C, 2*grid_h, 2*grid_w] fp32; 2 x 2
 * patches in raster order, patch vector index c*4 + dy*2 + dx; image
 * tokens first (grid_h * grid_w of them), then n_text text tokens, so
 * cfg->seq_len == grid_h * grid_w + n_text; bias-free embeddings
 * x_img = W_in p, x_txt = W_txt f; final layer on the image tokens:
 * h = rmsnorm(x) (1 + norm_f_w) (1 + scale_f) + shift_f with
 * [shift_f, scale_f] = W_tf SiLU(W_t1 e(t)), then v = W_out h
 * unpatchified. */
typedef struct {
  int32_t latent_ch;      /* C, even (4C is the patch vector)                  */
  int32_t grid_h, grid_w; /* latent patch grid, >= 1                           */
  int32_t n_text;         /* text tokens per sample, >= 0                      */
  int32_t txt_dim;        /* text feature width, % 8 == 0 (if n_text > 0)      */
  int32_t t_dim;          /* sinusoidal embedding width, even, 2..1024         */
} dit_model_config;

typedef struct {
  const void *w_in;      /* [D, 4C] dtype                                     */
  const void *w_txt;     /* [D, txt_dim] dtype (may be NULL when n_text == 0)  */
  const float *w_t1;     /* [D, t_dim] fp32 (as in dit_timestep_mod)          */
  const float *w_t2;     /* [6D, D] fp32 shared block modulation              */
  const float *w_tf;     /* [2D, D] fp32 final-norm shift / scale             */
  const float *norm_f_w; /* [D] fp32 zero-centred gain; NULL means 0          */
  const void *w_out;     /* [4C, D] dtype                                     */
} dit_model_weights;

/* Workspace bytes of dit_model_velocity and dit_sample (0 if invalid). */
size_t dit_model_workspace_size(const dit_config *cfg /* host */, const dit_model_config *mc /* host */);

/* The model as a velocity field at time t (host value, the same for every
 * sample): embeddings, the n_blocks-block stack (with the optional
 * prologue `pro`, NULL = none) under the shared modulation W_t2 SiLU(W_t1
 * e(t)), the final layer; v_out [B, C, Hl, Wl] fp32.  z [B, C, Hl, Wl]
 * fp32, txt [B, n_text, txt_dim] dtype.  v_out must not overlap z, txt or
 * ws. */
dit_status dit_model_velocity(const dit_config *cfg /* host */, const dit_model_config *mc /* host */,
                              const dit_prologue *pro /* host */, const dit_model_weights *mw /* host */,
                              int32_t n_blocks, const dit_block_weights *blocks /* host [n_blocks] */,
                              const float *z, float t, const void *txt, float *v_out, void *ws, size_t ws_bytes,
                              void *stream);

/* n_steps Euler steps of the rectified-flow sampler on z (in place, fp32):
 *   t_i = s u_i / (1 + (s - 1) u_i), u_i = 1 - i / n_steps (t_0 = 1, t_n = 0),
 *   z <- z + (t_{i+1} - t_i) v(z, t_i)
 * with v as in dit_model_velocity (dit_sample_cfg adds classifier-free
 * guidance).  n_steps >= 1, shift s > 0. */
dit_status dit_sample(const dit_config *cfg /* host */, const dit_model_config *mc /* host */,
                      const dit_prologue *pro /* host */, const dit_model_weights *mw /* host */, int32_t n_blocks,
                      const dit_block_weights *blocks /* host [n_blocks] */, float *z, int32_t n_steps,
                      float shift, const void *txt, void *ws, size_t ws_bytes, void *stream);

/* The sampler with classifier-free guidance (page "Krea 2 技术报告",
 * 训练 › 强化学习: guidance stays an optional control at inference; the
 * guidance of Ho and Salimans cited there): every step's velocity is
 *   v = v_u + guidance (v_c - v_u),
 * v_c the model's velocity under the text features txt, v_u under txt_null
 * (the caller's unconditional features, e.g. those of the empty prompt; the
 * pages do not say which), both evaluated as one batch of 2B samples (cfg
 * describes the B samples of z).  guidance = 1 gives dit_sample's steps
 * (up to rounding order), 0 the unconditional ones.  z [B, C, Hl, Wl] fp32
 * in place; txt, txt_null [B, n_text, txt_dim] dtype (txt_null may be NULL
 * only when n_text == 0).  Workspace: dit_sample_cfg_workspace_size bytes
 * (the model call at 2B, z twice and both text halves); it must not overlap
 * z, txt, txt_null or any weight.  Errors as dit_sample, plus DIT_ERR_SHAPE
 * for a non-finite guidance. */
size_t dit_sample_cfg_workspace_size(const dit_config *cfg /* host */, const dit_model_config *mc /* host */);
dit_status dit_sample_cfg(const dit_config *cfg /* host */, const dit_model_config *mc /* host */,
                          const dit_prologue *pro /* host */, const dit_model_weights *mw /* host */,
                          int32_t n_blocks, const dit_block_weights *blocks /* host [n_blocks] */, float *z,
                          int32_t n_steps, float shift, float guidance, const void *txt, const void *txt_null,
                          void *ws, size_t ws_bytes, void *stream);

/* Shared timestep modulation of every sample:
 *   e = [cos(1000 t f_i), sin(1000 t f_i)], f_i = 10000^(-i/(t_dim/2)),
 *   mod_out[b] = W_t2 * SiLU(W_t1 * e)  reshaped to [6, D].
 *   t [B] fp32; w_t1 [D, t_dim] fp32; w_t2 [6D, D] fp32; mod_out [B, 6, D].
 * t_dim even, 2 <= t_dim <= 1024.  ws needs B*D*4 bytes (dit_workspace_size
 * is always enough).  The pages name a sinusoidal time embedding and a
 * per-block bias in place of per-block MLPs (page "Krea 2 技术报告",
 * 架构 › 时间步条件化); the shared two-layer map is this library's reading. */
dit_status dit_timestep_mod(const dit_config *cfg /* host */, int32_t t_dim, const float *t,
                            const float *w_t1, const float *w_t2, float *mod_out, void *ws,
                            size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * dit_timestep_mod without the workspace argument.  Same kernels, same
 * result as dit_timestep_mod; the hidden activations [B, D] fp32 go to a
 * fixed scratch array of DIT_NOALLOC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on until the process ends (looked up on the current
 * device at the first call there; the stream must belong to the current
 * device).  Nothing is allocated or freed.  B * hidden * 4 bytes must fit
 * the scratch (else DIT_ERR_WORKSPACE: e.g. B <= 128 at hidden 4096).
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (each call writes all it reads): calls that overlap in
 * time on one GPU, on any streams, race. */
#define DIT_NOALLOC_SCRATCH_BYTES (2u << 20)
dit_status dit_timestep_mod_noalloc(const dit_config *cfg /* host */, int32_t t_dim, const float *t,
                                    const float *w_t1, const float *w_t2, float *mod_out, void *stream);

/* ---- the individual steps of the block (same kernels dit_block_fwd runs) */

/* Modulated zero-centred RMSNorm over rows of x [T, D] (page
 * "Krea 2 技术报告", 架构 › 归一化):
 *   h = x / sqrt(mean(x^2) + eps) * (1 + gain) * (1 + scale) + shift
 * with shift = mod[b][3*which] + bias[3*which], scale = mod[b][3*which+1]
 * + bias[3*which+1], b = row / seq_len.  which: 0 = first norm, 1 = second.
 * x_dtype may be DIT_F32 or cfg->dtype; h has cfg->dtype.  gain may be NULL. */
dit_status dit_modnorm(const dit_config *cfg /* host */, const void *x, dit_dtype x_dtype, void *h,
                       const float *mod, const float *bias, const float *gain, int32_t which,
                       void *stream);

/* C[M, N] = A[M, K] * W[N, K]^T in dtype with fp32 accumulation.
 * K % 8 == 0; M, N, K > 0; M*K, N*K elements each below 2^30. */
dit_status dit_gemm(dit_dtype dtype, int32_t m, int32_t n, int32_t k, const void *a, const void *w,
                    void *c, void *stream);

/* U[M, F] = SiLU(A W1^T) * (A W3^T) with W13 = [W1; W3] of shape [2F, K]
 * (page "Krea 2 技术报告", 架构 › Transformer块: SwiGLU MLP). */
dit_status dit_gemm_swiglu(dit_dtype dtype, int32_t m, int32_t f, int32_t k, const void *a,
                           const void *w13, void *u, void *stream);

/* The same products with an explicit tile configuration, for tuning and
 * tests: variant 0 forces whole 256 x 256 output tiles, 1 whole 192 x 256
 * tiles (the two whole-tile plans the block chooses from; 2 and above ->
 * DIT_ERR_UNSUPPORTED); group_m (0 = default, else 1..64) is
 * the number of row tiles walked together so their operands share an L2.
 * Every choice computes the same result up to fp32 summation order.
 * swiglu = 0: C[M, N] = A W^T with W [N, K]; swiglu = 1: as
 * dit_gemm_swiglu with F = n and W = W13 [2n, K].  The tile variant is
 * ignored by the fp32 path.  group_m outside 0..64 -> DIT_ERR_SHAPE. */
dit_status dit_gemm_variant(dit_dtype dtype, int32_t variant, int32_t group_m, int32_t swiglu,
                            int32_t m, int32_t n, int32_t k, const void *a, const void *w, void *c,
                            void *stream);

/* (host only, no GPU call) The configuration dit_block_fwd uses for a bf16
 * product of this shape when its workspace holds the partial tiles: tile
 * variant (as in dit_gemm_variant) and, when sk_tiles > 0, the split tail
 * of dit_gemm_splitk (256 x 256 tiles) with its fp32 partial bytes.  Non-
 * positive sizes or swiglu outside 0..1 -> DIT_ERR_SHAPE; NULL outputs ->
 * DIT_ERR_NULL. */
dit_status dit_gemm_plan(int32_t m, int32_t n, int32_t k, int32_t swiglu, int32_t *variant, int32_t *sk_tiles,
                         int32_t *segs, size_t *part_bytes);

/* The bf16 product (swiglu = 0: C = A W^T; 1: the SwiGLU hidden as in
 * dit_gemm_swiglu with F = n) on 256 x 256 output tiles (256 x 128 output
 * columns for SwiGLU), with the last sk_tiles tiles of the tile order each
 * split into segs contiguous ranges of K (64-element stages, segs <= the
 * stage count): every range is one workgroup that stores an fp32 partial
 * tile in ws, and a second pass sums the partials of each tile in range
 * order and applies the output step, so the result is deterministic.  This
 * is how the block keeps all CUs busy when the tile count leaves a mostly
 * empty last round; the block chooses sk_tiles and segs itself and this
 * entry point exposes the split for tests and tuning.
 * ws: sk_tiles * segs * 256 * 256 floats (may be NULL when that is 0),
 * 16-byte aligned, overlapping no operand.  dtype must be DIT_BF16
 * (DIT_F32 -> DIT_ERR_UNSUPPORTED).  sk_tiles outside 0..tiles, segs
 * outside 1..min(64, stages) -> DIT_ERR_SHAPE; ws too small ->
 * DIT_ERR_WORKSPACE. */
dit_status dit_gemm_splitk(dit_dtype dtype, int32_t swiglu, int32_t m, int32_t n, int32_t k, const void *a,
                           const void *w, void *c, int32_t sk_tiles, int32_t segs, void *ws, size_t ws_bytes,
                           void *stream);

/* ---- 8-bit projections (page "Krea 2 技术报告", 训练 › 预训练: 8-bit
 * training with row-wise scaling).  Format: OCP FP8 e4m3 (largest finite
 * 448), one float32 scale per row.
 *
 * Row-wise quantisation: for each row r of x [m, k] (dtype),
 *   amax = max |x[r, :]|,  scale[r] = amax / 448,
 *   q[r, c] = e4m3(x[r, c] * (448 / amax))  (round to nearest, ties even);
 * both divisions and the product are float32; an all-zero row gets
 * scale 1 and zeros.  q [m, k] bytes.  k % 16 == 0 (else
 * DIT_ERR_UNSUPPORTED); q and scale must not overlap x. */
dit_status dit_quantize_fp8(dit_dtype dtype, int32_t m, int32_t k, const void *x, void *q, float *scale,
                            void *stream);

/* Tensor-wise quantisation (the pages' 256 px scheme): one amax over all of
 * x, the same float32 scale amax / 448 and quotient x * (448 / amax) for
 * every element; scale [m] receives that scale for every row (so
 * dit_gemm_fp8 serves both schemes).  ws: 16 bytes of device scratch.
 * Three launches: row maxima (into scale), their maximum, the codes. */
dit_status dit_quantize_fp8_tensor(dit_dtype dtype, int32_t m, int32_t k, const void *x, void *q, float *scale,
                                   void *ws, void *stream);

/* C = (qa qw^T) * sa[:, None] * sw[None, :] in fp32 accumulation, stored
 * bf16: qa [m, k], qw [n, k] e4m3 bytes, sa [m], sw [n] fp32 (swiglu = 0);
 * or, swiglu = 1, the SwiGLU hidden U [m, n] = SiLU(C1) * C3 with
 * qw = [W1; W3] [2n, k] and sw [2n].  256 x 256 output tiles of
 * v_mfma_f32_16x16x128 f8 operations.  k % 16 == 0. */
dit_status dit_gemm_fp8(int32_t swiglu, int32_t m, int32_t n, int32_t k, const void *qa, const float *sa,
                        const void *qw, const float *sw, void *c, void *stream);

/* One block's weights for the 8-bit block (host struct of device pointers):
 * each projection matrix as row-wise e4m3 codes with one float32 scale per
 * row (W ~ codes * scale[row]; dit_quantize_fp8 of the bf16 matrix makes
 * them, dit_quantize_fp8_tensor the tensor-wise form), in the layouts of
 * dit_block_weights; the fp32 modulation bias and norm gains as there. */
typedef struct {
  const void *w_qkvg, *w_o, *w_13, *w_2;  /* e4m3 bytes                                  */
  const float *s_qkvg, *s_o, *s_13, *s_2; /* [rows] fp32 scales of the four matrices     */
  const float *mod_bias;                  /* [6, D]                                      */
  const float *norm1_w, *norm2_w;         /* [D] or NULL                                 */
} dit_block_weights_fp8;

/* Workspace bytes of dit_block_fwd_fp8 (0 if cfg is invalid for it). */
size_t dit_workspace_size_fp8(const dit_config *cfg /* host */);

/* The block with its four projections in 8 bits (page "Krea 2 技术报告",
 * 训练 › 预训练: 8-bit matrix products with tensor-wise / row-wise
 * scaling): the activation rows entering each product are quantised
 * row-wise to e4m3 as in dit_quantize_fp8 (h1 and h2 by the norm kernels
 * from their fp32 rows, Og and U from their bf16 storage) and multiplied
 * with the weight codes as in dit_gemm_fp8 (fp32 accumulation, both scales
 * applied); the rest is the bf16 block of dit_block_fwd (queries leave the
 * QKVG product pre-scaled for the attention; with seq_len a multiple of 64
 * the value heads go straight to the attention's V^T layout).
 * cfg->dtype must be DIT_BF16 (x_in, x_out bf16), head_dim 128, and hidden,
 * H*d and ffn multiples of 16 (else DIT_ERR_UNSUPPORTED / DIT_ERR_DTYPE).
 * Other arguments and errors as in dit_block_fwd. */
dit_status dit_block_fwd_fp8(const dit_config *cfg /* host */, const dit_block_weights_fp8 *w /* host */,
                             const void *x_in, void *x_out, const float *mod, void *ws, size_t ws_bytes,
                             void *stream);

/* Workspace bytes of dit_stack_fwd_fp8 (0 if cfg is invalid for it). */
size_t dit_stack_workspace_size_fp8(const dit_config *cfg /* host */);

/* n_blocks 8-bit blocks in order (blocks: host array of n_blocks weight
 * structs as for dit_block_fwd_fp8), all under the shared modulation mod:
 * the stack of dit_stack_fwd with every projection in row-wise e4m3.  The
 * residual stream between blocks stays fp32 in the workspace; x_in, x_out
 * bf16.  Arguments, checks and errors as in dit_block_fwd_fp8 and
 * dit_stack_fwd (n_blocks >= 1; the workspace must not overlap any input or
 * weight). */
dit_status dit_stack_fwd_fp8(const dit_config *cfg /* host */, int32_t n_blocks,
                             const dit_block_weights_fp8 *blocks /* host [n_blocks] */, const void *x_in,
                             void *x_out, const float *mod, void *ws, size_t ws_bytes, void *stream);

/* Gated grouped-query attention over the rows of qkvg [T, (2H+2Hkv)*d]
 * (column blocks Q | K | V | G, as produced by the QKVG projection):
 *   og[b, l, h*d:(h+1)*d] = softmax_keys(Q_h K_j^T / sqrt(d)) V_j * sigmoid(G_h)
 * within each sample, all keys, no mask (page "Krea 2 技术报告",
 * 架构 › Transformer块).  og [T, H*d] in cfg->dtype.  ws receives the
 * transposed V of every KV head (B*Hkv*d*ceil(L/64)*64 elements;
 * dit_workspace_size(cfg) is always enough) and must not overlap qkvg or og. */
dit_status dit_attention(const dit_config *cfg /* host */, const void *qkvg, void *og, void *ws,
                         size_t ws_bytes, void *stream);

/* dit_attention with the choice of query scaling.  q_prescaled = 1 (bf16
 * only): the query columns of qkvg already carry the factor
 * log2(e)/sqrt(d), applied in fp32 before their rounding to bf16 (this is
 * what the block path's projection epilogue produces), so the scores are in
 * base-2 units and the kernel applies no per-score scale:
 *   og = softmax_keys(2^(Q_h K_j^T) / sum) V_j * sigmoid(G_h),
 * the same attention as dit_attention's up to the rounding of the scaled Q.
 * q_prescaled = 0 is dit_attention.  Other values: DIT_ERR_SHAPE;
 * q_prescaled = 1 with cfg->dtype = DIT_F32: DIT_ERR_UNSUPPORTED. */
dit_status dit_attention_ex(const dit_config *cfg /* host */, const void *qkvg, void *og, void *ws,
                            size_t ws_bytes, int32_t q_prescaled, void *stream);

/* out = x + gate * y over rows of [T, D], gate = mod[b][3*which+2] +
 * bias[3*which+2] (page "Krea 2 技术报告", 架构 › 残差设计).
 * x_dtype and out_dtype may be DIT_F32 or cfg->dtype; y has cfg->dtype. */
dit_status dit_gated_residual(const dit_config *cfg /* host */, const void *x, dit_dtype x_dtype,
                              const void *y, const float *mod, const float *bias, int32_t which,
                              void *out, dit_dtype out_dtype, void *stream);

/* ---- diagnostics */

const char *dit_status_str(dit_status s);
/* hipError_t of this thread's last DIT_ERR_HIP (0 if none). */
int dit_last_hip_error(void);

/* Timing hook: while started, every launch of kernel class `kind` made by
 * this library is bracketed by a pair of HIP events recorded on the
 * launch's own stream (at most `capacity` launches).  dit_timer_stop
 * synchronises those events and returns the summed duration in ms and the
 * number of launches.  Global to the process; not for concurrent use. */
dit_status dit_timer_start(int32_t kind, int32_t capacity);
dit_status dit_timer_stop(double *total_ms /* host */, int32_t *n_launches /* host */);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H */
