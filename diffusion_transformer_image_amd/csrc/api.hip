// C ABI of libdit: argument checking, workspace carving, the block and
// stack drivers, and the timing hook.  Every entry point checks all of its
// arguments before the first HIP call; no exception crosses the ABI.
#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/dit.h"
#include "dit_kernels.h"

using namespace dit;

namespace {

thread_local int g_last_hip = 0;

dit_status hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return DIT_ERR_HIP;
}

// ---------------------------------------------------------------- fixed scratch
// Scratch of dit_timestep_mod_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  On the host the array's name is
// only a stand-in symbol, never a device address: host code passes the
// address hipGetSymbolAddress returns for the current device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) char scratch[DIT_NOALLOC_SCRATCH_BYTES];

namespace {

// The current device's copy of `scratch` (looked up once per device).
dit_status scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return DIT_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p) return hip_fail(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DIT_OK;
}

// ---------------------------------------------------------------- timing hook
struct Timer {
  std::mutex mu;
  bool active = false;
  int kind = -1;
  int capacity = 0;
  int count = 0;
  std::vector<hipEvent_t> ev0, ev1;
} g_timer;

template <typename F>
hipError_t timed(int kind, hipStream_t s, F &&launch) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_timer.mu);
    if (g_timer.active && g_timer.kind == kind && g_timer.count < g_timer.capacity) {
      e0 = g_timer.ev0[g_timer.count];
      e1 = g_timer.ev1[g_timer.count];
      ++g_timer.count;
    }
  }
  if (e0) {
    hipError_t e = hipEventRecord(e0, s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (e != hipSuccess) return e;
  if (e1) return hipEventRecord(e1, s);
  return hipSuccess;
}

// ---------------------------------------------------------------- checks
constexpr size_t kAlign = 256;
constexpr uint64_t kMaxSpan = 0x7FFFFFF0ull;  // buffer-descriptor byte range

size_t esize(dit_dtype t) { return t == DIT_BF16 ? 2 : 4; }
bool dtype_ok(int t) { return t == DIT_F32 || t == DIT_BF16; }
bool aligned(const void *p) { return ((uintptr_t)p & 15u) == 0; }
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

dit_status check_cfg(const dit_config *c) {
  if (!c) return DIT_ERR_NULL;
  if (!dtype_ok(c->dtype)) return DIT_ERR_DTYPE;
  if (c->batch <= 0 || c->seq_len <= 0 || c->hidden <= 0 || c->n_heads <= 0 ||
      c->n_kv_heads <= 0 || c->head_dim <= 0 || c->ffn <= 0 || !(c->eps >= 0.f))
    return DIT_ERR_SHAPE;
  if ((int64_t)c->n_heads * c->head_dim != c->hidden) return DIT_ERR_SHAPE;
  if (c->n_heads % c->n_kv_heads != 0) return DIT_ERR_SHAPE;
  // the attention kernels exist for 1, 2 and 4 query heads per KV head
  const int group = c->n_heads / c->n_kv_heads;
  if (group != 1 && group != 2 && group != 4) return DIT_ERR_UNSUPPORTED;
  if (c->dtype == DIT_BF16 ? c->head_dim != 128 : (c->head_dim != 64 && c->head_dim != 128))
    return DIT_ERR_UNSUPPORTED;
  if (c->hidden % 8 || c->ffn % 8) return DIT_ERR_UNSUPPORTED;
  if (c->hidden > 8192) return DIT_ERR_UNSUPPORTED;  // norms keep a row in registers, 3 vectors in LDS
  const uint64_t es = esize(c->dtype);
  const uint64_t nqkvg = (uint64_t)(2 * c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
  // byte ranges addressed through one buffer descriptor must stay below 2^31
  if ((uint64_t)c->seq_len * nqkvg * es > kMaxSpan) return DIT_ERR_UNSUPPORTED;
  if ((2ull * c->ffn + 256) * c->hidden * es > kMaxSpan) return DIT_ERR_UNSUPPORTED;
  if ((uint64_t)c->batch * c->seq_len > 0x7FFFFFFFull) return DIT_ERR_SHAPE;
  return DIT_OK;
}

struct Dims {
  size_t T, D, nqkvg, hd, F, es;
};
Dims dims(const dit_config *c) {
  Dims d;
  d.T = (size_t)c->batch * c->seq_len;
  d.D = c->hidden;
  d.nqkvg = (size_t)(2 * c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
  d.hd = (size_t)c->n_heads * c->head_dim;
  d.F = c->ffn;
  d.es = esize(c->dtype);
  return d;
}

struct BlockWs {
  char *h, *qkvg, *og, *br, *x1, *vt;
  float *part;        // fp32 K-split partials of the projections (bf16 only)
  size_t part_bytes;
  size_t bytes;
};

// fp32 partial bytes the default GEMM choices of one block need
size_t block_part_bytes(const dit_config *c) {
  if (c->dtype != DIT_BF16) return 0;
  const int T = c->batch * c->seq_len, D = c->hidden, F = c->ffn;
  const int nq = (2 * c->n_heads + 2 * c->n_kv_heads) * c->head_dim, hd = c->n_heads * c->head_dim;
  size_t b = gemm_choose(T, nq, D, false).part_bytes;
  b = std::max(b, gemm_choose(T, D, hd, false).part_bytes);
  b = std::max(b, gemm_choose(T, F, D, true).part_bytes);
  b = std::max(b, gemm_choose(T, D, F, false).part_bytes);
  return b;
}
BlockWs carve(const dit_config *c, void *ws) {
  const Dims d = dims(c);
  BlockWs w;
  char *p = (char *)ws;
  size_t off = 0;
  auto take = [&](size_t n) {
    char *r = p ? p + off : nullptr;
    off += round_up(n);
    return r;
  };
  w.h = take(d.T * d.D * d.es);
  w.qkvg = take(d.T * (d.nqkvg > d.F ? d.nqkvg : d.F) * d.es);
  w.og = take(d.T * d.hd * d.es);
  w.br = take(d.T * d.D * d.es);
  w.x1 = take(d.T * d.D * 4);  // x1 = x + gate1 * A stays fp32 (one rounding, at x_out)
  w.vt = take(attention_vt_bytes(c->dtype == DIT_F32, c->batch, c->seq_len, c->n_kv_heads, c->head_dim));
  w.part_bytes = block_part_bytes(c);
  w.part = (float *)take(w.part_bytes);
  const size_t tmod = (size_t)c->batch * c->hidden * 4;
  w.bytes = off > tmod ? off : tmod;
  return w;
}

// Workspace of the 8-bit block: the bf16 block's buffers but h (QKVG / U,
// Og, the branch output, x1, V^T; its K-split partials sized for the 8-bit
// products) plus the codes of one activation matrix [T, max(D, H*d, F)]
// bytes and its row scales [T] (the norms write their codes there).
struct Fp8Ws {
  BlockWs b;
  uint8_t *codes;
  float *scales;
  size_t bytes;
};
Fp8Ws carve_fp8(const dit_config *c, void *ws) {
  const Dims d = dims(c);
  Fp8Ws w;
  char *p = (char *)ws;
  size_t off = 0;
  auto take = [&](size_t n) {
    char *r = p ? p + off : nullptr;
    off += round_up(n);
    return r;
  };
  w.b.h = nullptr;
  w.b.qkvg = take(d.T * (d.nqkvg > d.F ? d.nqkvg : d.F) * d.es);
  w.b.og = take(d.T * d.hd * d.es);
  w.b.br = take(d.T * d.D * d.es);
  w.b.x1 = take(d.T * d.D * 4);
  w.b.vt = take(attention_vt_bytes(false, c->batch, c->seq_len, c->n_kv_heads, c->head_dim));
  const int T = (int)d.T, D = (int)d.D, F = (int)d.F, hd = (int)d.hd, nq = (int)d.nqkvg;
  size_t pb = gemm_choose_fp8(T, nq, D, false).part_bytes;
  pb = std::max(pb, gemm_choose_fp8(T, D, hd, false).part_bytes);
  pb = std::max(pb, gemm_choose_fp8(T, F, D, true).part_bytes);
  pb = std::max(pb, gemm_choose_fp8(T, D, F, false).part_bytes);
  w.b.part_bytes = pb;
  w.b.part = (float *)take(pb);
  w.codes = (uint8_t *)take(d.T * std::max(std::max(d.D, d.hd), d.F));
  w.scales = (float *)take(d.T * 4);
  const size_t tmod = (size_t)c->batch * c->hidden * 4;
  w.bytes = off > tmod ? off : tmod;
  w.b.bytes = w.bytes;
  return w;
}

dit_status check_cfg_fp8(const dit_config *c) {
  dit_status st = check_cfg(c);
  if (st != DIT_OK) return st;
  if (c->dtype != DIT_BF16) return DIT_ERR_DTYPE;
  if (c->hidden % 16 || (c->n_heads * c->head_dim) % 16 || c->ffn % 16) return DIT_ERR_UNSUPPORTED;
  // the 8-bit operands go through 32-bit buffer descriptors too
  if ((2ull * c->ffn + 256) * c->hidden > kMaxSpan) return DIT_ERR_UNSUPPORTED;
  return DIT_OK;
}

dit_status check_weights_fp8(const dit_config *c, const dit_block_weights_fp8 *w, const void *ws, size_t n) {
  if (!w) return DIT_ERR_NULL;
  if (!w->w_qkvg || !w->w_o || !w->w_13 || !w->w_2 || !w->s_qkvg || !w->s_o || !w->s_13 || !w->s_2 ||
      !w->mod_bias)
    return DIT_ERR_NULL;
  if (!aligned(w->w_qkvg) || !aligned(w->w_o) || !aligned(w->w_13) || !aligned(w->w_2) || !aligned(w->s_qkvg) ||
      !aligned(w->s_o) || !aligned(w->s_13) || !aligned(w->s_2) || !aligned(w->mod_bias) || !aligned(w->norm1_w) ||
      !aligned(w->norm2_w))
    return DIT_ERR_ALIGN;
  const Dims d = dims(c);
  const size_t D = d.D;
  if (overlap(ws, n, w->w_qkvg, d.nqkvg * D) || overlap(ws, n, w->w_o, D * d.hd) ||
      overlap(ws, n, w->w_13, 2 * d.F * D) || overlap(ws, n, w->w_2, D * d.F) ||
      overlap(ws, n, w->s_qkvg, d.nqkvg * 4) || overlap(ws, n, w->s_o, D * 4) || overlap(ws, n, w->s_13, 2 * d.F * 4) ||
      overlap(ws, n, w->s_2, D * 4) || overlap(ws, n, w->mod_bias, 6 * D * 4) ||
      overlap(ws, n, w->norm1_w, w->norm1_w ? D * 4 : 0) || overlap(ws, n, w->norm2_w, w->norm2_w ? D * 4 : 0))
    return DIT_ERR_SHAPE;
  return DIT_OK;
}

dit_status check_weights(const dit_block_weights *w) {
  if (!w) return DIT_ERR_NULL;
  if (!w->w_qkvg || !w->w_o || !w->w_13 || !w->w_2 || !w->mod_bias) return DIT_ERR_NULL;
  if (!aligned(w->w_qkvg) || !aligned(w->w_o) || !aligned(w->w_13) || !aligned(w->w_2) ||
      !aligned(w->mod_bias) || !aligned(w->norm1_w) || !aligned(w->norm2_w) || !aligned(w->q_norm_w) ||
      !aligned(w->k_norm_w))
    return DIT_ERR_ALIGN;
  return DIT_OK;
}

// True if [p, p + n) overlaps any buffer of one block's weights (the
// workspace must not alias an input: it is written before the weights are
// last read).
bool overlaps_weights(const dit_config *c, const dit_block_weights *w, const void *p, size_t n) {
  const Dims d = dims(c);
  const size_t D = d.D;
  return overlap(p, n, w->w_qkvg, d.nqkvg * D * d.es) || overlap(p, n, w->w_o, D * d.hd * d.es) ||
         overlap(p, n, w->w_13, 2 * d.F * D * d.es) || overlap(p, n, w->w_2, D * d.F * d.es) ||
         overlap(p, n, w->mod_bias, 6 * D * 4) || overlap(p, n, w->norm1_w, w->norm1_w ? D * 4 : 0) ||
         overlap(p, n, w->norm2_w, w->norm2_w ? D * 4 : 0) ||
         overlap(p, n, w->q_norm_w, w->q_norm_w ? (size_t)c->head_dim * 4 : 0) ||
         overlap(p, n, w->k_norm_w, w->k_norm_w ? (size_t)c->head_dim * 4 : 0);
}

// NULL is valid (no prologue)
dit_status check_prologue(const dit_config *c, const dit_prologue *p) {
  if (!p) return DIT_OK;
  if ((p->qk_norm != 0 && p->qk_norm != 1) || (p->rope != 0 && p->rope != 1)) return DIT_ERR_SHAPE;
  if (p->rope) {
    if (p->grid_h < 1 || p->grid_w < 1 || (int64_t)p->grid_h * p->grid_w > c->seq_len) return DIT_ERR_SHAPE;
    int64_t sum = 0;
    for (int i = 0; i < 3; ++i) {
      if (p->axes[i] < 0 || (p->axes[i] & 1)) return DIT_ERR_SHAPE;
      sum += p->axes[i];
    }
    if (sum != c->head_dim || !(p->theta > 0.f)) return DIT_ERR_SHAPE;
  }
  return DIT_OK;
}
bool prologue_on(const dit_prologue *p) { return p && (p->qk_norm || p->rope); }

#define DIT_TRY(expr)                     \
  do {                                    \
    hipError_t e_ = (expr);               \
    if (e_ != hipSuccess) return hip_fail(e_); \
  } while (0)

// The residual and norm passes can be one kernel (three staged fp32
// vectors per sample in LDS within the default 64 KiB window).
bool fused_resid_norm(int D) { return 3 * (size_t)D * sizeof(float) <= 64 * 1024; }

// One block, on the carved workspace.  x_in has dtype xin_f32 ? f32 : dtype;
// x_out has xout_f32 ? f32 : dtype; x1 (fp32) is stored in x1buf.
// h1_ready: ws.h already holds this block's first norm of x_in (the previous
// block of a stack computed it with its second residual).  defer_resid2:
// the block stops after the W2 product (M in ws.br, x1 in x1buf) and the
// caller applies the second residual.
dit_status run_block(const dit_config *c, const dit_prologue *pro, const dit_block_weights *w,
                     const void *x_in, bool xin_f32, void *x_out, bool xout_f32, const float *mod,
                     const BlockWs &ws, void *x1buf, hipStream_t s, bool h1_ready = false,
                     bool defer_resid2 = false) {
  const bool x1_f32 = true;
  const Dims d = dims(c);
  const bool f32 = c->dtype == DIT_F32;
  const int T = (int)d.T, D = (int)d.D, L = c->seq_len;
  if (!h1_ready) {
    DIT_TRY(timed(DIT_K_MODNORM, s, [&] {
      return launch_modnorm(xin_f32, f32, x_in, ws.h, mod, w->mod_bias, w->norm1_w, T, L, D, c->eps, 0, s);
    }));
  }
  // bf16: the attention's score factor rides on the query heads, applied in
  // fp32 before their one rounding (by the projection's epilogue, or by the
  // prologue pass, which would normalise it away), so the attention kernel
  // spends no per-score multiply
  const bool pre = !f32;
  const float qsc = pre ? attn_score_scale(c->head_dim) : 1.f;
  const bool pro_on = prologue_on(pro);
  // bf16 with whole 64-key tiles and no K split of the projection: its
  // epilogue writes the value heads straight into the attention's V^T
  // layout (no separate transpose pass, and V never reaches the QKVG rows)
  const int vc0 = (c->n_heads + c->n_kv_heads) * c->head_dim;
  const GemmVt gvt{ws.vt, vc0, vc0 + c->n_kv_heads * c->head_dim, L};
  const bool vt_by_gemm = !f32 && L % 64 == 0 && gemm_choose(T, (int)d.nqkvg, D, false).sk_tiles == 0;
  DIT_TRY(timed(DIT_K_GEMM_QKVG, s, [&] {
    return launch_gemm(f32, ws.h, w->w_qkvg, ws.qkvg, T, (int)d.nqkvg, D, s, -1, 0, ws.part, ws.part_bytes,
                       pre && !pro_on ? (int)d.hd : 0, qsc, vt_by_gemm ? &gvt : nullptr);
  }));
  if (pro_on) {
    DIT_TRY(timed(DIT_K_PROLOGUE, s, [&] {
      return launch_qk_prologue(f32, c->head_dim, ws.qkvg, w->q_norm_w, w->k_norm_w, T, L, c->n_heads,
                                c->n_kv_heads, pro->qk_norm, pro->rope, pro->grid_h, pro->grid_w, pro->axes,
                                pro->theta, c->eps, s, qsc);
    }));
  }
  DIT_TRY(timed(DIT_K_ATTN, s, [&] {
    return launch_attention(f32, c->head_dim, ws.qkvg, ws.vt, ws.og, c->batch, L, c->n_heads, c->n_kv_heads, s,
                            pre, vt_by_gemm);
  }));
  DIT_TRY(timed(DIT_K_GEMM_O, s, [&] {
    return launch_gemm(f32, ws.og, w->w_o, ws.br, T, D, (int)d.hd, s, -1, 0, ws.part, ws.part_bytes);
  }));
  if (fused_resid_norm(D)) {
    // x1 = x + gate1 * A (fp32) fused with h2 = modnorm(x1; norm 2)
    DIT_TRY(timed(DIT_K_RESID, s, [&] {
      return launch_resid_modnorm(xin_f32, f32, x_in, ws.br, (float *)x1buf, ws.h, mod, w->mod_bias, 0,
                                  w->mod_bias, w->norm2_w, 1, T, L, D, c->eps, s);
    }));
  } else {  // the three staged vectors would not fit the default LDS window
    DIT_TRY(timed(DIT_K_RESID, s, [&] {
      return launch_resid(xin_f32, f32, x1_f32, x_in, ws.br, x1buf, mod, w->mod_bias, T, L, D, 0, s);
    }));
    DIT_TRY(timed(DIT_K_MODNORM, s, [&] {
      return launch_modnorm(x1_f32, f32, x1buf, ws.h, mod, w->mod_bias, w->norm2_w, T, L, D, c->eps, 1, s);
    }));
  }
  DIT_TRY(timed(DIT_K_GEMM_W13, s, [&] {
    return launch_gemm_swiglu(f32, ws.h, w->w_13, ws.qkvg, T, (int)d.F, D, s, -1, 0, ws.part, ws.part_bytes);
  }));
  DIT_TRY(timed(DIT_K_GEMM_W2, s, [&] {
    return launch_gemm(f32, ws.qkvg, w->w_2, ws.br, T, D, (int)d.F, s, -1, 0, ws.part, ws.part_bytes);
  }));
  if (defer_resid2) return DIT_OK;
  DIT_TRY(timed(DIT_K_RESID, s, [&] {
    return launch_resid(x1_f32, f32, xout_f32, x1buf, ws.br, x_out, mod, w->mod_bias, T, L, D, 1, s);
  }));
  return DIT_OK;
}

// The 8-bit block: each product's activation rows quantised to e4m3 (one
// scale per row) and multiplied with the pre-quantised weight rows.
// x_in / x_out: bf16, or fp32 where xin_f32 / xout_f32 (the stack's
// residual stream); h1_ready and defer_resid2 as in run_block (h1's codes
// already in ws.codes; stop after the W2 product).
dit_status run_block_fp8(const dit_config *c, const dit_block_weights_fp8 *w, const void *x_in, void *x_out,
                         const float *mod, const Fp8Ws &ws, hipStream_t s, bool xin_f32 = false,
                         bool xout_f32 = false, bool h1_ready = false, bool defer_resid2 = false) {
  const Dims d = dims(c);
  const int T = (int)d.T, D = (int)d.D, L = c->seq_len, F = (int)d.F, hd = (int)d.hd, nq = (int)d.nqkvg;
  const BlockWs &b = ws.b;
  auto quant = [&](const void *x, int k) {
    return timed(DIT_K_QUANT, s, [&] { return launch_quantize_fp8(false, x, ws.codes, ws.scales, T, k, s); });
  };
  // the norms hand their rows over as codes quantised from fp32 (no bf16 h)
  if (!h1_ready) {
    DIT_TRY(timed(DIT_K_MODNORM, s, [&] {
      return launch_modnorm_fp8(xin_f32, x_in, ws.codes, ws.scales, mod, w->mod_bias, w->norm1_w, T, L, D, c->eps,
                                0, s);
    }));
  }
  // as in the bf16 block: the query columns leave the product pre-scaled
  // for the attention, and with whole 64-key tiles and no K split the value
  // heads go straight to V^T
  const float qsc = attn_score_scale(c->head_dim);
  const int vc0 = (c->n_heads + c->n_kv_heads) * c->head_dim;
  const GemmVt gvt{b.vt, vc0, vc0 + c->n_kv_heads * c->head_dim, L};
  const bool vt_by_gemm = L % 64 == 0 && gemm_choose_fp8(T, nq, D, false).sk_tiles == 0;
  DIT_TRY(timed(DIT_K_GEMM_QKVG, s, [&] {
    return launch_gemm_fp8(false, ws.codes, ws.scales, w->w_qkvg, w->s_qkvg, b.qkvg, T, nq, D, s, b.part,
                           b.part_bytes, hd, qsc, vt_by_gemm ? &gvt : nullptr);
  }));
  DIT_TRY(timed(DIT_K_ATTN, s, [&] {
    return launch_attention(false, c->head_dim, b.qkvg, b.vt, b.og, c->batch, L, c->n_heads, c->n_kv_heads, s,
                            true, vt_by_gemm);
  }));
  DIT_TRY(quant(b.og, hd));
  DIT_TRY(timed(DIT_K_GEMM_O, s, [&] {
    return launch_gemm_fp8(false, ws.codes, ws.scales, w->w_o, w->s_o, b.br, T, D, hd, s, b.part, b.part_bytes);
  }));
  if (fused_resid_norm(D)) {
    DIT_TRY(timed(DIT_K_RESID, s, [&] {
      return launch_resid_modnorm_fp8(xin_f32, x_in, b.br, (float *)b.x1, ws.codes, ws.scales, mod, w->mod_bias,
                                      0, w->mod_bias, w->norm2_w, 1, T, L, D, c->eps, s);
    }));
  } else {
    DIT_TRY(timed(DIT_K_RESID, s, [&] {
      return launch_resid(xin_f32, false, true, x_in, b.br, b.x1, mod, w->mod_bias, T, L, D, 0, s);
    }));
    DIT_TRY(timed(DIT_K_MODNORM, s, [&] {
      return launch_modnorm_fp8(true, b.x1, ws.codes, ws.scales, mod, w->mod_bias, w->norm2_w, T, L, D, c->eps, 1,
                                s);
    }));
  }
  DIT_TRY(timed(DIT_K_GEMM_W13, s, [&] {
    return launch_gemm_fp8(true, ws.codes, ws.scales, w->w_13, w->s_13, b.qkvg, T, F, D, s, b.part, b.part_bytes);
  }));
  DIT_TRY(quant(b.qkvg, F));
  DIT_TRY(timed(DIT_K_GEMM_W2, s, [&] {
    return launch_gemm_fp8(false, ws.codes, ws.scales, w->w_2, w->s_2, b.br, T, D, F, s, b.part, b.part_bytes);
  }));
  if (defer_resid2) return DIT_OK;
  DIT_TRY(timed(DIT_K_RESID, s, [&] {
    return launch_resid(true, false, xout_f32, b.x1, b.br, x_out, mod, w->mod_bias, T, L, D, 1, s);
  }));
  return DIT_OK;
}

// n_blocks 8-bit blocks: the fp32 residual stream between blocks after the
// carved block workspace, each block's second residual joined with the
// next block's first norm (whose codes the next QKVG product reads)
dit_status run_stack_fp8(const dit_config *cfg, int n_blocks, const dit_block_weights_fp8 *blocks,
                         const void *x_in, void *x_out, const float *mod, void *ws, hipStream_t s) {
  const Fp8Ws fw = carve_fp8(cfg, ws);
  char *xa = (char *)ws + fw.bytes;
  const Dims d = dims(cfg);
  const int T = (int)d.T, D = (int)d.D, L = cfg->seq_len;
  const bool chain = fused_resid_norm(D);
  for (int i = 0; i < n_blocks; ++i) {
    const bool first = i == 0, last = i == n_blocks - 1;
    dit_status st = run_block_fp8(cfg, &blocks[i], first ? x_in : xa, last ? x_out : xa, mod, fw, s, !first,
                                  !last, chain && !first, chain && !last);
    if (st != DIT_OK) return st;
    if (chain && !last) {
      hipError_t e = timed(DIT_K_RESID, s, [&] {
        return launch_resid_modnorm_fp8(true, fw.b.x1, fw.b.br, (float *)xa, fw.codes, fw.scales, mod,
                                        blocks[i].mod_bias, 1, blocks[i + 1].mod_bias, blocks[i + 1].norm1_w, 0, T,
                                        L, D, cfg->eps, s);
      });
      if (e != hipSuccess) return hip_fail(e);
    }
  }
  return DIT_OK;
}

// n_blocks blocks on a stack workspace (dit_stack_workspace_size bytes at ws)
dit_status run_stack(const dit_config *cfg, const dit_prologue *pro, int n_blocks, const dit_block_weights *blocks,
                     const void *x_in, void *x_out, const float *mod, void *ws, hipStream_t s) {
  const BlockWs bw = carve(cfg, ws);
  char *xa = (char *)ws + bw.bytes;  // fp32 residual stream between blocks
  const bool f32 = cfg->dtype == DIT_F32;
  const Dims d = dims(cfg);
  const int T = (int)d.T, D = (int)d.D, L = cfg->seq_len;
  // between two blocks, one pass: block i's second residual (x2 -> the fp32
  // stream) and block i+1's first norm of x2 (-> its h1)
  const bool chain = fused_resid_norm(D);
  for (int i = 0; i < n_blocks; ++i) {
    const bool first = i == 0, last = i == n_blocks - 1;
    dit_status st = run_block(cfg, pro, &blocks[i], first ? x_in : xa, first ? f32 : true, last ? x_out : xa,
                              last ? f32 : true, mod, bw, bw.x1, s, chain && !first, chain && !last);
    if (st != DIT_OK) return st;
    if (chain && !last) {
      hipError_t e = timed(DIT_K_RESID, s, [&] {
        return launch_resid_modnorm(true, f32, bw.x1, bw.br, (float *)xa, bw.h, mod, blocks[i].mod_bias, 1,
                                    blocks[i + 1].mod_bias, blocks[i + 1].norm1_w, 0, T, L, D, cfg->eps, s);
      });
      if (e != hipSuccess) return hip_fail(e);
    }
  }
  return DIT_OK;
}

// ---------------------------------------------------------------- model around the stack
dit_status check_model(const dit_config *c, const dit_model_config *mc, const dit_model_weights *mw) {
  if (!mc || !mw) return DIT_ERR_NULL;
  if (mc->latent_ch < 2 || (mc->latent_ch & 1) || mc->grid_h < 1 || mc->grid_w < 1 || mc->n_text < 0)
    return DIT_ERR_SHAPE;
  if ((int64_t)mc->grid_h * mc->grid_w + mc->n_text != c->seq_len) return DIT_ERR_SHAPE;
  if (mc->n_text > 0 && (mc->txt_dim <= 0 || mc->txt_dim % 8)) return DIT_ERR_SHAPE;
  if (mc->t_dim < 2 || mc->t_dim > 1024 || (mc->t_dim & 1)) return DIT_ERR_SHAPE;
  if (!mw->w_in || !mw->w_t1 || !mw->w_t2 || !mw->w_tf || !mw->w_out) return DIT_ERR_NULL;
  if (mc->n_text > 0 && !mw->w_txt) return DIT_ERR_NULL;
  if (!aligned(mw->w_in) || !aligned(mw->w_txt) || !aligned(mw->w_t1) || !aligned(mw->w_t2) ||
      !aligned(mw->w_tf) || !aligned(mw->norm_f_w) || !aligned(mw->w_out))
    return DIT_ERR_ALIGN;
  const uint64_t es = esize(c->dtype);
  if ((uint64_t)6 * c->hidden * c->hidden > 0x7FFFFFFFull) return DIT_ERR_UNSUPPORTED;
  if ((uint64_t)(c->hidden + 256) * mc->txt_dim * es > kMaxSpan) return DIT_ERR_UNSUPPORTED;
  if ((uint64_t)c->batch * 4 * mc->latent_ch * mc->grid_h * mc->grid_w > 0x7FFFFFFFull) return DIT_ERR_UNSUPPORTED;
  return DIT_OK;
}

struct ModelWs {
  char *stack, *x, *y, *p, *vt;
  float *mod, *modf, *zero, *zs, *t;
  size_t bytes;
};
ModelWs carve_model(const dit_config *c, const dit_model_config *mc, void *ws) {
  const Dims d = dims(c);
  const size_t nimg = (size_t)c->batch * mc->grid_h * mc->grid_w, pv = 4 * (size_t)mc->latent_ch;
  ModelWs w;
  char *p = (char *)ws;
  size_t off = 0;
  auto take = [&](size_t n) {
    char *r = p ? p + off : nullptr;
    off += round_up(n);
    return r;
  };
  w.stack = take(dit_stack_workspace_size(c));
  w.x = take(d.T * d.D * d.es);
  w.y = take(d.T * d.D * d.es);
  w.p = take(nimg * pv * d.es);
  w.vt = take(nimg * pv * d.es);
  w.mod = (float *)take((size_t)c->batch * 6 * d.D * 4);
  w.modf = (float *)take((size_t)c->batch * 2 * d.D * 4);
  w.zero = (float *)take(2 * d.D * 4);
  w.zs = (float *)take((size_t)c->batch * d.D * 4);
  w.t = (float *)take((size_t)c->batch * 4);
  w.bytes = off;
  return w;
}

// v(z, t) into vtok (token layout) -- everything but the unpatchify
dit_status model_tokens(const dit_config *c, const dit_model_config *mc, const dit_prologue *pro,
                        const dit_model_weights *mw, int n_blocks, const dit_block_weights *blocks, const float *z,
                        float t, const void *txt, const ModelWs &w, hipStream_t s) {
  const Dims d = dims(c);
  const bool f32 = c->dtype == DIT_F32;
  const int B = c->batch, L = c->seq_len, D = (int)d.D, C = mc->latent_ch;
  const int Hl = 2 * mc->grid_h, Wl = 2 * mc->grid_w, nimg = mc->grid_h * mc->grid_w, pv = 4 * C;
  DIT_TRY(launch_fill(w.t, t, (size_t)B, s));
  DIT_TRY(timed(DIT_K_TMOD, s, [&] {
    hipError_t e = launch_tmod(w.t, mw->w_t1, mw->w_t2, w.mod, w.zs, B, D, mc->t_dim, s);
    return e != hipSuccess ? e : launch_tmod_map(w.zs, mw->w_tf, w.modf, B, D, 2 * D, s);
  }));
  DIT_TRY(launch_patchify(f32, z, w.p, B, C, Hl, Wl, s));
  for (int b = 0; b < B; ++b) {
    DIT_TRY(launch_gemm(f32, w.p + (size_t)b * nimg * pv * d.es, mw->w_in, w.x + (size_t)b * L * D * d.es, nimg, D,
                        pv, s));
    if (mc->n_text > 0)
      DIT_TRY(launch_gemm(f32, (const char *)txt + (size_t)b * mc->n_text * mc->txt_dim * d.es, mw->w_txt,
                          w.x + ((size_t)b * L + nimg) * D * d.es, mc->n_text, D, mc->txt_dim, s));
  }
  dit_status st = run_stack(c, pro, n_blocks, blocks, w.x, w.y, w.mod, w.stack, s);
  if (st != DIT_OK) return st;
  DIT_TRY(launch_fill(w.zero, 0.f, 2 * d.D, s));
  for (int b = 0; b < B; ++b)  // final norm on the image rows; its output reuses x
    DIT_TRY(launch_modnorm(f32, f32, w.y + (size_t)b * L * D * d.es, w.x + (size_t)b * nimg * D * d.es,
                           w.modf + (size_t)b * 2 * D, w.zero, mw->norm_f_w, nimg, nimg, D, c->eps, 0, s));
  DIT_TRY(launch_gemm(f32, w.x, mw->w_out, w.vt, B * nimg, pv, D, s));
  return DIT_OK;
}

}  // namespace

extern "C" {

const char *dit_status_str(dit_status s) {
  switch (s) {
    case DIT_OK: return "ok";
    case DIT_ERR_NULL: return "null pointer";
    case DIT_ERR_SHAPE: return "invalid or inconsistent shape (or aliasing buffers)";
    case DIT_ERR_UNSUPPORTED: return "unsupported configuration";
    case DIT_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case DIT_ERR_WORKSPACE: return "workspace missing or too small";
    case DIT_ERR_DTYPE: return "unknown dtype";
    case DIT_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int dit_last_hip_error(void) { return g_last_hip; }

size_t dit_workspace_size(const dit_config *cfg) {
  if (check_cfg(cfg) != DIT_OK) return 0;
  return carve(cfg, nullptr).bytes;
}

size_t dit_stack_workspace_size(const dit_config *cfg) {
  if (check_cfg(cfg) != DIT_OK) return 0;
  const Dims d = dims(cfg);
  return carve(cfg, nullptr).bytes + round_up(d.T * d.D * 4);
}

dit_status dit_block_fwd_ex(const dit_config *cfg, const dit_prologue *pro, const dit_block_weights *w,
                            const void *x_in, void *x_out, const float *mod, void *ws, size_t ws_bytes,
                            void *stream) {
  dit_status st = check_cfg(cfg);
  if (st != DIT_OK) return st;
  if ((st = check_prologue(cfg, pro)) != DIT_OK) return st;
  if ((st = check_weights(w)) != DIT_OK) return st;
  if (!x_in || !x_out || !mod) return DIT_ERR_NULL;
  if (!ws) return DIT_ERR_WORKSPACE;
  if (!aligned(x_in) || !aligned(x_out) || !aligned(mod) || !aligned(ws)) return DIT_ERR_ALIGN;
  const Dims d = dims(cfg);
  const BlockWs need = carve(cfg, nullptr);
  if (ws_bytes < need.bytes) return DIT_ERR_WORKSPACE;
  const size_t xb = d.T * d.D * d.es;
  if (overlap(x_in, xb, x_out, xb)) return DIT_ERR_SHAPE;
  if (overlap(ws, need.bytes, x_in, xb) || overlap(ws, need.bytes, x_out, xb) ||
      overlap(ws, need.bytes, mod, (size_t)cfg->batch * 6 * cfg->hidden * 4) ||
      overlaps_weights(cfg, w, ws, need.bytes))
    return DIT_ERR_SHAPE;
  const BlockWs bw = carve(cfg, ws);
  const bool f32 = cfg->dtype == DIT_F32;
  return run_block(cfg, pro, w, x_in, f32, x_out, f32, mod, bw, bw.x1, (hipStream_t)stream);
}

dit_status dit_block_fwd(const dit_config *cfg, const dit_block_weights *w, const void *x_in,
                         void *x_out, const float *mod, void *ws, size_t ws_bytes, void *stream) {
  return dit_block_fwd_ex(cfg, nullptr, w, x_in, x_out, mod, ws, ws_bytes, stream);
}

size_t dit_workspace_size_fp8(const dit_config *cfg) {
  if (check_cfg_fp8(cfg) != DIT_OK) return 0;
  return carve_fp8(cfg, nullptr).bytes;
}

dit_status dit_block_fwd_fp8(const dit_config *cfg, const dit_block_weights_fp8 *w, const void *x_in, void *x_out,
                             const float *mod, void *ws, size_t ws_bytes, void *stream) {
  dit_status st = check_cfg_fp8(cfg);
  if (st != DIT_OK) return st;
  if (!x_in || !x_out || !mod || !w) return DIT_ERR_NULL;
  if (!ws) return DIT_ERR_WORKSPACE;
  if (!aligned(x_in) || !aligned(x_out) || !aligned(mod) || !aligned(ws)) return DIT_ERR_ALIGN;
  const Dims d = dims(cfg);
  const size_t need = carve_fp8(cfg, nullptr).bytes;
  if (ws_bytes < need) return DIT_ERR_WORKSPACE;
  if ((st = check_weights_fp8(cfg, w, ws, need)) != DIT_OK) return st;
  const size_t xb = d.T * d.D * d.es;
  if (overlap(x_in, xb, x_out, xb)) return DIT_ERR_SHAPE;
  if (overlap(ws, need, x_in, xb) || overlap(ws, need, x_out, xb) ||
      overlap(ws, need, mod, (size_t)cfg->batch * 6 * cfg->hidden * 4))
    return DIT_ERR_SHAPE;
  return run_block_fp8(cfg, w, x_in, x_out, mod, carve_fp8(cfg, ws), (hipStream_t)stream);
}

size_t dit_stack_workspace_size_fp8(const dit_config *cfg) {
  if (check_cfg_fp8(cfg) != DIT_OK) return 0;
  const Dims d = dims(cfg);
  return carve_fp8(cfg, nullptr).bytes + round_up(d.T * d.D * 4);
}

dit_status dit_stack_fwd_fp8(const dit_config *cfg, int32_t n_blocks, const dit_block_weights_fp8 *blocks,
                             const void *x_in, void *x_out, const float *mod, void *ws, size_t ws_bytes,
                             void *stream) {
  dit_status st = check_cfg_fp8(cfg);
  if (st != DIT_OK) return st;
  if (n_blocks <= 0) return DIT_ERR_SHAPE;
  if (!blocks || !x_in || !x_out || !mod) return DIT_ERR_NULL;
  if (!ws) return DIT_ERR_WORKSPACE;
  if (!aligned(x_in) || !aligned(x_out) || !aligned(mod) || !aligned(ws)) return DIT_ERR_ALIGN;
  const Dims d = dims(cfg);
  const size_t need = dit_stack_workspace_size_fp8(cfg);
  if (ws_bytes < need) return DIT_ERR_WORKSPACE;
  for (int i = 0; i < n_blocks; ++i)
    if ((st = check_weights_fp8(cfg, &blocks[i], ws, need)) != DIT_OK) return st;
  const size_t xb = d.T * d.D * d.es;
  if (overlap(x_in, xb, x_out, xb)) return DIT_ERR_SHAPE;
  if (overlap(ws, need, x_in, xb) || overlap(ws, need, x_out, xb) ||
      overlap(ws, need, mod, (size_t)cfg->batch * 6 * cfg->hidden * 4))
    return DIT_ERR_SHAPE;
  return run_stack_fp8(cfg, n_blocks, blocks, x_in, x_out, mod, ws, (hipStream_t)stream);
}

dit_status dit_stack_fwd_ex(const dit_config *cfg, const dit_prologue *pro, int32_t n_blocks,
                            const dit_block_weights *blocks, const void *x_in, void *x_out, const float *mod,
                            void *ws, size_t ws_bytes, void *stream) {
  dit_status st = check_cfg(cfg);
  if (st != DIT_OK) return st;
  if ((st = check_prologue(cfg, pro)) != DIT_OK) return st;
  if (n_blocks <= 0) return DIT_ERR_SHAPE;
  if (!blocks) return DIT_ERR_NULL;
  for (int i = 0; i < n_blocks; ++i)
    if ((st = check_weights(&blocks[i])) != DIT_OK) return st;
  if (!x_in || !x_out || !mod) return DIT_ERR_NULL;
  if (!ws) return DIT_ERR_WORKSPACE;
  if (!aligned(x_in) || !aligned(x_out) || !aligned(mod) || !aligned(ws)) return DIT_ERR_ALIGN;
  const Dims d = dims(cfg);
  const size_t need = dit_stack_workspace_size(cfg);
  if (ws_bytes < need) return DIT_ERR_WORKSPACE;
  const size_t xb = d.T * d.D * d.es;
  if (overlap(x_in, xb, x_out, xb)) return DIT_ERR_SHAPE;
  if (overlap(ws, need, x_in, xb) || overlap(ws, need, x_out, xb) ||
      overlap(ws, need, mod, (size_t)cfg->batch * 6 * cfg->hidden * 4))
    return DIT_ERR_SHAPE;
  for (int i = 0; i < n_blocks; ++i)
    if (overlaps_weights(cfg, &blocks[i], ws, need)) return DIT_ERR_SHAPE;
  return run_stack(cfg, pro, n_blocks, blocks, x_in, x_out, mod, ws, (hipStream_t)stream);
}

dit_status dit_stack_fwd(const dit_config *cfg, int32_t n_blocks, const dit_block_weights *blocks,
                         const void *x_in, void *x_out, const float *mod, void *ws, size_t ws_bytes,
                         void *stream) {
  return dit_stack_fwd_ex(cfg, nullptr, n_blocks, blocks, x_in, x_out, mod, ws, ws_bytes, stream);
}

dit_status dit_qk_prologue(const dit_config *cfg, const dit_prologue *pro, const float *q_norm_w,
                           const float *k_norm_w, void *qkvg, void *stream) {
  dit_status st = check_cfg(cfg);
  if (st != DIT_OK) return st;
  if (!pro || !qkvg) return DIT_ERR_NULL;
  if ((st = check_prologue(cfg, pro)) != DIT_OK) return st;
  if (!aligned(qkvg) || !aligned(q_norm_w) || !aligned(k_norm_w)) return DIT_ERR_ALIGN;
  const Dims d = dims(cfg);
  if (overlap(qkvg, d.T * d.nqkvg * d.es, q_norm_w, q_norm_w ? cfg->head_dim * 4 : 0) ||
      overlap(qkvg, d.T * d.nqkvg * d.es, k_norm_w, k_norm_w ? cfg->head_dim * 4 : 0))
    return DIT_ERR_SHAPE;
  if (!prologue_on(pro)) return DIT_OK;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = timed(DIT_K_PROLOGUE, s, [&] {
    return launch_qk_prologue(cfg->dtype == DIT_F32, cfg->head_dim, qkvg, q_norm_w, k_norm_w, (int)d.T,
                              cfg->seq_len, cfg->n_heads, cfg->n_kv_heads, pro->qk_norm, pro->rope, pro->grid_h,
                              pro->grid_w, pro->axes, pro->theta, cfg->eps, s);
  });
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

size_t dit_model_workspace_size(const dit_config *cfg, const dit_model_config *mc) {
  if (check_cfg(cfg) != DIT_OK || !mc) return 0;
  if (mc->latent_ch < 2 || mc->grid_h < 1 || mc->grid_w < 1) return 0;
  return carve_model(cfg, mc, nullptr).bytes;
}

// io_batch: samples of z and txt when they differ from cfg->batch (the
// guided sampler's model call runs 2B samples on B-sample inputs); need:
// the workspace bytes when more than the model call's own.
static dit_status check_model_call(const dit_config *cfg, const dit_model_config *mc, const dit_prologue *pro,
                                   const dit_model_weights *mw, int32_t n_blocks, const dit_block_weights *blocks,
                                   const float *z, const void *txt, void *ws, size_t ws_bytes, int io_batch = -1,
                                   size_t need_total = 0) {
  dit_status st = check_cfg(cfg);
  if (st != DIT_OK) return st;
  if ((st = check_prologue(cfg, pro)) != DIT_OK) return st;
  if ((st = check_model(cfg, mc, mw)) != DIT_OK) return st;
  if (n_blocks < 0) return DIT_ERR_SHAPE;
  if (n_blocks > 0 && !blocks) return DIT_ERR_NULL;
  for (int i = 0; i < n_blocks; ++i)
    if ((st = check_weights(&blocks[i])) != DIT_OK) return st;
  if (n_blocks == 0) return DIT_ERR_SHAPE;
  if (!z || (mc->n_text > 0 && !txt)) return DIT_ERR_NULL;
  if (!ws) return DIT_ERR_WORKSPACE;
  if (!aligned(z) || !aligned(txt) || !aligned(ws)) return DIT_ERR_ALIGN;
  const size_t need = std::max(carve_model(cfg, mc, nullptr).bytes, need_total);
  if (ws_bytes < need) return DIT_ERR_WORKSPACE;
  const size_t nb = io_batch >= 0 ? (size_t)io_batch : (size_t)cfg->batch;
  const size_t zb = nb * mc->latent_ch * 4 * mc->grid_h * mc->grid_w * 4;
  const size_t tb = txt ? nb * mc->n_text * mc->txt_dim * esize(cfg->dtype) : 0;
  if (overlap(ws, need, z, zb) || overlap(ws, need, txt, tb)) return DIT_ERR_SHAPE;
  for (int i = 0; i < n_blocks; ++i)
    if (overlaps_weights(cfg, &blocks[i], ws, need)) return DIT_ERR_SHAPE;
  return DIT_OK;
}

dit_status dit_model_velocity(const dit_config *cfg, const dit_model_config *mc, const dit_prologue *pro,
                              const dit_model_weights *mw, int32_t n_blocks, const dit_block_weights *blocks,
                              const float *z, float t, const void *txt, float *v_out, void *ws, size_t ws_bytes,
                              void *stream) {
  dit_status st = check_model_call(cfg, mc, pro, mw, n_blocks, blocks, z, txt, ws, ws_bytes);
  if (st != DIT_OK) return st;
  if (!v_out) return DIT_ERR_NULL;
  if (!aligned(v_out)) return DIT_ERR_ALIGN;
  const size_t zb = (size_t)cfg->batch * mc->latent_ch * 4 * mc->grid_h * mc->grid_w * 4;
  const size_t tb = mc->n_text ? (size_t)cfg->batch * mc->n_text * mc->txt_dim * esize(cfg->dtype) : 0;
  if (overlap(v_out, zb, z, zb) || overlap(v_out, zb, txt, tb) || overlap(v_out, zb, ws, ws_bytes))
    return DIT_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  const ModelWs w = carve_model(cfg, mc, ws);
  if ((st = model_tokens(cfg, mc, pro, mw, n_blocks, blocks, z, t, txt, w, s)) != DIT_OK) return st;
  hipError_t e = launch_unpatchify_axpy(cfg->dtype == DIT_F32, w.vt, nullptr, v_out, 1.0f, cfg->batch,
                                        mc->latent_ch, 2 * mc->grid_h, 2 * mc->grid_w, s);
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_sample(const dit_config *cfg, const dit_model_config *mc, const dit_prologue *pro,
                      const dit_model_weights *mw, int32_t n_blocks, const dit_block_weights *blocks, float *z,
                      int32_t n_steps, float shift, const void *txt, void *ws, size_t ws_bytes, void *stream) {
  dit_status st = check_model_call(cfg, mc, pro, mw, n_blocks, blocks, z, txt, ws, ws_bytes);
  if (st != DIT_OK) return st;
  if (n_steps < 1 || n_steps > 100000 || !(shift > 0.f)) return DIT_ERR_SHAPE;
  {  // z is written in place: it must not overlap the text features
    const size_t zb = (size_t)cfg->batch * mc->latent_ch * 4 * mc->grid_h * mc->grid_w * 4;
    const size_t tb = mc->n_text ? (size_t)cfg->batch * mc->n_text * mc->txt_dim * esize(cfg->dtype) : 0;
    if (overlap(z, zb, txt, tb)) return DIT_ERR_SHAPE;
  }
  hipStream_t s = (hipStream_t)stream;
  const ModelWs w = carve_model(cfg, mc, ws);
  auto sched = [&](int i) {  // s u / (1 + (s - 1) u), u = 1 - i / n
    const double u = 1.0 - (double)i / n_steps, sh = shift;
    return sh * u / (1.0 + (sh - 1.0) * u);
  };
  for (int i = 0; i < n_steps; ++i) {
    const double t0 = sched(i), t1 = sched(i + 1);
    if ((st = model_tokens(cfg, mc, pro, mw, n_blocks, blocks, z, (float)t0, txt, w, s)) != DIT_OK) return st;
    hipError_t e = launch_unpatchify_axpy(cfg->dtype == DIT_F32, w.vt, z, z, (float)(t1 - t0), cfg->batch,
                                          mc->latent_ch, 2 * mc->grid_h, 2 * mc->grid_w, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  return DIT_OK;
}

// Classifier-free guidance runs the model once on 2B samples: the
// workspace of that model call, then z twice [2B, C, Hl, Wl] fp32 and the
// text features of both halves [2B, n_text, txt_dim].
struct CfgWs {
  ModelWs m;
  float *z2;
  char *txt2;
  size_t bytes;
};
static dit_config doubled(const dit_config *c) {
  dit_config c2 = *c;
  c2.batch = 2 * c->batch;
  return c2;
}
static CfgWs carve_cfg(const dit_config *c, const dit_model_config *mc, void *ws) {
  const dit_config c2 = doubled(c);
  CfgWs w;
  w.m = carve_model(&c2, mc, ws);
  char *p = (char *)ws;
  size_t off = w.m.bytes;
  auto take = [&](size_t n) {
    char *r = p ? p + off : nullptr;
    off += round_up(n);
    return r;
  };
  w.z2 = (float *)take((size_t)c2.batch * mc->latent_ch * 4 * mc->grid_h * mc->grid_w * 4);
  w.txt2 = take((size_t)c2.batch * mc->n_text * mc->txt_dim * esize(c->dtype));
  w.bytes = off;
  return w;
}

size_t dit_sample_cfg_workspace_size(const dit_config *cfg, const dit_model_config *mc) {
  if (check_cfg(cfg) != DIT_OK || !mc || cfg->batch > 0x3FFFFFFF) return 0;
  const dit_config c2 = doubled(cfg);
  if (check_cfg(&c2) != DIT_OK) return 0;
  if (mc->latent_ch < 2 || mc->grid_h < 1 || mc->grid_w < 1) return 0;
  return carve_cfg(cfg, mc, nullptr).bytes;
}

dit_status dit_sample_cfg(const dit_config *cfg, const dit_model_config *mc, const dit_prologue *pro,
                          const dit_model_weights *mw, int32_t n_blocks, const dit_block_weights *blocks, float *z,
                          int32_t n_steps, float shift, float guidance, const void *txt, const void *txt_null,
                          void *ws, size_t ws_bytes, void *stream) {
  dit_status st = check_cfg(cfg);
  if (st != DIT_OK) return st;
  if (cfg->batch > 0x3FFFFFFF) return DIT_ERR_SHAPE;
  if (!mc) return DIT_ERR_NULL;
  // every kernel runs the doubled batch: the model call is checked at 2B
  // samples on B-sample inputs, against the whole workspace
  const dit_config c2 = doubled(cfg);
  if ((st = check_model_call(&c2, mc, pro, mw, n_blocks, blocks, z, txt, ws, ws_bytes, cfg->batch,
                             carve_cfg(cfg, mc, nullptr).bytes)) != DIT_OK)
    return st;
  const size_t need = carve_cfg(cfg, mc, nullptr).bytes;
  if (n_steps < 1 || n_steps > 100000 || !(shift > 0.f) || !std::isfinite(guidance)) return DIT_ERR_SHAPE;
  if (mc->n_text > 0 && !txt_null) return DIT_ERR_NULL;
  if (!aligned(txt_null)) return DIT_ERR_ALIGN;
  const size_t zb = (size_t)cfg->batch * mc->latent_ch * 4 * mc->grid_h * mc->grid_w * 4;
  const size_t tb = mc->n_text ? (size_t)cfg->batch * mc->n_text * mc->txt_dim * esize(cfg->dtype) : 0;
  if (overlap(ws, need, z, zb) || overlap(ws, need, txt, tb) || overlap(ws, need, txt_null, tb) ||
      overlap(z, zb, txt, tb) || overlap(z, zb, txt_null, tb))
    return DIT_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  const CfgWs w = carve_cfg(cfg, mc, ws);
  if (tb) {  // samples 0..B-1 conditional, B..2B-1 unconditional
    DIT_TRY(hipMemcpyAsync(w.txt2, txt, tb, hipMemcpyDeviceToDevice, s));
    DIT_TRY(hipMemcpyAsync(w.txt2 + tb, txt_null, tb, hipMemcpyDeviceToDevice, s));
  }
  auto sched = [&](int i) {  // s u / (1 + (s - 1) u), u = 1 - i / n
    const double u = 1.0 - (double)i / n_steps, sh = shift;
    return sh * u / (1.0 + (sh - 1.0) * u);
  };
  const size_t half_tok = (size_t)cfg->batch * mc->grid_h * mc->grid_w * 4 * mc->latent_ch * esize(cfg->dtype);
  for (int i = 0; i < n_steps; ++i) {
    const double t0 = sched(i), t1 = sched(i + 1);
    DIT_TRY(hipMemcpyAsync(w.z2, z, zb, hipMemcpyDeviceToDevice, s));
    DIT_TRY(hipMemcpyAsync((char *)w.z2 + zb, z, zb, hipMemcpyDeviceToDevice, s));
    if ((st = model_tokens(&c2, mc, pro, mw, n_blocks, blocks, w.z2, (float)t0, w.txt2, w.m, s)) != DIT_OK)
      return st;
    // velocity tokens: the conditional half first, then the unconditional
    hipError_t e = launch_unpatchify_axpy(cfg->dtype == DIT_F32, w.m.vt, z, z, (float)(t1 - t0), cfg->batch,
                                          mc->latent_ch, 2 * mc->grid_h, 2 * mc->grid_w, s, w.m.vt + half_tok,
                                          guidance);
    if (e != hipSuccess) return hip_fail(e);
  }
  return DIT_OK;
}

dit_status dit_timestep_mod(const dit_config *cfg, int32_t t_dim, const float *t, const float *w_t1,
                            const float *w_t2, float *mod_out, void *ws, size_t ws_bytes,
                            void *stream) {
  dit_status st = check_cfg(cfg);
  if (st != DIT_OK) return st;
  if (t_dim < 2 || t_dim > 1024 || (t_dim & 1)) return DIT_ERR_SHAPE;
  if (!t || !w_t1 || !w_t2 || !mod_out) return DIT_ERR_NULL;
  if (!ws) return DIT_ERR_WORKSPACE;
  if (!aligned(t) || !aligned(w_t1) || !aligned(w_t2) || !aligned(mod_out) || !aligned(ws))
    return DIT_ERR_ALIGN;
  if (ws_bytes < (size_t)cfg->batch * cfg->hidden * 4) return DIT_ERR_WORKSPACE;
  if ((uint64_t)6 * cfg->hidden * cfg->hidden > 0x7FFFFFFFull) return DIT_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = timed(DIT_K_TMOD, s, [&] {
    return launch_tmod(t, w_t1, w_t2, mod_out, (float *)ws, cfg->batch, cfg->hidden, t_dim, s);
  });
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_timestep_mod_noalloc(const dit_config *cfg, int32_t t_dim, const float *t, const float *w_t1,
                                    const float *w_t2, float *mod_out, void *stream) {
  dit_status st = check_cfg(cfg);
  if (st != DIT_OK) return st;
  if (t_dim < 2 || t_dim > 1024 || (t_dim & 1)) return DIT_ERR_SHAPE;
  if (!t || !w_t1 || !w_t2 || !mod_out) return DIT_ERR_NULL;
  if (!aligned(t) || !aligned(w_t1) || !aligned(w_t2) || !aligned(mod_out)) return DIT_ERR_ALIGN;
  if ((uint64_t)6 * cfg->hidden * cfg->hidden > 0x7FFFFFFFull) return DIT_ERR_UNSUPPORTED;
  // the hidden activations [B, D] fp32 live in the fixed scratch
  if ((uint64_t)cfg->batch * cfg->hidden * 4 > DIT_NOALLOC_SCRATCH_BYTES) return DIT_ERR_WORKSPACE;
  void *zs = nullptr;
  if ((st = scratch_address(&zs)) != DIT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // stage 1 writes every element of zs before stage 2 reads it, so nothing
  // has to be cleared between calls
  hipError_t e = timed(DIT_K_TMOD, s, [&] {
    return launch_tmod(t, w_t1, w_t2, mod_out, (float *)zs, cfg->batch, cfg->hidden, t_dim, s);
  });
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_modnorm(const dit_config *cfg, const void *x, dit_dtype x_dtype, void *h,
                       const float *mod, const float *bias, const float *gain, int32_t which,
                       void *stream) {
  dit_status st = check_cfg(cfg);
  if (st != DIT_OK) return st;
  if (!dtype_ok(x_dtype)) return DIT_ERR_DTYPE;
  if (x_dtype != DIT_F32 && x_dtype != cfg->dtype) return DIT_ERR_DTYPE;
  if (which != 0 && which != 1) return DIT_ERR_SHAPE;
  if (!x || !h || !mod || !bias) return DIT_ERR_NULL;
  if (!aligned(x) || !aligned(h) || !aligned(mod) || !aligned(bias) || !aligned(gain))
    return DIT_ERR_ALIGN;
  const Dims d = dims(cfg);
  if (overlap(x, d.T * d.D * esize(x_dtype), h, d.T * d.D * d.es)) return DIT_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = timed(DIT_K_MODNORM, s, [&] {
    return launch_modnorm(x_dtype == DIT_F32, cfg->dtype == DIT_F32, x, h, mod, bias, gain, (int)d.T,
                          cfg->seq_len, (int)d.D, cfg->eps, which, s);
  });
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

static dit_status check_gemm(dit_dtype dtype, int32_t m, int32_t n, int32_t k, const void *a,
                             const void *w, void *c, int64_t w_rows) {
  if (!dtype_ok(dtype)) return DIT_ERR_DTYPE;
  if (m <= 0 || n <= 0 || k <= 0) return DIT_ERR_SHAPE;
  if (k % 8) return DIT_ERR_UNSUPPORTED;
  if (!a || !w || !c) return DIT_ERR_NULL;
  if (!aligned(a) || !aligned(w) || !aligned(c)) return DIT_ERR_ALIGN;
  const uint64_t es = esize(dtype);
  if ((uint64_t)w_rows * k * es > kMaxSpan) return DIT_ERR_UNSUPPORTED;
  if ((uint64_t)256 * k * es > kMaxSpan) return DIT_ERR_UNSUPPORTED;
  return DIT_OK;
}

dit_status dit_gemm(dit_dtype dtype, int32_t m, int32_t n, int32_t k, const void *a, const void *w,
                    void *c, void *stream) {
  dit_status st = check_gemm(dtype, m, n, k, a, w, c, 256);  // a tile spans <= 256 W rows
  if (st != DIT_OK) return st;
  const size_t es = esize(dtype);
  if (overlap(c, (size_t)m * n * es, a, (size_t)m * k * es) ||
      overlap(c, (size_t)m * n * es, w, (size_t)n * k * es))
    return DIT_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_gemm(dtype == DIT_F32, a, w, c, m, n, k, s);
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_gemm_swiglu(dit_dtype dtype, int32_t m, int32_t f, int32_t k, const void *a,
                           const void *w13, void *u, void *stream) {
  dit_status st = check_gemm(dtype, m, f, k, a, w13, u, 2 * (int64_t)f + 256);
  if (st != DIT_OK) return st;
  const size_t es = esize(dtype);
  if (overlap(u, (size_t)m * f * es, a, (size_t)m * k * es) ||
      overlap(u, (size_t)m * f * es, w13, (size_t)2 * f * k * es))
    return DIT_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_gemm_swiglu(dtype == DIT_F32, a, w13, u, m, f, k, s);
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_gemm_variant(dit_dtype dtype, int32_t variant, int32_t group_m, int32_t swiglu,
                            int32_t m, int32_t n, int32_t k, const void *a, const void *w, void *c,
                            void *stream) {
  if (variant < 0 || variant >= kGemmVariants) return DIT_ERR_UNSUPPORTED;
  if (group_m < 0 || group_m > 64) return DIT_ERR_SHAPE;
  if (swiglu != 0 && swiglu != 1) return DIT_ERR_SHAPE;
  dit_status st = check_gemm(dtype, m, n, k, a, w, c, swiglu ? 2 * (int64_t)n + 256 : 256);
  if (st != DIT_OK) return st;
  const size_t es = esize(dtype);
  const size_t wrows = swiglu ? 2 * (size_t)n : (size_t)n;
  if (overlap(c, (size_t)m * n * es, a, (size_t)m * k * es) || overlap(c, (size_t)m * n * es, w, wrows * k * es))
    return DIT_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = swiglu ? launch_gemm_swiglu(dtype == DIT_F32, a, w, c, m, n, k, s, variant, group_m)
                        : launch_gemm(dtype == DIT_F32, a, w, c, m, n, k, s, variant, group_m);
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_quantize_fp8(dit_dtype dtype, int32_t m, int32_t k, const void *x, void *q, float *scale,
                            void *stream) {
  if (!dtype_ok(dtype)) return DIT_ERR_DTYPE;
  if (m <= 0 || k <= 0) return DIT_ERR_SHAPE;
  if (k % 16) return DIT_ERR_UNSUPPORTED;
  if (!x || !q || !scale) return DIT_ERR_NULL;
  if (!aligned(x) || !aligned(q) || !aligned(scale)) return DIT_ERR_ALIGN;
  const size_t xb = (size_t)m * k * esize(dtype), qb = (size_t)m * k;
  if (overlap(x, xb, q, qb) || overlap(x, xb, scale, (size_t)m * 4) || overlap(q, qb, scale, (size_t)m * 4))
    return DIT_ERR_SHAPE;
  hipError_t e = launch_quantize_fp8(dtype == DIT_F32, x, q, scale, m, k, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_quantize_fp8_tensor(dit_dtype dtype, int32_t m, int32_t k, const void *x, void *q, float *scale,
                                   void *ws, void *stream) {
  if (!dtype_ok(dtype)) return DIT_ERR_DTYPE;
  if (m <= 0 || k <= 0) return DIT_ERR_SHAPE;
  if (k % 16) return DIT_ERR_UNSUPPORTED;
  if (!x || !q || !scale) return DIT_ERR_NULL;
  if (!ws) return DIT_ERR_WORKSPACE;
  if (!aligned(x) || !aligned(q) || !aligned(scale) || !aligned(ws)) return DIT_ERR_ALIGN;
  const size_t xb = (size_t)m * k * esize(dtype), qb = (size_t)m * k, sb = (size_t)m * 4;
  if (overlap(x, xb, q, qb) || overlap(x, xb, scale, sb) || overlap(q, qb, scale, sb) || overlap(ws, 16, x, xb) ||
      overlap(ws, 16, q, qb) || overlap(ws, 16, scale, sb))
    return DIT_ERR_SHAPE;
  hipError_t e = launch_quantize_fp8_tensor(dtype == DIT_F32, x, q, scale, (float *)ws, m, k, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_gemm_fp8(int32_t swiglu, int32_t m, int32_t n, int32_t k, const void *qa, const float *sa,
                        const void *qw, const float *sw, void *c, void *stream) {
  if (swiglu != 0 && swiglu != 1) return DIT_ERR_SHAPE;
  if (m <= 0 || n <= 0 || k <= 0) return DIT_ERR_SHAPE;
  if (k % 16) return DIT_ERR_UNSUPPORTED;
  if (!qa || !sa || !qw || !sw || !c) return DIT_ERR_NULL;
  if (!aligned(qa) || !aligned(sa) || !aligned(qw) || !aligned(sw) || !aligned(c)) return DIT_ERR_ALIGN;
  const uint64_t wrows = swiglu ? 2ull * n : (uint64_t)n;
  if ((wrows + 256) * k > kMaxSpan || 256ull * k > kMaxSpan) return DIT_ERR_UNSUPPORTED;
  const size_t cb = (size_t)m * n * 2;
  if (overlap(c, cb, qa, (size_t)m * k) || overlap(c, cb, qw, wrows * k) || overlap(c, cb, sa, (size_t)m * 4) ||
      overlap(c, cb, sw, wrows * 4))
    return DIT_ERR_SHAPE;
  hipError_t e = launch_gemm_fp8(swiglu == 1, qa, sa, qw, sw, c, m, n, k, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_gemm_plan(int32_t m, int32_t n, int32_t k, int32_t swiglu, int32_t *variant, int32_t *sk_tiles,
                         int32_t *segs, size_t *part_bytes) {
  if (m <= 0 || n <= 0 || k <= 0 || (swiglu != 0 && swiglu != 1)) return DIT_ERR_SHAPE;
  if (!variant || !sk_tiles || !segs || !part_bytes) return DIT_ERR_NULL;
  const GemmChoice ch = gemm_choose(m, n, k, swiglu == 1);
  *variant = ch.variant;
  *sk_tiles = ch.sk_tiles;
  *segs = ch.segs;
  *part_bytes = ch.part_bytes;
  return DIT_OK;
}

dit_status dit_gemm_splitk(dit_dtype dtype, int32_t swiglu, int32_t m, int32_t n, int32_t k, const void *a,
                           const void *w, void *c, int32_t sk_tiles, int32_t segs, void *ws, size_t ws_bytes,
                           void *stream) {
  if (dtype != DIT_BF16) return dtype_ok(dtype) ? DIT_ERR_UNSUPPORTED : DIT_ERR_DTYPE;
  if (swiglu != 0 && swiglu != 1) return DIT_ERR_SHAPE;
  dit_status st = check_gemm(dtype, m, n, k, a, w, c, swiglu ? 2 * (int64_t)n + 256 : 256);
  if (st != DIT_OK) return st;
  const int64_t tiles = (int64_t)((m + 255) / 256) * ((n + (swiglu ? 127 : 255)) / (swiglu ? 128 : 256));
  const int nk = (k + 63) / 64;
  if (sk_tiles < 0 || sk_tiles > tiles || segs < 1 || segs > 64 || segs > nk) return DIT_ERR_SHAPE;
  const size_t need = (size_t)sk_tiles * segs * 256 * 256 * sizeof(float);
  if (need && !ws) return DIT_ERR_WORKSPACE;
  if (ws_bytes < need) return DIT_ERR_WORKSPACE;
  if (ws && !aligned(ws)) return DIT_ERR_ALIGN;
  const size_t wrows = swiglu ? 2 * (size_t)n : (size_t)n;
  if (overlap(c, (size_t)m * n * 2, a, (size_t)m * k * 2) || overlap(c, (size_t)m * n * 2, w, wrows * k * 2))
    return DIT_ERR_SHAPE;
  if (need && (overlap(ws, need, a, (size_t)m * k * 2) || overlap(ws, need, w, wrows * k * 2) ||
               overlap(ws, need, c, (size_t)m * n * 2)))
    return DIT_ERR_SHAPE;
  hipError_t e = launch_gemm_split(swiglu == 1, a, w, c, m, n, k, sk_tiles, segs, (float *)ws, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_attention(const dit_config *cfg, const void *qkvg, void *og, void *ws, size_t ws_bytes,
                         void *stream) {
  return dit_attention_ex(cfg, qkvg, og, ws, ws_bytes, 0, stream);
}

dit_status dit_attention_ex(const dit_config *cfg, const void *qkvg, void *og, void *ws, size_t ws_bytes,
                            int32_t q_prescaled, void *stream) {
  dit_status st = check_cfg(cfg);
  if (st != DIT_OK) return st;
  if (q_prescaled != 0 && q_prescaled != 1) return DIT_ERR_SHAPE;
  if (q_prescaled && cfg->dtype == DIT_F32) return DIT_ERR_UNSUPPORTED;
  if (!qkvg || !og) return DIT_ERR_NULL;
  if (!ws) return DIT_ERR_WORKSPACE;
  if (!aligned(qkvg) || !aligned(og) || !aligned(ws)) return DIT_ERR_ALIGN;
  const Dims d = dims(cfg);
  const size_t vtb = attention_vt_bytes(cfg->dtype == DIT_F32, cfg->batch, cfg->seq_len, cfg->n_kv_heads,
                                        cfg->head_dim);
  if (ws_bytes < vtb) return DIT_ERR_WORKSPACE;
  if (overlap(qkvg, d.T * d.nqkvg * d.es, og, d.T * d.hd * d.es) || overlap(ws, vtb, qkvg, d.T * d.nqkvg * d.es) ||
      overlap(ws, vtb, og, d.T * d.hd * d.es))
    return DIT_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = timed(DIT_K_ATTN, s, [&] {
    return launch_attention(cfg->dtype == DIT_F32, cfg->head_dim, qkvg, ws, og, cfg->batch,
                            cfg->seq_len, cfg->n_heads, cfg->n_kv_heads, s, q_prescaled == 1);
  });
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_gated_residual(const dit_config *cfg, const void *x, dit_dtype x_dtype,
                              const void *y, const float *mod, const float *bias, int32_t which,
                              void *out, dit_dtype out_dtype, void *stream) {
  dit_status st = check_cfg(cfg);
  if (st != DIT_OK) return st;
  if (!dtype_ok(x_dtype) || !dtype_ok(out_dtype)) return DIT_ERR_DTYPE;
  if ((x_dtype != DIT_F32 && x_dtype != cfg->dtype) || (out_dtype != DIT_F32 && out_dtype != cfg->dtype))
    return DIT_ERR_DTYPE;
  if (which != 0 && which != 1) return DIT_ERR_SHAPE;
  if (!x || !y || !mod || !bias || !out) return DIT_ERR_NULL;
  if (!aligned(x) || !aligned(y) || !aligned(mod) || !aligned(bias) || !aligned(out))
    return DIT_ERR_ALIGN;
  const Dims d = dims(cfg);
  const size_t n = d.T * d.D;
  if (overlap(out, n * esize(out_dtype), y, n * d.es)) return DIT_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = timed(DIT_K_RESID, s, [&] {
    return launch_resid(x_dtype == DIT_F32, cfg->dtype == DIT_F32, out_dtype == DIT_F32, x, y, out,
                        mod, bias, (int)d.T, cfg->seq_len, (int)d.D, which, s);
  });
  return e == hipSuccess ? DIT_OK : hip_fail(e);
}

dit_status dit_timer_start(int32_t kind, int32_t capacity) {
  if (kind < 0 || kind >= DIT_K_COUNT || capacity <= 0 || capacity > 1 << 16) return DIT_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(g_timer.mu);
  auto release = [] {
    for (hipEvent_t ev : g_timer.ev0)
      if (ev) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : g_timer.ev1)
      if (ev) (void)hipEventDestroy(ev);
    g_timer.ev0.clear();
    g_timer.ev1.clear();
    g_timer.active = false;
    g_timer.kind = -1;
    g_timer.capacity = g_timer.count = 0;
  };
  release();
  g_timer.ev0.assign(capacity, nullptr);
  g_timer.ev1.assign(capacity, nullptr);
  for (int i = 0; i < capacity; ++i) {
    hipError_t e = hipEventCreate(&g_timer.ev0[i]);
    if (e == hipSuccess) e = hipEventCreate(&g_timer.ev1[i]);
    if (e != hipSuccess) {
      release();  // every event created so far; the timer stays off
      return hip_fail(e);
    }
  }
  g_timer.kind = kind;
  g_timer.capacity = capacity;
  g_timer.count = 0;
  g_timer.active = true;
  return DIT_OK;
}

dit_status dit_timer_stop(double *total_ms, int32_t *n_launches) {
  if (!total_ms || !n_launches) return DIT_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_timer.mu);
  double tot = 0.0;
  for (int i = 0; i < g_timer.count; ++i) {
    hipError_t e = hipEventSynchronize(g_timer.ev1[i]);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_timer.ev0[i], g_timer.ev1[i]);
    if (e != hipSuccess) return hip_fail(e);
    tot += ms;
  }
  *total_ms = tot;
  *n_launches = g_timer.count;
  g_timer.active = false;
  g_timer.count = 0;
  return DIT_OK;
}

}  // extern "C"
