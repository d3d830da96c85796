// Host-side launchers of the gfx950 kernels (internal to libdit).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

namespace dit {

hipError_t launch_modnorm(bool x_f32, bool h_f32, const void *x, void *h, const float *mod,
                          const float *bias, const float *gain, int rows, int seq_len, int D,
                          float eps, int which, hipStream_t s);
hipError_t launch_resid(bool x_f32, bool y_f32, bool out_f32, const void *x, const void *y,
                        void *out, const float *mod, const float *bias, int rows, int seq_len,
                        int D, int which, hipStream_t s);
// x1 = x + gate * y (fp32), h = modnorm of x1: the gate of residual gw
// (0: first, 1: second) with bias gbias, the norm nw with bias nbias and
// gain ngain (may be NULL)
hipError_t launch_resid_modnorm(bool x_f32, bool f32, const void *x, const void *y, float *x1, void *h,
                                const float *mod, const float *gbias, int gw, const float *nbias,
                                const float *ngain, int nw, int rows, int seq_len, int D, float eps,
                                hipStream_t s);
// The two norms again with h leaving as row-wise e4m3 codes q [rows][D]
// and row scales qs [rows] (x1 of the fused pass is still stored in fp32;
// y is bf16)
hipError_t launch_modnorm_fp8(bool x_f32, const void *x, uint8_t *q, float *qs, const float *mod,
                              const float *bias, const float *gain, int rows, int seq_len, int D, float eps,
                              int which, hipStream_t s);
hipError_t launch_resid_modnorm_fp8(bool x_f32, const void *x, const void *y, float *x1, uint8_t *q, float *qs,
                                    const float *mod, const float *gbias, int gw, const float *nbias,
                                    const float *ngain, int nw, int rows, int seq_len, int D, float eps,
                                    hipStream_t s);
hipError_t launch_tmod(const float *t, const float *w1, const float *w2, float *mod, float *zs,
                       int B, int D, int tdim, hipStream_t s);
// out[b][o] = sum_r w[o][r] zs[b][r], o < O: a second map of the hidden zs
hipError_t launch_tmod_map(const float *zs, const float *w, float *out, int B, int D, int O, hipStream_t s);
// boundary layers of the stack
hipError_t launch_fill(float *p, float v, size_t n, hipStream_t s);
hipError_t launch_patchify(bool f32, const float *z, void *p, int B, int C, int Hl, int Wl, hipStream_t s);
// out = z + dt * unpatchify(vtok) (z may alias out, or be NULL for dt * v);
// with vtok_uncond, the velocity is vu + guidance * (v - vu)
hipError_t launch_unpatchify_axpy(bool f32, const void *vtok, const float *z, float *out, float dt, int B, int C,
                                  int Hl, int Wl, hipStream_t s, const void *vtok_uncond = nullptr,
                                  float guidance = 1.f);
// variant < 0 picks the default tile configuration for the shape (0 / 1:
// whole 256- / 192-row tiles); group_m <= 0 the default tile-grouping width
// (row tiles per L2 group).  part (fp32, part_bytes) lets the default
// configuration split the tail tiles along K.  Columns [0, scale_cols) of C
// are multiplied by col_scale before rounding.
// Value heads of a QKVG product written transposed for the attention
// kernel (bf16 only, seq_len L % 64 == 0, M a multiple of L): columns [c0,
// c1) of C go to vt ([B][Hkv][d][L], the layout of the V^T pass) instead of
// to C.
struct GemmVt {
  void *vt;
  int c0, c1, L;
};
hipError_t launch_gemm(bool f32, const void *a, const void *w, void *c, int M, int N, int K,
                       hipStream_t s, int variant = -1, int group_m = 0, float *part = nullptr,
                       size_t part_bytes = 0, int scale_cols = 0, float col_scale = 1.f,
                       const GemmVt *vt = nullptr);
hipError_t launch_gemm_swiglu(bool f32, const void *a, const void *w13, void *u, int M, int F,
                              int K, hipStream_t s, int variant = -1, int group_m = 0,
                              float *part = nullptr, size_t part_bytes = 0);
// The default choice for a bf16 product (variant 0: 256 x 256 tiles, the
// only ones split when sk_tiles > 0; 1: 192 x 256 tiles) and the fp32
// partial bytes its K split needs.
struct GemmChoice {
  int variant, sk_tiles, segs;
  size_t part_bytes;
};
GemmChoice gemm_choose(int M, int N, int K, bool swiglu);
// 256 x 256 tiles (bf16) with the last sk_tiles tiles split into segs K
// segments; part holds sk_tiles * segs * 256 * 256 floats.
hipError_t launch_gemm_split(bool swiglu, const void *a, const void *w, void *c, int M, int N, int K,
                             int sk_tiles, int segs, float *part, hipStream_t s);
constexpr int kGemmVariants = 2;
// vt: scratch of attention_vt_bytes() for the transposed V of every KV head
size_t attention_vt_bytes(bool f32, int B, int L, int Hkv, int head_dim);
// The attention's score factor in base-2 units, log2(e) / sqrt(head_dim).
inline float attn_score_scale(int head_dim) { return 1.4426950408889634f / sqrtf((float)head_dim); }
// q_prescaled (bf16 only): the query heads of qkvg already carry the factor
// attn_score_scale(head_dim), applied before their rounding to bf16.
// vt_ready: vt already holds V^T (written by the QKVG product's epilogue),
// so the V^T pass is skipped.
hipError_t launch_attention(bool f32, int head_dim, const void *qkvg, void *vt, void *og, int B,
                            int L, int H, int Hkv, hipStream_t s, bool q_prescaled = false,
                            bool vt_ready = false);

// QKNorm and 3D axial RoPE in place on the Q and K heads of qkvg rows; the
// query heads are multiplied by q_scale before they are rounded (1: none)
hipError_t launch_qk_prologue(bool f32, int head_dim, void *qkvg, const float *wq, const float *wk, int T,
                              int L, int H, int Hkv, int qk_norm, int rope, int grid_h, int grid_w,
                              const int axes[3], float theta, float eps, hipStream_t s, float q_scale = 1.f);

// FP8 (e4m3) projections with row-wise scales
hipError_t launch_quantize_fp8(bool f32, const void *x, void *q, float *scale, int M, int K, hipStream_t s);
// tensor-wise: scale[] receives the common scale for every row; tamax: 1 float
hipError_t launch_quantize_fp8_tensor(bool f32, const void *x, void *q, float *scale, float *tamax, int M, int K,
                                      hipStream_t s);
// part (fp32, part_bytes): lets the product split its last round of tiles
// along K as the bf16 one does (gemm_choose_fp8 says how much it needs).
// scale_cols / col_scale / vt as for launch_gemm (plain product only; vt
// only when gemm_choose_fp8 gives no split tiles)
hipError_t launch_gemm_fp8(bool swiglu, const void *aq, const float *sa, const void *wq, const float *sw, void *c,
                           int M, int N, int K, hipStream_t s, float *part = nullptr, size_t part_bytes = 0,
                           int scale_cols = 0, float col_scale = 1.f, const GemmVt *vt = nullptr);
GemmChoice gemm_choose_fp8(int M, int N, int K, bool swiglu);

}  // namespace dit
