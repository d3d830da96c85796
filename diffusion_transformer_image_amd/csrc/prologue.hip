// Attention prologue: QKNorm and 3D axial RoPE on the query and key heads
// (page "Krea 2 技术报告", 架构 › 归一化: RMSNorm as the QKNorm, zero-centred
// gain; 架构 › 位置编码: 3D axial RoPE over frame, height and width, text
// tokens at index zero).
//
// In place on the Q | K column blocks of the QKVG projection rows.  One
// wave per token row; a head of d dimensions is handled by d/8 lanes with
// 16-byte accesses (4 rotation pairs each).  The angles of a lane's pairs
// depend only on the token and the pair index: they are computed once per
// token (fp32 frequency and angle, accurate sincosf) and reused for every
// head.  The head's mean square is a DPP reduction over its d/8 lanes.
#include <cmath>

#include "dit_common.h"
#include "dit_kernels.h"
#include "qk_rope.h"

namespace dit {

// 8 consecutive elements (4 rotation pairs) of one head per lane.
template <typename T> struct Oct;
template <> struct Oct<bf16> {
  static __device__ __forceinline__ void load(const bf16 *p, float (&v)[8]) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)b[i];
  }
  static __device__ __forceinline__ void store(bf16 *p, const float (&v)[8]) {
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (bf16)v[i];
    *reinterpret_cast<u32x4 *>(p) = __builtin_bit_cast(u32x4, b);
  }
};
template <> struct Oct<float> {
  static __device__ __forceinline__ void load(const float *p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  static __device__ __forceinline__ void store(float *p, const float (&v)[8]) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
};

// DPP lane moves inside a row of 16 lanes (no LDS round trip, unlike a
// shuffle through ds_bpermute): rotate right by N, mirror each half row,
// swap neighbours / pairs in each quad.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
constexpr int DPP_ROW_ROR = 0x120, DPP_ROW_HALF_MIRROR = 0x141, DPP_QUAD_XOR1 = 0xb1, DPP_QUAD_XOR2 = 0x4e;

// Sum over the G consecutive lanes of a group (G a power of two <= 64),
// the result in every lane of the group.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G == 16) {  // rotations within the row: pairs, fours, eights, all
    v += dpp<DPP_ROW_ROR + 8>(v);
    v += dpp<DPP_ROW_ROR + 4>(v);
    v += dpp<DPP_ROW_ROR + 2>(v);
    v += dpp<DPP_ROW_ROR + 1>(v);
    return v;
  } else if constexpr (G == 8) {  // lane i + lane 7-i, then the quad's four
    v += dpp<DPP_ROW_HALF_MIRROR>(v);
    v += dpp<DPP_QUAD_XOR1>(v);
    v += dpp<DPP_QUAD_XOR2>(v);
    return v;
  } else {
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
  }
}

// One wave per token row.  A head of HD dimensions is HD/8 lanes holding 8
// consecutive elements (4 rotation pairs) each, so a wave covers 64 / (HD/8)
// heads per step; U steps' loads are issued before the first is used.
template <typename T, int HD>
__global__ __launch_bounds__(256) void qk_prologue_kernel(T *__restrict__ qkvg, const float *__restrict__ wq,
                                                          const float *__restrict__ wk, int T_rows, int L,
                                                          int H, int Hkv, int qk_norm, int rope, int grid_h,
                                                          int grid_w, int ax0, int ax1, float theta, float eps,
                                                          float q_scale) {
  constexpr int LPH = HD / 8;    // lanes per head
  constexpr int HPW = 64 / LPH;  // heads per wave step
  constexpr int U = 4;           // wave steps in flight together
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T_rows) return;
  const int e0 = (lane % LPH) * 8, hsub = lane / LPH;  // first element of this lane in its head
  T *base = qkvg + (size_t)row * (2 * H + 2 * Hkv) * HD + e0;
  const int nh = H + Hkv;  // query heads, then key heads
  float x[U][8];
  auto load_step = [&](int h0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int h = h0 + u * HPW + hsub;
      if (h < nh) Oct<T>::load(base + h * HD, x[u]);
      else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[u][i] = 0.f;
      }
    }
  };
  // the lane's 8 gains of each norm (16-byte loads, issued with the first
  // data loads so the two latencies overlap)
  float gq[8], gk[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) gq[i] = gk[i] = 0.f;
  if (qk_norm) {
    if (wq) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(wq + e0), b = *reinterpret_cast<const f32x4 *>(wq + e0 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) { gq[i] = a[i]; gq[4 + i] = b[i]; }
    }
    if (wk) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(wk + e0), b = *reinterpret_cast<const f32x4 *>(wk + e0 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) { gk[i] = a[i]; gk[4 + i] = b[i]; }
    }
  }
  load_step(0);  // in flight while the angles are computed
  // ---- rotations of this lane's 4 pairs j = e0/2 .. e0/2 + 3 at this token
  float c[4], s[4];
  {
    const QkParams p{qk_norm, rope, grid_h, grid_w, ax0, ax1, theta, eps, wq, wk};
    const float l2t = log2f(theta);
#pragma unroll
    for (int k = 0; k < 4; ++k) rope_cs<HD>(p, l2t, row % L, e0 / 2 + k, c[k], s[k]);
  }
  for (int h0 = 0; h0 < nh; h0 += U * HPW) {
    if (h0 > 0) load_step(h0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int h = h0 + u * HPW + hsub;
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = x[u][i];
      if (qk_norm) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
        const float inv = qk_inv_rms<HD>(group_sum<LPH>(ss), eps);
        const bool isq = h < H;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= inv * (1.f + (isq ? gq[i] : gk[i]));
      }
      rope_apply<4>(v, c, s);
      if (h < H && q_scale != 1.f) {  // the attention's score factor, before the one rounding
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= q_scale;
      }
      if (h < nh) Oct<T>::store(base + h * HD, v);
    }
  }
}

hipError_t launch_qk_prologue(bool f32, int head_dim, void *qkvg, const float *wq, const float *wk, int T,
                              int L, int H, int Hkv, int qk_norm, int rope, int grid_h, int grid_w,
                              const int axes[3], float theta, float eps, hipStream_t s, float q_scale) {
  const dim3 grid((T + 3) / 4), block(256);
#define DIT_QP(TT, HDV)                                                                                \
  hipLaunchKernelGGL((qk_prologue_kernel<TT, HDV>), grid, block, 0, s, (TT *)qkvg, wq, wk, T, L, H, Hkv, \
                     qk_norm, rope, grid_h, grid_w, axes[0], axes[1], theta, eps, q_scale)
  if (head_dim == 128) {
    if (f32) DIT_QP(float, 128); else DIT_QP(bf16, 128);
  } else if (head_dim == 64) {
    if (f32) DIT_QP(float, 64); else DIT_QP(bf16, 64);
  } else {
    return hipErrorInvalidValue;
  }
#undef DIT_QP
  return hipGetLastError();
}

}  // namespace dit
