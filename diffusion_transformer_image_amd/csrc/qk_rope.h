// QKNorm and 3D axial RoPE arithmetic of the attention prologue pass
// (page "Krea 2 技术报告", 架构 › 归一化: RMSNorm as the QKNorm with a
// zero-centred gain; 架构 › 位置编码: 3D axial RoPE over frame, height and
// width, text tokens at index zero).
#pragma once

#include <cmath>

#include "dit_common.h"

namespace dit {

// Parameters of the prologue as the kernels take them (by value).
struct QkParams {
  int qk_norm, rope;   // which of the two steps run
  int grid_h, grid_w;  // image tokens first, raster order: l -> (0, l / grid_w, l % grid_w)
  int ax0, ax1;        // rotation dims of the frame and height axes (width: head_dim - ax0 - ax1)
  float theta, eps;    // RoPE base, norm epsilon
  const float *wq, *wk;  // zero-centred gains of the query / key heads (head_dim each), or null
};

// Rotation (c, s) of pair j (dims 2j, 2j+1) of a head of HD dims at token
// position l of its sample: angle = pos_axis(l) * theta^(-2i / d_axis) for
// the axis the pair belongs to (i its index inside that axis).  fp32: the
// exponent's rounding moves the angle by at most ~2e-6 rad at position 84,
// the product by ~5e-6 rad, and sincosf reduces its argument exactly.
template <int HD>
__device__ __forceinline__ void rope_cs(const QkParams &p, float l2t, int l, int j, float &c, float &s) {
  c = 1.f;
  s = 0.f;
  if (!p.rope || l >= p.grid_h * p.grid_w) return;  // text token: position 0
  int pos = 0, i = 0, da = 1;
  if (2 * j >= p.ax0 && 2 * j < p.ax0 + p.ax1) {
    pos = l / p.grid_w; i = j - p.ax0 / 2; da = p.ax1;
  } else if (2 * j >= p.ax0 + p.ax1) {
    pos = l % p.grid_w; i = j - (p.ax0 + p.ax1) / 2; da = HD - p.ax0 - p.ax1;
  }  // frame axis: position 0 for an image
  if (pos != 0) {
    const float a = (float)pos * exp2f(-(2.0f * (float)i / (float)da) * l2t);
    sincosf(a, &s, &c);
  }
}

// Rotates consecutive pairs (v[2k], v[2k+1]) in place by (c[k], s[k]).
template <int NP>
__device__ __forceinline__ void rope_apply(float *v, const float (&c)[NP], const float (&s)[NP]) {
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const float a = v[2 * k], b = v[2 * k + 1];
    v[2 * k] = a * c[k] - b * s[k];
    v[2 * k + 1] = a * s[k] + b * c[k];
  }
}

// 1 / sqrt(mean square + eps) of a head from its sum of squares.
template <int HD>
__device__ __forceinline__ float qk_inv_rms(float ss, float eps) {
  return rsqrtf(ss / (float)HD + eps);
}

}  // namespace dit
