// HBM-bound kernels of the DiT block: the modulated zero-centred RMSNorm,
// the gated residual add and the timestep modulation (embedding + MLP).
//
// Page "Krea 2 技术报告" (Krea 2 technical report), section 架构:
//   归一化 (normalisation): RMSNorm everywhere, zero-centred gain;
//   时间步条件化 (timestep conditioning): AdaLN shift/scale/gate from a shared
//     timestep vector plus a per-block bias;
//   残差设计 (residual design): standard residual, here scaled by the gate.
#include "dit_common.h"
#include "dit_kernels.h"

namespace dit {

// ----------------------------------------------------------------- loads of 8
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  static __device__ __forceinline__ void load(const bf16 *p, float (&v)[8]) {
    u32x4 r = *reinterpret_cast<const u32x4 *>(p);
    bf16x8 b = __builtin_bit_cast(bf16x8, r);
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
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float *p, float (&v)[8]) {
    f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float *p, const float (&v)[8]) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
};
__device__ __forceinline__ void load8f(const float *p, float (&v)[8]) { Vec8<float>::load(p, v); }

// ----------------------------------------------------------------- modnorm
// One wave per token row; the row stays in registers between the
// sum-of-squares pass and the normalise pass (NCH chunks of 8 per lane).
// h = x * rsqrt(mean(x^2) + eps) * (1 + gain) * (1 + scale) + shift.
template <typename Tx, typename Th, int NCH>
__global__ __launch_bounds__(256) void modnorm_kernel(const Tx *__restrict__ x, Th *__restrict__ h,
                                                      const float *__restrict__ mod,
                                                      const float *__restrict__ bias,
                                                      const float *__restrict__ gain, int rows,
                                                      int seq_len, int D, float eps, int which) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nch = D >> 3;
  const Tx *xr = x + (size_t)row * D;
  float v[NCH][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      Vec8<Tx>::load(xr + ch * 8, v[c]);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += v[c][i] * v[c][i];
    }
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)D + eps);
  const int b = row / seq_len;
  const float *msh = mod + ((size_t)b * 6 + 3 * which) * D;
  const float *bsh = bias + (size_t)(3 * which) * D;
  Th *hr = h + (size_t)row * D;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      float sh[8], sc[8], bs0[8], bs1[8], g[8], o[8];
      load8f(msh + ch * 8, sh);
      load8f(msh + D + ch * 8, sc);
      load8f(bsh + ch * 8, bs0);
      load8f(bsh + D + ch * 8, bs1);
      if (gain) {
        load8f(gain + ch * 8, g);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        o[i] = v[c][i] * inv * (1.f + g[i]) * (1.f + (sc[i] + bs1[i])) + (sh[i] + bs0[i]);
      Vec8<Th>::store(hr + ch * 8, o);
    }
  }
}

template <typename Tx, typename Th>
static hipError_t launch_modnorm_t(const void *x, void *h, const float *mod, const float *bias,
                                   const float *gain, int rows, int seq_len, int D, float eps,
                                   int which, hipStream_t s) {
  const int nch = D / 8;
  const int per = (nch + 63) / 64;
  dim3 grid((rows + 3) / 4), block(256);
#define DIT_MN(N)                                                                                  \
  hipLaunchKernelGGL((modnorm_kernel<Tx, Th, N>), grid, block, 0, s, (const Tx *)x, (Th *)h, mod,  \
                     bias, gain, rows, seq_len, D, eps, which)
  if (per <= 1) DIT_MN(1);
  else if (per <= 2) DIT_MN(2);
  else if (per <= 4) DIT_MN(4);
  else if (per <= 8) DIT_MN(8);
  else if (per <= 16) DIT_MN(16);
  else if (per <= 32) DIT_MN(32);
  else return hipErrorInvalidValue;
#undef DIT_MN
  return hipGetLastError();
}

hipError_t launch_modnorm(bool x_f32, bool h_f32, const void *x, void *h, const float *mod,
                          const float *bias, const float *gain, int rows, int seq_len, int D,
                          float eps, int which, hipStream_t s) {
  if (x_f32 && h_f32) return launch_modnorm_t<float, float>(x, h, mod, bias, gain, rows, seq_len, D, eps, which, s);
  if (x_f32) return launch_modnorm_t<float, bf16>(x, h, mod, bias, gain, rows, seq_len, D, eps, which, s);
  if (h_f32) return launch_modnorm_t<bf16, float>(x, h, mod, bias, gain, rows, seq_len, D, eps, which, s);
  return launch_modnorm_t<bf16, bf16>(x, h, mod, bias, gain, rows, seq_len, D, eps, which, s);
}

// ----------------------------------------------------------------- residual
// out = x + gate * y, one 8-element chunk per thread (grid-stride).
template <typename Tx, typename Ty, typename To>
__global__ __launch_bounds__(256) void resid_kernel(const Tx *__restrict__ x, const Ty *__restrict__ y,
                                                    To *__restrict__ out,
                                                    const float *__restrict__ mod,
                                                    const float *__restrict__ bias, int rows,
                                                    int seq_len, int D, int which) {
  const int nch_row = D >> 3;
  const size_t total = (size_t)rows * nch_row;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(idx / nch_row);
    const int col = (int)(idx - (size_t)row * nch_row) * 8;
    const int b = row / seq_len;
    float xv[8], yv[8], gm[8], gb[8], o[8];
    Vec8<Tx>::load(x + (size_t)row * D + col, xv);
    Vec8<Ty>::load(y + (size_t)row * D + col, yv);
    load8f(mod + ((size_t)b * 6 + 3 * which + 2) * D + col, gm);
    load8f(bias + (size_t)(3 * which + 2) * D + col, gb);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = xv[i] + (gm[i] + gb[i]) * yv[i];
    Vec8<To>::store(out + (size_t)row * D + col, o);
  }
}

template <typename Tx, typename Ty, typename To>
static hipError_t launch_resid_t(const void *x, const void *y, void *out, const float *mod,
                                 const float *bias, int rows, int seq_len, int D, int which,
                                 hipStream_t s) {
  const size_t total = (size_t)rows * (D / 8);
  size_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL((resid_kernel<Tx, Ty, To>), dim3((unsigned)blocks), dim3(256), 0, s,
                     (const Tx *)x, (const Ty *)y, (To *)out, mod, bias, rows, seq_len, D, which);
  return hipGetLastError();
}

hipError_t launch_resid(bool x_f32, bool y_f32, bool out_f32, const void *x, const void *y,
                        void *out, const float *mod, const float *bias, int rows, int seq_len,
                        int D, int which, hipStream_t s) {
#define DIT_R(TX, TY, TO) return launch_resid_t<TX, TY, TO>(x, y, out, mod, bias, rows, seq_len, D, which, s)
  if (y_f32) {
    if (x_f32) { if (out_f32) DIT_R(float, float, float); else DIT_R(float, float, bf16); }
    else { if (out_f32) DIT_R(bf16, float, float); else DIT_R(bf16, float, bf16); }
  } else {
    if (x_f32) { if (out_f32) DIT_R(float, bf16, float); else DIT_R(float, bf16, bf16); }
    else { if (out_f32) DIT_R(bf16, bf16, float); else DIT_R(bf16, bf16, bf16); }
  }
#undef DIT_R
}

// ----------------------------------------------------------------- timestep MLP
// Stage 1: zs[b][r] = SiLU(sum_k W_t1[r][k] e_b[k]) with the sinusoidal
// embedding e_b = [cos(1000 t_b f_i), sin(1000 t_b f_i)], f_i =
// 10000^(-i/half), evaluated in double precision (arguments reach 1000 rad).
__global__ __launch_bounds__(256) void tmod_stage1(const float *__restrict__ t,
                                                   const float *__restrict__ w1,
                                                   float *__restrict__ zs, int B, int D, int tdim) {
  __shared__ float e[1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = tdim / 2;
  for (int b = 0; b < B; ++b) {
    __syncthreads();
    for (int i = threadIdx.x; i < half; i += blockDim.x) {
      const double f = exp(-log(10000.0) * (double)i / (double)half);
      const double a = 1000.0 * (double)t[b] * f;
      e[i] = (float)cos(a);
      e[half + i] = (float)sin(a);
    }
    __syncthreads();
    for (int rr = 0; rr < 4; ++rr) {
      const int r = blockIdx.x * 16 + wave * 4 + rr;
      if (r >= D) break;
      float acc = 0.f;
      for (int k = lane; k < tdim; k += 64) acc += w1[(size_t)r * tdim + k] * e[k];
      acc = wave_sum(acc);
      if (lane == 0) zs[(size_t)b * D + r] = acc / (1.0f + expf(-acc));
    }
  }
}

// Stage 2: mod[b][o] = sum_r W_t2[o][r] zs[b][r], o < 6D.  Each wave owns
// two output rows; a chunk of zs for up to 32 samples is staged in LDS and
// W_t2 is streamed from HBM once per 32 samples.
__global__ __launch_bounds__(256) void tmod_stage2(const float *__restrict__ zs,
                                                   const float *__restrict__ w2,
                                                   float *__restrict__ mod, int B, int D) {
  constexpr int KC = 256, BMAX = 32, NR = 2;
  __shared__ f32x4 zl[BMAX][KC / 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int O = 6 * D;
  const int o0 = (blockIdx.x * 4 + wave) * NR;
  for (int b0 = 0; b0 < B; b0 += BMAX) {
    const int nb = min(BMAX, B - b0);
    float acc[NR][BMAX];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int b = 0; b < BMAX; ++b) acc[r][b] = 0.f;
    for (int k0 = 0; k0 < D; k0 += KC) {
      __syncthreads();
      for (int i = threadIdx.x; i < nb * (KC / 4); i += blockDim.x) {
        const int b = i / (KC / 4), c = i % (KC / 4);
        const int k = k0 + 4 * c;
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        if (k < D) z = *reinterpret_cast<const f32x4 *>(zs + (size_t)(b0 + b) * D + k);
        zl[b][c] = z;
      }
      __syncthreads();
      const int k = k0 + 4 * lane;
      if (k < D) {
        f32x4 w[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r)
          w[r] = (o0 + r < O) ? *reinterpret_cast<const f32x4 *>(w2 + (size_t)(o0 + r) * D + k)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < BMAX; ++b) {
          if (b < nb) {
            const f32x4 z = zl[b][lane];
#pragma unroll
            for (int r = 0; r < NR; ++r)
              acc[r][b] += w[r].x * z.x + w[r].y * z.y + w[r].z * z.z + w[r].w * z.w;
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
      if (b < nb) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float s = wave_sum(acc[r][b]);
          if (lane == 0 && o0 + r < O) mod[(size_t)(b0 + b) * O + o0 + r] = s;
        }
      }
    }
  }
}

hipError_t launch_tmod(const float *t, const float *w1, const float *w2, float *mod, float *zs,
                       int B, int D, int tdim, hipStream_t s) {
  hipLaunchKernelGGL(tmod_stage1, dim3((D + 15) / 16), dim3(256), 0, s, t, w1, zs, B, D, tdim);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tmod_stage2, dim3((6 * D + 7) / 8), dim3(256), 0, s, zs, w2, mod, B, D);
  return hipGetLastError();
}

}  // namespace dit
