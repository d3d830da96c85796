// Row-wise FP8 (OCP e4m3) quantisation of the operands of the 8-bit
// projections (page "Krea 2 技术报告", 训练 › 预训练: 8-bit training with
// row-wise scaling): for each row, s = amax / 448 and q = e4m3(x * (448 /
// amax)), rounded to nearest even by the hardware conversion; both the
// scale and the quotient are float32 operations.  One wave per row, two
// passes over the row (the second hits L2), 8 elements per lane step.
#include "dit_common.h"
#include "dit_kernels.h"

namespace dit {

// MODE 0: row-wise (scale and codes per row); MODE 1: only each row's amax
// into scale[row]; MODE 2: codes with the tensor scale, amax = tscale[0]
// (written by amax_reduce), and scale[row] = amax / 448 for every row.
template <typename T, int MODE>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T *__restrict__ x, uint8_t *__restrict__ q,
                                                           float *__restrict__ scale, const float *__restrict__ tamax,
                                                           int M, int K) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const T *xr = x + (size_t)row * K;
  const int nch = K / 8;
  float amax = 0.f;
  if (MODE != 2)
  for (int c = lane; c < nch; c += 64) {
    float v[8];
    if constexpr (sizeof(T) == 2) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(xr + c * 8));
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (float)b[i];
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(xr + c * 8), b = *reinterpret_cast<const f32x4 *>(xr + c * 8 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  if (MODE == 1) {
    if (lane == 0) scale[row] = amax;
    return;
  }
  if (MODE == 2) amax = tamax[0];
  const float s = fp8_row_scale(amax);
  const float inv = fp8_row_inv(amax);
  if (lane == 0) scale[row] = s;
  uint8_t *qr = q + (size_t)row * K;
  for (int c = lane; c < nch; c += 64) {
    float v[8];
    if constexpr (sizeof(T) == 2) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(xr + c * 8));
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (float)b[i];
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(xr + c * 8), b = *reinterpret_cast<const f32x4 *>(xr + c * 8 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
    }
    *reinterpret_cast<u32x2 *>(qr + c * 8) = fp8_pack8(v, inv);
  }
}

// Row-wise codes of bf16 rows with the whole row held in registers (NCH
// 16-byte chunks per lane): one read of the row instead of two, every load
// of it in flight at once.  Same float32 decisions as MODE 0 above.
template <int NCH>
__global__ __launch_bounds__(256) void quantize_fp8_rows_reg(const bf16 *__restrict__ x, uint8_t *__restrict__ q,
                                                             float *__restrict__ scale, int M, int K) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const bf16 *xr = x + (size_t)row * K;
  const int nch = K / 8;
  u32x4 r[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) r[c] = *reinterpret_cast<const u32x4 *>(xr + ch * 8);
  }
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (lane + 64 * c < nch) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, r[c]);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)b[i]));
    }
  }
  amax = wave_max(amax);
  const float inv = fp8_row_inv(amax);
  if (lane == 0) scale[row] = fp8_row_scale(amax);
  uint8_t *qr = q + (size_t)row * K;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, r[c]);
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (float)b[i];
      *reinterpret_cast<u32x2 *>(qr + ch * 8) = fp8_pack8(v, inv);
    }
  }
}

// max over the M row maxima (one workgroup; the max is exact in any order)
__global__ __launch_bounds__(1024) void amax_reduce(const float *__restrict__ row_amax, float *__restrict__ out,
                                                    int M) {
  __shared__ float red[16];
  float m = 0.f;
  for (int i = threadIdx.x; i < M; i += blockDim.x) m = fmaxf(m, row_amax[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, red[w]);
    out[0] = r;
  }
}

hipError_t launch_quantize_fp8(bool f32, const void *x, void *q, float *scale, int M, int K, hipStream_t s) {
  const dim3 grid((M + 3) / 4), block(256);
  if (!f32) {  // bf16 rows of up to 16384 elements: one pass from registers
    const int per = (K / 8 + 63) / 64;
#define DIT_QR(N)                                                                                                \
  hipLaunchKernelGGL(quantize_fp8_rows_reg<N>, grid, block, 0, s, (const bf16 *)x, (uint8_t *)q, scale, M, K); \
  return hipGetLastError()
    if (per <= 8) { DIT_QR(8); }
    if (per <= 16) { DIT_QR(16); }
    if (per <= 24) { DIT_QR(24); }
    if (per <= 32) { DIT_QR(32); }
#undef DIT_QR
  }
  if (f32)
    hipLaunchKernelGGL((quantize_fp8_kernel<float, 0>), grid, block, 0, s, (const float *)x, (uint8_t *)q, scale,
                       nullptr, M, K);
  else
    hipLaunchKernelGGL((quantize_fp8_kernel<bf16, 0>), grid, block, 0, s, (const bf16 *)x, (uint8_t *)q, scale,
                       nullptr, M, K);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8_tensor(bool f32, const void *x, void *q, float *scale, float *tamax, int M, int K,
                                      hipStream_t s) {
  const dim3 grid((M + 3) / 4), block(256);
  if (f32)
    hipLaunchKernelGGL((quantize_fp8_kernel<float, 1>), grid, block, 0, s, (const float *)x, (uint8_t *)q, scale,
                       nullptr, M, K);
  else
    hipLaunchKernelGGL((quantize_fp8_kernel<bf16, 1>), grid, block, 0, s, (const bf16 *)x, (uint8_t *)q, scale,
                       nullptr, M, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(amax_reduce, dim3(1), dim3(1024), 0, s, scale, tamax, M);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (f32)
    hipLaunchKernelGGL((quantize_fp8_kernel<float, 2>), grid, block, 0, s, (const float *)x, (uint8_t *)q, scale,
                       tamax, M, K);
  else
    hipLaunchKernelGGL((quantize_fp8_kernel<bf16, 2>), grid, block, 0, s, (const bf16 *)x, (uint8_t *)q, scale,
                       tamax, M, K);
  return hipGetLastError();
}

}  // namespace dit
