// The layers around the block stack: 2 x 2 patches of the latent in and
// out, and the rectified-flow Euler update (page "Krea 2 技术报告": the DiT
// runs on autoencoder latent tokens; 训练 › 预训练: rectified-flow loss
// with v-parameterization).  Data movement only; the embeddings and the
// output projection are GEMMs, the final norm is the modulated norm.
//
// Patch layout: token (py, px) of a sample, raster order, holds
// z[c][2py + dy][2px + dx] at vector index c*4 + dy*2 + dx.
#include "dit_common.h"
#include "dit_kernels.h"

namespace dit {

__global__ __launch_bounds__(256) void fill_kernel(float *__restrict__ p, float v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_fill(float *p, float v, size_t n, hipStream_t s) {
  const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_kernel, dim3(grid > 0 ? grid : 1), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

// One thread per (token, c, dy): reads the 2 horizontally adjacent latent
// values (8 bytes) and writes 2 patch elements.
template <typename T>
__global__ __launch_bounds__(256) void patchify_kernel(const float *__restrict__ z, T *__restrict__ p, int B, int C,
                                                        int Hl, int Wl) {
  const int gw = Wl / 2, gh = Hl / 2, ntok = gh * gw;
  const size_t n = (size_t)B * ntok * C * 2;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int dy = (int)(i % 2);
    const int c = (int)((i / 2) % C);
    const size_t tok = i / (2 * C);  // b * ntok + py * gw + px
    const int b = (int)(tok / ntok), t = (int)(tok % ntok);
    const int py = t / gw, px = t % gw;
    const f32x2 v = *reinterpret_cast<const f32x2 *>(z + (((size_t)b * C + c) * Hl + 2 * py + dy) * Wl + 2 * px);
    T *dst = p + tok * (4 * C) + c * 4 + dy * 2;
    dst[0] = from_f32<T>(v[0]);
    dst[1] = from_f32<T>(v[1]);
  }
}

hipError_t launch_patchify(bool f32, const float *z, void *p, int B, int C, int Hl, int Wl, hipStream_t s) {
  const size_t n = (size_t)B * (Hl / 2) * (Wl / 2) * C * 2;
  const int grid = (int)std::min<size_t>((n + 255) / 256, 8192);
  if (f32) hipLaunchKernelGGL(patchify_kernel<float>, dim3(grid), dim3(256), 0, s, z, (float *)p, B, C, Hl, Wl);
  else hipLaunchKernelGGL(patchify_kernel<bf16>, dim3(grid), dim3(256), 0, s, z, (bf16 *)p, B, C, Hl, Wl);
  return hipGetLastError();
}

// One thread per (token, c, dy): out[b][c][2py+dy][2px + {0,1}] =
// z + dt * vtok[token][c*4 + dy*2 + {0,1}].  With vu (the unconditional
// velocity tokens of classifier-free guidance) the velocity is vu + g (v -
// vu) instead.
template <typename T>
__global__ __launch_bounds__(256) void unpatchify_axpy_kernel(const T *__restrict__ v, const float *z,
                                                               float *out, float dt, int B, int C, int Hl,
                                                               int Wl, const T *__restrict__ vu, float g) {
  const int gw = Wl / 2, gh = Hl / 2, ntok = gh * gw;
  const size_t n = (size_t)B * ntok * C * 2;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int dy = (int)(i % 2);
    const int c = (int)((i / 2) % C);
    const size_t tok = i / (2 * C);
    const int b = (int)(tok / ntok), t = (int)(tok % ntok);
    const int py = t / gw, px = t % gw;
    const T *src = v + tok * (4 * C) + c * 4 + dy * 2;
    const size_t o = (((size_t)b * C + c) * Hl + 2 * py + dy) * Wl + 2 * px;
    float v0 = to_f32(src[0]), v1 = to_f32(src[1]);
    if (vu) {
      const T *su = vu + tok * (4 * C) + c * 4 + dy * 2;
      const float u0 = to_f32(su[0]), u1 = to_f32(su[1]);
      v0 = u0 + g * (v0 - u0);
      v1 = u1 + g * (v1 - u1);
    }
    f32x2 r = {dt * v0, dt * v1};
    if (z) {
      const f32x2 zz = *reinterpret_cast<const f32x2 *>(z + o);
      r[0] += zz[0];
      r[1] += zz[1];
    }
    *reinterpret_cast<f32x2 *>(out + o) = r;
  }
}

hipError_t launch_unpatchify_axpy(bool f32, const void *vtok, const float *z, float *out, float dt, int B, int C,
                                  int Hl, int Wl, hipStream_t s, const void *vtok_uncond, float guidance) {
  const size_t n = (size_t)B * (Hl / 2) * (Wl / 2) * C * 2;
  const int grid = (int)std::min<size_t>((n + 255) / 256, 8192);
  if (f32)
    hipLaunchKernelGGL(unpatchify_axpy_kernel<float>, dim3(grid), dim3(256), 0, s, (const float *)vtok, z, out, dt,
                       B, C, Hl, Wl, (const float *)vtok_uncond, guidance);
  else
    hipLaunchKernelGGL(unpatchify_axpy_kernel<bf16>, dim3(grid), dim3(256), 0, s, (const bf16 *)vtok, z, out, dt,
                       B, C, Hl, Wl, (const bf16 *)vtok_uncond, guidance);
  return hipGetLastError();
}

}  // namespace dit
