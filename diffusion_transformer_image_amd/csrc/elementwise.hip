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

// ----------------------------------------------------------------- layout
// Every elementwise kernel runs one workgroup per (sample b, 8 token rows):
// the per-sample modulation vectors it needs (combined with the block bias
// and the norm gain) are computed once into LDS, then each of the 8 waves
// streams one row, 8 elements per lane-chunk, its loads issued before the
// staging.  Timed one launch at a time after a 640 MB read that evicts the
// last-level cache (1024 px, B = 2): 8 waves of one row each against 4
// waves of two rows: modnorm 33.7 -> 31.8 us, residual + norm 73.5 -> 72.2
// us, the stack's residual-and-next-norm pass 49.8 -> 47.7 us, the plain
// residual unchanged (54 us); a plain copy of modnorm's bytes takes 25 us
// (6.0 TB/s).  Fewer rows per wave or more rows per workgroup were slower.
constexpr int EW_ROWS = 8;  // rows per workgroup
constexpr int EW_WAVES = 8;
// the plain residual walks its rows flat; 4 rows on 4 waves measured best
// there (51 us against 54 us with 8 on 8)
constexpr int RES_ROWS = 4;
constexpr int RES_WAVES = 4;

// Per-sample vectors of length D sit in LDS split in two halves: elements
// 8c..8c+3 of chunk c at [4c, 4c+4), elements 8c+4..8c+7 at [D/2 + 4c, ...).
// A wave reading the chunks of 64 consecutive c then makes two reads of
// 1 KiB each, contiguous over its lanes (with the plain layout each 16-byte
// read had a 32-byte lane stride: two-way bank conflicts in the counters).
__device__ __forceinline__ int vec_slot(int i, int D) {  // i: multiple of 4
  return ((i >> 2) & 1) * (D >> 1) + ((i >> 3) << 2);
}
__device__ __forceinline__ void lds8v(const float *vec, int ch, int D, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(vec + ch * 4);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(vec + (D >> 1) + ch * 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Row-wise e4m3 quantisation of one row held in registers (chunk ch = lane
// + 64 c of NCH per lane): the row's amax is one wave reduction, then the
// codes go to qr and the scale amax / 448 to *qs.  The same float32
// decisions as the stand-alone quantiser, from the unrounded values.
template <typename T> struct is_u8 { static constexpr bool value = false; };
template <> struct is_u8<uint8_t> { static constexpr bool value = true; };
template <int NCH>
__device__ __forceinline__ void quant_row_store(const float (&v)[NCH][8], uint8_t *qr, float *qs, int lane,
                                                int nch) {
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    if (lane + 64 * c < nch) {
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
    }
  amax = wave_max(amax);
  const float inv = fp8_row_inv(amax);
  if (lane == 0) *qs = fp8_row_scale(amax);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) *reinterpret_cast<u32x2 *>(qr + ch * 8) = fp8_pack8(v[c], inv);
  }
}

// One row's NCH chunks of 8 elements per lane (chunk ch = lane + 64 c), held
// as raw 16-byte words so a row can be in flight while the previous one is
// computed: loads are issued by load(), converted by get().
template <typename T, int NCH>
struct RowBuf {
  static constexpr int W = sizeof(T) == 2 ? 1 : 2;  // 16-byte words per chunk
  u32x4 r[NCH][W];
  __device__ __forceinline__ void load(const T *row, int lane, int nch) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
#pragma unroll
        for (int w = 0; w < W; ++w) r[c][w] = *reinterpret_cast<const u32x4 *>(row + ch * 8 + w * 4);
      }
    }
  }
  __device__ __forceinline__ void get(int c, float (&v)[8]) const {
    if constexpr (W == 1) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, r[c][0]);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (float)b[i];
    } else {
      const f32x4 a = __builtin_bit_cast(f32x4, r[c][0]), b = __builtin_bit_cast(f32x4, r[c][1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
    }
  }
};

// A = (1 + gain) * (1 + scale), S = shift of norm `which`; G = gate of
// residual `which` (all with the per-block bias added to m[b]).
__device__ __forceinline__ void stage_norm_vectors(float *A, float *S, const float *mod, const float *bias,
                                                   const float *gain, int b, int D, int which) {
  const float *msh = mod + ((size_t)b * 6 + 3 * which) * D;
  const float *bsh = bias + (size_t)(3 * which) * D;
  for (int i = threadIdx.x * 4; i < D; i += blockDim.x * 4) {
    const f32x4 sh = *reinterpret_cast<const f32x4 *>(msh + i) + *reinterpret_cast<const f32x4 *>(bsh + i);
    const f32x4 sc = *reinterpret_cast<const f32x4 *>(msh + D + i) + *reinterpret_cast<const f32x4 *>(bsh + D + i);
    const f32x4 g = gain ? *reinterpret_cast<const f32x4 *>(gain + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4 *>(A + vec_slot(i, D)) = (1.0f + g) * (1.0f + sc);
    *reinterpret_cast<f32x4 *>(S + vec_slot(i, D)) = sh;
  }
}
__device__ __forceinline__ void stage_gate_vector(float *G, const float *mod, const float *bias, int b, int D,
                                                  int which) {
  const float *mg = mod + ((size_t)b * 6 + 3 * which + 2) * D;
  const float *bg = bias + (size_t)(3 * which + 2) * D;
  for (int i = threadIdx.x * 4; i < D; i += blockDim.x * 4)
    *reinterpret_cast<f32x4 *>(G + vec_slot(i, D)) =
        *reinterpret_cast<const f32x4 *>(mg + i) + *reinterpret_cast<const f32x4 *>(bg + i);
}

// ----------------------------------------------------------------- modnorm
// h = x * rsqrt(mean(x^2) + eps) * A + S; the row stays in registers
// (NCH chunks of 8 per lane) between the sum of squares and the output.
// Th = uint8_t: h leaves as row-wise e4m3 codes with its row scales in hs
// (the operand of an 8-bit product, quantised from the fp32 values).
template <typename Tx, typename Th, int NCH>
__global__ __launch_bounds__(EW_WAVES * 64) void modnorm_kernel(const Tx *__restrict__ x, Th *__restrict__ h,
                                                      float *__restrict__ hs,
                                                      const float *__restrict__ mod,
                                                      const float *__restrict__ bias,
                                                      const float *__restrict__ gain, int seq_len, int D,
                                                      float eps, int which) {
  extern __shared__ float ew_lds[];
  float *A = ew_lds, *S = ew_lds + D;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = D >> 3;
  constexpr int RPW = EW_ROWS / EW_WAVES;  // rows per wave
  auto row_at = [&](int rr) { return blockIdx.x * EW_ROWS + rr * EW_WAVES + wave; };
  // the first row's loads go out before the staging of the vectors, and
  // row rr+1's before row rr is computed (two memory latencies overlap)
  RowBuf<Tx, NCH> buf[2];
  if (row_at(0) < seq_len) buf[0].load(x + ((size_t)b * seq_len + row_at(0)) * D, lane, nch);
  stage_norm_vectors(A, S, mod, bias, gain, b, D, which);
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int l = row_at(rr);
    if (l >= seq_len) break;
    if (rr + 1 < RPW && row_at(rr + 1) < seq_len)
      buf[(rr + 1) & 1].load(x + ((size_t)b * seq_len + row_at(rr + 1)) * D, lane, nch);
    const size_t row = (size_t)b * seq_len + l;
    float v[NCH][8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
        buf[rr & 1].get(c, v[c]);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += v[c][i] * v[c][i];
      }
    }
    const float inv = rsqrtf(wave_sum(ss) / (float)D + eps);
    Th *hr = h + row * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
        float a[8], sh[8];
        lds8v(A, ch, D, a);
        lds8v(S, ch, D, sh);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[c][i] = v[c][i] * inv * a[i] + sh[i];
        if constexpr (!is_u8<Th>::value) Vec8<Th>::store(hr + ch * 8, v[c]);
      }
    }
    if constexpr (is_u8<Th>::value) quant_row_store<NCH>(v, hr, hs + row, lane, nch);
  }
}

static int nch_bucket(int D) {
  const int per = (D / 8 + 63) / 64;
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : per <= 16 ? 16 : -1;
}

template <typename Tx, typename Th>
static hipError_t launch_modnorm_t(const void *x, void *h, const float *mod, const float *bias,
                                   const float *gain, int rows, int seq_len, int D, float eps,
                                   int which, hipStream_t s, float *hs = nullptr) {
  const int B = rows / seq_len;
  dim3 grid((seq_len + EW_ROWS - 1) / EW_ROWS, B), block(EW_WAVES * 64);
  const size_t lds = 2 * (size_t)D * sizeof(float);
#define DIT_MN(N)                                                                                  \
  hipLaunchKernelGGL((modnorm_kernel<Tx, Th, N>), grid, block, lds, s, (const Tx *)x, (Th *)h, hs, mod, \
                     bias, gain, seq_len, D, eps, which)
  switch (nch_bucket(D)) {
    case 1: DIT_MN(1); break;
    case 2: DIT_MN(2); break;
    case 4: DIT_MN(4); break;
    case 8: DIT_MN(8); break;
    case 16: DIT_MN(16); break;
    default: return hipErrorInvalidValue;
  }
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

hipError_t launch_modnorm_fp8(bool x_f32, const void *x, uint8_t *q, float *qs, const float *mod,
                              const float *bias, const float *gain, int rows, int seq_len, int D, float eps,
                              int which, hipStream_t s) {
  if (x_f32) return launch_modnorm_t<float, uint8_t>(x, q, mod, bias, gain, rows, seq_len, D, eps, which, s, qs);
  return launch_modnorm_t<bf16, uint8_t>(x, q, mod, bias, gain, rows, seq_len, D, eps, which, s, qs);
}

// ----------------------------------------------------------------- residual
// out = x + G * y, G the gate of residual `which`.
template <typename Tx, typename Ty, typename To>
__global__ __launch_bounds__(RES_WAVES * 64) void resid_kernel(const Tx *__restrict__ x, const Ty *__restrict__ y,
                                                    To *__restrict__ out, const float *__restrict__ mod,
                                                    const float *__restrict__ bias, int seq_len, int D,
                                                    int which) {
  extern __shared__ float ew_lds[];
  float *G = ew_lds;
  const int b = blockIdx.y;
  const int nch = D >> 3;
  const int l0 = blockIdx.x * RES_ROWS;
  const int nrows = min(RES_ROWS, seq_len - l0);
  const int n = nrows * nch;
  // flat walk over (row, chunk) of this workgroup's rows, fully coalesced,
  // UR chunks per thread at a time with all their loads issued first (the
  // first batch before the gate vector is staged)
  constexpr int UR = 4;
  const size_t base = ((size_t)b * seq_len + l0) * D;
  auto batch = [&](int idx0, RowBuf<Tx, UR> &bx, RowBuf<Ty, UR> &by) {
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int idx = idx0 + u * blockDim.x;
      if (idx < n) {
        const int r = idx / nch, ch = idx - r * nch;
        const size_t off = base + (size_t)r * D + ch * 8;
#pragma unroll
        for (int w = 0; w < RowBuf<Tx, UR>::W; ++w) bx.r[u][w] = *reinterpret_cast<const u32x4 *>(x + off + w * 4);
#pragma unroll
        for (int w = 0; w < RowBuf<Ty, UR>::W; ++w) by.r[u][w] = *reinterpret_cast<const u32x4 *>(y + off + w * 4);
      }
    }
  };
  RowBuf<Tx, UR> bx;
  RowBuf<Ty, UR> by;
  int idx0 = threadIdx.x;
  batch(idx0, bx, by);
  stage_gate_vector(G, mod, bias, b, D, which);
  __syncthreads();
  for (; idx0 < n; idx0 += UR * blockDim.x) {
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int idx = idx0 + u * blockDim.x;
      if (idx < n) {
        const int r = idx / nch, ch = idx - r * nch;
        const size_t off = base + (size_t)r * D + ch * 8;
        float xv[8], yv[8], gv[8], o[8];
        bx.get(u, xv);
        by.get(u, yv);
        lds8v(G, ch, D, gv);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = xv[i] + gv[i] * yv[i];
        Vec8<To>::store(out + off, o);
      }
    }
    if (idx0 + UR * blockDim.x < n) batch(idx0 + UR * blockDim.x, bx, by);
  }
}

template <typename Tx, typename Ty, typename To>
static hipError_t launch_resid_t(const void *x, const void *y, void *out, const float *mod,
                                 const float *bias, int rows, int seq_len, int D, int which,
                                 hipStream_t s) {
  const int B = rows / seq_len;
  dim3 grid((seq_len + RES_ROWS - 1) / RES_ROWS, B);
  hipLaunchKernelGGL((resid_kernel<Tx, Ty, To>), grid, dim3(RES_WAVES * 64), (size_t)D * sizeof(float), s,
                     (const Tx *)x, (const Ty *)y, (To *)out, mod, bias, seq_len, D, which);
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

// ----------------------------------------------------------------- residual + norm
// A gated residual fused with the modulated norm that reads its result:
//   x1 = x + gate * y   (stored fp32),   h = modnorm(x1; norm),
// gate = residual `gw` with bias gbias, norm = norm `nw` with bias nbias and
// gain ngain.  Inside a block: the first residual and the second norm (one
// block's bias for both); between two blocks of a stack: the second
// residual of one block and the first norm of the next (each its own
// block's bias).  Saves writing x1 and reading it back between two passes.
template <typename Tx, typename Ty, typename Th, int NCH>
__global__ __launch_bounds__(EW_WAVES * 64) void resid_modnorm_kernel(const Tx *__restrict__ x, const Ty *__restrict__ y,
                                                            float *__restrict__ x1, Th *__restrict__ h,
                                                            float *__restrict__ hs,
                                                            const float *__restrict__ mod,
                                                            const float *__restrict__ gbias, int gw,
                                                            const float *__restrict__ nbias,
                                                            const float *__restrict__ ngain, int nw,
                                                            int seq_len, int D, float eps) {
  extern __shared__ float ew_lds[];
  float *G = ew_lds, *A = ew_lds + D, *S = ew_lds + 2 * D;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = D >> 3;
  constexpr int RPW = EW_ROWS / EW_WAVES;  // rows per wave
  auto row_at = [&](int rr) { return blockIdx.x * EW_ROWS + rr * EW_WAVES + wave; };
  // the first row's loads go out before the staging of the vectors, and
  // row rr+1's before row rr is computed (two memory latencies overlap)
  RowBuf<Tx, NCH> bx[2];
  RowBuf<Ty, NCH> by[2];
  if (row_at(0) < seq_len) {
    const size_t r0 = ((size_t)b * seq_len + row_at(0)) * D;
    bx[0].load(x + r0, lane, nch);
    by[0].load(y + r0, lane, nch);
  }
  stage_gate_vector(G, mod, gbias, b, D, gw);
  stage_norm_vectors(A, S, mod, nbias, ngain, b, D, nw);
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int l = row_at(rr);
    if (l >= seq_len) break;
    if (rr + 1 < RPW && row_at(rr + 1) < seq_len) {
      const size_t rn = ((size_t)b * seq_len + row_at(rr + 1)) * D;
      bx[(rr + 1) & 1].load(x + rn, lane, nch);
      by[(rr + 1) & 1].load(y + rn, lane, nch);
    }
    const size_t row = (size_t)b * seq_len + l;
    float v[NCH][8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
        float xv[8], yv[8], gv[8];
        bx[rr & 1].get(c, xv);
        by[rr & 1].get(c, yv);
        lds8v(G, ch, D, gv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[c][i] = xv[i] + gv[i] * yv[i];
          ss += v[c][i] * v[c][i];
        }
        Vec8<float>::store(x1 + row * D + ch * 8, v[c]);
      }
    }
    const float inv = rsqrtf(wave_sum(ss) / (float)D + eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
        float a[8], sh[8];
        lds8v(A, ch, D, a);
        lds8v(S, ch, D, sh);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[c][i] = v[c][i] * inv * a[i] + sh[i];
        if constexpr (!is_u8<Th>::value) Vec8<Th>::store(h + row * D + ch * 8, v[c]);
      }
    }
    if constexpr (is_u8<Th>::value) quant_row_store<NCH>(v, h + row * D, hs + row, lane, nch);
  }
}

template <typename Tx, typename Ty, typename Th>
static hipError_t launch_resid_modnorm_t(const void *x, const void *y, float *x1, void *h, const float *mod,
                                         const float *gbias, int gw, const float *nbias, const float *ngain,
                                         int nw, int rows, int seq_len, int D, float eps, hipStream_t s,
                                         float *hs = nullptr) {
  const int B = rows / seq_len;
  dim3 grid((seq_len + EW_ROWS - 1) / EW_ROWS, B), block(EW_WAVES * 64);
  const size_t lds = 3 * (size_t)D * sizeof(float);
#define DIT_RMN(N)                                                                                   \
  hipLaunchKernelGGL((resid_modnorm_kernel<Tx, Ty, Th, N>), grid, block, lds, s, (const Tx *)x,     \
                     (const Ty *)y, x1, (Th *)h, hs, mod, gbias, gw, nbias, ngain, nw, seq_len, D, eps)
  switch (nch_bucket(D)) {
    case 1: DIT_RMN(1); break;
    case 2: DIT_RMN(2); break;
    case 4: DIT_RMN(4); break;
    case 8: DIT_RMN(8); break;
    case 16: DIT_RMN(16); break;
    default: return hipErrorInvalidValue;
  }
#undef DIT_RMN
  return hipGetLastError();
}

hipError_t launch_resid_modnorm(bool x_f32, bool f32, const void *x, const void *y, float *x1, void *h,
                                const float *mod, const float *gbias, int gw, const float *nbias,
                                const float *ngain, int nw, int rows, int seq_len, int D, float eps,
                                hipStream_t s) {
  // y and h have the compute dtype (f32 ? fp32 : bf16); x is fp32 or that dtype
#define DIT_RMNT(TX, TY, TH) \
  launch_resid_modnorm_t<TX, TY, TH>(x, y, x1, h, mod, gbias, gw, nbias, ngain, nw, rows, seq_len, D, eps, s)
  if (f32) return DIT_RMNT(float, float, float);
  if (x_f32) return DIT_RMNT(float, bf16, bf16);
  return DIT_RMNT(bf16, bf16, bf16);
#undef DIT_RMNT
}

hipError_t launch_resid_modnorm_fp8(bool x_f32, const void *x, const void *y, float *x1, uint8_t *q, float *qs,
                                    const float *mod, const float *gbias, int gw, const float *nbias,
                                    const float *ngain, int nw, int rows, int seq_len, int D, float eps,
                                    hipStream_t s) {
  if (x_f32)
    return launch_resid_modnorm_t<float, bf16, uint8_t>(x, y, x1, q, mod, gbias, gw, nbias, ngain, nw, rows,
                                                        seq_len, D, eps, s, qs);
  return launch_resid_modnorm_t<bf16, bf16, uint8_t>(x, y, x1, q, mod, gbias, gw, nbias, ngain, nw, rows, seq_len,
                                                     D, eps, s, qs);
}

// ----------------------------------------------------------------- timestep MLP
// A 16-byte load marked non-temporal, for weight rows that are read exactly
// once per call: the stream does not displace cached lines that are reused
// (W_t2 at D = 4096: the two timestep kernels 109 -> 91 us).
__device__ __forceinline__ f32x4 stream_load(const float *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}

// Stage 1: zs[b][r] = SiLU(sum_k W_t1[r][k] e_b[k]) with the sinusoidal
// embedding e_b = [cos(1000 t_b f_i), sin(1000 t_b f_i)], f_i =
// 10000^(-i/half), evaluated in double precision (arguments reach 1000 rad).
// Each wave owns 4 rows of W_t1 and reads them once for up to TM1_NB
// samples (the embeddings of those samples sit in LDS), with the loads of
// 4 column steps of all 4 rows in flight before any is used.
constexpr int TM1_NB = 4;
__global__ __launch_bounds__(256) void tmod_stage1(const float *__restrict__ t,
                                                   const float *__restrict__ w1,
                                                   float *__restrict__ zs, int B, int D, int tdim) {
  __shared__ float e[TM1_NB][1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = tdim / 2;
  const int r0 = blockIdx.x * 16 + wave * 4;
  // one chunk of TM1_NB samples per grid row (at 256 px, B = 32, a loop over
  // the 8 chunks inside 256 workgroups took 59 us, latency-bound)
  {
    const int b0 = blockIdx.y * TM1_NB;
    const int nb = min(TM1_NB, B - b0);
    for (int idx = threadIdx.x; idx < nb * half; idx += blockDim.x) {
      const int bb = idx / half, i = idx - bb * half;
      const double f = exp(-log(10000.0) * (double)i / (double)half);
      const double a = 1000.0 * (double)t[b0 + bb] * f;
      e[bb][i] = (float)cos(a);
      e[bb][half + i] = (float)sin(a);
    }
    __syncthreads();
    float acc[4][TM1_NB];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int bb = 0; bb < TM1_NB; ++bb) acc[rr][bb] = 0.f;
    for (int k0 = 0; k0 < tdim; k0 += 4 * 64) {
      float wv[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int k = k0 + u * 64 + lane;
          wv[u][rr] = (k < tdim && r0 + rr < D) ? w1[(size_t)(r0 + rr) * tdim + k] : 0.f;
        }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = k0 + u * 64 + lane;
        if (k < tdim) {
#pragma unroll
          for (int bb = 0; bb < TM1_NB; ++bb) {
            if (bb < nb) {
              const float ev = e[bb][k];
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) acc[rr][bb] += wv[u][rr] * ev;
            }
          }
        }
      }
    }
#pragma unroll
    for (int bb = 0; bb < TM1_NB; ++bb) {
      if (bb < nb) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float v = wave_sum(acc[rr][bb]);
          if (lane == 0 && r0 + rr < D) zs[(size_t)(b0 + bb) * D + r0 + rr] = v / (1.0f + expf(-v));
        }
      }
    }
  }
}

// Stage 2: mod[b][o] = sum_r W[o][r] zs[b][r], o < O (O = 6D for the block
// modulation, 2D for the final norm's shift and scale).

// Stage 2 for few samples (B <= 4): the whole SiLU'd hidden of every sample
// sits in LDS, so each wave streams 4 rows of W_t2 at a time over the full K
// with 16 independent 16-byte loads in flight per lane and no barrier; a
// workgroup covers 64 rows so the staging is amortised.
constexpr int TM_NB = 4;
__global__ __launch_bounds__(256) void tmod_stage2_fewb(const float *__restrict__ zs,
                                                        const float *__restrict__ w2,
                                                        float *__restrict__ mod, int B, int D, int O) {
  extern __shared__ float zl[];  // [B][D]
  for (int i = threadIdx.x * 4; i < B * D; i += blockDim.x * 4)
    *reinterpret_cast<f32x4 *>(zl + i) = *reinterpret_cast<const f32x4 *>(zs + i);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // 64 rows per workgroup (4 passes of 4 rows per wave) amortise the staging
  for (int pass = 0; pass < 4; ++pass) {
  const int o0 = ((blockIdx.x * 4 + pass) * 4 + wave) * 4;
  if (o0 >= O) break;
  float acc[4][TM_NB];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int b = 0; b < TM_NB; ++b) acc[r][b] = 0.f;
  for (int k0 = 0; k0 < D; k0 += 4 * 256) {
    f32x4 w[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int k = k0 + u * 256 + lane * 4;
        w[u][r] = (k < D && o0 + r < O) ? stream_load(w2 + (size_t)(o0 + r) * D + k) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u * 256 + lane * 4;
      if (k < D) {
#pragma unroll
        for (int b = 0; b < TM_NB; ++b) {
          if (b < B) {
            const f32x4 z = *reinterpret_cast<const f32x4 *>(zl + b * D + k);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[r][b] += w[u][r].x * z.x + w[u][r].y * z.y + w[u][r].z * z.z + w[u][r].w * z.w;
          }
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < TM_NB; ++b) {
    if (b < B) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sum = wave_sum(acc[r][b]);
        if (lane == 0 && o0 + r < O) mod[(size_t)b * O + o0 + r] = sum;
      }
    }
  }
  }
}

// Stage 2 for more samples (B > 4): the map is a skinny fp32 product
// mod[B, O] = zs[B, D] W[O, D]^T, streamed once per 16 * NSB samples on
// the fp32 matrix cores (v_mfma_f32_16x16x4f32: W rows as the 16-row
// operand, samples as the 16 columns).  A workgroup owns TMM_RB blocks of 16
// rows; its TMM_W waves split K into contiguous ranges of 64-k chunks and
// their partial sums are added through LDS.  Each lane loads 16 bytes (4
// consecutive k) of one W row and of one sample per 16-k step, and the four
// k of a 16-byte piece feed four MFMAs in the same order on both operands,
// so every k is summed once.  zs (B * D floats) is read from L2.
// 4 K ranges per workgroup measured against 8 on one box: 256 px (B = 32)
// 218 against 227 us, 512 px (B = 8) 128 against 126 us; the previous VALU
// kernel (hidden vectors staged per 256-k chunk in LDS) took 367 and 144 us
constexpr int TMM_RB = 2, TMM_U = 4, TMM_W = 4;
template <int NSB>
__global__ __launch_bounds__(TMM_W * 64) void tmod_stage2_mfma(const float *__restrict__ zs,
                                                               const float *__restrict__ w2,
                                                               float *__restrict__ mod, int B, int D, int O) {
  __shared__ f32x4 red[TMM_W][TMM_RB * NSB][64];  // per wave: its partial C blocks, lane-major
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int o0 = blockIdx.x * (16 * TMM_RB);
  const int nc = (D + 16 * TMM_U - 1) / (16 * TMM_U);  // 64-k chunks
  const int c_beg = wave * nc / TMM_W, c_end = (wave + 1) * nc / TMM_W;
  for (int b0 = 0; b0 < B; b0 += 16 * NSB) {
    f32x4 acc[TMM_RB][NSB];
#pragma unroll
    for (int rb = 0; rb < TMM_RB; ++rb)
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) acc[rb][sb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // chunk c+1's loads are issued before chunk c's MFMAs (two register sets)
    f32x4 wv[TMM_U][TMM_RB], zv[TMM_U][NSB], wn[TMM_U][TMM_RB], zn[TMM_U][NSB];
    auto load_chunk = [&](int c, f32x4 (&w)[TMM_U][TMM_RB], f32x4 (&z)[TMM_U][NSB]) {
      const int k0 = c * 16 * TMM_U;
#pragma unroll
      for (int u = 0; u < TMM_U; ++u) {
        const int k = k0 + 16 * u + 4 * g;
        const bool kin = c < c_end && k < D;
#pragma unroll
        for (int rb = 0; rb < TMM_RB; ++rb) {
          const int o = o0 + rb * 16 + r16;
          w[u][rb] = (kin && o < O) ? stream_load(w2 + (size_t)o * D + k) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
          const int b = b0 + sb * 16 + r16;
          z[u][sb] = (kin && b < B) ? *reinterpret_cast<const f32x4 *>(zs + (size_t)b * D + k)
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    };
    load_chunk(c_beg, wn, zn);
    for (int c = c_beg; c < c_end; ++c) {
#pragma unroll
      for (int u = 0; u < TMM_U; ++u) {
#pragma unroll
        for (int rb = 0; rb < TMM_RB; ++rb) wv[u][rb] = wn[u][rb];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) zv[u][sb] = zn[u][sb];
      }
      load_chunk(c + 1, wn, zn);
#pragma unroll
      for (int u = 0; u < TMM_U; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int rb = 0; rb < TMM_RB; ++rb)
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
              acc[rb][sb] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[u][rb][j], zv[u][sb][j], acc[rb][sb], 0, 0, 0);
    }
    // the K ranges' partial blocks meet in LDS; each thread then adds the
    // TMM_W partials of (block, lane) slots
    __syncthreads();  // the previous sample group's slots have been read
#pragma unroll
    for (int rb = 0; rb < TMM_RB; ++rb)
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) red[wave][rb * NSB + sb][lane] = acc[rb][sb];
    __syncthreads();
    for (int e = threadIdx.x; e < TMM_RB * NSB * 64; e += blockDim.x) {
      const int blk = e / 64, l = e % 64;
      const int rb = blk / NSB, sb = blk % NSB;
      f32x4 v = red[0][blk][l];
#pragma unroll
      for (int w = 1; w < TMM_W; ++w) v += red[w][blk][l];
      // C of a 16x16 block: lane l holds rows 4 (l / 16) + i of column l % 16
      const int b = b0 + sb * 16 + (l & 15);
      if (b >= B) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = o0 + rb * 16 + 4 * (l >> 4) + i;
        if (o < O) mod[(size_t)b * O + o] = v[i];
      }
    }
  }
}

hipError_t launch_tmod(const float *t, const float *w1, const float *w2, float *mod, float *zs,
                       int B, int D, int tdim, hipStream_t s) {
  hipLaunchKernelGGL(tmod_stage1, dim3((D + 15) / 16, (B + TM1_NB - 1) / TM1_NB), dim3(256), 0, s, t, w1, zs, B, D,
                     tdim);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_tmod_map(zs, w2, mod, B, D, 6 * D, s);
}

hipError_t launch_tmod_map(const float *zs, const float *w, float *out, int B, int D, int O, hipStream_t s) {
  if (B <= TM_NB && (size_t)B * D * sizeof(float) <= 64 * 1024)
    hipLaunchKernelGGL(tmod_stage2_fewb, dim3((O + 63) / 64), dim3(256), (size_t)B * D * sizeof(float), s,
                       zs, w, out, B, D, O);
  else {
    // blocks of 16 samples per pass over W: as many as B needs, at most 4
    const dim3 grid((O + 16 * TMM_RB - 1) / (16 * TMM_RB)), block(TMM_W * 64);
    const int nsb = (B + 15) / 16;
    if (nsb <= 1)
      hipLaunchKernelGGL(tmod_stage2_mfma<1>, grid, block, 0, s, zs, w, out, B, D, O);
    else if (nsb <= 2)
      hipLaunchKernelGGL(tmod_stage2_mfma<2>, grid, block, 0, s, zs, w, out, B, D, O);
    else
      hipLaunchKernelGGL(tmod_stage2_mfma<4>, grid, block, 0, s, zs, w, out, B, D, O);
  }
  return hipGetLastError();
}

}  // namespace dit
