// Device-side helpers shared by the gfx950 kernels of the DiT block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer descriptor over [base, base + bytes).  Loads whose byte range
// is not inside it return zeros, which is how every tile edge is handled:
// an out-of-range chunk gets the offset kOOB.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}
constexpr uint32_t kOOB = 0x80000000u;

// 16 bytes per lane from global memory straight into LDS: lane i of the
// wave writes bytes [16 i, 16 i + 16) after the wave-uniform LDS address.
__device__ __forceinline__ void load_lds16(rsrc_t r, const void *lds_wave_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_wave_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ u32x4 load16(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}
__device__ __forceinline__ u32x2 load8(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt lgkmcnt(0) as a real instruction (not inline asm), so the
// compiler's wait-insertion pass sees it.  Placed before a main loop, it
// retires the scalar kernel-argument loads the scheduler tends to leave in
// flight: scalar loads return out of order, and while one is pending every
// LDS wait in the loop degrades to lgkmcnt(0), which serialises the
// software-pipelined fragment reads with the MFMAs.
// Encoding (gfx9): vmcnt = 63 (bits 3:0, 15:14), expcnt = 7, lgkmcnt = 0.
__device__ __forceinline__ void drain_lgkm() { __builtin_amdgcn_s_waitcnt(0xc07f); }

template <typename T> struct is_bf16 { static constexpr bool value = false; };
template <> struct is_bf16<bf16> { static constexpr bool value = true; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// One 16x16 MFMA "k-chunk": each lane supplies 16 bytes of A and of B.
// bf16: 8 elements -> one v_mfma_f32_16x16x32_bf16 (k = 32).
// f32 : 4 elements -> four v_mfma_f32_16x16x4_f32 (k = 16).
// Lane l contributes row (l % 16) of A / column (l % 16) of B at the
// k positions owned by lane group l / 16; A and B use the same k order, so
// the product sums every k exactly once.  C/D: lane l holds rows
// 4 (l / 16) + i, i = 0..3, of column l % 16.
template <typename T> __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mma16<bf16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mma16<float>(u32x4 a, u32x4 b, f32x4 c) {
  // Reinterpret the whole vector: a bit_cast of a single element of an
  // ext_vector (`a.y`) is miscompiled by this clang to read element 0.
  const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[0], bf[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[1], bf[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[2], bf[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[3], bf[3], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Eight values times inv as OCP e4m3 codes (the hardware conversion rounds
// to nearest even), packed little-endian: element i is byte i.
__device__ __forceinline__ u32x2 fp8_pack8(const float (&v)[8], float inv) {
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * inv, v[1] * inv, 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * inv, v[3] * inv, w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4] * inv, v[5] * inv, 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6] * inv, v[7] * inv, w1, true);
  return u32x2{(uint32_t)w0, (uint32_t)w1};
}
// The row-wise scale of a row with largest magnitude amax (s = amax / 448,
// an all-zero row gets s = 1) and the factor its values are multiplied by
// before the conversion (448 / amax, 0 for an all-zero row).
__device__ __forceinline__ float fp8_row_scale(float amax) { return amax > 0.f ? amax / 448.0f : 1.0f; }
__device__ __forceinline__ float fp8_row_inv(float amax) { return amax > 0.f ? 448.0f / amax : 0.0f; }

// z * sigmoid(z) with the hardware reciprocal (~1 ulp) instead of an IEEE
// division (a ~10-instruction sequence per element in the GEMM epilogues);
// z -> -inf gives -0, z -> +inf gives z
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

}  // namespace dit
