// Flash-style grouped-query attention with a sigmoid output gate for the
// single-stream DiT block (page "Krea 2 技术报告", 架构 › Transformer块:
// GQA, the report's reference 45, with the gated attention of its
// reference 47; one joint text+image sequence, no mask, no positions).
//
//   og[q, h*d:(h+1)*d] = softmax_k(Q_h[q] . K_j[k] / sqrt(d)) V_j * sigmoid(G_h[q])
//   with j = h / (H / Hkv).
//
// Design for gfx950:
//  * one workgroup = (sample b, KV head j, 64 query tokens) for ALL query
//    heads of the group: the K / V tiles of head j are brought to LDS once
//    and read by group * 2 waves (each wave: one query head, 32 queries);
//  * scores are computed transposed, S^T = K Q^T (MFMA 16x16), so each
//    lane owns one query column: the online-softmax statistics of a query
//    live in 4 lanes (one per lane group) and the probabilities P^T are
//    already in the register layout of the B operand of O^T = V^T P^T;
//  * V^T tiles are written to LDS transposed (4 keys x 16 bytes per
//    thread), with an XOR swizzle of the 4-key units by (d & 15);
//  * K tiles go HBM -> LDS directly (buffer_load ... lds), double-buffered;
//  * softmax in fp32 with exp2 and the 1/sqrt(d) scale folded into one FMA;
//    the running max is shared by the 4 lanes of a query via xor shuffles;
//  * epilogue: divide by the row sum, multiply by sigmoid(G), store.
#include "dit_common.h"
#include "dit_kernels.h"

namespace dit {

constexpr int ATT_BQ = 64;   // query tokens per workgroup
constexpr int ATT_QW = 32;   // query tokens per wave
constexpr int ATT_BK = 64;   // keys per tile

template <typename T, int HD, int MIN_THREADS>
__global__ __launch_bounds__(512) void attn_kernel(const T *__restrict__ qkvg, T *__restrict__ og,
                                                   int L, int H, int Hkv, float sc) {
  constexpr int ES = sizeof(T);
  constexpr int EPC = 16 / ES;          // elements per 16-byte chunk
  constexpr int KROW = HD * ES;         // bytes of one K row in LDS
  constexpr int NCK = KROW / 16;        // chunks per K row
  constexpr int KS = KROW / 64;         // MFMA k-steps over d (4 chunks each)
  constexpr int KTILE = ATT_BK * KROW;  // bytes of a K tile
  constexpr int VROW = ATT_BK * ES;     // bytes of one V^T row (64 keys)
  constexpr int UB = 4 * ES;            // bytes of a 4-key unit of V^T
  constexpr int VTILE = HD * VROW;
  constexpr int STAGE = KTILE + VTILE;
  constexpr int DB = HD / 16;           // 16-row blocks of d
  constexpr int QB = ATT_QW / 16;       // 16-column blocks of queries per wave
  constexpr int KB = ATT_BK / 16;       // 16-key blocks per tile
  static_assert(NCK >= 8, "K rows need >= 8 chunks for the swizzle");

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int nthreads = blockDim.x;
  const int group = H / Hkv;
  const int b = blockIdx.z, j = blockIdx.y;
  const int h = j * group + (wave >> 1);
  const int q0 = blockIdx.x * ATT_BQ + (wave & 1) * ATT_QW;
  const int g = lane >> 4, r16 = lane & 15;

  const int ldq = (2 * H + 2 * Hkv) * HD;  // elements per token row of qkvg
  const uint32_t ldqb = (uint32_t)ldq * ES;
  const T *base = qkvg + (size_t)b * L * ldq;
  const rsrc_t rq = make_rsrc(base, (uint32_t)L * ldqb);
  const uint32_t kcol = (uint32_t)(H + j) * HD * ES;
  const uint32_t vcol = (uint32_t)(H + Hkv + j) * HD * ES;

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers
  u32x4 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = q0 + qb * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t off = (uint32_t)q * ldqb + (uint32_t)h * HD * ES + (ks * 4 + g) * 16;
      qf[qb][ks] = load16(rq, q < L ? off : kOOB);
    }
  }

  // ---- tile loaders
  const int nwaves = nthreads >> 6;
  auto issue_k = [&](int t, int buf) {
    char *kb = smem + buf * STAGE;
    constexpr int ROWS_PER_BLK = 1024 / KROW;
    constexpr int NBLK = KTILE / 1024;
    for (int blk = wave; blk < NBLK; blk += nwaves) {
      const int row = blk * ROWS_PER_BLK + lane / NCK;
      const int pc = lane % NCK;
      const int lc = pc ^ (row & 7);
      const int key = t * ATT_BK + row;
      const uint32_t off = key < L ? (uint32_t)key * ldqb + kcol + lc * 16 : kOOB;
      load_lds16(rq, kb + blk * 1024, off);
    }
  };
  // V: each unit is 4 keys x EPC d-values; loaded to registers, then
  // written transposed.  Units per tile = 16 * HD / EPC.
  constexpr int NVU = (ATT_BK / 4) * (HD / EPC);
  constexpr int VU_PER_T = (NVU + MIN_THREADS - 1) / MIN_THREADS;
  u32x4 vreg[VU_PER_T][4];
  auto load_v = [&](int t) {
#pragma unroll
    for (int u = 0; u < VU_PER_T; ++u) {
      const int unit = tid + u * nthreads;
      if (unit < NVU) {
        const int kg = unit % (ATT_BK / 4), dc = unit / (ATT_BK / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = t * ATT_BK + kg * 4 + r;
          const uint32_t off = key < L ? (uint32_t)key * ldqb + vcol + dc * 16 : kOOB;
          vreg[u][r] = load16(rq, off);
        }
      }
    }
  };
  auto store_vt = [&](int buf) {
    char *vt = smem + buf * STAGE + KTILE;
#pragma unroll
    for (int u = 0; u < VU_PER_T; ++u) {
      const int unit = tid + u * nthreads;
      if (unit < NVU) {
        const int kg = unit % (ATT_BK / 4), dc = unit / (ATT_BK / 4);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int d = dc * EPC + e;
          char *dst = vt + d * VROW + ((kg ^ (d & 15)) * UB);
          if constexpr (ES == 2) {
            // element e of 4 consecutive key rows -> one 8-byte unit
            uint32_t w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t word = vreg[u][r][e >> 1];
              w[r] = (e & 1) ? (word >> 16) : (word & 0xFFFFu);
            }
            *reinterpret_cast<u32x2 *>(dst) = u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
          } else {
            *reinterpret_cast<u32x4 *>(dst) =
                u32x4{vreg[u][0][e], vreg[u][1][e], vreg[u][2][e], vreg[u][3][e]};
          }
        }
      }
    }
  };

  f32x4 o[DB][QB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int k = 0; k < QB; ++k) o[i][k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[QB], lrow[QB];
#pragma unroll
  for (int k = 0; k < QB; ++k) { mrow[k] = -INFINITY; lrow[k] = 0.f; }

  const int nt = (L + ATT_BK - 1) / ATT_BK;
  issue_k(0, 0);
  load_v(0);
  store_vt(0);
  wait_vmem();
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nt) {
      issue_k(t + 1, buf ^ 1);
      load_v(t + 1);
    }
    const char *kt = smem + buf * STAGE;
    const char *vt = kt + KTILE;

    // S^T[kb][qb]: lane holds keys kb*16 + 4g + i of query qb*16 + r16
    f32x4 s[KB][QB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int row = kb * 16 + r16;
        const u32x4 kf = *reinterpret_cast<const u32x4 *>(kt + row * KROW + (((ks * 4 + g) ^ (row & 7)) * 16));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mma16<T>(kf, qf[qb][ks], s[kb][qb]);
      }
    }

    // mask keys past the end of the sequence (last tile only)
    if ((t + 1) * ATT_BK > L) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t * ATT_BK + kb * 16 + 4 * g + i >= L)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb][i] = -INFINITY;
    }

    // online softmax per query column
    float alpha[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrow[qb], mx);
      alpha[qb] = __builtin_amdgcn_exp2f((mrow[qb] - mnew) * sc);
      mrow[qb] = mnew;
      const float msc = mnew * sc;
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][i], sc, -msc));
          s[kb][qb][i] = p;
          sum += p;
        }
      lrow[qb] = lrow[qb] * alpha[qb] + sum;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db][qb] *= alpha[qb];
    }

    // O^T[db][qb] += V^T[db rows] * P^T
    if constexpr (ES == 2) {
      // bf16: one MFMA (k = 32) per pair of 16-key blocks
#pragma unroll
      for (int pr = 0; pr < KB / 2; ++pr) {
        u32x4 pf[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          bf16x8 pv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pv[i] = (bf16)s[2 * pr][qb][i];
            pv[4 + i] = (bf16)s[2 * pr + 1][qb][i];
          }
          pf[qb] = __builtin_bit_cast(u32x4, pv);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 16 + r16;
          const char *rowp = vt + d * VROW;
          const u32x2 lo = *reinterpret_cast<const u32x2 *>(rowp + ((((2 * pr) * 4 + g) ^ r16) * UB));
          const u32x2 hi = *reinterpret_cast<const u32x2 *>(rowp + ((((2 * pr + 1) * 4 + g) ^ r16) * UB));
          const u32x4 vf = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[db][qb] = mma16<T>(vf, pf[qb], o[db][qb]);
        }
      }
    } else {
      // fp32: four MFMAs (k = 4 each) per 16-key block
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        u32x4 pf[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) pf[qb] = __builtin_bit_cast(u32x4, s[kb][qb]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 16 + r16;
          const u32x4 vf = *reinterpret_cast<const u32x4 *>(vt + d * VROW + (((kb * 4 + g) ^ r16) * UB));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[db][qb] = mma16<T>(vf, pf[qb], o[db][qb]);
        }
      }
    }

    if (t + 1 < nt) store_vt(buf ^ 1);
    wait_vmem();
    __syncthreads();
  }

  // ---- epilogue: row sums over the 4 lane groups, normalise, gate, store
  const uint32_t gcol = (uint32_t)(H + 2 * Hkv + h) * HD;
  const int ldo = H * HD;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l = lrow[qb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = 1.0f / l;
    const int q = q0 + qb * 16 + r16;
    if (q < L) {
      const T *grow = base + (size_t)q * ldq + gcol;
      T *orow = og + ((size_t)b * L + q) * ldo + (size_t)h * HD;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 16 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = to_f32(grow[d + i]);
          orow[d + i] = from_f32<T>(o[db][qb][i] * inv * sigmoid(gv));
        }
      }
    }
  }
}

template <typename T, int HD>
static hipError_t launch_attn_t(const void *qkvg, void *og, int B, int L, int H, int Hkv,
                                hipStream_t s) {
  const int group = H / Hkv;
  dim3 grid((L + ATT_BQ - 1) / ATT_BQ, Hkv, B);
  const int nthr = group * (ATT_BQ / ATT_QW) * 64;
  // log2(e) / sqrt(d): softmax in base 2 with the score scale in one FMA
  const float sc = 1.4426950408889634f / sqrtf((float)HD);
  if (nthr >= 256)
    hipLaunchKernelGGL((attn_kernel<T, HD, 256>), grid, dim3(nthr), 0, s, (const T *)qkvg, (T *)og, L, H, Hkv, sc);
  else
    hipLaunchKernelGGL((attn_kernel<T, HD, 128>), grid, dim3(nthr), 0, s, (const T *)qkvg, (T *)og, L, H, Hkv, sc);
  return hipGetLastError();
}

hipError_t launch_attention(bool f32, int head_dim, const void *qkvg, void *og, int B, int L, int H,
                            int Hkv, hipStream_t s) {
  if (f32) {
    if (head_dim == 64) return launch_attn_t<float, 64>(qkvg, og, B, L, H, Hkv, s);
    if (head_dim == 128) return launch_attn_t<float, 128>(qkvg, og, B, L, H, Hkv, s);
  } else {
    if (head_dim == 128) return launch_attn_t<bf16, 128>(qkvg, og, B, L, H, Hkv, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dit
