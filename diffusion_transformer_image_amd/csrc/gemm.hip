// MFMA GEMM for the projections of the DiT block: C[M,N] = A[M,K] * W[N,K]^T
// (nn.Linear layout: both operands K-contiguous), with an optional fused
// SwiGLU epilogue for the up/gate projection (page "Krea 2 技术报告",
// 架构 › Transformer块: SwiGLU MLP; grouped-query attention projections).
//
// Design for gfx950:
//  * a workgroup owns a BM x BN output tile; WM x WN waves each own a
//    (BM/WM) x (BN/WN) sub-tile of 16x16 MFMA blocks with fp32 accumulators;
//  * K advances 128 bytes per stage (64 bf16 / 32 fp32).  Operands go from
//    HBM straight into LDS with buffer_load ... lds (no VGPR staging),
//    double-buffered, one barrier per stage;
//  * LDS rows are 128 bytes; 16-byte chunk c of row r is stored at chunk
//    c ^ (r & 7), so the MFMA fragment reads (16 rows x one chunk per lane
//    group) spread over all banks;
//  * tails in M, N and K are zero-filled by the buffer descriptor's range
//    check (out-of-range chunks are given an out-of-range offset);
//  * workgroup ids are remapped so that each XCD (dispatch is round-robin
//    over the 8 XCDs) walks a contiguous band of tiles that share A rows.
#include "dit_common.h"
#include "dit_kernels.h"

namespace dit {

enum { EPI_STORE = 0, EPI_SWIGLU = 1 };

template <typename T, int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM *WN * 64) void gemm_kernel(const T *__restrict__ A,
                                                           const T *__restrict__ W,
                                                           T *__restrict__ C, int M, int N, int K,
                                                           int m_tiles, int n_tiles) {
  constexpr int NW = WM * WN;
  constexpr int ROWB = 128;               // bytes of K per LDS row per stage
  constexpr int EPC = 16 / sizeof(T);     // elements per 16-byte chunk
  constexpr int KSTAGE = ROWB / sizeof(T);  // K elements per stage
  constexpr int TM = BM / WM, TN = BN / WN;  // wave sub-tile
  constexpr int RB = TM / 16, CB = TN / 16;
  constexpr int ABLK = BM / 8, BBLK = BN / 8;  // 1 KiB blocks (8 rows) per stage
  constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  static_assert((ABLK + BBLK) % NW == 0, "blocks must split evenly over waves");
  static_assert(EPI != EPI_SWIGLU || (CB % 2 == 0), "SwiGLU pairs column blocks");

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile id: XCD-contiguous remap, then grouped (GM row tiles) order
  const int nwg = m_tiles * n_tiles;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  constexpr int GM = 8;
  const int group = pid / (GM * n_tiles);
  const int first_m = group * GM;
  const int gsz = min(m_tiles - first_m, GM);
  const int in_g = pid - group * GM * n_tiles;
  const int tm = first_m + in_g % gsz, tn = in_g / gsz;
  const int m0 = tm * BM;
  // SwiGLU: W holds [W1; W3] with N = F rows each; the tile covers F-columns
  // [f0, f0 + BN/2) and reads those rows of both halves.
  const int n0 = (EPI == EPI_SWIGLU) ? tn * (BN / 2) : tn * BN;

  // Descriptors span only the rows this tile may touch, so 32-bit offsets
  // suffice for any M (the host checks (2N + BN) * K * sizeof(T) < 2^31).
  const uint32_t ldb = (uint32_t)K * sizeof(T);  // row pitch in bytes
  const rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)min(M - m0, BM) * ldb);
  const rsrc_t rw = (EPI == EPI_SWIGLU)
                        ? make_rsrc(W + (size_t)n0 * K, (uint32_t)(N + min(N - n0, BN / 2)) * ldb)
                        : make_rsrc(W + (size_t)n0 * K, (uint32_t)min(N - n0, BN) * ldb);

  // ---- per-lane load offsets: lane writes LDS slot lane of a 1 KiB block =
  // row lane/8, physical chunk lane%8, which holds logical chunk
  // (lane%8) ^ (lane/8).
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow;
  constexpr int BPW = (ABLK + BBLK) / NW;
  uint32_t goff[BPW];
  bool gval[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int blk = wave + j * NW;
    if (blk < ABLK) {
      const int r = blk * 8 + lrow;
      gval[j] = (m0 + r) < M;
      goff[j] = (uint32_t)r * ldb + lchunk * 16;
    } else {
      const int r = (blk - ABLK) * 8 + lrow;
      if (EPI == EPI_SWIGLU) {
        // rows [0, BN/2) of the tile: W1 row n0 + r; rows [BN/2, BN): W3 row
        // N + n0 + r - BN/2 (offsets relative to the descriptor at row n0)
        const int rr = r < BN / 2 ? r : r - BN / 2;
        gval[j] = n0 + rr < N;
        goff[j] = (uint32_t)(r < BN / 2 ? rr : N + rr) * ldb + lchunk * 16;
      } else {
        gval[j] = (n0 + r) < N;
        goff[j] = (uint32_t)r * ldb + lchunk * 16;
      }
    }
  }

  auto issue_stage = [&](int kt, int buf) {
    const int k0 = kt * KSTAGE;
    const bool ktail = (k0 + KSTAGE) > K;
    const int kc_ok = ktail ? (K - k0) / EPC : 8;  // chunks of this stage inside K
    char *base = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int blk = wave + j * NW;
      const bool ok = gval[j] && (lchunk < kc_ok);
      const uint32_t off = ok ? goff[j] + (uint32_t)k0 * sizeof(T) : kOOB;
      load_lds16(blk < ABLK ? ra : rw, base + blk * 1024, off);
    }
  };

  f32x4 acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment rows inside the stage buffer
  const int g = lane >> 4, r16 = lane & 15;
  const int swz = lane & 7;  // (row & 7) for every fragment row this lane reads
  int arow[RB], brow[CB];
#pragma unroll
  for (int i = 0; i < RB; ++i) arow[i] = wm * TM + i * 16 + r16;
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    if (EPI == EPI_SWIGLU) {
      const int half = CB / 2, jj = j % half;
      brow[j] = BM + (j < half ? 0 : BN / 2) + wn * (TN / 2) + jj * 16 + r16;
    } else {
      brow[j] = BM + wn * TN + j * 16 + r16;
    }
  }

  const int nk = (K + KSTAGE - 1) / KSTAGE;
  issue_stage(0, 0);
  wait_vmem();
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) issue_stage(kt + 1, buf ^ 1);
    const char *sb = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int pc = ((ks * 4 + g) ^ swz) * 16;
      u32x4 af[RB], bfr[CB];
#pragma unroll
      for (int i = 0; i < RB; ++i) af[i] = *reinterpret_cast<const u32x4 *>(sb + arow[i] * ROWB + pc);
#pragma unroll
      for (int j = 0; j < CB; ++j) bfr[j] = *reinterpret_cast<const u32x4 *>(sb + brow[j] * ROWB + pc);
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = mma16<T>(af[i], bfr[j], acc[i][j]);
    }
    wait_vmem();
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4g+i of column r16 of every 16x16 block
  if (EPI == EPI_SWIGLU) {
    constexpr int half = CB / 2;
#pragma unroll
    for (int j = 0; j < half; ++j) {
      const int col = n0 + wn * (TN / 2) + j * 16 + r16;
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + wm * TM + i * 16 + 4 * g + e;
          if (row < M) {
            const float a = acc[i][j][e], b = acc[i][j + half][e];
            C[(size_t)row * N + col] = from_f32<T>(silu(a) * b);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int col = n0 + wn * TN + j * 16 + r16;
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + wm * TM + i * 16 + 4 * g + e;
          if (row < M) C[(size_t)row * N + col] = from_f32<T>(acc[i][j][e]);
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int WM, int WN, int EPI>
static hipError_t launch_gemm_t(const void *a, const void *w, void *c, int M, int N, int K,
                                hipStream_t s) {
  const int mt = (M + BM - 1) / BM;
  const int nt = (EPI == EPI_SWIGLU) ? (N + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI>), dim3(mt * nt), dim3(WM * WN * 64), 0,
                     s, (const T *)a, (const T *)w, (T *)c, M, N, K, mt, nt);
  return hipGetLastError();
}

hipError_t launch_gemm(bool f32, const void *a, const void *w, void *c, int M, int N, int K,
                       hipStream_t s) {
  if (f32) return launch_gemm_t<float, 256, 256, 2, 4, EPI_STORE>(a, w, c, M, N, K, s);
  // narrow outputs (N <= 4096) leave too few 256x256 tiles for 256 CUs
  if (N <= 4096) return launch_gemm_t<bf16, 256, 128, 4, 2, EPI_STORE>(a, w, c, M, N, K, s);
  return launch_gemm_t<bf16, 256, 256, 2, 4, EPI_STORE>(a, w, c, M, N, K, s);
}

hipError_t launch_gemm_swiglu(bool f32, const void *a, const void *w13, void *u, int M, int F,
                              int K, hipStream_t s) {
  if (f32) return launch_gemm_t<float, 256, 256, 2, 4, EPI_SWIGLU>(a, w13, u, M, F, K, s);
  return launch_gemm_t<bf16, 256, 256, 2, 4, EPI_SWIGLU>(a, w13, u, M, F, K, s);
}

}  // namespace dit
