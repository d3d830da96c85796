// MFMA GEMM for the projections of the DiT block: C[M,N] = A[M,K] * W[N,K]^T
// (nn.Linear layout: both operands K-contiguous), with an optional fused
// SwiGLU epilogue for the up/gate projection (page "Krea 2 技术报告",
// 架构 › Transformer块: SwiGLU MLP; the attention projections).
//
// Design for gfx950:
//  * a workgroup owns a BM x BN output tile; WM x WN waves each own a
//    (BM/WM) x (BN/WN) sub-tile of 16x16 MFMA blocks with fp32 accumulators;
//  * K advances BKB bytes per stage (64 or 128 bytes of every row).  Operands
//    go from HBM straight into LDS with buffer_load ... lds (no VGPR
//    staging) through a STAGES-deep ring: the loads of stage kt+STAGES-1 are
//    issued while stage kt is multiplied, and each wave waits only for its
//    own loads of the stage it is about to read (partial vmcnt), so one
//    barrier per stage is the only synchronisation; in the pipelined
//    two-stage loop the refill of a stage is spread over the MFMAs (one
//    load every few MFMAs) instead of leaving as a burst after the barrier;
//  * 16-byte chunk c of LDS row r sits at chunk c ^ swz(r), which spreads
//    the fragment reads (16 rows x one chunk per lane group) over all banks;
//  * tails in M, N and K are zero-filled by the buffer descriptor's range
//    check (out-of-range chunks are given an out-of-range offset);
//  * workgroup ids are remapped so that each XCD (dispatch is round-robin
//    over the 8 XCDs) walks a contiguous band of tiles, grouped gm row
//    tiles at a time, so tiles sharing A rows or W rows meet in one L2
//    (gm = 2 row tiles for the SwiGLU tile, 8 otherwise, unless the caller
//    sets it);
//  * the bf16 epilogue stages the whole output tile in LDS and each wave
//    stores whole rows (full cache lines).
#include <cmath>
#include <type_traits>

#include "dit_common.h"
#include "dit_kernels.h"

namespace dit {

enum { EPI_STORE = 0, EPI_SWIGLU = 1 };

template <int CPR>
__device__ __forceinline__ int chunk_swizzle(int row) {
  // CPR = 16-byte chunks per LDS row: 8 (128-byte rows) or 4 (64-byte rows)
  return CPR == 8 ? (row & 7) : ((row >> 1) & 3);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Split of the last tiles along K (stream-K style tail): tiles dp_tiles ..
// end of the grouped tile order are each computed by `segs` workgroups, one
// per contiguous range of K stages; those store fp32 partial tiles in `part`
// (slot = (tile - dp_tiles) * segs + segment, BM*BN floats each, in the
// accumulator register layout) and gemm_sk_fixup sums the segments of a tile
// in segment order and applies the epilogue.  segs == 1: no split.
struct SkPlan {
  int dp_tiles;
  int segs;
  float *part;
};

// Output columns [0, n) are multiplied by `scale` in fp32 before the one
// rounding to the output type (the attention score scale folded into the
// query columns of the QKVG product); n = 0: plain store.  Applies to the
// store epilogue only.
//
// vt != nullptr (bf16 store epilogue, whole tiles, no K split): output
// columns [vc0, vc1) -- the value heads of the QKVG product -- are written
// to vt in the transposed, key-permuted layout the attention kernel reads
// ([B][Hkv][d][L], see attention.hip: key k of a 64-key tile goes to chunk
// ((k >> 5) * 4 + ((k >> 2) & 3)) ^ (dd & 7), element ((k >> 4) & 1) * 4 +
// (k & 3)) instead of to C.  Needs L % 64 == 0, so every 32-row pair of
// 16-row blocks of a tile lies inside one sample and one half of a key
// tile: a lane then holds, for its column, keys 4g..4g+3 of both 16-key
// blocks of a chunk -- one 16-byte store.
struct ColScale {
  int n = 0;
  float scale = 1.f;
  bf16 *vt = nullptr;
  int vc0 = 0, vc1 = 0, L = 0;
  __device__ __forceinline__ float apply(int col, float v) const { return col < n ? v * scale : v; }
  __device__ __forceinline__ bool to_vt(int col) const { return vt && col >= vc0 && col < vc1; }
};

// The value columns of a wave's TM x TN sub-tile (rows row0.., columns
// col0..) into the V^T layout described at ColScale.
template <int TM, int TN>
__device__ __forceinline__ void store_vt(const f32x4 (&acc)[TM / 16][TN / 16], const ColScale &cs, int M,
                                         int row0, int col0, int lane) {
  constexpr int RB = TM / 16, CB = TN / 16;
  static_assert(RB % 2 == 0, "pairs of 16-row blocks");
  const int g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int col = col0 + j * 16 + r16;
    if (!cs.to_vt(col)) continue;
    const int cv = col - cs.vc0;
#pragma unroll
    for (int p = 0; p < RB / 2; ++p) {
      const int rb = row0 + 2 * p * 16;  // first row of the pair (a multiple of 32 inside its sample)
      if (rb >= M) continue;
      const int b = rb / cs.L, l = rb - b * cs.L;
      const int phys = ((((l >> 5) & 1) * 4) + g) ^ (cv & 7);
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = (bf16)acc[2 * p][j][e];
        v[4 + e] = (bf16)acc[2 * p + 1][j][e];
      }
      *reinterpret_cast<u32x4 *>(cs.vt + ((size_t)b * (cs.vc1 - cs.vc0) + cv) * cs.L + (l & ~63) + phys * 8) =
          __builtin_bit_cast(u32x4, v);
    }
  }
}

// Linear tile id -> (row tile, column tile): walks gm row tiles at a time,
// column-major inside a group, so tiles sharing operands run together.
__device__ __forceinline__ void tile_coords(int pid, int m_tiles, int n_tiles, int gm, int &tm, int &tn) {
  const int group = pid / (gm * n_tiles);
  const int first_m = group * gm;
  const int gsz = min(m_tiles - first_m, gm);
  const int in_g = pid - group * gm * n_tiles;
  tm = first_m + in_g % gsz;
  tn = in_g / gsz;
}

// One wave's TM x TN sub-tile straight to C (element stores), with the
// SwiGLU pairing of column blocks j and j + CB/2.
template <typename T, int TM, int TN, int EPI>
__device__ __forceinline__ void gemm_store_direct(const f32x4 (&acc)[TM / 16][TN / 16], T *__restrict__ C,
                                                  int M, int N, int row0, int col0, int lane,
                                                  const ColScale &cs) {
  constexpr int RB = TM / 16, CB = TN / 16;
  const int g = lane >> 4, r16 = lane & 15;
  if constexpr (EPI == EPI_STORE && is_bf16<T>::value)
    if (cs.vt) store_vt<TM, TN>(acc, cs, M, row0, col0, lane);
#pragma unroll
  for (int j = 0; j < CB / ((EPI == EPI_SWIGLU) ? 2 : 1); ++j) {
    const int col = col0 + j * 16 + r16;
    if (col >= N || (EPI == EPI_STORE && cs.to_vt(col))) continue;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = row0 + i * 16 + 4 * g + e;
        float v;
        if constexpr (EPI == EPI_SWIGLU) v = silu(acc[i][j][e]) * acc[i][j + CB / 2][e];
        else v = cs.apply(col, acc[i][j][e]);
        if (row < M) C[(size_t)row * N + col] = from_f32<T>(v);
      }
    }
  }
}

// Epilogue shared by the GEMM kernels: lane holds rows 4g+e of column r16 of
// every 16x16 block of its wave's TM x TN sub-tile.  bf16 output goes through
// LDS (16-byte chunks XOR-swizzled by row) and leaves as whole 16-byte chunks.
template <typename T, int BM, int BN, int NW, int WM, int WN, int EPI, int SMEM>
__device__ __forceinline__ void gemm_epilogue(const f32x4 (&acc)[BM / WM / 16][BN / WN / 16], char *smem,
                                              T *__restrict__ C, int M, int N, int m0, int n0,
                                              int wave, int lane, const ColScale &cs) {
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int RB = TM / 16, CB = TN / 16;
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4, r16 = lane & 15;
  constexpr int TNO = (EPI == EPI_SWIGLU) ? TN / 2 : TN;  // output columns per wave
  const int col0 = (EPI == EPI_SWIGLU) ? n0 + wn * (TN / 2) : n0 + wn * TN;
  const int row0 = m0 + wm * TM;
  auto out_val = [&](int i, int j, int e, int col) -> float {  // col: output column in C
    if constexpr (EPI == EPI_SWIGLU) return silu(acc[i][j][e]) * acc[i][j + CB / 2][e];
    else return cs.apply(col, acc[i][j][e]);
  };
  // (the XOR swizzle needs a power-of-two number of 16-byte chunks per row)
  constexpr int BNO = (EPI == EPI_SWIGLU) ? BN / 2 : BN;  // output columns of the tile
  constexpr int PITCH = BNO * 2;                           // bytes per tile row in LDS
  constexpr int CPRO = PITCH / 16;                         // 16-byte chunks per row
  if constexpr (sizeof(T) == 2 && CPRO >= 4 && (CPRO & (CPRO - 1)) == 0 && BM * PITCH <= SMEM &&
                BM % NW == 0) {
    // bf16: stage the whole BM x BNO output tile in LDS (16-byte chunks
    // XOR-swizzled by row), then each wave writes BM/NW whole rows of
    // PITCH contiguous bytes: every store instruction covers whole cache
    // lines (a wave's own sub-tile row is only 64 bytes for the SwiGLU
    // tile, half a line, which costs the L2 a merge per line).
    if constexpr (EPI == EPI_STORE)
      if (cs.vt) store_vt<TM, TN>(acc, cs, M, row0, col0, lane);
    __syncthreads();  // all waves are done reading the operand stages
#pragma unroll
    for (int j = 0; j < CB / ((EPI == EPI_SWIGLU) ? 2 : 1); ++j) {
      const int col = wn * TNO + j * 16 + r16;  // column inside the tile
#pragma unroll
      for (int i = 0; i < RB; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = wm * TM + i * 16 + 4 * g + e;
          const int off = row * PITCH + (((col >> 3) ^ (row & (CPRO - 1))) << 4) + (col & 7) * 2;
          *reinterpret_cast<bf16 *>(smem + off) = (bf16)out_val(i, j, e, n0 + col);
        }
      }
    }
    __syncthreads();  // the whole tile is staged
    constexpr int RPW = BM / NW;  // rows stored by each wave
#pragma unroll
    for (int q = lane; q < RPW * CPRO; q += 64) {
      const int row = wave * RPW + q / CPRO, c = q % CPRO;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(smem + row * PITCH + ((c ^ (row & (CPRO - 1))) << 4));
      const int gr = m0 + row, gc = n0 + c * 8;
      if (gr < M && (EPI != EPI_STORE || !cs.to_vt(gc))) {  // value columns went to V^T
        T *dst = C + (size_t)gr * N + gc;
        if (gc + 8 <= N && (N & 7) == 0) {
          *reinterpret_cast<u32x4 *>(dst) = v;
        } else {
          const bf16x8 vb = __builtin_bit_cast(bf16x8, v);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gc + e < N) dst[e] = vb[e];
        }
      }
    }
  } else {
    gemm_store_direct<T, TM, TN, EPI>(acc, C, M, N, row0, col0, lane, cs);
  }
}

// 16-byte LDS DMA with the K offset as the scalar offset (part of the
// descriptor's range check).
__device__ __forceinline__ void load_lds16_k(rsrc_t r, const void *lds_wave_base, uint32_t voff,
                                             uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_wave_base, 16, voff, soff, 0, 0);
}

// PIPE (two-stage ring only): software-pipelined main loop.  The fragments
// of k-step ks+1 are read from LDS while the MFMAs of k-step ks run, and the
// stage barrier sits between the last two MFMA bursts of a stage: the wave
// first reads its last fragments of stage kt, issues the MFMAs of the
// previous k-step, then waits for stage kt+1 and the barrier, reads the
// first fragments of stage kt+1 and refills the buffer stage kt used while
// its last MFMAs of stage kt execute.  When K is a whole number of stages
// the refill's DMA loads are spread one per RB*CB/BPW MFMAs instead of
// leaving as one burst right after the barrier (a burst from all waves
// queues in the texture path and raises the L2 latency every wave sees).
template <typename T, int BM, int BN, int BKB, int STAGES, int WM, int WN, int EPI, bool PIPE = false>
__global__ __launch_bounds__(WM *WN * 64) void gemm_kernel(const T *__restrict__ A,
                                                           const T *__restrict__ W,
                                                           T *__restrict__ C, int M, int N, int K,
                                                           int m_tiles, int n_tiles, int gm, SkPlan sk,
                                                           ColScale cs) {
  constexpr int NW = WM * WN;
  constexpr int CPR = BKB / 16;             // 16-byte chunks per row per stage
  constexpr int RPB = 1024 / BKB;           // rows per 1 KiB DMA block
  constexpr int EPC = 16 / sizeof(T);       // elements per chunk
  constexpr int KSTAGE = BKB / sizeof(T);   // K elements per stage
  constexpr int KSTEPS = CPR / 4;           // MFMA k-steps per stage (4 chunks each)
  constexpr int TM = BM / WM, TN = BN / WN;  // wave sub-tile
  constexpr int RB = TM / 16, CB = TN / 16;
  constexpr int ABLK = BM / RPB, BBLK = BN / RPB;  // DMA blocks per stage
  constexpr int STAGE_BYTES = (BM + BN) * BKB;
  constexpr int BPW = (ABLK + BBLK) / NW;   // DMA loads per wave per stage
  static_assert((ABLK + BBLK) % NW == 0, "blocks must split evenly over waves");
  static_assert(EPI != EPI_SWIGLU || (CB % 2 == 0), "SwiGLU pairs column blocks");
  static_assert(STAGES >= 2 && BPW * (STAGES - 2) < 64, "vmcnt range");
  static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile id: whole tiles first (XCD-contiguous remap, then grouped
  // order), then the K segments of the split tail tiles
  const int nk_all = (K + KSTAGE - 1) / KSTAGE;
  int pid, kb = 0, nk = nk_all, slot = -1;
  if ((int)blockIdx.x < sk.dp_tiles) {
    const int nwg = sk.dp_tiles;
    pid = blockIdx.x;
    if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  } else {
    slot = blockIdx.x - sk.dp_tiles;
    const int seg = slot % sk.segs;
    pid = sk.dp_tiles + slot / sk.segs;
    kb = seg * nk_all / sk.segs;
    nk = (seg + 1) * nk_all / sk.segs - kb;
  }
  int tm, tn;
  tile_coords(pid, m_tiles, n_tiles, gm, tm, tn);
  const int m0 = tm * BM;
  // SwiGLU: W holds [W1; W3] with N = F rows each; the tile covers F-columns
  // [n0, n0 + BN/2) and reads those rows of both halves.
  const int n0 = (EPI == EPI_SWIGLU) ? tn * (BN / 2) : tn * BN;

  // Descriptors span only the rows this tile may touch, so 32-bit offsets
  // suffice for any M (the host checks (2N + 256) * K * sizeof(T) < 2^31).
  const uint32_t ldb = (uint32_t)K * sizeof(T);  // row pitch in bytes
  const rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)min(M - m0, BM) * ldb);
  const rsrc_t rw = (EPI == EPI_SWIGLU)
                        ? make_rsrc(W + (size_t)n0 * K, (uint32_t)(N + min(N - n0, BN / 2)) * ldb)
                        : make_rsrc(W + (size_t)n0 * K, (uint32_t)min(N - n0, BN) * ldb);

  // ---- per-lane DMA offsets: lane writes LDS slot `lane` of a 1 KiB block
  // = row lane / CPR, physical chunk lane % CPR, which holds logical chunk
  // (lane % CPR) ^ swz(row).
  const int lrow = lane / CPR;
  const int lchunk = (lane % CPR) ^ chunk_swizzle<CPR>(lrow);
  uint32_t goff[BPW];
  bool gval[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int blk = wave + j * NW;
    if (blk < ABLK) {
      const int r = blk * RPB + lrow;
      gval[j] = (m0 + r) < M;
      goff[j] = (uint32_t)r * ldb + lchunk * 16;
    } else {
      const int r = (blk - ABLK) * RPB + lrow;
      if (EPI == EPI_SWIGLU) {
        // tile rows [0, BN/2): W1 row n0 + r; rows [BN/2, BN): W3 row
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
    const int k0 = (kb + kt) * KSTAGE;
    const int kc_ok = (k0 + KSTAGE > K) ? (K - k0) / EPC : CPR;  // chunks inside K
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

  // fragment rows inside a stage buffer (A rows first, then W rows)
  const int g = lane >> 4, r16 = lane & 15;
  const int swz = chunk_swizzle<CPR>(r16);  // every fragment row this lane reads is r16 mod 16
  int arow[RB], brow[CB];
#pragma unroll
  for (int i = 0; i < RB; ++i) arow[i] = (wm * TM + i * 16 + r16) * BKB;
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    int r;
    if (EPI == EPI_SWIGLU) {
      const int half = CB / 2, jj = j % half;
      r = BM + (j < half ? 0 : BN / 2) + wn * (TN / 2) + jj * 16 + r16;
    } else {
      r = BM + wn * TN + j * 16 + r16;
    }
    brow[j] = r * BKB;
  }

  auto load_frags = [&](const char *sb, int ks, u32x4(&af)[RB], u32x4(&bf)[CB]) {
    const int pc = ((ks * 4 + g) ^ swz) * 16;
#pragma unroll
    for (int i = 0; i < RB; ++i) af[i] = *reinterpret_cast<const u32x4 *>(sb + arow[i] + pc);
#pragma unroll
    for (int j = 0; j < CB; ++j) bf[j] = *reinterpret_cast<const u32x4 *>(sb + brow[j] + pc);
  };
  auto mmas = [&](const u32x4(&af)[RB], const u32x4(&bf)[CB]) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) acc[i][j] = mma16<T>(af[i], bf[j], acc[i][j]);
  };

  if constexpr (PIPE) {
  static_assert(STAGES == 2 && KSTEPS == 2, "pipelined loop: two stages of two k-steps");
  // PIPE with K a whole number of stages: the K offset of a stage is the
  // DMA's scalar offset; rows outside the operand carry an out-of-range
  // vector offset at every stage, and the stage past the end of K gets an
  // out-of-range scalar offset: its loads land in a buffer that is not read
  // again (zeros, or for a row outside the operand, whose two out-of-range
  // offsets may wrap to offset 0 in 32 bits, bytes from the start of the
  // operand: in bounds either way)
  uint32_t goffs[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) goffs[j] = gval[j] ? goff[j] : kOOB;
  auto issue_spread = [&](int kt, int buf) {
    const uint32_t soff = kt < nk ? (uint32_t)(kb + kt) * KSTAGE * sizeof(T) : kOOB;
    char *base = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int blk = wave + j * NW;
      load_lds16_k(blk < ABLK ? ra : rw, base + blk * 1024, goffs[j], soff);
    }
  };
  if (K % KSTAGE == 0) {
    // both buffers are free at the start: stage 1 goes out with stage 0
    issue_spread(0, 0);
    issue_spread(1, 1);
    wait_vmcnt<BPW>();  // this wave's loads of stage 0 (they complete in issue order)
    __syncthreads();
    u32x4 a0[RB], b0[CB], a1[RB], b1[CB];
    load_frags(smem, 0, a0, b0);
    drain_lgkm();
    for (int kt = 0; kt < nk - 1; ++kt) {
      const char *sb = smem + (kt & 1) * STAGE_BYTES;
      load_frags(sb, 1, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      mmas(a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();  // this wave's DMA of stage kt+1
      __syncthreads();  // stage kt+1 visible; every wave holds its stage-kt fragments
      // the second half of the stage (fragment reads, the refill spread over
      // the MFMAs) runs at raised wave priority: the SIMD's other wave, in
      // its first burst or at the barrier, then does not delay this wave's
      // loads and MFMAs.  The priority is raised before the reads and loads,
      // not between them and the MFMAs: s_setprio bounds the scheduling
      // groups, and placed there it leaves the refill as one burst
      __builtin_amdgcn_s_setprio(1);
      load_frags(smem + ((kt + 1) & 1) * STAGE_BYTES, 0, a0, b0);
      issue_spread(kt + 2, kt & 1);
      mmas(a1, b1);
      // scheduling groups: the fragment reads first, then BPW times (two
      // MFMAs, one DMA load), then the rest of the MFMAs: the refill leaves
      // within the first 2*BPW MFMAs (one load per 2 MFMAs measured best:
      // per 1, 3 or 4 MFMAs, or all loads first, were 1-3 % slower on W13)
#pragma unroll
      for (int q = 0; q < RB + CB; ++q) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int q = 0; q < BPW; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      static_assert(RB * CB >= 2 * BPW, "two MFMAs per refill load");
      __builtin_amdgcn_sched_group_barrier(0x008, RB * CB - 2 * BPW, 0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    }
    load_frags(smem + ((nk - 1) & 1) * STAGE_BYTES, 1, a1, b1);
    mmas(a0, b0);
    mmas(a1, b1);
    wait_vmcnt<0>();  // the stage past the end has landed before LDS is reused
  } else {
    issue_stage(0, 0);
    wait_vmcnt<0>();
    __syncthreads();
    if (nk > 1) issue_stage(1, 1);
    u32x4 a0[RB], b0[CB], a1[RB], b1[CB];
    load_frags(smem, 0, a0, b0);
    drain_lgkm();
    // The last stage is peeled so the loop body is straight-line: a branch
    // inside it would merge a path with the next stage's fragment reads in
    // flight into the wait before the second MFMA burst.
    // sched_barrier(0) keeps the instruction scheduler from moving the
    // fragment reads next to the MFMAs that consume them.
    for (int kt = 0; kt < nk - 1; ++kt) {
      const char *sb = smem + (kt & 1) * STAGE_BYTES;
      load_frags(sb, 1, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      mmas(a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();  // this wave's DMA of stage kt+1
      __syncthreads();  // stage kt+1 visible; every wave holds its stage-kt fragments
      if (kt + 2 < nk) issue_stage(kt + 2, kt & 1);
      load_frags(smem + ((kt + 1) & 1) * STAGE_BYTES, 0, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mmas(a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    }
    load_frags(smem + ((nk - 1) & 1) * STAGE_BYTES, 1, a1, b1);
    mmas(a0, b0);
    mmas(a1, b1);
  }
  } else {
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue_stage(s, s);

  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of stage kt are done once at most the loads of the
    // (up to STAGES-2) later stages already issued are still in flight
    if (kt + STAGES - 2 < nk) wait_vmcnt<BPW * (STAGES - 2)>();
    else wait_vmcnt<0>();
    __syncthreads();  // every wave's part of stage kt has landed; stage kt-1 is consumed
    if (kt + STAGES - 1 < nk) issue_stage(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    const char *sb = smem + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int pc = ((ks * 4 + g) ^ swz) * 16;
      u32x4 af[RB], bfr[CB];
#pragma unroll
      for (int i = 0; i < RB; ++i) af[i] = *reinterpret_cast<const u32x4 *>(sb + arow[i] + pc);
#pragma unroll
      for (int j = 0; j < CB; ++j) bfr[j] = *reinterpret_cast<const u32x4 *>(sb + brow[j] + pc);
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = mma16<T>(af[i], bfr[j], acc[i][j]);
    }
  }
  }

  if (slot >= 0) {  // a K segment of a split tile: fp32 partial, register layout
    float *dst = sk.part + (size_t)slot * BM * BN + (size_t)wave * RB * CB * 256 + lane * 4;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) *reinterpret_cast<f32x4 *>(dst + (i * CB + j) * 256) = acc[i][j];
    return;
  }
  gemm_epilogue<T, BM, BN, NW, WM, WN, EPI, STAGES * STAGE_BYTES>(acc, smem, C, M, N, m0, n0, wave,
                                                                 lane, cs);
}

// Sums the K-segment partials of each split tile in segment order and
// stores the result through the epilogue.  One workgroup (one wave) covers
// FRB of the RB row blocks of one wave sub-tile of one split tile, so the
// pass runs RB / FRB times more waves than the tiles have sub-tiles.
template <typename T, int BM, int BN, int WM, int WN, int EPI, int FRB>
__global__ __launch_bounds__(64) void gemm_sk_fixup(const float *__restrict__ part, T *__restrict__ C,
                                                    int M, int N, int m_tiles, int n_tiles, int gm,
                                                    int dp_tiles, int segs, ColScale cs) {
  constexpr int NW = WM * WN, TM = BM / WM, TN = BN / WN, RB = TM / 16, CB = TN / 16;
  static_assert(RB % FRB == 0, "row-block split");
  constexpr int NP = RB / FRB;  // workgroups per wave sub-tile
  const int lane = threadIdx.x;
  const int piece = blockIdx.x % NP, wave = (blockIdx.x / NP) % NW, t = blockIdx.x / (NP * NW);
  const int wm = wave / WN, wn = wave % WN;
  f32x4 acc[FRB][CB];
#pragma unroll
  for (int i = 0; i < FRB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sgm = 0; sgm < segs; ++sgm) {
    const float *src = part + (size_t)(t * segs + sgm) * BM * BN + (size_t)wave * RB * CB * 256 + lane * 4;
#pragma unroll
    for (int i = 0; i < FRB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j)
        acc[i][j] += *reinterpret_cast<const f32x4 *>(src + ((piece * FRB + i) * CB + j) * 256);
  }
  int tm, tn;
  tile_coords(dp_tiles + t, m_tiles, n_tiles, gm, tm, tn);
  const int row0 = tm * BM + wm * TM + piece * FRB * 16;
  const int col0 = (EPI == EPI_SWIGLU) ? tn * (BN / 2) + wn * (TN / 2) : tn * BN + wn * TN;
  gemm_store_direct<T, FRB * 16, TN, EPI>(acc, C, M, N, row0, col0, lane, cs);
}

// ---------------------------------------------------------------------------
// FP8 (OCP e4m3) GEMM with row-wise scales (the pages' 8-bit projections,
// page "Krea 2 技术报告", 训练 › 预训练: row-wise scaling):
//   C[m, n] = sa[m] sw[n] sum_k qa[m, k] qw[n, k]      (bf16 out)
// and the SwiGLU form over W13 = [W1; W3] (sw13 holds both halves' scales).
// Same tile, waves, LDS-DMA ring and epilogue as the bf16 kernel; a stage
// is 128 bytes of every row = 128 K elements = one v_mfma 16x16x128 f8
// k-step, so each lane's fragment is 32 bytes (two 16-byte chunks of its
// row).  The accumulators are scaled by sa[row] * sw[col] before the
// shared epilogue.
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int EPI>
__global__ __launch_bounds__(512) void gemm_fp8_kernel(const uint8_t *__restrict__ A, const float *__restrict__ sa,
                                                       const uint8_t *__restrict__ W, const float *__restrict__ sw,
                                                       bf16 *__restrict__ C, int M, int N, int K, int m_tiles,
                                                       int n_tiles, int gm, SkPlan sk, ColScale ocs) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4, NW = 8;
  constexpr int TM = BM / WM, TN = BN / WN, RB = TM / 16, CB = TN / 16;
  constexpr int BKB = 128, CPR = 8, RPB = 1024 / BKB;
  constexpr int ABLK = BM / RPB, BBLK = BN / RPB, STAGE = (BM + BN) * BKB, BPW = (ABLK + BBLK) / NW;
  // the ring, then the tile's row scales (sa of its BM rows) and the scales
  // of its BN operand rows of W, fetched at the start so their latency
  // overlaps the main loop instead of preceding the epilogue (one LDS
  // object: with a second one the compiler no longer keeps the fragment
  // reads clear of the in-flight DMA and waits for it before each read)
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE + (BM + BN) * 4];
  float *s_scale = reinterpret_cast<float *>(smem + 2 * STAGE);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  // whole tiles first (XCD-contiguous remap), then the K segments of the
  // split tail tiles, as in gemm_kernel (stages of 128 K elements)
  const int nk_all = (K + BKB - 1) / BKB;
  int pid, kb = 0, nk = nk_all, slot = -1;
  if ((int)blockIdx.x < sk.dp_tiles) {
    const int nwg = sk.dp_tiles;
    pid = blockIdx.x;
    if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  } else {
    slot = blockIdx.x - sk.dp_tiles;
    const int seg = slot % sk.segs;
    pid = sk.dp_tiles + slot / sk.segs;
    kb = seg * nk_all / sk.segs;
    nk = (seg + 1) * nk_all / sk.segs - kb;
  }
  int tm, tn;
  tile_coords(pid, m_tiles, n_tiles, gm, tm, tn);
  const int m0 = tm * BM;
  const int n0 = (EPI == EPI_SWIGLU) ? tn * (BN / 2) : tn * BN;
  // (called right after the first stage's DMA is issued, so the two
  // latencies overlap)
  auto stage_scales = [&]() {
    static_assert(BM + BN == 512, "one scale per thread");
    if (tid < BM) {
      s_scale[tid] = m0 + tid < M ? sa[m0 + tid] : 0.f;
    } else {
      // operand row r of the W tile: W1 rows n0.. then W3 rows N + n0..
      // for the SwiGLU tile, else rows n0..
      const int r = tid - BM;
      const int rr = (EPI == EPI_SWIGLU && r >= BN / 2) ? r - BN / 2 : r;
      const int wr = (EPI == EPI_SWIGLU && r >= BN / 2) ? N + n0 + rr : n0 + rr;
      s_scale[tid] = n0 + rr < N ? sw[wr] : 0.f;
    }
  };
  const uint32_t ldb = (uint32_t)K;
  const rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)min(M - m0, BM) * ldb);
  const rsrc_t rw = (EPI == EPI_SWIGLU)
                        ? make_rsrc(W + (size_t)n0 * K, (uint32_t)(N + min(N - n0, BN / 2)) * ldb)
                        : make_rsrc(W + (size_t)n0 * K, (uint32_t)min(N - n0, BN) * ldb);
  const int lrow = lane / CPR;
  const int lchunk = (lane % CPR) ^ (lrow & 7);
  uint32_t goff[BPW];
  bool gval[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int blk = wave + j * NW;
    if (blk < ABLK) {
      const int r = blk * RPB + lrow;
      gval[j] = (m0 + r) < M;
      goff[j] = (uint32_t)r * ldb + lchunk * 16;
    } else {
      const int r = (blk - ABLK) * RPB + lrow;
      if (EPI == EPI_SWIGLU) {
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
    const int k0 = (kb + kt) * BKB;
    const int kc_ok = (k0 + BKB > K) ? (K - k0) / 16 : CPR;
    char *base = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int blk = wave + j * NW;
      const bool ok = gval[j] && (lchunk < kc_ok);
      load_lds16(blk < ABLK ? ra : rw, base + blk * 1024, ok ? goff[j] + (uint32_t)k0 : kOOB);
    }
  };
  // lane group g supplies the k-chunks g and g + 4 of the 128-byte stage
  // (any k order works when A and B share it): each of the two reads then
  // has the bf16 kernel's conflict-free pattern, where chunks 2g and 2g + 1
  // measured ~3 bank-conflict cycles per LDS instruction cycle
  const int g = lane >> 4, r16 = lane & 15, swz = r16 & 7;
  const int c0 = (g ^ swz) * 16, c1 = ((g + 4) ^ swz) * 16;
  int arow[RB], brow[CB];
#pragma unroll
  for (int i = 0; i < RB; ++i) arow[i] = (wm * TM + i * 16 + r16) * BKB;
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    int r;
    if (EPI == EPI_SWIGLU) {
      const int half = CB / 2, jj = j % half;
      r = BM + (j < half ? 0 : BN / 2) + wn * (TN / 2) + jj * 16 + r16;
    } else {
      r = BM + wn * TN + j * 16 + r16;
    }
    brow[j] = r * BKB;
  }
  f32x4 acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto frag = [&](const char *sb, int row) {
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(sb + row + c0);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(sb + row + c1);
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  auto mmas = [&](const char *sb) {
    i32x8 bf[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) bf[j] = frag(sb, brow[j]);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const i32x8 af = frag(sb, arow[i]);
#pragma unroll
      for (int j = 0; j < CB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
  };
  if (K % BKB == 0) {
    // K a whole number of stages: the K offset is the DMA's scalar offset
    // (rows outside the operand keep an out-of-range vector offset; the
    // stage past the end gets an out-of-range scalar offset), and the 8
    // loads of the next stage are spread over the first half of the
    // stage's MFMAs, the A fragment reads of row block i+1 issued beside the
    // MFMAs of block i
    uint32_t goffs[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) goffs[j] = gval[j] ? goff[j] : kOOB;
    auto issue_spread = [&](int kt, int buf) {
      const uint32_t soff = kt < nk ? (uint32_t)(kb + kt) * BKB : kOOB;
      char *base = smem + buf * STAGE;
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const int blk = wave + j * NW;
        load_lds16_k(blk < ABLK ? ra : rw, base + blk * 1024, goffs[j], soff);
      }
    };
    static_assert(BPW == RB && RB % 2 == 0, "two DMA loads per row block over the first half");
    issue_spread(0, 0);
    stage_scales();
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<0>();  // this wave's DMA of stage kt
      __syncthreads();  // stage kt visible to all; every wave is done with stage kt-1
      const char *sb = smem + (kt & 1) * STAGE;
      char *nb = smem + ((kt + 1) & 1) * STAGE;
      const uint32_t soff = kt + 1 < nk ? (uint32_t)(kb + kt + 1) * BKB : kOOB;
      // program order: the fragment reads of stage kt, then the DMA loads
      // of stage kt+1 one per row block (the DMA writes the other buffer;
      // in this order the compiler may keep the loads beside the MFMAs)
      i32x8 bf[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) bf[j] = frag(sb, brow[j]);
      i32x8 af = frag(sb, arow[0]);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const i32x8 an = i + 1 < RB ? frag(sb, arow[i + 1]) : af;
        // the refill leaves two loads per row block over the first half of
        // the stage (one per block over all of it: the four products 1.83
        // -> 1.80 ms at 1024 px)
        if (2 * i < RB) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int blk = wave + (2 * i + h) * NW;
            load_lds16_k(blk < ABLK ? ra : rw, nb + blk * 1024, goffs[2 * i + h], soff);
          }
        }
#pragma unroll
        for (int j = 0; j < CB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
        af = an;
      }
    }
    wait_vmcnt<0>();  // the stage past the end has landed before LDS is reused
  } else {
    issue_stage(0, 0);
    stage_scales();
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<0>();  // this wave's DMA of stage kt
      __syncthreads();  // stage kt visible to all; every wave is done with stage kt-1
      if (kt + 1 < nk) issue_stage(kt + 1, (kt + 1) & 1);
      mmas(smem + (kt & 1) * STAGE);
    }
  }

  // ---- row and column scales (staged in LDS at the start; the main
  // loop's barriers made them visible), then the shared epilogue
  const float *s_row = s_scale, *s_col = s_scale + BM;
  float cs[CB];
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    if (EPI == EPI_SWIGLU)
      cs[j] = s_col[(j < CB / 2 ? 0 : BN / 2) + wn * (TN / 2) + (j % (CB / 2)) * 16 + r16];
    else
      cs[j] = s_col[wn * TN + j * 16 + r16];
  }
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float rs = s_row[wm * TM + i * 16 + 4 * g + e];
#pragma unroll
      for (int j = 0; j < CB; ++j) acc[i][j][e] *= rs * cs[j];
    }
  if (slot >= 0) {  // a K segment of a split tile: the scaled fp32 partial (the scales are per row and column)
    float *dst = sk.part + (size_t)slot * BM * BN + (size_t)wave * RB * CB * 256 + lane * 4;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) *reinterpret_cast<f32x4 *>(dst + (i * CB + j) * 256) = acc[i][j];
    return;
  }
  gemm_epilogue<bf16, BM, BN, NW, WM, WN, EPI, 2 * STAGE>(acc, smem, C, M, N, m0, n0, wave, lane, ocs);
}

template <int EPI>
static hipError_t launch_fp8_t(const void *aq, const float *sa, const void *wq, const float *sw, void *c, int M,
                               int N, int K, hipStream_t s, int sk_tiles, int segs, float *part, ColScale cs = {}) {
  const int mt = (M + 255) / 256, nt = (EPI == EPI_SWIGLU) ? (N + 127) / 128 : (N + 255) / 256;
  const int gm = (EPI == EPI_SWIGLU) ? 4 : 8;
  if (segs <= 1 || !part) sk_tiles = 0;
  const SkPlan plan{mt * nt - sk_tiles, sk_tiles ? segs : 1, part};
  hipLaunchKernelGGL(gemm_fp8_kernel<EPI>, dim3(plan.dp_tiles + sk_tiles * plan.segs), dim3(512), 0, s,
                     (const uint8_t *)aq, sa, (const uint8_t *)wq, sw, (bf16 *)c, M, N, K, mt, nt, gm, plan, cs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sk_tiles == 0) return e;
  // the partials carry the scales already: the bf16 fixup sums them and
  // applies the epilogue (same tile and accumulator layout)
  hipLaunchKernelGGL((gemm_sk_fixup<bf16, 256, 256, 2, 4, EPI, 2>), dim3(sk_tiles * 8 * 4), dim3(64), 0, s,
                     (const float *)part, (bf16 *)c, M, N, mt, nt, gm, plan.dp_tiles, plan.segs, cs);
  return hipGetLastError();
}

GemmChoice gemm_choose_fp8(int M, int N, int K, bool swiglu) {
  // the bf16 cost model on 128-element stages: a round costs about 0.6 of
  // the bf16 one, so the fixed cost of the partials weighs more; 192-row
  // tiles do not exist in FP8 (variant 0 only)
  GemmChoice ch = gemm_choose(M, N, (K + 1) / 2, swiglu);
  if (ch.sk_tiles == 0) return GemmChoice{0, 0, 1, 0};
  const int nk = (K + 127) / 128;
  if (ch.segs > nk / 2) return GemmChoice{0, 0, 1, 0};
  ch.variant = 0;
  return ch;
}

// A value-head request of launch_gemm (whole tiles only): checked and
// copied into the epilogue's column settings.
static bool set_vt(ColScale &cs, const GemmVt *vt, int M, int N) {
  if (!vt) return true;
  if (vt->L <= 0 || vt->L % 64 || M % vt->L || vt->c0 % 16 || vt->c1 % 16 || vt->c0 < 0 || vt->c1 <= vt->c0 ||
      vt->c1 > N)
    return false;
  cs.vt = (bf16 *)vt->vt;
  cs.vc0 = vt->c0;
  cs.vc1 = vt->c1;
  cs.L = vt->L;
  return true;
}

hipError_t launch_gemm_fp8(bool swiglu, const void *aq, const float *sa, const void *wq, const float *sw, void *c,
                           int M, int N, int K, hipStream_t s, float *part, size_t part_bytes, int scale_cols,
                           float col_scale, const GemmVt *vt) {
  GemmChoice ch{0, 0, 1, 0};
  if (part) {
    ch = gemm_choose_fp8(M, N, K, swiglu);
    if (part_bytes < ch.part_bytes) ch = GemmChoice{0, 0, 1, 0};
  }
  ColScale cs{scale_cols, col_scale};
  // the value heads go to V^T from whole tiles only (the caller checks
  // gemm_choose_fp8 first); the SwiGLU product has no column settings
  if (!set_vt(cs, vt, M, N) || (vt && (swiglu || ch.sk_tiles > 0)) || (swiglu && scale_cols))
    return hipErrorInvalidValue;
  if (swiglu) return launch_fp8_t<EPI_SWIGLU>(aq, sa, wq, sw, c, M, N, K, s, ch.sk_tiles, ch.segs, part);
  return launch_fp8_t<EPI_STORE>(aq, sa, wq, sw, c, M, N, K, s, ch.sk_tiles, ch.segs, part, cs);
}

template <typename T, int BM, int BN, int BKB, int STAGES, int WM, int WN, int EPI, bool PIPE = false>
static hipError_t launch_gemm_t(const void *a, const void *w, void *c, int M, int N, int K,
                                hipStream_t s, int gm, int sk_tiles = 0, int segs = 1, float *part = nullptr,
                                ColScale cs = {}) {
  const int mt = (M + BM - 1) / BM;
  const int nt = (EPI == EPI_SWIGLU) ? (N + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  if (segs <= 1 || !part) sk_tiles = 0;
  const SkPlan plan{mt * nt - sk_tiles, sk_tiles ? segs : 1, part};
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BKB, STAGES, WM, WN, EPI, PIPE>),
                     dim3(plan.dp_tiles + sk_tiles * plan.segs), dim3(WM * WN * 64), 0, s, (const T *)a,
                     (const T *)w, (T *)c, M, N, K, mt, nt, gm, plan, cs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sk_tiles == 0) return e;
  constexpr int FRB = (BM / WM / 16) % 2 == 0 ? 2 : 1;  // row blocks per fixup wave
  hipLaunchKernelGGL((gemm_sk_fixup<T, BM, BN, WM, WN, EPI, FRB>), dim3(sk_tiles * WM * WN * (BM / WM / 16 / FRB)),
                     dim3(64), 0, s, (const float *)part, (T *)c, M, N, mt, nt, gm, plan.dp_tiles, plan.segs,
                     cs);
  return hipGetLastError();
}

// Default configuration of a bf16 product, in units of one round of
// 256 x 256 tiles over the 256 CUs:
//  * whole 256 x 256 tiles: ceil(tiles / 256) rounds;
//  * whole 192 x 256 tiles: ceil(tiles192 / 256) rounds of ~0.85 (measured
//    per-round cost of the smaller tile);
//  * 256 x 256 tiles with the partial last round split along K into `segs`
//    segments per tile (2 <= segs <= min(8, 256 / tail tiles, nk / 2), the
//    cheapest): full rounds + 1/segs + the fp32 partials and the fixup pass,
//    ~5 us + 0.13 us per 256 KiB partial (written once, read once), against
//    a round of ~97 us per 4096 of K (measured on the block's shapes).
//    Needs the partial buffer (segs * tail * 256 KiB).
GemmChoice gemm_choose(int M, int N, int K, bool swiglu) {
  GemmChoice ch{0, 0, 1, 0};
  const int ncols = swiglu ? 128 : 256;  // output columns per tile
  const long nt = (N + ncols - 1) / ncols;
  const long t256 = (long)((M + 255) / 256) * nt, t192 = (long)((M + 191) / 192) * nt;
  const double r256 = std::ceil(t256 / 256.0), r192 = std::ceil(t192 / 256.0) * 0.85;
  double best = r256;
  if (r192 < best) { best = r192; ch.variant = 1; }
  const long full = t256 / 256, tail = t256 % 256;
  const int nk = (K + 63) / 64;
  if (full >= 1 && tail > 0) {
    const int smax = (int)std::min<long>(std::min<long>(8, 256 / tail), nk / 2);
    const double round_us = 97.0 * K / 4096.0;
    for (int segs = 2; segs <= smax; ++segs) {
      const double rsk = full + 1.0 / segs + (5.0 + 0.131 * tail * segs) / round_us;
      if (rsk < best) {
        best = rsk;
        ch = GemmChoice{0, (int)tail, segs, (size_t)tail * segs * 256 * 256 * sizeof(float)};
      }
    }
  }
  return ch;
}

// Tile configurations: variant < 0 picks the default plan; 0 / 1 force whole
// 256 x 256 / 192 x 256 tiles.
template <int EPI>
static hipError_t gemm_dispatch(bool f32, int variant, int gm, const void *a, const void *w,
                                void *c, int M, int N, int K, hipStream_t s, float *part,
                                size_t part_bytes, ColScale cs = {}) {
  // L2 grouping width: 2 row tiles for the SwiGLU tile (it reads W1 and W3
  // rows), else 8.  W13 at 1024 px, B = 2, same box: 2 -> 1192, 4 -> 1216,
  // 8 -> 1200, 16 -> 1250 us; 2 against 4 also 1.7 % faster at 512 px,
  // 0.7 % at 256 px and within 1 % at B = 1.  (The bf16 tile only: the FP8
  // SwiGLU tile measured the same with 2 and 4.)
  if (gm <= 0) gm = (EPI == EPI_SWIGLU) ? 2 : 8;
  if (f32) return launch_gemm_t<float, 256, 256, 128, 2, 2, 4, EPI>(a, w, c, M, N, K, s, gm, 0, 1, nullptr, cs);
  if (variant < 0) {
    const GemmChoice ch = gemm_choose(M, N, K, EPI == EPI_SWIGLU);
    if (ch.sk_tiles > 0 && part && part_bytes >= ch.part_bytes)
      return launch_gemm_t<bf16, 256, 256, 128, 2, 2, 4, EPI, true>(a, w, c, M, N, K, s, gm, ch.sk_tiles,
                                                                    ch.segs, part, cs);
    // without the partial buffer: whole tiles, the fuller of 192 / 256 rows
    const int ncols = (EPI == EPI_SWIGLU) ? 128 : 256;
    auto fill = [&](int bm) {
      const double tiles = (double)((M + bm - 1) / bm) * ((N + ncols - 1) / ncols);
      return tiles / (std::ceil(tiles / 256.0) * 256.0);
    };
    variant = ch.sk_tiles > 0 ? ((fill(192) > fill(256) + 0.02) ? 1 : 0) : ch.variant;
    if (variant == 0) return launch_gemm_t<bf16, 256, 256, 128, 2, 2, 4, EPI, true>(a, w, c, M, N, K, s, gm, 0, 1,
                                                                                   nullptr, cs);
    return launch_gemm_t<bf16, 192, 256, 128, 2, 2, 4, EPI, true>(a, w, c, M, N, K, s, gm, 0, 1, nullptr, cs);
  }
  switch (variant) {  // the two whole-tile plans, for tests and tuning
    case 0: return launch_gemm_t<bf16, 256, 256, 128, 2, 2, 4, EPI, true>(a, w, c, M, N, K, s, gm, 0, 1, nullptr, cs);
    case 1: return launch_gemm_t<bf16, 192, 256, 128, 2, 2, 4, EPI, true>(a, w, c, M, N, K, s, gm, 0, 1, nullptr, cs);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(bool f32, const void *a, const void *w, void *c, int M, int N, int K,
                       hipStream_t s, int variant, int group_m, float *part, size_t part_bytes, int scale_cols,
                       float col_scale, const GemmVt *vt) {
  ColScale cs{scale_cols, col_scale};
  if ((vt && f32) || !set_vt(cs, vt, M, N)) return hipErrorInvalidValue;
  return gemm_dispatch<EPI_STORE>(f32, variant, group_m, a, w, c, M, N, K, s, part, part_bytes, cs);
}

hipError_t launch_gemm_swiglu(bool f32, const void *a, const void *w13, void *u, int M, int F,
                              int K, hipStream_t s, int variant, int group_m, float *part,
                              size_t part_bytes) {
  return gemm_dispatch<EPI_SWIGLU>(f32, variant, group_m, a, w13, u, M, F, K, s, part, part_bytes);
}

hipError_t launch_gemm_split(bool swiglu, const void *a, const void *w, void *c, int M, int N, int K,
                             int sk_tiles, int segs, float *part, hipStream_t s) {
  if (swiglu)
    return launch_gemm_t<bf16, 256, 256, 128, 2, 2, 4, EPI_SWIGLU, true>(a, w, c, M, N, K, s, 4, sk_tiles,
                                                                         segs, part);
  return launch_gemm_t<bf16, 256, 256, 128, 2, 2, 4, EPI_STORE, true>(a, w, c, M, N, K, s, 8, sk_tiles, segs,
                                                                      part);
}

}  // namespace dit
