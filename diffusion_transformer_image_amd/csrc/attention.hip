// Flash-style grouped-query attention with a sigmoid output gate for the
// single-stream DiT block (page "Krea 2 技术报告", 架构 › Transformer块:
// GQA, the report's reference 45, with the gated attention of its
// reference 47; one joint text+image sequence, no mask, no positions).
//
//   og[q, h*d:(h+1)*d] = softmax_k(Q_h[q] . K_j[k] / sqrt(d)) V_j * sigmoid(G_h[q])
//   with j = h / (H / Hkv).
//
// Design for gfx950:
//  * a small pass first writes V^T ([B][Hkv][d][Lp], keys contiguous, Lp =
//    L rounded up to the key tile, zero padded), so both operand tiles of
//    the main loop go HBM -> LDS by DMA (buffer_load ... lds) with no VALU
//    work, through a ring of tiles (each wave waits only for its own DMA
//    of tile t, then one barrier);
//  * one workgroup = (sample b, KV head j, WPH*QW query tokens) for ALL
//    query heads of the group: the K / V^T tiles of head j are brought to
//    LDS once and read by group * WPH waves (each wave: one query head, QW
//    queries).  bf16 with 4 query heads per KV head: one wave per head,
//    QW = 48, a 2-deep ring, two 4-wave workgroups per CU that run out of
//    phase; otherwise two waves per head (QW = 48 in bf16, 32 in fp32)
//    and a 3-deep ring;
//  * scores are computed transposed, S^T = K Q^T (MFMA 16x16), so each
//    lane owns one query column: the softmax statistics of a query live in
//    4 lanes (one per lane group) and the probabilities P^T are already in
//    the register layout of the B operand of O^T = V^T P^T;
//  * softmax in fp32 base 2 with the 1/sqrt(d) scale folded into one FMA
//    (or, for queries that carry the factor already, into the queries: then
//    each score chain starts from -reference and a numerator is one exp2),
//    against a lazy reference: the numerators of a tile are computed with
//    the current reference and packed to bf16 (the B operand of P V), and
//    the row sums are taken from the packed values with v_dot2 (two keys
//    per instruction).  Only if a lane's partial sum leaves [0, 2^30] (a
//    score > 30 log2 units above the reference, or no reference yet) does
//    the wave recompute the tile's scores, take their maximum, rescale the
//    accumulators and redo the numerators; the quotient O / l does not
//    depend on the reference.  No per-tile maximum, no shuffles;
//  * LDS data is XOR-swizzled (K by 16-byte chunk at DMA time, V^T when
//    the V^T pass writes it, which also groups each lane's keys of one
//    MFMA into one chunk) so every fragment is one ds_read_b128 and 16
//    rows hit distinct banks (checked with SQ_LDS_BANK_CONFLICT); both
//    products read their fragments a rolling window ahead of the MFMAs
//    that consume them;
//  * epilogue: divide by the row sum, multiply by sigmoid(G), store.
#include <cmath>

#include "dit_common.h"
#include "dit_kernels.h"

namespace dit {

constexpr int ATT_BK = 64;   // keys per tile

__host__ __device__ constexpr int att_lpad(int L) { return (L + ATT_BK - 1) / ATT_BK * ATT_BK; }

// ---------------------------------------------------------------- V^T pass
// vt[b][j][dd][l] = qkvg[b*L + l][(H + Hkv + j)*HD + dd], zero for l >= L,
// with the keys of each 64-key tile of a row dd rearranged so that every
// 16-byte chunk holds exactly the keys one lane feeds one MFMA, and the
// chunks XOR-swizzled by dd:
//   bf16: logical chunk c = pr*4 + g holds keys (2pr)*16 + 4g + {0..3} and
//         (2pr+1)*16 + 4g + {0..3}; it is stored at chunk c ^ (dd & 7);
//   fp32: logical chunk c holds keys 4c + {0..3}; stored at c ^ (dd & 15).
// A straight 16-byte DMA copy of a tile row then gives the LDS layout the
// fragment reads want: one conflict-free ds_read_b128 per fragment.
template <typename T>
__device__ __forceinline__ int vt_chunk_key(int c, int e) {  // e < 16 / sizeof(T)
  if constexpr (sizeof(T) == 2) return (2 * (c >> 2) + (e >> 2)) * 16 + 4 * (c & 3) + (e & 3);
  else return 4 * c + e;
}
template <typename T>
__device__ __forceinline__ int vt_swizzle(int dd) { return sizeof(T) == 2 ? (dd & 7) : (dd & 15); }

template <typename T, int HD>
__global__ __launch_bounds__(256) void vtrans_kernel(const T *__restrict__ qkvg, T *__restrict__ vt,
                                                     int L, int H, int Hkv) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  __shared__ __attribute__((aligned(16))) T tile[ATT_BK][HD + EPC];
  const int l0 = blockIdx.x * ATT_BK, j = blockIdx.y, b = blockIdx.z;
  const int Lp = att_lpad(L);
  const size_t ldq = (size_t)(2 * H + 2 * Hkv) * HD;
  const T *src = qkvg + (size_t)b * L * ldq + (size_t)(H + Hkv + j) * HD;
  // all of this thread's row chunks are requested before any is stored;
  // each lands in the padded tile as one 16-byte write (the row pitch,
  // (HD + EPC) elements, is a multiple of 16 bytes)
  constexpr int NLD = ATT_BK * (HD / EPC) / 256;
  static_assert(NLD * 256 == ATT_BK * (HD / EPC), "whole chunks per thread");
  u32x4 v[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    const int idx = threadIdx.x + 256 * k;
    const int r = idx / (HD / EPC), c = (idx % (HD / EPC)) * EPC;
    v[k] = u32x4{0u, 0u, 0u, 0u};
    if (l0 + r < L) v[k] = *reinterpret_cast<const u32x4 *>(src + (size_t)(l0 + r) * ldq + c);
  }
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    const int idx = threadIdx.x + 256 * k;
    const int r = idx / (HD / EPC), c = (idx % (HD / EPC)) * EPC;
    *reinterpret_cast<u32x4 *>(&tile[r][c]) = v[k];
  }
  __syncthreads();
  T *dst = vt + ((size_t)b * Hkv + j) * HD * Lp + l0;
  static_assert(HD * (ATT_BK / EPC) % 256 == 0, "whole output chunks per thread");
#pragma unroll
  for (int idx = threadIdx.x; idx < HD * (ATT_BK / EPC); idx += 256) {
    // consecutive lanes store consecutive chunks of one V^T row (whole
    // 128-byte row pieces per 8 lanes for bf16)
    const int dd = idx / (ATT_BK / EPC), pc = idx % (ATT_BK / EPC);  // physical 16-byte chunk of the row
    const int lc = pc ^ vt_swizzle<T>(dd);   // logical chunk stored there
    T w[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) w[e] = tile[vt_chunk_key<T>(lc, e)][dd];
    u32x4 v;
    __builtin_memcpy(&v, w, 16);
    *reinterpret_cast<u32x4 *>(dst + (size_t)dd * Lp + pc * EPC) = v;
  }
}

// ---------------------------------------------------------------- main kernel
template <int N>
__device__ __forceinline__ void att_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// NW = waves per workgroup, WPH per query head of the group (NW = group *
// WPH); QW = query tokens per wave (32 or 48), so a workgroup covers
// WPH * QW query tokens.  WPH = 2: one workgroup per CU with a 3-deep
// K / V^T ring; WPH = 1 (bf16, 4 query heads per key head): 4-wave
// workgroups with a 2-deep ring, two per CU (64 KiB of LDS each), which
// drift out of phase so one's softmax runs beside the other's MFMAs
// (1024 px: 626-628 -> 601-605 us, same box, for twice the K / V reads).
// PRE: the query heads in qkvg already carry the factor sc = log2(e)/sqrt(d)
// (applied before their one rounding, by the projection's epilogue or the
// prologue pass), so scores come out of the MFMAs in base-2 units; each
// score chain then starts from -reference (the first MFMA reads it as its
// accumulator input) and a numerator is one exp2, with no per-score FMA.
template <typename T, int HD, int NW, int QW, bool PRE, int WPH>
__global__ __launch_bounds__(NW * 64, WPH == 1 ? 2 : 1) void attn_kernel(const T *__restrict__ qkvg, const T *__restrict__ vt,
                                                       T *__restrict__ og, int L, int H, int Hkv, float sc) {
  static_assert(!PRE || sizeof(T) == 2, "pre-scaled queries: bf16 only");
  constexpr int ES = sizeof(T);
  constexpr int KROW = HD * ES;         // bytes of one K row in LDS
  constexpr int NCK = KROW / 16;        // 16-byte chunks per K row (16 or 32)
  constexpr int KS = KROW / 64;         // MFMA k-steps over d (4 chunks each)
  constexpr int KTILE = ATT_BK * KROW;  // bytes of a K tile
  constexpr int VROW = ATT_BK * ES;     // bytes of one V^T row (64 keys)
  constexpr int VCH = VROW / 16;        // chunks per V^T row (8 or 16)
  constexpr int VTILE = HD * VROW;
  constexpr int STAGE = KTILE + VTILE;
  constexpr int DB = HD / 16;           // 16-row blocks of d
  constexpr int QB = QW / 16;           // 16-column blocks of queries per wave
  constexpr int KB = ATT_BK / 16;       // 16-key blocks per tile
  constexpr int NSTAGE = (WPH == 2 && 3 * STAGE <= 160 * 1024) ? 3 : 2;  // K / V^T ring depth
  constexpr int PD = NSTAGE - 1;        // tiles in flight ahead of the one in use
  constexpr int KBLK = KTILE / 1024, VBLK = VTILE / 1024;
  constexpr int DMA_PER_TILE = (KBLK + NW - 1) / NW + (VBLK + NW - 1) / NW;  // per wave
  static_assert(NCK >= 16, "K rows need >= 16 chunks for the swizzle");
  static_assert(KBLK % NW == 0 && VBLK % NW == 0, "tile blocks split evenly over the waves");
  static_assert(NSTAGE * STAGE <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int group = H / Hkv;
  const int b = blockIdx.z, j = blockIdx.y;
  const int h = j * group + wave / WPH;
  const int q0 = blockIdx.x * (WPH * QW) + (wave % WPH) * QW;
  const int g = lane >> 4, r16 = lane & 15;
  const int Lp = att_lpad(L);

  const int ldq = (2 * H + 2 * Hkv) * HD;  // elements per token row of qkvg
  const uint32_t ldqb = (uint32_t)ldq * ES;
  const T *base = qkvg + (size_t)b * L * ldq;
  const rsrc_t rq = make_rsrc(base, (uint32_t)L * ldqb);
  const rsrc_t rv = make_rsrc(vt + ((size_t)b * Hkv + j) * HD * Lp, (uint32_t)HD * Lp * ES);
  const uint32_t kcol = (uint32_t)(H + j) * HD * ES;

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

  // ---- tile loaders (DMA; each wave writes whole 1 KiB blocks, blocks
  // wave, wave + NW, ...: a trip count known at compile time, so the loads
  // are straight-line code)
  auto issue_tile = [&](int t, int buf) {
    char *kt = smem + buf * STAGE;
    constexpr int KRPB = 1024 / KROW;
#pragma unroll
    for (int i = 0; i < KBLK / NW; ++i) {
      const int blk = wave + i * NW;
      const int row = blk * KRPB + lane / NCK;
      const int lc = (lane % NCK) ^ (row & 15);
      const int key = t * ATT_BK + row;
      const uint32_t off = key < L ? (uint32_t)key * ldqb + kcol + lc * 16 : kOOB;
      load_lds16(rq, kt + blk * 1024, off);
    }
    char *vtl = kt + KTILE;
    constexpr int VRPB = 1024 / VROW;
#pragma unroll
    for (int i = 0; i < VBLK / NW; ++i) {
      const int blk = wave + i * NW;
      // rows of V^T are stored pre-swizzled: copy them verbatim
      const int d = blk * VRPB + lane / VCH;
      const uint32_t off = (uint32_t)d * Lp * ES + (uint32_t)t * VROW + (lane % VCH) * 16;
      load_lds16(rv, vtl + blk * 1024, off);
    }
  };

  f32x4 o[DB][QB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int k = 0; k < QB; ++k) o[i][k] = f32x4{0.f, 0.f, 0.f, 0.f};
  // mref: the running reference per query column (raw score units, or
  // base-2 units when PRE); PRE keeps it finite (0 until the first tile,
  // which always takes the recompute path) and negm = -mref in the layout
  // of a score accumulator
  float mref[QB], lrow[QB];
  f32x4 negm[QB];
#pragma unroll
  for (int k = 0; k < QB; ++k) {
    mref[k] = PRE ? 0.f : -INFINITY;
    lrow[k] = 0.f;
    negm[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nt = (L + ATT_BK - 1) / ATT_BK;
#pragma unroll
  for (int p = 0; p < PD; ++p)
    if (p < nt) issue_tile(p, p);

  // lane-dependent parts of the fragment addresses inside a stage buffer
  // (the 16-row block and the buffer base are added as immediates / one
  // uniform offset per tile)
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = r16 * KROW + (((ks * 4 + g) ^ r16) * 16);
  const int vrow = KTILE + r16 * VROW;

  // S^T[kb][qb] = K Q^T for the tile in buffer kt: lane holds keys
  // kb*16 + 4g + i of query qb*16 + r16; keys past the end of the sequence
  // get -inf.  PRE: S^T - mref.  The 16-byte K fragments f = kb*KS + ks are
  // read KPF ahead of their MFMAs (a rolling window: each read goes out as
  // soon as the MFMAs of the fragment KPF places earlier are issued, so the
  // LDS latency runs beside the matrix work instead of after it).
  constexpr int KPF = 8;
  auto scores = [&](const char *kt, int t, f32x4(&s)[KB][QB]) {
    constexpr int NF = KB * KS;
    u32x4 kf[NF];
#pragma unroll
    for (int f = 0; f < KPF; ++f)
      kf[f] = *reinterpret_cast<const u32x4 *>(kt + koff[f % KS] + (f / KS) * 16 * KROW);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int kb = f / KS, ks = f % KS;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        s[kb][qb] = mma16<T>(kf[f], qf[qb][ks], ks ? s[kb][qb] : (PRE ? negm[qb] : f32x4{0.f, 0.f, 0.f, 0.f}));
      if (f + KPF < NF)
        kf[f + KPF] = *reinterpret_cast<const u32x4 *>(kt + koff[(f + KPF) % KS] + ((f + KPF) / KS) * 16 * KROW);
    }
#pragma unroll
    for (int f = 0; f < KPF; ++f) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      if (f + KPF < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if ((t + 1) * ATT_BK > L) {
      // a real branch (the empty volatile asm cannot be speculated): without
      // it the compiler turns the mask into selects on every tile
      asm volatile("" ::: "memory");
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t * ATT_BK + kb * 16 + 4 * g + i >= L)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb][i] = -INFINITY;
    }
  };

  // Numerators p = 2^(s*sc - mref*sc) against the running reference (PRE:
  // p = 2^s, the reference already subtracted), as the B operand of
  // O^T += V^T P^T (bf16: one 16-byte fragment per pair of 16-key blocks;
  // fp32: the values themselves), and this lane's partial row sums, taken
  // from the values the MFMA will use.
  constexpr int NPF = (ES == 2) ? KB / 2 : KB;
  auto numerators = [&](f32x4(&s)[KB][QB], u32x4(&pf)[NPF][QB], float (&lp)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float msc = mref[qb] * sc;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[kb][qb][i] = __builtin_amdgcn_exp2f(PRE ? s[kb][qb][i] : fmaf(s[kb][qb][i], sc, -msc));
      float sum = 0.f;
      if constexpr (ES == 2) {
#pragma unroll
        for (int pr = 0; pr < KB / 2; ++pr) {
          bf16x8 pv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pv[i] = (bf16)s[2 * pr][qb][i];
            pv[4 + i] = (bf16)s[2 * pr + 1][qb][i];
          }
          pf[pr][qb] = __builtin_bit_cast(u32x4, pv);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bf16x2 two = {pv[2 * i], pv[2 * i + 1]};
            sum = __builtin_amdgcn_fdot2_f32_bf16(two, bf16x2{(bf16)1.0f, (bf16)1.0f}, sum, false);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          pf[kb][qb] = __builtin_bit_cast(u32x4, s[kb][qb]);
#pragma unroll
          for (int i = 0; i < 4; ++i) sum += s[kb][qb][i];
        }
      }
      lp[qb] = sum;
    }
  };

  // V^T fragments of the P V product: the one of row d = db*16 + r16 for
  // k-slice c is one 16-byte chunk at c ^ swizzle(d).  bf16: one MFMA
  // (k = 32) per pair of 16-key blocks, the lane's 8 keys (2pr)*16 + 4g +
  // {0..3} and (2pr+1)*16 + 4g + {0..3} (chunk pr*4 + g); fp32: four MFMAs
  // (k = 4 each) per 16-key block, chunk kb*4 + g.
  constexpr int NVF = NPF * DB;
  // rolling depth VPF; VPF0 of those are requested before the numerators
  constexpr int VPF = 6, VPF0 = 2;
  auto read_vf = [&](const char *kt, int f) {
    const int ksl = f / DB, db = f % DB;
    const int cpos = ES == 2 ? ((ksl * 4 + g) ^ (r16 & 7)) * 16 : ((ksl * 4 + g) ^ r16) * 16;
    return *reinterpret_cast<const u32x4 *>(kt + vrow + db * 16 * VROW + cpos);
  };

  for (int t = 0; t < nt; ++t) {
    // this wave's DMA of tile t is done once only the (up to PD-1) later
    // tiles already issued may be pending
    if (t + PD - 1 < nt) att_wait_vmcnt<DMA_PER_TILE * (PD - 1)>();
    else att_wait_vmcnt<0>();
    __syncthreads();  // all of tile t landed; every wave is done with tile t-1
    if (t + PD < nt) issue_tile(t + PD, (t + PD) % NSTAGE);
    const char *kt = smem + (t % NSTAGE) * STAGE;

    f32x4 s[KB][QB];
    scores(kt, t, s);
    // the first VPF0 V^T fragments of the tile are requested before the
    // numerators (their LDS latency runs beside the exponentials; more than
    // two do not fit in the registers left); the rare recompute path reads
    // them again, so they are not held across it
    u32x4 vf[NVF];
#pragma unroll
    for (int f = 0; f < VPF0; ++f) vf[f] = read_vf(kt, f);
    u32x4 pf[NPF][QB];
    float lp[QB];
    // Lazy reference: a lane's partial row sum above 2^30 (or not finite)
    // means a score more than 30 (log2 units) above the reference, or no
    // reference yet (first tile; PRE: always taken there).  Then the wave
    // recomputes the tile's scores, raises the reference to the running
    // maximum, rescales the accumulators and redoes the numerators; O / l
    // does not depend on the reference, which only keeps the numerators in
    // range.
    bool big = PRE && t == 0;
    if (!big) {
      numerators(s, pf, lp);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) big |= !(lp[qb] <= 0x1p30f);
    }
    if (__any(big)) {
      scores(kt, t, s);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if constexpr (PRE) {
          // s = score - mref: the new reference is mref + max(mx, 0) (the
          // first tile: mref + mx); delta <= 0 except on the first tile,
          // where o and l are still zero
          const float mnew = mref[qb] + (t == 0 ? mx : fmaxf(mx, 0.f));
          const float delta = mref[qb] - mnew;
          const float alpha = __builtin_amdgcn_exp2f(fminf(delta, 0.f));
          mref[qb] = mnew;
          negm[qb] = f32x4{-mnew, -mnew, -mnew, -mnew};
          lrow[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db][qb] *= alpha;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) s[kb][qb] += delta;
        } else {
          const float mnew = fmaxf(mref[qb], mx);
          const float alpha = __builtin_amdgcn_exp2f((mref[qb] - mnew) * sc);  // 0 when mref = -inf
          mref[qb] = mnew;
          lrow[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db][qb] *= alpha;
        }
      }
      numerators(s, pf, lp);
#pragma unroll
      for (int f = 0; f < VPF0; ++f) vf[f] = read_vf(kt, f);
    }
#pragma unroll
    for (int f = VPF0; f < VPF; ++f) vf[f] = read_vf(kt, f);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lrow[qb] += lp[qb];

    // O^T[db][qb] += V^T[db rows] * P^T, fragment f = kslice * DB + db;
    // the reads roll VPF ahead of the MFMAs
#pragma unroll
    for (int f = 0; f < NVF; ++f) {
      const int ksl = f / DB, db = f % DB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) o[db][qb] = mma16<T>(vf[f], pf[ksl][qb], o[db][qb]);
      if (f + VPF < NVF) vf[f + VPF] = read_vf(kt, f + VPF);
    }
#pragma unroll
    for (int f = 0; f < NVF; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      if (f + VPF < NVF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
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
        const int d = db * 16 + 4 * g;  // 4 consecutive channels per lane
        if constexpr (ES == 2) {
          const bf16x4 gv = *reinterpret_cast<const bf16x4 *>(grow + d);
          bf16x4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ov[i] = (bf16)(o[db][qb][i] * inv * __builtin_amdgcn_rcpf(1.0f + __expf(-(float)gv[i])));
          *reinterpret_cast<bf16x4 *>(orow + d) = ov;
        } else {
          const f32x4 gv = *reinterpret_cast<const f32x4 *>(grow + d);
          f32x4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = o[db][qb][i] * inv / (1.0f + __expf(-gv[i]));
          *reinterpret_cast<f32x4 *>(orow + d) = ov;
        }
      }
    }
  }
}

size_t attention_vt_bytes(bool f32, int B, int L, int Hkv, int head_dim) {
  return (size_t)B * Hkv * head_dim * att_lpad(L) * (f32 ? 4 : 2);
}

template <typename T, int HD, int QW, bool PRE>
static void launch_attn_q(const T *q, const T *v, T *og, int B, int L, int H, int Hkv, float sc,
                          hipStream_t s) {
  const int group = H / Hkv;
#define DIT_ATT(NWV, WPHV)                                                                             \
  hipLaunchKernelGGL((attn_kernel<T, HD, NWV, QW, PRE, WPHV>), dim3((L + WPHV * QW - 1) / (WPHV * QW), Hkv, B), \
                     dim3(NWV * 64), 0, s, q, v, og, L, H, Hkv, sc)
  switch (group) {
    case 1: DIT_ATT(2, 2); break;
    case 2: DIT_ATT(4, 2); break;
    case 4:
      if constexpr (sizeof(T) == 2) DIT_ATT(4, 1);  // one wave per head, two workgroups per CU
      else DIT_ATT(8, 2);
      break;
  }
#undef DIT_ATT
}

template <typename T, int HD, bool PRE>
static hipError_t launch_attn_t(const void *qkvg, void *vt, void *og, int B, int L, int H, int Hkv,
                                hipStream_t s, bool vt_ready) {
  const int group = H / Hkv;
  if (group != 1 && group != 2 && group != 4) return hipErrorInvalidValue;
  if (!vt_ready) {
    hipLaunchKernelGGL((vtrans_kernel<T, HD>), dim3(att_lpad(L) / ATT_BK, Hkv, B), dim3(256), 0, s,
                       (const T *)qkvg, (T *)vt, L, H, Hkv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // softmax in base 2 with the score scale in one FMA (PRE: in the queries)
  const float sc = attn_score_scale(HD);
  const auto *q = (const T *)qkvg;
  const auto *v = (const T *)vt;
  // bf16: 48 queries per wave (more MFMAs per K / V fragment read); with two
  // workgroups per CU the finer launch balances itself, and 48 measured
  // faster than 32 at every size here (256 px 243 -> 229 us, 512 px 298 ->
  // 283 us, 1024 px equal, the 60-block stack at B = 1 110 -> 108 ms)
  if constexpr (sizeof(T) == 2)
    launch_attn_q<T, HD, 48, PRE>(q, v, (T *)og, B, L, H, Hkv, sc, s);
  else
    launch_attn_q<T, HD, 32, PRE>(q, v, (T *)og, B, L, H, Hkv, sc, s);
  return hipGetLastError();
}

hipError_t launch_attention(bool f32, int head_dim, const void *qkvg, void *vt, void *og, int B,
                            int L, int H, int Hkv, hipStream_t s, bool q_prescaled, bool vt_ready) {
  if (vt_ready && (f32 || L % ATT_BK)) return hipErrorInvalidValue;  // V^T by the projection: whole key tiles
  if (f32) {
    if (q_prescaled) return hipErrorInvalidValue;
    if (head_dim == 64) return launch_attn_t<float, 64, false>(qkvg, vt, og, B, L, H, Hkv, s, false);
    if (head_dim == 128) return launch_attn_t<float, 128, false>(qkvg, vt, og, B, L, H, Hkv, s, false);
  } else if (head_dim == 128) {
    if (q_prescaled) return launch_attn_t<bf16, 128, true>(qkvg, vt, og, B, L, H, Hkv, s, vt_ready);
    return launch_attn_t<bf16, 128, false>(qkvg, vt, og, B, L, H, Hkv, s, vt_ready);
  }
  return hipErrorInvalidValue;
}

}  // namespace dit
