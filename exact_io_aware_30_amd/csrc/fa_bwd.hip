// Backward kernels: the delta pre-pass, then dK/dV with key blocks in the
// outer loop, then dQ with query blocks in the outer loop ("flash-attn-triton"
// docs, "Where things live" and "Scope": backward kernels rebuild P from the
// saved L instead of reading it back; "flash attention" note, "Key
// Mechanisms": backward recomputation).  The gradient formulas are those of
// the softmax-attention definition:
//   P = 2^(S c - L log2 e)  (S = Q K^T, c = scale log2 e, masked entries 0)
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = scale dS K,
//   dK = scale dS^T Q,  with D_i = sum_k dO_ik O_ik from the pre-pass.
// No atomics: every output element is written by exactly one lane.
#include "fa_device.h"
#include "fa_launch.h"

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

// Device memory of the backward entry point that allocates nothing: the
// head-split float32 partial sums live here instead of in a caller
// workspace.  Every device the library runs on holds its own copy from the
// time the code object is loaded until the process ends; every call on a
// device shares it (see fa::scratch_region).
static __device__ __align__(256) unsigned char scratch[fa::kScratchBytes];

// Tile configuration (compile-time; defaults chosen by measurement).
#ifndef FA_BWD_STAGES
#define FA_BWD_STAGES 2
#endif
namespace fa {

// ---------------------------------------------------------------------------
// D_i = sum_k dO_ik O_ik.  D/8 lanes per row, 16 bytes per lane, fp32 sum.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(256) void preprocess_kernel(const void* __restrict__ op, const void* __restrict__ dop,
                                                         float* __restrict__ delta, long rows) {
  constexpr int CPR = D / 8, RPB = 256 / CPR;
  const int tid = threadIdx.x;
  const int ch = tid % CPR;
  for (long row0 = (long)blockIdx.x * RPB; row0 < rows; row0 += (long)gridDim.x * RPB) {
    const long row = row0 + tid / CPR;
    float s = 0.f;
    if (row < rows) {
      const u32x4 a = *((const u32x4*)op + row * CPR + ch);
      const u32x4 b = *((const u32x4*)dop + row * CPR + ch);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s = __builtin_fmaf(Elem<T>::lo(a[i]), Elem<T>::lo(b[i]), s);
        s = __builtin_fmaf(Elem<T>::hi(a[i]), Elem<T>::hi(b[i]), s);
      }
    }
#pragma unroll
    for (int m = CPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (ch == 0 && row < rows) delta[row] = s;
  }
}

constexpr int kBwdWaves = 4, kBwdStages = FA_BWD_STAGES;
// dQ: MFMAs' worth of LDS operand reads kept in flight in the S/dP and dQ
// runs of the tile without the interleave.
#ifndef FA_DQ_PRE1
#define FA_DQ_PRE1 6
#endif
#ifndef FA_DQ_PRE2
#define FA_DQ_PRE2 3
#endif
// dQ key tile rows and ring depth.
#ifdef FA_DQ_TILE
template <int D>
constexpr int kDqTile = FA_DQ_TILE;
#else
template <int D>
constexpr int kDqTile = D == 128 ? 32 : 64;
#endif
#ifdef FA_DQ_STAGES
template <int D>
constexpr int kDqStages = FA_DQ_STAGES;
#else
template <int D>
constexpr int kDqStages = kBwdStages;
#endif
// dK/dV kernel configuration per head dimension (chosen by measurement):
// query tile rows (32 or 64), workgroups per CU the registers are limited
// for, ring depth, MFMAs' worth of LDS operand reads kept in flight in the
// S/dP and dV/dK phases, and whether V's operand is read from LDS instead of
// being held in registers.  FA_DKDV_* macros override every head dimension.
template <int D>
struct DkdvCfg {
  static constexpr int kTile = D == 32 ? 64 : 32;
  // Minimum workgroups per CU for the register allocator (d = 128: 1 lets
  // it schedule more freely; the kernel still fits two per CU).
  static constexpr int kOcc = D == 128 ? 1 : D == 64 ? 3 : 1;
  static constexpr bool kVLds = D == 128;
  static constexpr int kStages = 2, kPre1 = D == 32 ? 6 : 4, kPre2 = 3;
};
#ifdef FA_DKDV_TILE
#define FA_DKDV_CFG_TILE FA_DKDV_TILE
#else
#define FA_DKDV_CFG_TILE DkdvCfg<D>::kTile
#endif
#ifdef FA_DKDV_OCC
#define FA_DKDV_CFG_OCC FA_DKDV_OCC
#else
#define FA_DKDV_CFG_OCC DkdvCfg<D>::kOcc
#endif
#ifdef FA_DKDV_VLDS
#define FA_DKDV_CFG_VLDS (FA_DKDV_VLDS != 0)
#else
#define FA_DKDV_CFG_VLDS DkdvCfg<D>::kVLds
#endif
#ifdef FA_DKDV_STAGES
#define FA_DKDV_CFG_STAGES FA_DKDV_STAGES
#else
#define FA_DKDV_CFG_STAGES DkdvCfg<D>::kStages
#endif
#ifdef FA_DKDV_PRE1
#define FA_DKDV_CFG_PRE1 FA_DKDV_PRE1
#else
#define FA_DKDV_CFG_PRE1 DkdvCfg<D>::kPre1
#endif
#ifdef FA_DKDV_PRE2
#define FA_DKDV_CFG_PRE2 FA_DKDV_PRE2
#else
#define FA_DKDV_CFG_PRE2 DkdvCfg<D>::kPre2
#endif
template <int D>
struct Dkdv {
  static constexpr int kTile = FA_DKDV_CFG_TILE, kOcc = FA_DKDV_CFG_OCC, kStages = FA_DKDV_CFG_STAGES;
  static constexpr int kPre1 = FA_DKDV_CFG_PRE1, kPre2 = FA_DKDV_CFG_PRE2;
  static constexpr bool kVLds = FA_DKDV_CFG_VLDS;
  static_assert(kTile == 32 || kTile == 64, "dK/dV query tile");
};
// A tile's dV MFMAs issued before its dK MFMAs with dS formed between them
// (1), or dS formed in the vector phase and the two kinds alternating (0).
// Bit-identical either way; 1 is 3% faster at d = 32 (fp16 [3,12,2000,32]
// full), and at d = 128 causal 5% slower, so it is the default at d = 32
// only.  Not used for general windows, whose mask tests leave no registers
// for it.  FA_DKDV_DV_FIRST=0/1 forces one form for every head dimension.
#ifdef FA_DKDV_DV_FIRST
template <int D>
constexpr bool kDvFirst = FA_DKDV_DV_FIRST != 0;
#else
template <int D>
constexpr bool kDvFirst = D == 32;
#endif
// L and D of a query tile: one dword per lane of a wave, so 64 rows of each
// are copied (rows past the tile are not read).
constexpr int kStatsRows = 64;

// The wave's V rows as the B operand of dP^T (k = head dimension, n = key).
struct VRegs {
  static constexpr int kReads = 0;
  const u32x4* f;
  __device__ __forceinline__ u32x4 operator()(int kk, int) const { return f[kk]; }
};
template <int D>
struct VLds {
  static constexpr int kReads = 1;
  const lds_char* tile;  // the workgroup's key rows of V, swizzled like the Q tile
  int row0;              // the wave's first row in it
  __device__ __forceinline__ u32x4 operator()(int kk, int lane) const {
    return lds_rows_operand<D>(tile, row0, kk, lane);
  }
};

// The three phases of one query tile of the dK/dV kernels for one wave.
// Phase 1 (MFMA): S^T and dP^T of the tile (lane = key, registers = query).
// The V operand is negated (the workgroup's V rows are stored with their
// signs flipped) and the dP^T accumulator starts from the tile's D values,
// so the MFMAs leave D - dP, and dS = P (dP - D) is -(P (D - dP)): the sign
// is carried into the final dK scale.  st + kStatsRows holds the tile's D.
template <class T, int D, int NA, class VOp>
__device__ __forceinline__ void dkdv_scores(const lds_char* qt, const lds_char* dot, const u32x4* kf, const VOp& vop,
                                            const float* st, f32x16* s, f32x16* dp, int lane) {
  constexpr int NKK = D / 16;
  const int h = lane >> 5;
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    s[a] = (f32x16){};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 dd = *(const f32x4*)(st + kStatsRows + 32 * a + 8 * g + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[a][4 * g + e] = dd[e];
    }
  }
  prio_mfma_begin();
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      s[a] = Elem<T>::mma(lds_rows_operand<D>(qt, 32 * a, kk, lane), kf[kk], s[a]);
      dp[a] = Elem<T>::mma(lds_rows_operand<D>(dot, 32 * a, kk, lane), vop(kk, lane), dp[a]);
    }
  {
    constexpr int NM = 2 * NA * NKK, TR = NM + NA * NKK * VOp::kReads;
    sched_mfma_reads<NM, TR, (TR < Dkdv<D>::kPre1 ? TR : Dkdv<D>::kPre1)>();
  }
  prio_mfma_end();
}

// Scores of queries outside the lane's key window to -inf: query i sees key
// krow iff krow - right <= i <= krow + left, compared as offsets
// 32a + 8(r/4) + r%4 from i0 + 4h.
template <int NA>
__device__ __forceinline__ void dkdv_mask(f32x16* s, int i0, int krow, Win win, int h) {
  const int rlo = (win.right < 0 ? kUnbounded : krow - win.right) - i0 - 4 * h;
  const int rhi = (win.left < 0 ? (1 << 30) : krow + win.left) - i0 - 4 * h;
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 32 * a + 8 * (r >> 2) + (r & 3);
      if ((win.right >= 0 && off < rlo) || (win.left >= 0 && off > rhi)) s[a][r] = -INFINITY;
    }
}

// Phase 2 (VALU): mask (only when `edge`: the tile crosses an edge of the
// window of some of the wave's keys), P = 2^(S c - L log2 e),
// -dS = P (D - dP) from the accumulator, packed into MFMA operands.  st holds
// the tile's L (st[0..63]) and D (st[64..127]).
template <class T, int NA>
__device__ __forceinline__ void dkdv_probs(f32x16* s, f32x16* dp, const float* st, u32x4* pf, u32x4* dsf, bool edge,
                                           int i0, int krow, Win win, float c, int lane) {
  const int h = lane >> 5;
  if (edge) dkdv_mask<NA>(s, i0, krow, win, h);
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qi = 32 * a + 8 * g + 4 * h;
      const f32x4 l2 = *(const f32x4*)(st + qi) * kLog2e;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        const float p = exp2_fast(__builtin_fmaf(s[a][r], c, -l2[e]));
        s[a][r] = p;
        dp[a][r] = p * dp[a][r];
      }
    }
#pragma unroll
  for (int j = 0; j < 2 * NA; ++j) {
    pf[j] = pack8<T>(s[j >> 1], j & 1);
    dsf[j] = pack8<T>(dp[j >> 1], j & 1);
  }
}

// Phase 2 when dS is formed in phase 3 (kDvFirst): the mask,
// P = 2^(S c - L log2 e) and its packing; dp keeps D - dP.
template <class T, int NA>
__device__ __forceinline__ void dkdv_probs_p(f32x16* s, const float* st, u32x4* pf, bool edge, int i0, int krow,
                                             Win win, float c, int lane) {
  const int h = lane >> 5;
  if (edge) dkdv_mask<NA>(s, i0, krow, win, h);
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l2 = *(const f32x4*)(st + 32 * a + 8 * g + 4 * h) * kLog2e;
#pragma unroll
      for (int e = 0; e < 4; ++e) s[a][4 * g + e] = exp2_fast(__builtin_fmaf(s[a][4 * g + e], c, -l2[e]));
    }
#pragma unroll
  for (int j = 0; j < 2 * NA; ++j) pf[j] = pack8<T>(s[j >> 1], j & 1);
}

// Phase 3 with the dV MFMAs first: dV^T += dO^T P, then -dS = P (D - dP)
// and its packing written after them (so that they can issue while those
// MFMAs run), then dK^T += Q^T dS.  Each accumulator sums its products in
// the same order as dkdv_accum: bit-identical results.
template <class T, int D, int NA>
__device__ __forceinline__ void dkdv_accum_dv_first(const lds_char* qt, const lds_char* dot, const u32x4* pf,
                                                    const f32x16* s, f32x16* dp, f32x16* dka, f32x16* dva, int lane) {
  constexpr int NB = D / 32;
  u32x4 dsf[2 * NA];
  prio_mfma_begin();
#pragma unroll
  for (int j = 0; j < 2 * NA; ++j)
#pragma unroll
    for (int b = 0; b < NB; ++b) dva[b] = Elem<T>::mma(lds_cols_operand<D>(dot, j, 32 * b, lane), pf[j], dva[b]);
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[a][r] = s[a][r] * dp[a][r];
#pragma unroll
  for (int j = 0; j < 2 * NA; ++j) dsf[j] = pack8<T>(dp[j >> 1], j & 1);
#pragma unroll
  for (int j = 0; j < 2 * NA; ++j)
#pragma unroll
    for (int b = 0; b < NB; ++b) dka[b] = Elem<T>::mma(lds_cols_operand<D>(qt, j, 32 * b, lane), dsf[j], dka[b]);
  sched_mfma_lds<4 * NA * NB, 2, (4 * NA * NB < Dkdv<D>::kPre2 ? 4 * NA * NB : Dkdv<D>::kPre2)>();
  prio_mfma_end();
}

// Phase 3 (MFMA): dV^T += dO^T P and dK^T += Q^T dS, A operands by
// transposed LDS reads.
template <class T, int D, int NA>
__device__ __forceinline__ void dkdv_accum(const lds_char* qt, const lds_char* dot, const u32x4* pf, const u32x4* dsf,
                                           f32x16* dka, f32x16* dva, int lane) {
  constexpr int NB = D / 32;
  prio_mfma_begin();
#pragma unroll
  for (int j = 0; j < 2 * NA; ++j)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      dva[b] = Elem<T>::mma(lds_cols_operand<D>(dot, j, 32 * b, lane), pf[j], dva[b]);
      dka[b] = Elem<T>::mma(lds_cols_operand<D>(qt, j, 32 * b, lane), dsf[j], dka[b]);
    }
  sched_mfma_lds<4 * NA * NB, 2, (4 * NA * NB < Dkdv<D>::kPre2 ? 4 * NA * NB : Dkdv<D>::kPre2)>();
  prio_mfma_end();
}

// One query tile of the dK/dV kernel for one wave, the three phases in a
// row.  One code path for every tile, so the accumulator registers need no
// copies at merges.
template <class T, int D, int NA, bool DVF, class VOp>
__device__ __forceinline__ void dkdv_tile(const lds_char* qt, const lds_char* dot, const float* st, const u32x4* kf,
                                          const VOp& vop, f32x16* dka, f32x16* dva, bool edge, int i0, int krow,
                                          Win win, float c, int lane) {
  f32x16 s[NA], dp[NA];
  u32x4 pf[2 * NA], dsf[2 * NA];
  dkdv_scores<T, D, NA>(qt, dot, kf, vop, st, s, dp, lane);
  if constexpr (DVF) {
    dkdv_probs_p<T, NA>(s, st, pf, edge, i0, krow, win, c, lane);
    dkdv_accum_dv_first<T, D, NA>(qt, dot, pf, s, dp, dka, dva, lane);
  } else {
    dkdv_probs<T, NA>(s, dp, st, pf, dsf, edge, i0, krow, win, c, lane);
    dkdv_accum<T, D, NA>(qt, dot, pf, dsf, dka, dva, lane);
  }
}

// Enqueue the DMA of query tile i0: Q rows, dO rows, then L and D (one
// dword per lane, waves 0 and 1).  Rows past N load as zeros: their Q and
// dO rows are zero, so they add nothing to dV (dO = 0) or to dK
// (dS = P (0 - 0) = 0) whatever P is.
template <int D>
__device__ __forceinline__ void dkdv_issue(lds_char* b, int i0, const DmaTile<Dkdv<D>::kTile, D, kBwdWaves>& dma, Rsrc rq,
                                           Rsrc rdo, Rsrc rl, Rsrc rd, int w, int lane) {
  constexpr int TILE = Dkdv<D>::kTile * D * 2;
  dma.issue(rq, b, i0, w);
  dma.issue(rdo, b + TILE, i0, w);
  if (w < 2) dma4(w == 0 ? rl : rd, b + 2 * TILE + w * kStatsRows * 4, (uint32_t)((i0 + lane) * 4));
}

// One ring step on query tile t, held in ring buffer IDX = t % S (a
// compile-time index, so LDS operand addresses are register + immediate):
// wait and barrier, DMA of tile t + S - 1, then the math.  Tile t starts
// at row i_first + t walk: walk = -BMQ walks the tiles from the last one
// down, walk = BMQ from the first one up (see dkdv_kernel).
template <class T, int D, bool MASK, bool DVF, int IDX, class VOp>
__device__ __forceinline__ void dkdv_step(lds_char* lds, int t, int nt, int i_first, int walk,
                                          const DmaTile<Dkdv<D>::kTile, D, kBwdWaves>& dma, Rsrc rq, Rsrc rdo, Rsrc rl,
                                          Rsrc rd, const u32x4* kf, const VOp& vop, f32x16* dka, f32x16* dva,
                                          int wk0, int krow, Win win, float c, int w, int lane) {
  constexpr int S = Dkdv<D>::kStages, BMQ = Dkdv<D>::kTile, TILE = BMQ * D * 2, BUF = 2 * TILE + 2 * kStatsRows * 4;
  constexpr int PT = 2 * DmaTile<Dkdv<D>::kTile, D, kBwdWaves>::PER;  // per tile; waves 0, 1 add an L or D dword
  if (w < 2)
    ring_wait<S, PT + 1>(t, nt);
  else
    ring_wait<S, PT>(t, nt);
  const int i0 = i_first + t * walk;
  if (t + S - 1 < nt) dkdv_issue<D>(lds + ((IDX + S - 1) % S) * BUF, i0 + (S - 1) * walk, dma, rq, rdo, rl, rd, w, lane);
  __builtin_amdgcn_sched_barrier(0);
  // No query of the tile sees any key of the wave.
  if (MASK && (i0 + BMQ <= win.query_lo(wk0) || i0 >= win.query_hi(wk0 + 31, 1 << 30))) return;
  const lds_char* cur = lds + IDX * BUF;
  const float* st = (const float*)(cur + 2 * TILE);
  const bool edge = MASK && !win.all_visible(i0, i0 + BMQ - 1, wk0, wk0 + 31);
  dkdv_tile<T, D, BMQ / 32, DVF>(cur, cur + TILE, st, kf, vop, dka, dva, edge, i0, krow, win, c, lane);
}

// ---------------------------------------------------------------------------
// dK, dV.  Workgroup = 128 keys of one head (wave w owns keys k0 + 32w ..
// k0 + 32w + 31, with its K and V rows resident as MFMA B operands), looping
// over query tiles of 64 rows: Q and dO tiles plus their L and D copied by
// buffer DMA into swizzled LDS through a ring of S buffers (tiles t+1 ..
// t+S-1 in flight during tile t).  Per tile and wave:
//   S = Q K^T, dP = dO V^T          (lane = key, registers = queries)
//   P = 2^(S c - L2), dS = P (dP - D)
//   dV^T += dO^T P, dK^T += Q^T dS  (A operands by transposed LDS reads)
// With a window (the causal mask is one) the query tiles cover only the
// queries that see some key of the block, and only tiles that cross an edge
// of a key's window are masked.
// ---------------------------------------------------------------------------
// The ring loop over query tiles, once per query head g0 .. g0 + ng - 1 of
// the key/value head's group (G = 1 without grouping: the gradients of a
// shared K and V are the sums over the heads that read them), and the final
// store of dK and dV, or of their float32 partial sums over those heads when
// the group is split over several workgroups.  The first head's first tiles
// were issued by the caller.
template <class T, int D, bool MASK, bool SPLIT, bool DVF, class VOp, class Dst>
__device__ __forceinline__ void dkdv_run(lds_char* lds, int nt, int i_first, int walk, const DmaTile<Dkdv<D>::kTile, D, kBwdWaves>& dma,
                                         const void* qp, const void* dop, const float* lsep, const float* deltap,
                                         const Geom& geo, int b, int hk, int g0, int ng, int N, const u32x4* kf,
                                         const VOp& vop, Dst rdk, Dst rdv,
                                         int wk0, int krow, Win win, float c, float scale, int w, int lane) {
  constexpr int S = Dkdv<D>::kStages, NB = D / 32, BMQ = Dkdv<D>::kTile;
  constexpr int BUF = 2 * BMQ * D * 2 + 2 * kStatsRows * 4;
  const uint32_t bytes = (uint32_t)N * D * 2;
  f32x16 dka[NB], dva[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) dka[b] = dva[b] = (f32x16){};
  for (int g = 0; g < ng; ++g) {
    long qr0, kvr0;
    int len;
    geo.slice(b, hk * geo.G + g0 + g, qr0, kvr0, len);
    const size_t head = (size_t)qr0 * D * 2;
    const Rsrc rq = make_rsrc_words((const char*)qp + head, bytes);
    const Rsrc rdo = make_rsrc_words((const char*)dop + head, bytes);
    const Rsrc rl = make_rsrc_words(lsep + qr0, (uint32_t)N * 4);
    const Rsrc rd = make_rsrc_words(deltap + qr0, (uint32_t)N * 4);
    if (g > 0) {
      // Every wave is done with the previous head's ring before it refills.
      dma_wait_barrier<0>();
      dkdv_issue<D>(lds, i_first, dma, rq, rdo, rl, rd, w, lane);
      if (S > 2 && nt > 1) dkdv_issue<D>(lds + (1 % S) * BUF, i_first + walk, dma, rq, rdo, rl, rd, w, lane);
      if (S > 3 && nt > 2) dkdv_issue<D>(lds + (2 % S) * BUF, i_first + 2 * walk, dma, rq, rdo, rl, rd, w, lane);
    }
    for (int t = 0; t < nt; t += S) {
      dkdv_step<T, D, MASK, DVF, 0>(lds, t, nt, i_first, walk, dma, rq, rdo, rl, rd, kf, vop, dka, dva, wk0, krow, win, c, w,
                               lane);
      if (t + 1 < nt)
        dkdv_step<T, D, MASK, DVF, 1>(lds, t + 1, nt, i_first, walk, dma, rq, rdo, rl, rd, kf, vop, dka, dva, wk0, krow, win, c,
                                 w, lane);
      if constexpr (S > 2)
        if (t + 2 < nt)
          dkdv_step<T, D, MASK, DVF, 2 % S>(lds, t + 2, nt, i_first, walk, dma, rq, rdo, rl, rd, kf, vop, dka, dva, wk0, krow,
                                       win, c, w, lane);
      if constexpr (S > 3)
        if (t + 3 < nt)
          dkdv_step<T, D, MASK, DVF, 3 % S>(lds, t + 3, nt, i_first, walk, dma, rq, rdo, rl, rd, kf, vop, dka, dva, wk0, krow,
                                       win, c, w, lane);
    }
  }
  if constexpr (SPLIT) {
    // float32 partial rows (built here, after the loop, to keep the
    // descriptors out of the loop's registers)
    store_rows_f32<D>(make_rsrc(rdk, (uint32_t)N * D * 4), krow, dka, lane);
    store_rows_f32<D>(make_rsrc(rdv, (uint32_t)N * D * 4), krow, dva, lane);
  } else {
    store_rows<T, D>(rdk, krow, dka, -scale, lane);  // dka holds -dK / scale
    store_rows<T, D>(rdv, krow, dva, 1.0f, lane);
  }
}

// Grid: key blocks x head splits x key/value heads (BHkv = B * H / G of
// them); the query heads of key/value head hk are hk G .. hk G + G - 1 of
// the same batch.  With GS = 1 a workgroup takes the whole group and stores
// dK and dV; with GS > 1 (GS divides G) split s takes heads s G/GS ..
// (s + 1) G/GS - 1 and stores float32 sums (dK as -dK / scale, the sign
// convention of dkdv_scores) into part[s][row][D] (dK) and
// part[GS + s][row][D] (dV), rows numbered as in the K tensor (R of them),
// for dkdv_reduce_kernel to add up.
template <class T, int D, int MODE, bool SPLIT>
__global__ __launch_bounds__(64 * kBwdWaves, Dkdv<D>::kOcc) void dkdv_kernel(
    const void* __restrict__ qp, const void* __restrict__ kp, const void* __restrict__ vp,
    const void* __restrict__ dop, const float* __restrict__ lsep, const float* __restrict__ deltap,
    void* __restrict__ dkp, void* __restrict__ dvp, float* __restrict__ part, int GS_in, Geom geo, int BHkv,
    Win win_in, float c, float scale, int gen) {
  // MODE 0: no window (full mask); 1: the causal window (-1, 0), a
  // compile-time constant so that every window test folds; 2: any window.
  constexpr bool MASK = MODE != 0;
  const Win win = MODE == 1 ? Win{-1, 0} : win_in;
  constexpr int NW = kBwdWaves, BNK = 32 * NW, BMQ = Dkdv<D>::kTile, NKK = D / 16;
  constexpr int TILE = BMQ * D * 2;
  constexpr int S = Dkdv<D>::kStages;
  constexpr bool VL = Dkdv<D>::kVLds;
  constexpr int BUF = 2 * TILE + 2 * kStatsRows * 4;  // Q tile, dO tile, L[64], D[64]
  constexpr int VTILE = VL ? BNK * D * 2 : 0;  // the workgroup's V rows
  __shared__ __attribute__((aligned(16))) char smem[S * BUF + VTILE];
  lds_char* const lds = (lds_char*)smem;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
  const int GS = SPLIT ? GS_in : 1;
  const int x = blockIdx.x;
  const int kb = x / (BHkv * GS), rest = x - kb * (BHkv * GS);
  // Uniform across the workgroup: kept in scalar registers.
  const int split = SPLIT ? __builtin_amdgcn_readfirstlane(rest / BHkv) : 0, bhkv = rest - split * BHkv;
  const int ng = SPLIT ? __builtin_amdgcn_readfirstlane(geo.G / GS) : geo.G;
  const int Hkv = geo.H / geo.G, g0 = split * ng;
  const int b = bhkv / Hkv, hk = bhkv % Hkv;
  const int k0 = kb * BNK;
  long qr0, kvr0;  // the split's first query head, and the key/value head
  int N;
  geo.slice(b, hk * geo.G + g0, qr0, kvr0, N);
  if (k0 >= N) return;  // past the end of a shorter packed sequence (the whole workgroup)
  const size_t headkv = (size_t)kvr0 * D * 2;
  const size_t head0 = (size_t)qr0 * D * 2;
  const uint32_t bytes = (uint32_t)N * D * 2;
  const auto rk = make_rsrc((const char*)kp + headkv, bytes);
  // dK and dV destinations: buffer descriptors of the output rows, or with
  // SPLIT the float32 partial rows of this split.
  using Dst = std::conditional_t<SPLIT, const float*, __amdgpu_buffer_rsrc_t>;
  Dst rdk, rdv;
  if constexpr (SPLIT) {
    const long R = geo.cu ? (long)Hkv * geo.T : (long)BHkv * geo.N;
    rdk = part + ((long)split * R + kvr0) * D;
    rdv = rdk + (long)GS * R * D;
  } else {
    rdk = make_rsrc((char*)dkp + headkv, bytes);
    rdv = make_rsrc((char*)dvp + headkv, bytes);
  }

  // Query rows i_start .. i_end - 1 hold every query that sees a key of the block.
  const int i_start = MASK ? win.query_lo(k0) : 0, i_end = MASK ? win.query_hi(k0 + BNK - 1, N) : N;
  const int nt = (i_end - i_start + BMQ - 1) / BMQ;
  // Walk direction.  The co-resident key blocks of a head share a Q or dO
  // tile through L2 only if they read it at about the same time.  Under the
  // causal mask the blocks are dispatched heavy first, `gen` workgroups at a
  // time (the number resident at once; 0 when the grid holds fewer than two
  // such generations).  Generation 0 starts together and walks down from the
  // last tile, so its blocks move in step; they finish one by one at their
  // diagonals, lightest first, and the blocks of generation 1 start in their
  // places, staggered by as much as their lengths differ.  Walking up from
  // their diagonals, they then reach each row at the same time and finish
  // together at the last tile, so generation 2 starts together and walks
  // down, and so on.  Every other case walks down (without a mask all blocks
  // start and end together).  Measured at bf16 causal: walking every block
  // down was 1.2% faster than walking every block up at [2,16,8192,128] and
  // 8% at [8,16,1024,64]; alternating keeps that time and reads a third
  // fewer bytes from beyond L2 at [2,16,8192,128] (40% fewer at N = 16384).
  // Not at d = 64, whose occupancy of three workgroups per CU leaves no
  // register for the direction.
  const bool up = MODE == 1 && !SPLIT && D != 64 && gen > 0 && ((x / gen) & 1) != 0;
  const int i_first = up ? i_start : i_start + (nt - 1) * BMQ;
  const int walk = up ? BMQ : -BMQ;
  DmaTile<BMQ, D, NW> dma;
  dma.init(w, lane);
  {
    const Rsrc rq = make_rsrc_words((const char*)qp + head0, bytes);
    const Rsrc rdo = make_rsrc_words((const char*)dop + head0, bytes);
    const Rsrc rl = make_rsrc_words(lsep + qr0, (uint32_t)N * 4);
    const Rsrc rd = make_rsrc_words(deltap + qr0, (uint32_t)N * 4);
    dkdv_issue<D>(lds, i_first, dma, rq, rdo, rl, rd, w, lane);
  }
  lds_char* const vt = lds + S * BUF;
  if constexpr (VL) {
    DmaTile<BNK, D, NW> dmav;
    dmav.init(w, lane);
    dmav.issue(make_rsrc_words((const char*)vp + headkv, bytes), vt, k0, w);
  }

  const int wk0 = k0 + 32 * w;
  const int krow = wk0 + (lane & 31);
  u32x4 kf[NKK], vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kf[kk] = bload16(rk, (uint32_t)((krow * D + 16 * kk + 8 * h) * 2));
  if constexpr (!VL) {
    const auto rv = make_rsrc((const char*)vp + headkv, bytes);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) vf[kk] = bload16(rv, (uint32_t)((krow * D + 16 * kk + 8 * h) * 2));
  }
  // K and V (and with them tile 0 and the V tile) land before the ring starts.
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    land(kf[kk]);
    if constexpr (!VL) land(vf[kk]);
  }
  // The signs of the workgroup's V rows flipped once (exact), for the
  // dP^T accumulation that starts from D (dkdv_scores).
  if constexpr (VL) {
    // Every wave's share of the V tile landed before its K loads; after the
    // barrier each lane flips 16-byte chunks of the whole tile, and the
    // ring's first barrier (after an lgkmcnt(0) wait) publishes them.
    __builtin_amdgcn_s_barrier();
    lds_u32x4* const v4 = (lds_u32x4*)vt;
    for (int i = tid; i < VTILE / 16; i += 64 * NW) v4[i] ^= kSignBits16;
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) vf[kk] ^= kSignBits16;
  }
  {
    const Rsrc rq = make_rsrc_words((const char*)qp + head0, bytes);
    const Rsrc rdo = make_rsrc_words((const char*)dop + head0, bytes);
    const Rsrc rl = make_rsrc_words(lsep + qr0, (uint32_t)N * 4);
    const Rsrc rd = make_rsrc_words(deltap + qr0, (uint32_t)N * 4);
    if (S > 2 && nt > 1) dkdv_issue<D>(lds + (1 % S) * BUF, i_first + walk, dma, rq, rdo, rl, rd, w, lane);
    if (S > 3 && nt > 2) dkdv_issue<D>(lds + (2 % S) * BUF, i_first + 2 * walk, dma, rq, rdo, rl, rd, w, lane);
  }
  if constexpr (VL)
    dkdv_run<T, D, MASK, SPLIT, kDvFirst<D> && MODE != 2>(lds, nt, i_first, walk, dma, qp, dop, lsep, deltap, geo, b, hk, g0, ng, N, kf,
                                VLds<D>{vt, 32 * w}, rdk, rdv, wk0, krow, win, c, scale, w, lane);
  else
    dkdv_run<T, D, MASK, SPLIT, kDvFirst<D> && MODE != 2>(lds, nt, i_first, walk, dma, qp, dop, lsep, deltap, geo, b, hk, g0, ng, N, kf, VRegs{vf},
                                rdk, rdv, wk0, krow, win, c, scale, w, lane);
}

// Sum of the GS float32 partials of dK and dV (split 0 first, so the bits
// depend only on GS), dK times `scale` (the launcher passes -scale, undoing
// the partials' sign), rounded to the element type.  One
// workgroup per dK/dV key block: rows k0 .. k0 + 127 of one key/value head,
// D / 4 lanes per row, four columns per lane.
template <class T, int D>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float* __restrict__ part, void* __restrict__ dkp,
                                                          void* __restrict__ dvp, int GS, Geom geo, int BHkv,
                                                          float scale) {
  constexpr int BNK = 32 * kBwdWaves, LPR = D / 4, RPI = 256 / LPR;
  const int x = blockIdx.x, kb = x / BHkv, bhkv = x % BHkv;
  const int Hkv = geo.H / geo.G, b = bhkv / Hkv, hk = bhkv % Hkv;
  long qr0, kvr0;
  int N;
  geo.slice(b, hk * geo.G, qr0, kvr0, N);
  const int k0 = kb * BNK;
  if (k0 >= N) return;
  const int rows = min(BNK, N - k0);
  const long R = geo.cu ? (long)Hkv * geo.T : (long)BHkv * geo.N;
  const long plane = R * D;
  const int c4 = threadIdx.x % LPR;
  for (int r = threadIdx.x / LPR; r < rows; r += RPI) {
    const long e = (kvr0 + k0 + r) * D + 4 * c4;
    float4 sk = *(const float4*)(part + e), sv = *(const float4*)(part + GS * plane + e);
    for (int s = 1; s < GS; ++s) {
      const float4 pk = *(const float4*)(part + s * plane + e), pv = *(const float4*)(part + (GS + s) * plane + e);
      sk.x += pk.x; sk.y += pk.y; sk.z += pk.z; sk.w += pk.w;
      sv.x += pv.x; sv.y += pv.y; sv.z += pv.z; sv.w += pv.w;
    }
    const u32x2 ok = {Elem<T>::pack2(sk.x * scale, sk.y * scale), Elem<T>::pack2(sk.z * scale, sk.w * scale)};
    const u32x2 ov = {Elem<T>::pack2(sv.x, sv.y), Elem<T>::pack2(sv.z, sv.w)};
    *(u32x2*)((char*)dkp + e * 2) = ok;
    *(u32x2*)((char*)dvp + e * 2) = ov;
  }
}

// One key tile of the dQ kernel for one wave (`edge`: the tile crosses an
// edge of the window of some of the wave's queries, or the end of N).  One
// code path for every tile, so the accumulator registers need no copies at
// merges.
template <class T, int D, bool MASK, int NA>
__device__ __forceinline__ void dq_tile(const lds_char* kt, const lds_char* vt, const u32x4* qf, const u32x4* dof,
                                        f32x16* dqa, float l2, float dd, bool edge, int j0, int qrow, int N, Win win,
                                        float c, int lane) {
  constexpr int NKK = D / 16, NB = D / 32;
  const int h = lane >> 5;
  f32x16 s[NA], dp[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) s[a] = dp[a] = (f32x16){};
  prio_mfma_begin();
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      s[a] = Elem<T>::mma(lds_rows_operand<D>(kt, 32 * a, kk, lane), qf[kk], s[a]);
      dp[a] = Elem<T>::mma(lds_rows_operand<D>(vt, 32 * a, kk, lane), dof[kk], dp[a]);
    }
  sched_mfma_lds<2 * NA * NKK, 1, (2 * NA * NKK < FA_DQ_PRE1 ? 2 * NA * NKK : FA_DQ_PRE1)>();
  prio_mfma_end();
  if (edge) {
    const int klo = MASK ? win.lo(qrow) : kUnbounded, khi = MASK ? win.hi(qrow, N) : N - 1;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * a + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key > khi || (MASK && win.left >= 0 && key < klo)) s[a][r] = -INFINITY;
      }
  }
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(__builtin_fmaf(s[a][r], c, -l2));
      dp[a][r] = p * (dp[a][r] - dd);
    }
  u32x4 dsf[2 * NA];
#pragma unroll
  for (int j = 0; j < 2 * NA; ++j) dsf[j] = pack8<T>(dp[j >> 1], j & 1);
  prio_mfma_begin();
#pragma unroll
  for (int j = 0; j < 2 * NA; ++j)
#pragma unroll
    for (int b = 0; b < NB; ++b) dqa[b] = Elem<T>::mma(lds_cols_operand<D>(kt, j, 32 * b, lane), dsf[j], dqa[b]);
  sched_mfma_lds<2 * NA * NB, 2, (2 * NA * NB < FA_DQ_PRE2 ? 2 * NA * NB : FA_DQ_PRE2)>();
  prio_mfma_end();
}

// The same tile as three MFMA runs with the tile's VALU work written
// between them in issue order (each MFMA followed by its share, fenced so
// that the compiler keeps the order): S^T; dP^T with P = 2^(S c - L2) of two
// elements per MFMA; dQ^T with dS = P (dP - D) formed one packed operand
// ahead of the MFMAs that take it.  The MFMA pipe then runs while the wave's
// own softmax work issues.
// Used at every head dimension (10% and 5% faster dQ on the ragged fp16
// d = 32 and bf16 d = 64 workloads; at d = 128 it fits the registers with
// 32-key tiles and is 1.6% faster on the causal workload, even on the full
// one).  FA_DQ_PIPE=0/1 forces one form for every head dimension.
#ifdef FA_DQ_PIPE
template <int D>
constexpr bool kDqPipe = FA_DQ_PIPE != 0;
#else
template <int D>
constexpr bool kDqPipe = true;
#endif
// LDS operand reads run this many MFMAs ahead in the score runs and the dQ run.
#ifdef FA_DQ_PIPE_PRE1
template <int D>
constexpr int kDqPipePre1 = FA_DQ_PIPE_PRE1;
#else
template <int D>
constexpr int kDqPipePre1 = D == 64 ? 1 : 2;
#endif
#ifndef FA_DQ_PIPE_PRE3
#define FA_DQ_PIPE_PRE3 1
#endif

template <class T, int D, bool MASK, int NA>
__device__ __forceinline__ void dq_tile_pipe(const lds_char* kt, const lds_char* vt, const u32x4* qf,
                                             const u32x4* dof, f32x16* dqa, float l2, float dd, bool edge, int j0,
                                             int qrow, int N, Win win, float c, int lane) {
  constexpr int NKK = D / 16, NB = D / 32, NM = NA * NKK, NM3 = 2 * NA * NB;
  constexpr int E = 16 * NA / NM, F = 16 * NA / NM3;  // elements per MFMA in runs 2 and 3
  constexpr int PRE = kDqPipePre1<D>, PRE3 = FA_DQ_PIPE_PRE3;
  const int h = lane >> 5;
  f32x16 s[NA], dp[NA];
  u32x4 dsf[2 * NA];

  // Run 1: S^T = K Q^T (MFMA i: kk = i / NA, a = i % NA).
  {
    u32x4 ko[NM];
#pragma unroll
    for (int a = 0; a < NA; ++a) s[a] = dp[a] = (f32x16){};
#pragma unroll
    for (int i = 0; i < PRE; ++i) ko[i] = lds_rows_operand<D>(kt, 32 * (i % NA), i / NA, lane);
    prio_mfma_begin();
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + PRE < NM) ko[i + PRE] = lds_rows_operand<D>(kt, 32 * ((i + PRE) % NA), (i + PRE) / NA, lane);
      s[i % NA] = Elem<T>::mma(ko[i], qf[i / NA], s[i % NA]);
      __builtin_amdgcn_sched_barrier(0);
    }
    prio_mfma_end();
  }
  if (edge) {
    const int klo = MASK ? win.lo(qrow) : kUnbounded, khi = MASK ? win.hi(qrow, N) : N - 1;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * a + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key > khi || (MASK && win.left >= 0 && key < klo)) s[a][r] = -INFINITY;
      }
  }
  __builtin_amdgcn_sched_barrier(0);

  // Run 2: dP^T = V dO^T, and P = 2^(S c - L2) of E elements after each MFMA.
  {
    u32x4 vo[NM];
#pragma unroll
    for (int i = 0; i < PRE; ++i) vo[i] = lds_rows_operand<D>(vt, 32 * (i % NA), i / NA, lane);
    prio_mfma_begin();
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + PRE < NM) vo[i + PRE] = lds_rows_operand<D>(vt, 32 * ((i + PRE) % NA), (i + PRE) / NA, lane);
      dp[i % NA] = Elem<T>::mma(vo[i], dof[i / NA], dp[i % NA]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int x = i * E + e;
        s[x / 16][x % 16] = exp2_fast(__builtin_fmaf(s[x / 16][x % 16], c, -l2));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    prio_mfma_end();
  }

  // Run 3: dQ^T += K^T dS^T (MFMA i: j = i / NB, b = i % NB).  dS operand j
  // (elements 8j .. 8j + 7) is formed before the first MFMA, operand j + 1
  // under the MFMAs of operand j, F elements after each.
  {
    auto ds_elem = [&](int x) {
      dp[x / 16][x % 16] = s[x / 16][x % 16] * (dp[x / 16][x % 16] - dd);
      if (x % 8 == 7) dsf[x / 8] = pack8<T>(dp[x / 16], (x % 16) / 8);
    };
#pragma unroll
    for (int x = 0; x < 8; ++x) ds_elem(x);
    u32x4 to[NM3];
#pragma unroll
    for (int i = 0; i < PRE3; ++i) to[i] = lds_cols_operand<D>(kt, i / NB, 32 * (i % NB), lane);
    prio_mfma_begin();
#pragma unroll
    for (int i = 0; i < NM3; ++i) {
      if (i + PRE3 < NM3) to[i + PRE3] = lds_cols_operand<D>(kt, (i + PRE3) / NB, 32 * ((i + PRE3) % NB), lane);
      dqa[i % NB] = Elem<T>::mma(to[i], dsf[i / NB], dqa[i % NB]);
      if (i / NB + 1 < 2 * NA) {
#pragma unroll
        for (int e = 0; e < F; ++e) ds_elem(8 * (i / NB + 1) + F * (i % NB) + e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    prio_mfma_end();
  }
}

// DMA of key tile t (K then V) into ring buffer IDX.
template <int D, int IDX>
__device__ __forceinline__ void dq_issue(lds_char* lds, int t, const DmaTile<kDqTile<D>, D, kBwdWaves>& dma, Rsrc rk,
                                         Rsrc rv, int w) {
  constexpr int TILE = kDqTile<D> * D * 2;
  lds_char* b = lds + IDX * 2 * TILE;
  dma.issue(rk, b, t * kDqTile<D>, w);
  dma.issue(rv, b + TILE, t * kDqTile<D>, w);
}

// One ring step on key tile t, held in ring buffer IDX = t % S.
template <class T, int D, bool MASK, int IDX>
__device__ __forceinline__ void dq_step(lds_char* lds, int t, int nt, int tb, const DmaTile<kDqTile<D>, D, kBwdWaves>& dma,
                                        Rsrc rk, Rsrc rv, const u32x4* qf, const u32x4* dof, f32x16* dqa, float l2,
                                        float dd, int wq0, int qrow, int N, Win win, float c, int w, int lane) {
  constexpr int S = kDqStages<D>, BN = kDqTile<D>, TILE = BN * D * 2;
  ring_wait<S, 2 * DmaTile<kDqTile<D>, D, kBwdWaves>::PER>(t, nt);
  if (t + S - 1 < nt) dq_issue<D, (IDX + S - 1) % S>(lds, tb + t + S - 1, dma, rk, rv, w);
  __builtin_amdgcn_sched_barrier(0);
  const int j0 = (tb + t) * BN;
  // No key of the tile is visible to any query of the wave.
  if (MASK && (j0 + BN <= win.key_lo(wq0) || j0 >= win.key_hi(wq0 + 31, N))) return;
  const lds_char* cur = lds + IDX * 2 * TILE;
  const bool edge = (j0 + BN > N) || (MASK && !win.all_visible(wq0, wq0 + 31, j0, j0 + BN - 1));
  if constexpr (kDqPipe<D>)
    dq_tile_pipe<T, D, MASK, BN / 32>(cur, cur + TILE, qf, dof, dqa, l2, dd, edge, j0, qrow, N, win, c, lane);
  else
    dq_tile<T, D, MASK, BN / 32>(cur, cur + TILE, qf, dof, dqa, l2, dd, edge, j0, qrow, N, win, c, lane);
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup = 128 queries of one head (wave w owns 32, with its Q and dO
// rows resident as MFMA B operands and its L and D in registers), looping
// over key tiles of 64 rows (K and V copied by buffer DMA into swizzled LDS
// through a ring of S buffers):
//   S^T = K Q^T, dP^T = V dO^T   (lane = query, registers = keys)
//   P = 2^(S c - L2), dS = P (dP - D)
//   dQ^T += K^T dS^T             (A operand by transposed LDS reads)
// ---------------------------------------------------------------------------
template <class T, int D, int MODE>
__global__ __launch_bounds__(64 * kBwdWaves, 2) void dq_kernel(const void* __restrict__ qp, const void* __restrict__ kp,
                                                            const void* __restrict__ vp, const void* __restrict__ dop,
                                                            const float* __restrict__ lsep,
                                                            const float* __restrict__ deltap, void* __restrict__ dqp,
                                                            Geom geo, int BH, int nqb, Win win_in, float c,
                                                            float scale) {
  // MODE 0: no window (full mask); 1: the causal window (-1, 0), a
  // compile-time constant so that every window test folds; 2: any window.
  constexpr bool MASK = MODE != 0;
  const Win win = MODE == 1 ? Win{-1, 0} : win_in;
  constexpr int NW = kBwdWaves, BM = 32 * NW, BN = kDqTile<D>, NKK = D / 16, NB = D / 32;
  constexpr int S = kDqStages<D>, TILE = BN * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[S * 2 * TILE];
  lds_char* const lds = (lds_char*)smem;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
  const int x = blockIdx.x;
  const int qb = MASK ? (nqb - 1 - x / BH) : (x / BH);
  const int bh = x % BH;
  const int q0 = qb * BM;
  // This (batch, head) slice: query head h reads key/value head h / G.
  long qr0, kvr0;
  int N;
  geo.slice(bh / geo.H, bh % geo.H, qr0, kvr0, N);
  if (q0 >= N) return;  // past the end of a shorter packed sequence (the whole workgroup)
  const size_t head = (size_t)qr0 * D * 2, headkv = (size_t)kvr0 * D * 2;
  const uint32_t bytes = (uint32_t)N * D * 2;
  const auto rq = make_rsrc((const char*)qp + head, bytes);
  const auto rdo = make_rsrc((const char*)dop + head, bytes);
  const auto rdq = make_rsrc((char*)dqp + head, bytes);
  const Rsrc rk = make_rsrc_words((const char*)kp + headkv, bytes);
  const Rsrc rv = make_rsrc_words((const char*)vp + headkv, bytes);

  // Key tiles tb .. tb + nt - 1 hold every key visible to the block.
  const int kbeg = MASK ? win.key_lo(q0) : 0, kend = MASK ? win.key_hi(q0 + BM - 1, N) : N;
  const int tb = kbeg / BN, nt = (kend + BN - 1) / BN - tb;
  DmaTile<BN, D, NW> dma;
  dma.init(w, lane);
  dq_issue<D, 0>(lds, tb, dma, rk, rv, w);

  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + (lane & 31);
  u32x4 qf[NKK], dof[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qf[kk] = bload16(rq, (uint32_t)((qrow * D + 16 * kk + 8 * h) * 2));
    dof[kk] = bload16(rdo, (uint32_t)((qrow * D + 16 * kk + 8 * h) * 2));
  }
  const float l2 = qrow < N ? lsep[(size_t)qr0 + qrow] * kLog2e : INFINITY;
  const float dd = qrow < N ? deltap[(size_t)qr0 + qrow] : 0.f;
  // Q, dO, L, D (and with them tile 0) land before the ring starts.
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    land(qf[kk]);
    land(dof[kk]);
  }
  land(l2);
  land(dd);
  if (S > 2 && nt > 1) dq_issue<D, 1 % S>(lds, tb + 1, dma, rk, rv, w);
  if (S > 3 && nt > 2) dq_issue<D, 2 % S>(lds, tb + 2, dma, rk, rv, w);
  f32x16 dqa[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) dqa[b] = (f32x16){};

  for (int t = 0; t < nt; t += S) {
    dq_step<T, D, MASK, 0>(lds, t, nt, tb, dma, rk, rv, qf, dof, dqa, l2, dd, wq0, qrow, N, win, c, w, lane);
    if (t + 1 < nt)
      dq_step<T, D, MASK, 1>(lds, t + 1, nt, tb, dma, rk, rv, qf, dof, dqa, l2, dd, wq0, qrow, N, win, c, w, lane);
    if constexpr (S > 2)
      if (t + 2 < nt)
        dq_step<T, D, MASK, 2 % S>(lds, t + 2, nt, tb, dma, rk, rv, qf, dof, dqa, l2, dd, wq0, qrow, N, win, c, w,
                                   lane);
    if constexpr (S > 3)
      if (t + 3 < nt)
        dq_step<T, D, MASK, 3 % S>(lds, t + 3, nt, tb, dma, rk, rv, qf, dof, dqa, l2, dd, wq0, qrow, N, win, c, w,
                                   lane);
  }
  store_rows<T, D>(rdq, qrow, dqa, scale, lane);
}

// ---------------------------------------------------------------------------
// The static scratch array's device address on the current device, looked
// up once per device (with that device current) and kept: in host code the
// array's name is not a device address, so kernels only ever receive the
// address returned here.
// ---------------------------------------------------------------------------
namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_region(void** base) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_addr[dev] = p;
  }
  *base = scratch_addr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <class T, int D>
static hipError_t launch_pre_t(const PreArgs& a, hipStream_t st) {
  const long rows = (long)a.B * a.H * a.N;
  const int rpb = 256 / (D / 8);
  const long grid = std::min<long>((rows + rpb - 1) / rpb, 1L << 20);
  hipLaunchKernelGGL((preprocess_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, st, a.o, a.dO, a.delta, rows);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_pre_e(const PreArgs& a, hipStream_t st) {
  switch (a.d) {
    case 32: return launch_pre_t<T, 32>(a, st);
    case 64: return launch_pre_t<T, 64>(a, st);
    default: return launch_pre_t<T, 128>(a, st);
  }
}

hipError_t launch_preprocess(const PreArgs& a, hipStream_t st) {
  return a.bf16 ? launch_pre_e<bf16_tag>(a, st) : launch_pre_e<f16_tag>(a, st);
}

// Workgroups of `kernel` (256 threads) resident on the current device at
// once (compute units x workgroups per compute unit), looked up once per
// device into `cache`; 0 if either query fails.
static int resident_workgroups(const void* kernel, std::atomic<int>* cache) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, per_cu = 0;
    const bool ok = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                    hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) == hipSuccess;
    // A failed query must not surface as the launch's error (the caller
    // reads hipGetLastError after the launch): clear it and walk down.
    if (!ok) (void)hipGetLastError();
    v = ok && cus > 0 && per_cu > 0 ? cus * per_cu : -1;  // 0 is "not looked up yet"
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v > 0 ? v : 0;
}

// The generation size passed to the causal dK/dV kernel's choice of walk
// direction: the resident workgroups, or 0 (every block walks down) when the
// grid holds fewer than two generations, where alternating only reorders.
static int walk_generation(int resident, long long grid) { return grid >= 2LL * resident ? resident : 0; }

template <class T, int D>
static int dkdv_resident() {
  static std::atomic<int> cache[kMaxDevices] = {};
  return resident_workgroups(reinterpret_cast<const void*>(dkdv_kernel<T, D, 1, false>), cache);
}

template <class T, int D, int MODE>
static hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t st) {
  const int BHkv = a.B * a.Hkv;
  const int nkb = (a.N + 127) / 128;
  const Geom geo{a.N, a.H, a.H / a.Hkv, a.cu, a.T};
  if (!a.part) {
    const long long grid = static_cast<long long>(nkb) * BHkv;
    const int gen = MODE == 1 && D != 64 ? walk_generation(dkdv_resident<T, D>(), grid) : 0;
    hipLaunchKernelGGL((dkdv_kernel<T, D, MODE, false>), dim3(nkb * BHkv), dim3(256), 0, st, a.q, a.k, a.v, a.dO,
                       a.lse, a.delta, a.dk, a.dv, nullptr, 1, geo, BHkv, Win{a.wl, a.wr}, a.scale * kLog2e, a.scale,
                       gen);
    return hipGetLastError();
  }
  const int GS = a.splits;
  hipLaunchKernelGGL((dkdv_kernel<T, D, MODE, true>), dim3(nkb * BHkv * GS), dim3(256), 0, st, a.q, a.k, a.v, a.dO,
                     a.lse, a.delta, a.dk, a.dv, a.part, GS, geo, BHkv, Win{a.wl, a.wr}, a.scale * kLog2e, a.scale,
                     0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The partials hold -dK / scale (the dK/dV kernel's sign convention).
  hipLaunchKernelGGL((dkdv_reduce_kernel<T, D>), dim3(nkb * BHkv), dim3(256), 0, st, a.part, a.dk, a.dv, GS, geo,
                     BHkv, -a.scale);
  return hipGetLastError();
}

template <class T, int D, int MODE>
static hipError_t launch_dq_t(const BwdArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  const int nqb = (a.N + 127) / 128;
  const Geom geo{a.N, a.H, a.H / a.Hkv, a.cu, a.T};
  hipLaunchKernelGGL((dq_kernel<T, D, MODE>), dim3(nqb * BH), dim3(256), 0, st, a.q, a.k, a.v, a.dO, a.lse,
                     a.delta, a.dq, geo, BH, nqb, Win{a.wl, a.wr}, a.scale * kLog2e, a.scale);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_dkdv_d(const BwdArgs& a, hipStream_t st) {
  switch (win_mode(a.wl, a.wr)) {
    case 0: return launch_dkdv_t<T, D, 0>(a, st);
    case 1: return launch_dkdv_t<T, D, 1>(a, st);
    default: return launch_dkdv_t<T, D, 2>(a, st);
  }
}
template <class T, int D>
static hipError_t launch_dq_d(const BwdArgs& a, hipStream_t st) {
  switch (win_mode(a.wl, a.wr)) {
    case 0: return launch_dq_t<T, D, 0>(a, st);
    case 1: return launch_dq_t<T, D, 1>(a, st);
    default: return launch_dq_t<T, D, 2>(a, st);
  }
}

template <class T>
static hipError_t launch_dkdv_e(const BwdArgs& a, hipStream_t st) {
  switch (a.d) {
    case 32: return launch_dkdv_d<T, 32>(a, st);
    case 64: return launch_dkdv_d<T, 64>(a, st);
    default: return launch_dkdv_d<T, 128>(a, st);
  }
}
template <class T>
static hipError_t launch_dq_e(const BwdArgs& a, hipStream_t st) {
  switch (a.d) {
    case 32: return launch_dq_d<T, 32>(a, st);
    case 64: return launch_dq_d<T, 64>(a, st);
    default: return launch_dq_d<T, 128>(a, st);
  }
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t st) {
  return a.bf16 ? launch_dkdv_e<bf16_tag>(a, st) : launch_dkdv_e<f16_tag>(a, st);
}
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st) {
  return a.bf16 ? launch_dq_e<bf16_tag>(a, st) : launch_dq_e<f16_tag>(a, st);
}

}  // namespace fa
