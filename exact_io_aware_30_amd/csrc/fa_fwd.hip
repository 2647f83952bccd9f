// Forward kernel: exact attention with the online softmax, one workgroup per
// BM query rows of one head ("flash-attn-triton" docs, "Tiling softmax is
// exact algebra" and Fig. 3 "the update, per tile"; FlashAttention-2 layout:
// queries in the outer loop, accumulator in registers, one divide after the
// loop, grid split over the sequence).
//
// Workgroup: NW waves; wave w owns queries q0 + 32w .. q0 + 32w + 31.
// Per key tile of BN = 32 NA rows (K and V copied global -> LDS by buffer DMA
// into a swizzled layout, through a ring of S buffers, so tiles t+1 .. t+S-1
// are in flight during tile t's math):
//   S^T = K Q^T          MFMA, A = K rows from LDS, B = Q^T kept in registers;
//                        lane l holds query l % 32 and half of the tile's keys
//   mask                 only on tiles that cross the diagonal or the end of N
//   row max              in-lane max, then one v_permlane32_swap
//   p = 2^(S c - ref), c = scale * log2(e); l += rowsum p
//   O^T += V^T P^T       MFMA, A = V^T by transposed LDS reads, B = P^T
//                        converted from the S^T registers in place
// The reference ref (a running row maximum in base-2 units) moves only when a
// row maximum exceeds it by more than 2^8; then l and acc are rescaled by
// alpha = 2^(ref_old - ref_new).  After the last tile: O = acc / l and
// L = (ref + log2 l) ln 2.
//
// Two forms: fwd_kernel (above per tile, a 3-deep ring) and, at d = 128,
// fwd_pipe_kernel, which overlaps tile t's softmax with tile t+1's QK^T
// inside each wave (see the comment at its step function).
#include "fa_device.h"
#include "fa_launch.h"

// Tile configuration (compile-time; defaults chosen by measurement).
// FA_FWD_WAVES / FA_FWD_KEYBLOCKS / FA_FWD_STAGES, when defined, apply to
// every head dimension.

namespace fa {

// Per head dimension: waves per workgroup (32 query rows each), key tile of
// 32 * kNA rows, LDS ring depth of the plain kernel.  At d = 32 a workgroup
// of 4 waves with a 2-deep ring (many workgroups per CU) is 20% faster than
// 8 waves with a 3-deep ring; at d = 64 and 128 the smaller workgroup is
// 3-9% slower on the large workloads.
template <int D>
struct FwdCfg {
#ifdef FA_FWD_WAVES
  static constexpr int kWaves = FA_FWD_WAVES;
#else
  static constexpr int kWaves = D == 32 ? 4 : 8;
#endif
#ifdef FA_FWD_KEYBLOCKS
  static constexpr int kNA = FA_FWD_KEYBLOCKS;
#else
  static constexpr int kNA = 2;
#endif
  static constexpr int kBN = 32 * kNA;
#ifdef FA_FWD_STAGES
  static constexpr int kStages = FA_FWD_STAGES;
#else
  static constexpr int kStages = D == 32 ? 2 : 3;
#endif
};

// Short sequences (N <= kShortSeq, the longest sequence when packed) use
// the plain kernel with 4 waves (128 query rows) and a 2-deep ring at every
// head dimension: causal grids of short sequences are a few blocks per head
// with very uneven work, and the smaller blocks pack the compute units
// better.  Measured (bf16 causal, same box): 10-13% faster at d = 64 for
// [8,16,1024] and [4,16,2048], 12% and 4% at d = 128 for [8,16,1024] and
// [4,16,2048]; at N = 4096 (d = 128) and 65536 (d = 64) the default shapes
// are 5% and 3% faster, hence the cut.
constexpr int kShortSeq = 2048, kShortWaves = 4, kShortStages = 2;
// Windows bounded on both sides and at most kNarrowWindow keys wide take the
// same kernel at any N: a block visits the keys of its rows' windows, so
// 128-row blocks visit fewer masked keys at the window's edges than 256-row
// ones.  Measured (bf16 [2,16,8192,d], same box, outputs bit-identical):
// windows (256, 0) 26% faster at d = 128 and 14% at d = 64, (512, 512) 12%,
// (1024, 0) 14% and 6%, (2047, 0) 9% and 7%, (3071, 0) 4%, (4095, 0) 2-3%.
constexpr long kNarrowWindow = 4096;

// Rescale threshold in base-2 units: the reference maximum used for the
// exponentials is moved only when a row's maximum exceeds it by more than
// this, so p = 2^(S c - ref) stays below 2^8 and most tiles skip the
// rescale of l and acc.  O = acc / l and L = ref + log2 l hold for any
// reference, so the result is the same up to rounding.
constexpr float kRescaleSlack = 8.0f;

// Wave priority around MFMA runs in the forward kernels (FA_FWD_PRIO=0 turns
// it off; the backward kernels use FA_SETPRIO).
#ifndef FA_FWD_PRIO
#define FA_FWD_PRIO 0
#endif
__device__ __forceinline__ void fwd_prio_begin() {
  if constexpr (FA_FWD_PRIO != 0) prio_mfma_begin_always();
}
__device__ __forceinline__ void fwd_prio_end() {
  if constexpr (FA_FWD_PRIO != 0) prio_mfma_end_always();
}

// Row sums of the plain kernel's tile added before its PV MFMAs (0) or
// after them in source order (1), where they issue beside the MFMAs: 0.3-1.6%
// faster at d = 32 and 64, bit-identical (same order of the adds).
#ifndef FA_FWD_PLAIN_SUM_AFTER_PV
#define FA_FWD_PLAIN_SUM_AFTER_PV 1
#endif
constexpr bool kPlainSumAfterPv = FA_FWD_PLAIN_SUM_AFTER_PV != 0;

// One key tile for one wave: S^T, mask (only when `edge`: the tile crosses
// an edge of the window or the end of N), online-softmax update, PV.  One
// code path for every tile, so the accumulator registers need no copies at
// merges.
template <class T, int D, bool MASK>
__device__ __forceinline__ void fwd_tile(const lds_char* kt, const lds_char* vt, const u32x4* qf, f32x16* acc,
                                         float& mref, float& l, bool edge, int j0, int qrow, int N, Win win,
                                         float c, int lane) {
  constexpr int NKK = D / 16, NB = D / 32, NA = FwdCfg<D>::kNA;
  const int h = lane >> 5;
  f32x16 s[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) s[a] = (f32x16){};
  fwd_prio_begin();
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
    for (int a = 0; a < NA; ++a) s[a] = Elem<T>::mma(lds_rows_operand<D>(kt, 32 * a, kk, lane), qf[kk], s[a]);
  sched_mfma_lds<NA * NKK, 1, (NA * NKK < 6 ? NA * NKK : 6)>();
  fwd_prio_end();
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
  float mx = s[0][0];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[a][r]);
  const float mxc = max_with_partner(mx) * c;  // row max in base-2 units
  if (__builtin_amdgcn_ballot_w64(mxc > mref + kRescaleSlack)) {
    const float mnew = fmaxf(mref, mxc);
    // 0 on a row's first visible tile (mref = -inf); rows with nothing
    // visible yet keep l = 0, acc = 0.
    const float alpha = mnew == -INFINITY ? 1.f : exp2_fast(mref - mnew);
    mref = mnew;
    l *= alpha;
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] *= alpha;
  }
  float rs = 0.f;
  const float mr = mref == -INFINITY ? 0.f : mref;  // all of a row masked so far: p = 0
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(__builtin_fmaf(s[a][r], c, -mr));
      s[a][r] = p;
      if constexpr (!kPlainSumAfterPv) rs += p;
    }
  if constexpr (!kPlainSumAfterPv) l += rs;
  u32x4 pf[2 * NA];
#pragma unroll
  for (int j = 0; j < 2 * NA; ++j) pf[j] = pack8<T>(s[j >> 1], j & 1);
  fwd_prio_begin();
#pragma unroll
  for (int j = 0; j < 2 * NA; ++j)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = Elem<T>::mma(lds_cols_operand<D>(vt, j, 32 * b, lane), pf[j], acc[b]);
  if constexpr (kPlainSumAfterPv) {
    // The row sums after the PV MFMAs in source order: only the packed P
    // must be ready before them, so the adds can issue while they run.
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) rs += s[a][r];
    l += rs;
  }
  sched_mfma_lds<2 * NA * NB, 2, (2 * NA * NB < 3 ? 2 * NA * NB : 3)>();
  fwd_prio_end();
}

// DMA of key tile t (K then V) into ring buffer IDX.
template <int D, int IDX, int NW>
__device__ __forceinline__ void fwd_issue(lds_char* lds, int t, const DmaTile<FwdCfg<D>::kBN, D, NW>& dma, Rsrc rk,
                                          Rsrc rv, int w) {
  constexpr int TILE = FwdCfg<D>::kBN * D * 2;
  lds_char* b = lds + IDX * 2 * TILE;
  dma.issue(rk, b, t * FwdCfg<D>::kBN, w);
  dma.issue(rv, b + TILE, t * FwdCfg<D>::kBN, w);
}

// Ring step on tile t, which sits in buffer IDX = t % S (a compile-time
// index, so that every LDS operand address is a register plus an immediate):
// wait and barrier, DMA of tile t + S - 1 into the buffer tile t - 1 used,
// then the math.
template <class T, int D, bool MASK, int IDX, int NW, int S>
__device__ __forceinline__ void fwd_step(lds_char* lds, int t, int nt, int tb, const DmaTile<FwdCfg<D>::kBN, D, NW>& dma,
                                         Rsrc rk, Rsrc rv, const u32x4* qf, f32x16* acc, float& mref, float& l,
                                         int wq0, int qrow, int N, Win win, float c, int w, int lane) {
  constexpr int BN = FwdCfg<D>::kBN, TILE = BN * D * 2;
  ring_wait<S, 2 * DmaTile<FwdCfg<D>::kBN, D, NW>::PER>(t, nt);
  if (t + S - 1 < nt) fwd_issue<D, (IDX + S - 1) % S, NW>(lds, tb + t + S - 1, dma, rk, rv, w);
  __builtin_amdgcn_sched_barrier(0);
  const int j0 = (tb + t) * BN;
  // No key of the tile is visible to any query of the wave.
  if (MASK && (j0 + BN <= win.key_lo(wq0) || j0 >= win.key_hi(wq0 + 31, N))) return;
  const lds_char* cur = lds + IDX * 2 * TILE;
  const bool edge = (j0 + BN > N) || (MASK && !win.all_visible(wq0, wq0 + 31, j0, j0 + BN - 1));
  fwd_tile<T, D, MASK>(cur, cur + TILE, qf, acc, mref, l, edge, j0, qrow, N, win, c, lane);
}

// ---------------------------------------------------------------------------
// Software-pipelined form: per wave, the QK^T MFMAs of tile t+1 are issued
// interleaved with the exponentials and bf16/fp16 packing of tile t, and the
// PV MFMAs of tile t interleaved with the row sums of tile t and the row
// maximum of tile t+1, so one wave's VALU work runs under its own MFMAs.  Every tile needs K
// of t+1 and V of t in LDS, so the ring is four tiles deep: tiles t, t+1 are
// read while t+2 lands and t+3 is being issued into the buffer of t-1.
// ---------------------------------------------------------------------------
constexpr int kPipeStages = 4;
// LDS operand reads run this many MFMAs ahead of their use in the QK^T and
// PV runs.
#ifndef FA_FWD_PIPE_PRE1
#define FA_FWD_PIPE_PRE1 3
#endif
#ifndef FA_FWD_PIPE_PRE2
#define FA_FWD_PIPE_PRE2 2
#endif
constexpr int kPipePre1 = FA_FWD_PIPE_PRE1, kPipePre2 = FA_FWD_PIPE_PRE2;
// Where the row sums of tile t are added: under the QK^T MFMAs of tile t+1
// beside the exponentials (0), or under the PV MFMAs of tile t beside the
// row maximum (1).  With 1 the QK^T run's vector work per MFMA (two
// exponentials, two FMAs, half a pack) fits in the MFMA's 32 cycles and the
// PV run, which had little besides the maximum, takes the adds: 2-3%
// faster at d = 128, bit-identical (the adds run in the same order).
#ifndef FA_FWD_SUM_IN_PV
#define FA_FWD_SUM_IN_PV 1
#endif
constexpr bool kSumInPv = FA_FWD_SUM_IN_PV != 0;
// Used at d = 128, where a tile's VALU work fits under its MFMAs; at d = 64
// and 32 (half and a quarter of the MFMAs per score) the plain kernel is
// faster.  FA_FWD_PIPE=0/1 forces one form for every head dimension.
#ifdef FA_FWD_PIPE
template <int D>
constexpr bool kFwdPipelined = FA_FWD_PIPE != 0;
#else
template <int D>
constexpr bool kFwdPipelined = D == 128;
#endif

// S^T of one key tile into s (lane = query, registers = keys).
template <class T, int D>
__device__ __forceinline__ void fwd_scores(const lds_char* kt, const u32x4* qf, f32x16* s, int lane) {
  constexpr int NKK = D / 16, NA = FwdCfg<D>::kNA;
#pragma unroll
  for (int a = 0; a < NA; ++a) s[a] = (f32x16){};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
    for (int a = 0; a < NA; ++a) s[a] = Elem<T>::mma(lds_rows_operand<D>(kt, 32 * a, kk, lane), qf[kk], s[a]);
}

// Keys past N, and keys outside the lane's query window, to -inf: key
// j0 + 32a + 8(r/4) + 4h + r%4 is dropped when it lies outside the query's
// [lo, hi] (hi = N - 1 without a window), compared as offsets against
// lo - j0 - 4h and hi - j0 - 4h.  The bounds pass through an empty asm
// statement so that the compares stay inside the caller's branch.
template <bool MASK, int NA>
__device__ __forceinline__ void fwd_mask(f32x16* s, int j0, int qrow, int N, Win win, int lane) {
  int rhi = (MASK ? win.hi(qrow, N) : N - 1) - j0 - 4 * (lane >> 5);
  int rlo = (MASK ? win.lo(qrow) : kUnbounded) - j0 - 4 * (lane >> 5);
  asm volatile("" : "+v"(rhi), "+v"(rlo));
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 32 * a + 8 * (r >> 2) + (r & 3);
      if (off > rhi || (MASK && win.left >= 0 && off < rlo)) s[a][r] = -INFINITY;
    }
}

// Row maximum of s in base-2 units (both lane halves).
template <int NA>
__device__ __forceinline__ float fwd_rowmax(const f32x16* s, float c) {
  float mx = s[0][0];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[a][r]);
  return max_with_partner(mx) * c;
}

// Move the reference when some row's maximum exceeds it by more than the
// slack; l and acc are rescaled with it.
template <int NB>
__device__ __forceinline__ void fwd_rescale(float mxc, f32x16* acc, float& mref, float& l) {
  if (__builtin_amdgcn_ballot_w64(mxc > mref + kRescaleSlack)) {
    const float mnew = fmaxf(mref, mxc);
    // 0 on a row's first visible tile (mref = -inf); rows with nothing
    // visible yet keep l = 0, acc = 0.
    const float alpha = mnew == -INFINITY ? 1.f : exp2_fast(mref - mnew);
    mref = mnew;
    l *= alpha;
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] *= alpha;
  }
}

// Ring layout of the pipelined kernel: the K tiles of all buffers first,
// then the V tiles, so that within each half every buffer is an immediate
// offset (under 64 KiB) from one base address.
template <int D, int IDX>
__device__ __forceinline__ void fwd_pipe_issue(lds_char* lds, int t, const DmaTile<FwdCfg<D>::kBN, D, FwdCfg<D>::kWaves>& dma,
                                               Rsrc rk, Rsrc rv, int w) {
  constexpr int TILE = FwdCfg<D>::kBN * D * 2;
  dma.issue(rk, lds + IDX * TILE, t * FwdCfg<D>::kBN, w);
  dma.issue(rv, lds + (kPipeStages + IDX) * TILE, t * FwdCfg<D>::kBN, w);
}

// Wait until tile t+1 has landed (tile t already has), allowing the DMA of
// tile t+2 to be in flight, then the workgroup barrier.
template <int PT>
__device__ __forceinline__ void pipe_wait(int t, int nt) {
  if (t + 2 < nt)
    dma_wait_barrier<PT>();
  else
    dma_wait_barrier<0>();
}

// One pipelined step: tile t in buffer IDX (its V is read), tile t+1 in
// buffer IDX+1 (its K is read); s_cur holds S^T of tile t (masked, the
// reference already moved for it), s_nxt receives S^T of tile t+1.
// The two MFMA runs are written out in issue order, each MFMA followed by
// its share of VALU work and the LDS reads for a later MFMA, with
// scheduling fences between the groups so that the compiler keeps this
// order (a wave issues VALU work while its own MFMAs execute).
template <class T, int D, bool MASK, int IDX>
__device__ __forceinline__ void fwd_pipe_step(lds_char* lds, lds_char* ldsd, int t, int nt, int ntw, int tb,
                                              const DmaTile<FwdCfg<D>::kBN, D, FwdCfg<D>::kWaves>& dma, Rsrc rk, Rsrc rv,
                                              const u32x4* qf, uint32_t* koff, uint32_t* voff,
                                              f32x16* acc, f32x16* s_cur, f32x16* s_nxt, float& mref, float& l,
                                              int wq0, int qrow, int N, Win win, float c, int w, int lane) {
  constexpr int S = kPipeStages, BN = FwdCfg<D>::kBN, TILE = BN * D * 2, NB = D / 32, NKK = D / 16, NA = FwdCfg<D>::kNA;
  pipe_wait<2 * DmaTile<FwdCfg<D>::kBN, D, FwdCfg<D>::kWaves>::PER>(t, nt);
  if (t + S - 1 < nt) fwd_pipe_issue<D, (IDX + S - 1) % S>(ldsd, tb + t + S - 1, dma, rk, rv, w);
  __builtin_amdgcn_sched_barrier(0);
  if (t >= ntw) return;  // no key from tile t on is visible to any query of the wave
  // The per-lane operand addresses (absolute: K's are relative to ring
  // buffer 0, V's to V buffer 0) are made opaque in place each step (no
  // instruction is emitted), so that the compiler does not hoist a full set
  // of per-buffer addresses out of the loop; the buffer and row-block terms
  // are then immediates folded into the read instructions' offsets, with
  // no address arithmetic left in the step.
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(koff[kk]));
#pragma unroll
  for (int x = 0; x < 2 * NB; ++x) asm volatile("" : "+v"(voff[x]));
  const lds_char* kp[NKK];
  const lds_char* vp[NB][2];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kp[kk] = (const lds_char*)(uintptr_t)koff[kk] + ((IDX + 1) % S) * TILE;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int x = 0; x < 2; ++x) vp[b][x] = (const lds_char*)(uintptr_t)voff[2 * b + x] + IDX * TILE;

  // Run 1: S^T(t+1) = K(t+1) Q^T, MFMA i = (kk = i / NA, a = i % NA), and
  // p = 2^(S(t) c - mref) and packing of tile t (with kSumInPv off, also its
  // row sums), E elements per MFMA.  K of tile t+1 is read even past the wave's (or the sequence's)
  // last tile: the buffer is in bounds and such scores are masked below.
  {
    constexpr int NM = NA * NKK, E = 16 * NA / NM, PRE = NM < kPipePre1 ? NM : kPipePre1;
    u32x4 kop[NM];
    float rs = 0.f;
    const float mr = mref == -INFINITY ? 0.f : mref;  // all of a row masked so far: p = 0
    u32x4 pf[2 * NA];
#pragma unroll
    for (int i = 0; i < PRE; ++i) kop[i] = *(const u32x4*)(kp[i / NA] + 64 * D * (i % NA));
#pragma unroll
    for (int a = 0; a < NA; ++a) s_nxt[a] = (f32x16){};
    fwd_prio_begin();
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + PRE < NM) kop[i + PRE] = *(const u32x4*)(kp[(i + PRE) / NA] + 64 * D * ((i + PRE) % NA));
      s_nxt[i % NA] = Elem<T>::mma(kop[i], qf[i / NA], s_nxt[i % NA]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int x = i * E + e, a = x / 16, r = x % 16;
        s_cur[a][r] = exp2_fast(__builtin_fmaf(s_cur[a][r], c, -mr));  // P in place
        if constexpr (!kSumInPv) rs += s_cur[a][r];
        if (r % 8 == 7) pf[x / 8] = pack8<T>(s_cur[a], (r / 8));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    fwd_prio_end();
    // Pin P (and l) here, or the compiler sinks their VALU work past the
    // branch below, away from the MFMAs it is meant to run under.
#pragma unroll
    for (int j = 0; j < 2 * NA; ++j) land(pf[j]);
    if constexpr (!kSumInPv) {
      l += rs;
      land(l);
    }

    const int j1 = (tb + t + 1) * BN;
    if ((j1 + BN > N) || (MASK && !win.all_visible(wq0, wq0 + 31, j1, j1 + BN - 1)))
      fwd_mask<MASK, NA>(s_nxt, j1, qrow, N, win, lane);
    __builtin_amdgcn_sched_barrier(0);

    // Run 2: O^T += V(t)^T P(t)^T, MFMA i = (j = i / NB, b = i % NB), and the
    // row maximum of S(t+1) and the row sums of P(t), F elements per MFMA.
    constexpr int NM2 = 2 * NA * NB, F = 16 * NA / NM2, PRE2 = NM2 < kPipePre2 ? NM2 : kPipePre2;
    u32x4 vop[NM2];
#pragma unroll
    for (int i = 0; i < PRE2; ++i)
      vop[i] = lds_cols_at<0>(vp[i % NB][0] + 32 * D * (i / NB), vp[i % NB][1] + 32 * D * (i / NB));
    float mx = -INFINITY;
    fwd_prio_begin();
#pragma unroll
    for (int i = 0; i < NM2; ++i) {
      if (i + PRE2 < NM2) {
        const int n = i + PRE2;
        vop[n] = lds_cols_at<0>(vp[n % NB][0] + 32 * D * (n / NB), vp[n % NB][1] + 32 * D * (n / NB));
      }
      acc[i % NB] = Elem<T>::mma(vop[i], pf[i / NB], acc[i % NB]);
#pragma unroll
      for (int e = 0; e < F; ++e) {
        const int x = i * F + e;
        mx = fmaxf(mx, s_nxt[x / 16][x % 16]);
        if constexpr (kSumInPv) rs += s_cur[x / 16][x % 16];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    fwd_prio_end();
    if constexpr (kSumInPv) l += rs;
    fwd_rescale<NB>(max_with_partner(mx) * c, acc, mref, l);
  }
}

template <class T, int D, int MODE>
__global__ __launch_bounds__(64 * FwdCfg<D>::kWaves, 2) void fwd_pipe_kernel(const void* __restrict__ qp,
                                                                     const void* __restrict__ kp,
                                                                     const void* __restrict__ vp,
                                                                     void* __restrict__ op, float* __restrict__ lsep,
                                                                     Geom geo, int BH, int nqb, Win win_in, float c) {
  // MODE 0: no window (full mask); 1: the causal window (-1, 0), a
  // compile-time constant so that every window test folds; 2: any window.
  constexpr bool MASK = MODE != 0;
  const Win win = MODE == 1 ? Win{-1, 0} : win_in;
  constexpr int NW = FwdCfg<D>::kWaves, S = kPipeStages, BM = 32 * NW, BN = FwdCfg<D>::kBN, NKK = D / 16, NB = D / 32;
  constexpr int TILE = BN * D * 2, BUF = 2 * TILE;
  using Dma = DmaTile<BN, D, NW>;
  constexpr int PT = 2 * Dma::PER;
  __shared__ __attribute__((aligned(16))) char smem[S * BUF];
  // The LDS base goes through an empty asm statement: with its bits unknown
  // the compiler adds (instead of ORing) constant offsets to per-lane
  // addresses and folds them into the read instructions' immediate offsets.
  uint32_t lds_base = (uint32_t)(uintptr_t)(lds_char*)smem;
  asm volatile("" : "+v"(lds_base));
  lds_char* const lds = (lds_char*)(uintptr_t)lds_base;
  // DMA destinations from the array's own address, which the compiler keeps
  // in scalar registers: M0 is then set without a v_readfirstlane (a vector
  // to scalar dependency in every copy).
  lds_char* const ldsd = (lds_char*)smem;

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
  const auto ro = make_rsrc((char*)op + head, bytes);
  const Rsrc rk = make_rsrc_words((const char*)kp + headkv, bytes);
  const Rsrc rv = make_rsrc_words((const char*)vp + headkv, bytes);

  // Key tiles tb .. tb + nt - 1 hold every key visible to the block.
  const int kbeg = MASK ? win.key_lo(q0) : 0, kend = MASK ? win.key_hi(q0 + BM - 1, N) : N;
  const int tb = kbeg / BN, nt = (kend + BN - 1) / BN - tb;
  const int wq0 = q0 + 32 * w;  // first query of this wave
  // This wave computes tiles 0 .. ntw - 1 of the block's (those past its
  // last visible key are skipped; leading tiles it cannot see are masked).
  const int ntw = MASK ? min(nt, (win.key_hi(wq0 + 31, N) + BN - 1) / BN - tb) : nt;
  Dma dma;
  dma.init(w, lane);
  fwd_pipe_issue<D, 0>(ldsd, tb, dma, rk, rv, w);

  const int qrow = wq0 + (lane & 31);  // this lane's query
  u32x4 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = bload16(rq, (uint32_t)((qrow * D + 16 * kk + 8 * h) * 2));
  uint32_t koff[NKK], voff[2 * NB];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) koff[kk] = lds_base + rows_offset<D>(kk, lane);
#pragma unroll
  for (int x = 0; x < 2 * NB; ++x) voff[x] = lds_base + S * TILE + cols_offset<D>(32 * (x / 2), x % 2, lane);
  // Q has landed (and with it tile 0) before the ring starts: no load the
  // compiler tracks may be pending inside the loop.
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) land(qf[kk]);
  if (nt > 1) fwd_pipe_issue<D, 1>(ldsd, tb + 1, dma, rk, rv, w);
  if (nt > 2) fwd_pipe_issue<D, 2>(ldsd, tb + 2, dma, rk, rv, w);
  // Tile 0 landed (waited above); tiles 1 and 2 may be in flight.
  dma_wait_barrier<63>();

  f32x16 acc[NB], sa[FwdCfg<D>::kNA], sb[FwdCfg<D>::kNA];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = (f32x16){};
  float mref = -INFINITY, l = 0.f;  // reference max (base 2) and this lane's part of the row sum
  fwd_scores<T, D>(lds, qf, sa, lane);
  {
    const int j0 = tb * BN;
    if (j0 + BN > N || (MASK && !win.all_visible(wq0, wq0 + 31, j0, j0 + BN - 1)))
      fwd_mask<MASK, FwdCfg<D>::kNA>(sa, j0, qrow, N, win, lane);
  }
  fwd_rescale<NB>(fwd_rowmax<FwdCfg<D>::kNA>(sa, c), acc, mref, l);

  for (int t = 0; t < nt; t += 4) {
    fwd_pipe_step<T, D, MASK, 0>(lds, ldsd, t, nt, ntw, tb, dma, rk, rv, qf, koff, voff, acc, sa, sb, mref, l, wq0, qrow, N, win, c, w,
                                  lane);
    if (t + 1 < nt)
      fwd_pipe_step<T, D, MASK, 1>(lds, ldsd, t + 1, nt, ntw, tb, dma, rk, rv, qf, koff, voff, acc, sb, sa, mref, l, wq0, qrow, N, win,
                                    c, w, lane);
    if (t + 2 < nt)
      fwd_pipe_step<T, D, MASK, 2>(lds, ldsd, t + 2, nt, ntw, tb, dma, rk, rv, qf, koff, voff, acc, sa, sb, mref, l, wq0, qrow, N, win,
                                    c, w, lane);
    if (t + 3 < nt)
      fwd_pipe_step<T, D, MASK, 3>(lds, ldsd, t + 3, nt, ntw, tb, dma, rk, rv, qf, koff, voff, acc, sb, sa, mref, l, wq0, qrow, N, win,
                                    c, w, lane);
  }

  const float lt = sum_with_partner(l);
  store_rows<T, D>(ro, qrow, acc, 1.0f / lt, lane);
  if (h == 0 && qrow < N) lsep[(size_t)qr0 + qrow] = (mref + log2_fast(lt)) * kLn2;
}

template <class T, int D, int MODE, int NW, int S>
__global__ __launch_bounds__(64 * NW, 2) void fwd_kernel(const void* __restrict__ qp,
                                                                const void* __restrict__ kp,
                                                                const void* __restrict__ vp, void* __restrict__ op,
                                                                float* __restrict__ lsep, Geom geo, int BH, int nqb,
                                                                Win win_in, float c) {
  // MODE 0: no window (full mask); 1: the causal window (-1, 0), a
  // compile-time constant so that every window test folds; 2: any window.
  constexpr bool MASK = MODE != 0;
  const Win win = MODE == 1 ? Win{-1, 0} : win_in;
  constexpr int BM = 32 * NW, BN = FwdCfg<D>::kBN, NKK = D / 16, NB = D / 32;
  constexpr int TILE = BN * D * 2, BUF = 2 * TILE;
  using Dma = DmaTile<BN, D, NW>;
  __shared__ __attribute__((aligned(16))) char smem[S * BUF];
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
  const auto ro = make_rsrc((char*)op + head, bytes);
  const Rsrc rk = make_rsrc_words((const char*)kp + headkv, bytes);
  const Rsrc rv = make_rsrc_words((const char*)vp + headkv, bytes);

  // Key tiles tb .. tb + nt - 1 hold every key visible to the block.
  const int kbeg = MASK ? win.key_lo(q0) : 0, kend = MASK ? win.key_hi(q0 + BM - 1, N) : N;
  const int tb = kbeg / BN, nt = (kend + BN - 1) / BN - tb;
  Dma dma;
  dma.init(w, lane);
  fwd_issue<D, 0, NW>(lds, tb, dma, rk, rv, w);

  const int qrow = q0 + 32 * w + (lane & 31);  // this lane's query
  u32x4 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = bload16(rq, (uint32_t)((qrow * D + 16 * kk + 8 * h) * 2));
  // Q has landed (and with it tile 0) before the ring starts: no load the
  // compiler tracks may be pending inside the loop.
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) land(qf[kk]);
  if (S > 2 && nt > 1) fwd_issue<D, 1 % S, NW>(lds, tb + 1, dma, rk, rv, w);
  if (S > 3 && nt > 2) fwd_issue<D, 2 % S, NW>(lds, tb + 2, dma, rk, rv, w);

  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = (f32x16){};
  float mref = -INFINITY, l = 0.f;  // reference max (base 2) and this lane's part of the row sum
  const int wq0 = q0 + 32 * w;      // first query of this wave

  for (int t = 0; t < nt; t += S) {
    fwd_step<T, D, MASK, 0, NW, S>(lds, t, nt, tb, dma, rk, rv, qf, acc, mref, l, wq0, qrow, N, win, c, w, lane);
    if (t + 1 < nt)
      fwd_step<T, D, MASK, 1, NW, S>(lds, t + 1, nt, tb, dma, rk, rv, qf, acc, mref, l, wq0, qrow, N, win, c, w, lane);
    if constexpr (S > 2)
      if (t + 2 < nt)
        fwd_step<T, D, MASK, 2 % S, NW, S>(lds, t + 2, nt, tb, dma, rk, rv, qf, acc, mref, l, wq0, qrow, N, win, c, w,
                                           lane);
    if constexpr (S > 3)
      if (t + 3 < nt)
        fwd_step<T, D, MASK, 3 % S, NW, S>(lds, t + 3, nt, tb, dma, rk, rv, qf, acc, mref, l, wq0, qrow, N, win, c, w,
                                           lane);
  }

  const float lt = sum_with_partner(l);
  store_rows<T, D>(ro, qrow, acc, 1.0f / lt, lane);
  if (h == 0 && qrow < N) lsep[(size_t)qr0 + qrow] = (mref + log2_fast(lt)) * kLn2;
}

// The plain kernel with NW waves and an S-deep ring.
template <class T, int D, int MODE, int NW, int S>
static void launch_fwd_plain(const FwdArgs& a, const Geom& geo, const Win& win, hipStream_t st) {
  const int BH = a.B * a.H, BM = 32 * NW;
  const int nqb = (a.N + BM - 1) / BM;  // a.N: the longest sequence when packed
  hipLaunchKernelGGL((fwd_kernel<T, D, MODE, NW, S>), dim3(nqb * BH), dim3(64 * NW), 0, st, a.q, a.k, a.v, a.o, a.lse,
                     geo, BH, nqb, win, a.scale * kLog2e);
}

template <class T, int D, int MODE>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  const Win win{a.wl, a.wr};
  const Geom geo{a.N, a.H, a.H / a.Hkv, a.cu, a.T};
  constexpr bool kShortIsDefault = !kFwdPipelined<D> && FwdCfg<D>::kWaves == kShortWaves &&
                                   FwdCfg<D>::kStages == kShortStages;
  const bool narrow = MODE == 2 && a.wl >= 0 && a.wr >= 0 && static_cast<long>(a.wl) + a.wr + 1 <= kNarrowWindow;
  if (!kShortIsDefault && (a.N <= kShortSeq || narrow)) {
    launch_fwd_plain<T, D, MODE, kShortWaves, kShortStages>(a, geo, win, st);
  } else if constexpr (kFwdPipelined<D>) {
    const int BM = 32 * FwdCfg<D>::kWaves;
    const int nqb = (a.N + BM - 1) / BM;
    hipLaunchKernelGGL((fwd_pipe_kernel<T, D, MODE>), dim3(nqb * BH), dim3(64 * FwdCfg<D>::kWaves), 0, st, a.q, a.k, a.v,
                       a.o, a.lse, geo, BH, nqb, win, a.scale * kLog2e);
  } else {
    launch_fwd_plain<T, D, MODE, FwdCfg<D>::kWaves, FwdCfg<D>::kStages>(a, geo, win, st);
  }
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t st) {
  switch (win_mode(a.wl, a.wr)) {
    case 0: return launch_fwd_t<T, D, 0>(a, st);
    case 1: return launch_fwd_t<T, D, 1>(a, st);
    default: return launch_fwd_t<T, D, 2>(a, st);
  }
}

template <class T>
static hipError_t launch_fwd_e(const FwdArgs& a, hipStream_t st) {
  switch (a.d) {
    case 32: return launch_fwd_d<T, 32>(a, st);
    case 64: return launch_fwd_d<T, 64>(a, st);
    default: return launch_fwd_d<T, 128>(a, st);
  }
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  return a.bf16 ? launch_fwd_e<bf16_tag>(a, st) : launch_fwd_e<f16_tag>(a, st);
}

}  // namespace fa
