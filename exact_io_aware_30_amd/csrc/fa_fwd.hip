// Forward kernel: exact attention with the online softmax, one workgroup per
// BM query rows of one head ("flash-attn-triton" docs, "Tiling softmax is
// exact algebra" and Fig. 3 "the update, per tile"; FlashAttention-2 layout:
// queries in the outer loop, accumulator in registers, one divide after the
// loop, grid split over the sequence).
//
// Workgroup: 4 waves; wave w owns queries q0 + 32w .. q0 + 32w + 31.
// Per key tile of BN = 64 rows (K and V copied global -> LDS by buffer DMA into
// a swizzled layout, double buffered, the next tile in flight during this
// tile's math):
//   S^T = K Q^T          MFMA, A = K rows from LDS, B = Q^T kept in registers;
//                        lane l holds query l % 32 and 32 of the 64 keys
//   mask                 only on tiles that cross the diagonal or the end of N
//   m_new = max(m, rowmax S)     in-lane max, then one v_permlane32_swap
//   p = 2^(S c - m_new c), alpha = 2^((m - m_new) c), c = scale * log2(e)
//   l = alpha l + rowsum p;  acc = alpha acc
//   O^T += V^T P^T       MFMA, A = V^T by transposed LDS reads, B = P^T
//                        converted from the S^T registers in place
// After the last tile: O = acc / l, L = (m c + log2 l) ln 2.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// Rescale threshold in base-2 units: the reference maximum used for the
// exponentials is moved only when a row's maximum exceeds it by more than
// this, so p = 2^(S c - ref) stays below 2^8 and most tiles skip the
// rescale of l and acc.  O = acc / l and L = ref + log2 l hold for any
// reference, so the result is the same up to rounding.
constexpr float kRescaleSlack = 8.0f;

// One key tile for one wave: S^T, optional mask, online-softmax update, PV.
template <class T, int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void fwd_tile(const lds_char* kt, const lds_char* vt, const u32x4* qf, f32x16* acc,
                                         float& mref, float& l, int j0, int qrow, int N, float c, int lane) {
  constexpr int NKK = D / 16, NB = D / 32;
  const int h = lane >> 5;
  f32x16 s[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    s[a] = (f32x16){};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) s[a] = Elem<T>::mma(lds_rows_operand<D>(kt, 32 * a, kk, lane), qf[kk], s[a]);
  }
  if constexpr (MASK) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * a + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key >= N || (CAUSAL && key > qrow)) s[a][r] = -INFINITY;
      }
  }
  float mx = s[0][0];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[a][r]);
  const float mxc = max_with_partner(mx) * c;  // row max in base-2 units
  if (__builtin_amdgcn_ballot_w64(mxc > mref + kRescaleSlack)) {
    const float mnew = fmaxf(mref, mxc);
    const float alpha = exp2_fast(mref - mnew);  // 0 on the first tile (mref = -inf)
    mref = mnew;
    l *= alpha;
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] *= alpha;
  }
  float rs = 0.f;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(__builtin_fmaf(s[a][r], c, -mref));
      s[a][r] = p;
      rs += p;
    }
  l += rs;
  u32x4 pf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pf[j] = pack8<T>(s[j >> 1], j & 1);
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[b] = Elem<T>::mma(lds_cols_operand<D>(vt, j, 32 * b, lane), pf[j], acc[b]);
}

// One pipeline step: wait for tile t in `cur`, start the DMA of tile t + 1
// into `nxt` (every wave is past its reads of `nxt`), then the math on `cur`.
template <class T, int D, bool CAUSAL>
__device__ __forceinline__ void fwd_step(lds_char* cur, lds_char* nxt, int t, int nt, const DmaTile<64, D, 4>& dma,
                                         __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, const u32x4* qf,
                                         f32x16* acc, float& mref, float& l, int wq0, int qrow, int N, float c, int w,
                                         int lane) {
  constexpr int BN = 64, TILE = BN * D * 2;
  dma_barrier();
  if (t + 1 < nt) {
    dma.issue(rk, nxt, (t + 1) * BN, w);
    dma.issue(rv, nxt + TILE, (t + 1) * BN, w);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int j0 = t * BN;
  if (CAUSAL && j0 > wq0 + 31) return;  // every key of the tile follows every query of the wave
  if ((j0 + BN > N) || (CAUSAL && j0 + BN - 1 > wq0))
    fwd_tile<T, D, CAUSAL, true>(cur, cur + TILE, qf, acc, mref, l, j0, qrow, N, c, lane);
  else
    fwd_tile<T, D, CAUSAL, false>(cur, cur + TILE, qf, acc, mref, l, j0, qrow, N, c, lane);
}

template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const void* __restrict__ qp, const void* __restrict__ kp,
                                                  const void* __restrict__ vp, void* __restrict__ op,
                                                  float* __restrict__ lsep, int N, int BH, int nqb,
                                                  float c) {
  constexpr int BM = 128, BN = 64, NW = 4, NKK = D / 16, NB = D / 32;
  constexpr int TILE = BN * D * 2;
  // Two K/V buffers as separate objects, so that the compiler can tell the
  // tile being read from the tile being filled by DMA.
  __shared__ __attribute__((aligned(16))) char buf0[2 * TILE];
  __shared__ __attribute__((aligned(16))) char buf1[2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  const int x = blockIdx.x;
  const int qb = CAUSAL ? (nqb - 1 - x / BH) : (x / BH);
  const int bh = x % BH;
  const int q0 = qb * BM;
  const size_t head = (size_t)bh * N * D * 2;
  const uint32_t bytes = (uint32_t)N * D * 2;
  const auto rq = make_rsrc((const char*)qp + head, bytes);
  const auto rk = make_rsrc((const char*)kp + head, bytes);
  const auto rv = make_rsrc((const char*)vp + head, bytes);
  const auto ro = make_rsrc((char*)op + head, bytes);

  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int nt = (kend + BN - 1) / BN;
  DmaTile<BN, D, NW> dma;
  dma.init(w, lane);
  dma.issue(rk, (lds_char*)buf0, 0, w);
  dma.issue(rv, (lds_char*)buf0 + TILE, 0, w);

  const int qrow = q0 + 32 * w + (lane & 31);  // this lane's query
  u32x4 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = bload16(rq, (uint32_t)((qrow * D + 16 * kk + 8 * h) * 2));

  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = (f32x16){};
  float mref = -INFINITY, l = 0.f;  // reference max (base 2) and this lane's part of the row sum
  const int wq0 = q0 + 32 * w;      // first query of this wave

  for (int t = 0; t < nt; t += 2) {
    fwd_step<T, D, CAUSAL>((lds_char*)buf0, (lds_char*)buf1, t, nt, dma, rk, rv, qf, acc, mref, l, wq0, qrow, N, c,
                           w, lane);
    if (t + 1 < nt)
      fwd_step<T, D, CAUSAL>((lds_char*)buf1, (lds_char*)buf0, t + 1, nt, dma, rk, rv, qf, acc, mref, l, wq0, qrow,
                             N, c, w, lane);
  }

  const float lt = sum_with_partner(l);
  store_rows<T, D>(ro, qrow, acc, 1.0f / lt, lane);
  if (h == 0 && qrow < N) lsep[(size_t)bh * N + qrow] = (mref + log2_fast(lt)) * kLn2;
}

template <class T, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  const int nqb = (a.N + 127) / 128;
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL>), dim3(nqb * BH), dim3(256), 0, st, a.q, a.k, a.v, a.o,
                     a.lse, a.N, BH, nqb, a.scale * kLog2e);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t st) {
  return a.causal ? launch_fwd_t<T, D, true>(a, st) : launch_fwd_t<T, D, false>(a, st);
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
