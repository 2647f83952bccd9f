// Device building blocks shared by the gfx950 attention kernels.
//
// MFMA: v_mfma_f32_32x32x16_{bf16,f16}.  Lane layouts (checked on the device):
//   A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//   B (16 x 32): lane l holds B[8 * (l / 32) + e][l % 32]
//   C (32 x 32): register r of lane l holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// The reduction index k of one MFMA may be any permutation shared by A and
// B.  The kernels use the permutation that makes a C tile, converted to
// 16-bit, directly usable as an A or B operand: within a 16-wide chunk, lane
// half h and element e stand for position 8 * (e / 4) + 4 * h + e % 4.
//
// LDS tiles are [rows][D] 16-bit, rows of D*2 bytes with no padding; the
// 16-byte chunk c of row r lives at chunk (c ^ swz(r)).  swz() is chosen so
// that both ways the kernels read a tile hit 64 distinct banks per 256 bytes:
//   * ds_read_b128 of 16 consecutive rows at one chunk (operand rows), and
//   * ds_read_b64_tr_b16 of 4 consecutive rows x 64 bytes per 32 lanes
//     (operands whose reduction index runs along the rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit format, gfx9

struct bf16_tag {};
struct f16_tag {};

template <class T>
struct Elem;

template <>
struct Elem<bf16_tag> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Two floats to two round-to-nearest-even bf16 in one dword (x low).
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x, y}, bf16x2));
  }
  static __device__ __forceinline__ float lo(unsigned u) { return __uint_as_float(u << 16); }
  static __device__ __forceinline__ float hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }
};

template <>
struct Elem<f16_tag> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x, y}, f16x2));
  }
  static __device__ __forceinline__ float lo(unsigned u) {
    return (float)__builtin_bit_cast(f16x2, u)[0];
  }
  static __device__ __forceinline__ float hi(unsigned u) {
    return (float)__builtin_bit_cast(f16x2, u)[1];
  }
};

// ---------------------------------------------------------------------------
// Where the (batch b, query head h) slice of each tensor lives, in rows of d
// elements.  Batched tensors: Q, O, dO, dQ [B, H, N, d]; K, V, dK, dV
// [B, H/G, N, d]; L, D [B, H, N].  Packed variable-length tensors (cu not
// null): [H, T, d], [H/G, T, d] and [H, T], sequence b at rows cu[b] ..
// cu[b+1] - 1 of every head.  Offsets read from cu are clamped to [0, T], so
// malformed offsets cannot address rows outside the tensors.
// ---------------------------------------------------------------------------
struct Geom {
  int N;          // batched: rows per sequence; packed: the longest sequence
  int H, G;       // query heads; query heads per key/value head
  const int* cu;  // packed: B + 1 row offsets in device memory; batched: null
  int T;          // packed: total rows
  // First row of the slice in the query-side tensors (and L, D), first row
  // in the key/value-side tensors, and its number of rows.
  __device__ __forceinline__ void slice(int b, int h, long& qrow0, long& kvrow0, int& len) const {
    if (cu) {
      const int s = min(max(cu[b], 0), T), e = min(max(cu[b + 1], s), T);
      qrow0 = (long)h * T + s;
      kvrow0 = (long)(h / G) * T + s;
      len = e - s;
    } else {
      qrow0 = ((long)b * H + h) * N;
      kvrow0 = ((long)b * (H / G) + h / G) * N;
      len = N;
    }
  }
};

// ---------------------------------------------------------------------------
// Attention window: key j is visible to query i iff i - left <= j <= i + right,
// a negative bound meaning unbounded.  The causal mask is the window
// (left, right) = (-1, 0); kernels compiled without a window (the full mask)
// skip every window test.  Every row sees its own key (the window contains
// the diagonal), so no row is ever fully masked.
// ---------------------------------------------------------------------------
constexpr int kUnbounded = -(1 << 30);  // lower key bound standing for "none"

// Kernel mask mode for a window (wl, wr): 0 none (full mask), 1 causal, 2 other.
inline int win_mode(int wl, int wr) { return (wl < 0 && wr < 0) ? 0 : (wl < 0 && wr == 0) ? 1 : 2; }

struct Win {
  int left, right;
  // Keys visible to some query of [qlo, qhi]: [key_lo, key_hi), within [0, N).
  __device__ __forceinline__ int key_lo(int qlo) const { return left < 0 ? 0 : max(0, qlo - left); }
  __device__ __forceinline__ int key_hi(int qhi, int N) const { return right < 0 ? N : min(N, qhi + right + 1); }
  // Queries that see some key of [klo, khi]: [query_lo, query_hi), within [0, N).
  __device__ __forceinline__ int query_lo(int klo) const { return right < 0 ? 0 : max(0, klo - right); }
  __device__ __forceinline__ int query_hi(int khi, int N) const { return left < 0 ? N : min(N, khi + left + 1); }
  // Every query of [qlo, qhi] sees every key of [klo, khi].
  __device__ __forceinline__ bool all_visible(int qlo, int qhi, int klo, int khi) const {
    return (left < 0 || qhi - left <= klo) && (right < 0 || khi <= qlo + right);
  }
  // Visible keys of query i: [lo(i), hi(i, N)] (inclusive; lo may be kUnbounded).
  __device__ __forceinline__ int lo(int i) const { return left < 0 ? kUnbounded : i - left; }
  __device__ __forceinline__ int hi(int i, int N) const { return right < 0 ? N - 1 : min(N - 1, i + right); }
};

// ---------------------------------------------------------------------------
// Buffer resources: a head slice [N, D] addressed with byte offsets.  Loads
// past num_records return zero and stores past it are dropped, which is how
// the ragged tail (rows >= N) is zero-filled on load and never written.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// Sign bits of the two 16-bit elements in each dword (fp16 and bf16 alike):
// XOR negates every element exactly.
constexpr u32x4 kSignBits16 = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Swizzled LDS tile of ROWS x D 16-bit elements.
// ---------------------------------------------------------------------------
template <int D>
struct Swz {
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "D must be 32, 64 or 128");
  static __device__ __forceinline__ int f(int r) {
    if constexpr (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else if constexpr (CPR == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return (r >> 2) & 3;
  }
  // Byte offset of 16-byte chunk c of row r.
  static __device__ __forceinline__ int chunk(int r, int c) { return (r * CPR + (c ^ f(r))) << 4; }
  // Byte offset of element column col (multiple of 4) of row r, for 8-byte reads.
  static __device__ __forceinline__ int elem4(int r, int col) {
    return chunk(r, col >> 3) + ((col & 4) << 1);
  }
};

// Operand with rows along the MFMA M/N index: lane l reads row (row0 + l % 32),
// 8 elements starting at column 16 * kk + 8 * (l / 32).
template <int D>
__device__ __forceinline__ u32x4 lds_rows_operand(const lds_char* tile, int row0, int kk, int lane) {
  const int r = row0 + (lane & 31);
  const int c = 2 * kk + (lane >> 5);
  return *(const u32x4*)(tile + Swz<D>::chunk(r, c));
}

__device__ __forceinline__ u32x2 ds_read_tr16(const lds_char* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Operand whose reduction index runs along the tile rows: lane l gets column
// (col0 + l % 32) and the 8 rows of 16-row chunk kc in the permuted order
// (rows 16kc + 4h + 0..3, then 16kc + 8 + 4h + 0..3, h = l / 32).
// ds_read_b64_tr_b16 works on 16-lane groups: lane t of a group names row
// (base + t / 4) and 4 columns starting at 4 * (t % 4); after the transpose
// lane i of the group holds column i of those 4 rows.
template <int D>
__device__ __forceinline__ u32x4 lds_cols_operand(const lds_char* tile, int kc, int col0, int lane) {
  const int g = lane >> 4, t = lane & 15, h = lane >> 5;
  const int col = col0 + 16 * (g & 1) + 4 * (t & 3);
  const int r0 = 16 * kc + 4 * h + (t >> 2);
  u32x2 a = ds_read_tr16(tile + Swz<D>::elem4(r0, col));
  u32x2 b = ds_read_tr16(tile + Swz<D>::elem4(r0 + 8, col));
  return (u32x4){a.x, a.y, b.x, b.y};
}

// The same two operands through per-lane byte offsets computed once.  The
// swizzle depends only on a row's index modulo 16, so moving the first row
// by a multiple of 16 moves every lane's address by the same amount: a rows
// operand of row block 32a is rows_offset(kk) + 32a * 2D bytes from the tile,
// and a cols operand of row chunk kc is cols_offset(col0, half) + kc * 32D
// bytes.  Kernels add the per-lane offsets to a tile base once per tile and
// let the row-block terms fold into the read instructions' immediates.
template <int D>
__device__ __forceinline__ uint32_t rows_offset(int kk, int lane) {
  return (uint32_t)Swz<D>::chunk(lane & 31, 2 * kk + (lane >> 5));
}
template <int D>
__device__ __forceinline__ uint32_t cols_offset(int col0, int half, int lane) {
  const int g = lane >> 4, t = lane & 15, h = lane >> 5;
  return (uint32_t)Swz<D>::elem4(4 * h + (t >> 2) + 8 * half, col0 + 16 * (g & 1) + 4 * (t & 3));
}
// Reads at p + OFF (a compile-time byte offset).
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16_at(const lds_char* p) {
  return *(const u32x4*)(p + OFF);
}
template <int OFF>
__device__ __forceinline__ u32x4 lds_cols_at(const lds_char* p0, const lds_char* p1) {
  u32x2 a = ds_read_tr16(p0 + OFF);
  u32x2 b = ds_read_tr16(p1 + OFF);
  return (u32x4){a.x, a.y, b.x, b.y};
}

// ---------------------------------------------------------------------------
// Global -> LDS copies without registers: buffer_load_dword{,x4} ... lds.  One
// instruction moves 64 lanes x 4 or 16 bytes; lane l's bytes land at LDS
// M0 + l * size, so a wave fills a contiguous LDS range and each lane chooses
// the global chunk that belongs in its slot.  Lanes past num_records write
// zeros.  The loads are issued from inline assembly on purpose: the compiler
// then does not track them, and all waiting for them is explicit (counted
// vmcnt waits before the workgroup barrier of a multi-buffer ring) instead of
// the compiler's conservative vmcnt(0) before every LDS read, which would wait
// for the prefetch of later tiles too.  Kernels must therefore have no
// compiler-tracked vector-memory load pending inside the ring loop.
// ---------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));
struct Rsrc {
  i32x4 v;  // buffer resource words: base lo, base hi | stride 0, num_records, format
};
__device__ __forceinline__ Rsrc make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  Rsrc r;
  r.v = (i32x4){(int)__builtin_amdgcn_readfirstlane((uint32_t)a),
                (int)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu),
                (int)__builtin_amdgcn_readfirstlane(bytes), (int)kRsrcWord3};
  return r;
}
// M0 is saved and restored around each copy; one wait state separates the
// M0 write from the load that reads it.
__device__ __forceinline__ void dma16(Rsrc src, lds_char* dst, uint32_t voffset) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voffset), "s"(src.v)
      : "memory");
}
__device__ __forceinline__ void dma4(Rsrc src, lds_char* dst, uint32_t voffset) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voffset), "s"(src.v)
      : "memory");
}

// Force a value loaded from memory to have landed (the compiler waits for its
// load before this point); used to drain compiler-tracked loads before a
// DMA ring loop.
template <class V>
__device__ __forceinline__ void land(const V& v) {
  asm volatile("" ::"v"(v));
}

template <int ROWS, int D, int NW>
struct DmaTile {
  static constexpr int CPR = D / 8;
  static constexpr int SLOTS = ROWS * CPR;
  static constexpr int NI = SLOTS / 64;              // wave-instructions per tile
  static constexpr int PER = (NI + NW - 1) / NW;     // per wave (waves past NI issue fewer)
  static_assert(SLOTS % 64 == 0, "tile must be a whole number of 1 KiB DMA instructions");
  // Every wave issues either PER or no instructions per tile, so a counted
  // vmcnt wait based on PER is exact for the waves that issue any.
  static_assert(NI % NW == 0 || NI < NW, "uneven DMA split");
  uint32_t off[PER];  // per-lane byte offset of its chunk relative to the tile's first row
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int slot = (i * NW + w) * 64 + lane;
      const int r = (slot / CPR) % ROWS, p = slot % CPR;
      off[i] = (uint32_t)((r * D + 8 * (p ^ Swz<D>::f(r))) * 2);
    }
  }
  // Enqueue the tile whose first row is row0 (the row offset is added per
  // lane so that the out-of-range check sees the full offset).  With an even
  // split the per-wave test is false at compile time: no branches.
  __device__ __forceinline__ void issue(Rsrc src, lds_char* tile, int row0, int w) const {
    const uint32_t base = (uint32_t)(row0 * D * 2);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (NI % NW == 0 || i * NW + w < NI) dma16(src, tile + (i * NW + w) * 1024, base + off[i]);
  }
};

// s_waitcnt vmcnt(N) lgkmcnt(0), expcnt left alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier for the DMA ring: this wave's DMA instructions older than
// its last N have landed in LDS and its LDS reads are done, then every wave
// arrives.  Unlike __syncthreads() there is no memory fence, which would wait
// for all outstanding DMA (vmcnt(0)) and defeat the ring.  The empty asm
// statements keep the compiler from moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void dma_wait_barrier() {
  asm volatile("" ::: "memory");
  wait_vmcnt_lgkm0<N>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Ring of S LDS buffers fed by DMA: before working on tile t a wave waits
// until at most its DMA instructions for tiles t+1 .. t+S-2 are in flight
// (PT instructions per tile), then the workgroup barrier.  After it, tile t
// is in LDS for every wave and every wave is done with tile t - 1, whose
// buffer can receive tile t + S - 1.
template <int S, int PT>
__device__ __forceinline__ void ring_wait(int t, int nt) {
  static_assert(S >= 2 && S <= 4, "ring depth");
  if constexpr (S == 2) {
    dma_wait_barrier<0>();
  } else if constexpr (S == 3) {
    if (t + 1 < nt)
      dma_wait_barrier<PT>();
    else
      dma_wait_barrier<0>();
  } else {
    if (t + 2 < nt)
      dma_wait_barrier<2 * PT>();
    else if (t + 1 < nt)
      dma_wait_barrier<PT>();
    else
      dma_wait_barrier<0>();
  }
}

// Scheduling hints for a straight run of MFMAs that each consume RPM LDS
// reads: the scheduler keeps PRE MFMAs' worth of reads issued ahead of the
// MFMA that uses them, so LDS latency overlaps earlier MFMAs instead of
// stalling each one.  Masks: 0x008 MFMA, 0x100 LDS read, 0x002 VALU.
template <int NM, int RPM, int PRE, int SYNC = 0>
__device__ __forceinline__ void sched_mfma_lds() {
  static_assert(PRE <= NM, "prefetch depth");
  __builtin_amdgcn_sched_group_barrier(0x100, PRE * RPM, SYNC);
#pragma unroll
  for (int i = 0; i < NM - PRE; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, SYNC);
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, SYNC);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PRE, SYNC);
}

// Same, for a run of NM MFMAs that consume TR LDS reads in all (spread
// evenly over the MFMAs), with PRE reads issued ahead of the first MFMA.
template <int NM, int TR, int PRE, int I, int DONE>
__device__ __forceinline__ void sched_mfma_reads_tail() {
  if constexpr (I < NM) {
    constexpr int want = PRE + ((I + 1) * TR) / NM;
    constexpr int tgt = want < TR ? want : TR;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (tgt > DONE) __builtin_amdgcn_sched_group_barrier(0x100, tgt - DONE, 0);
    sched_mfma_reads_tail<NM, TR, PRE, I + 1, (tgt > DONE ? tgt : DONE)>();
  }
}
template <int NM, int TR, int PRE>
__device__ __forceinline__ void sched_mfma_reads() {
  static_assert(PRE <= TR, "prefetch depth");
  __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
  sched_mfma_reads_tail<NM, TR, PRE, 0, PRE>();
}

// Wave priority around an MFMA run: while its MFMAs issue, a wave wins issue
// arbitration over a wave that is in its VALU phase on the same SIMD.  The
// scheduling fences keep the priority changes where they are written.
#ifndef FA_SETPRIO
#define FA_SETPRIO 1
#endif
__device__ __forceinline__ void prio_mfma_begin_always() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void prio_mfma_end_always() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void prio_mfma_begin() {
  if constexpr (FA_SETPRIO != 0) prio_mfma_begin_always();
}
__device__ __forceinline__ void prio_mfma_end() {
  if constexpr (FA_SETPRIO != 0) prio_mfma_end_always();
}

// Value of x in lane l ^ 32, combined with x: returns {x_own, x_partner} as
// the two halves of v_permlane32_swap (order depends on the lane half).
__device__ __forceinline__ float max_with_partner(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Pack the 8 C-registers c[8*j .. 8*j+7] into an A/B operand (see header).
template <class T>
__device__ __forceinline__ u32x4 pack8(const f32x16& c, int j) {
  return (u32x4){Elem<T>::pack2(c[8 * j + 0], c[8 * j + 1]), Elem<T>::pack2(c[8 * j + 2], c[8 * j + 3]),
                 Elem<T>::pack2(c[8 * j + 4], c[8 * j + 5]), Elem<T>::pack2(c[8 * j + 6], c[8 * j + 7])};
}

// Store a wave's [32 rows x D] fp32 result held with lane = row (C tiles of
// the transposed product: register r of tile b is column 32b + 8(r/4) +
// 4h + r%4) as 16-bit rows of a [N, D] slice, scaled by `mul`.
template <class T, int D>
__device__ __forceinline__ void store_rows(__amdgpu_buffer_rsrc_t dst, int row, const f32x16* acc,
                                           float mul, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * b + 8 * g + 4 * h;
      u32x2 v = {Elem<T>::pack2(acc[b][4 * g + 0] * mul, acc[b][4 * g + 1] * mul),
                 Elem<T>::pack2(acc[b][4 * g + 2] * mul, acc[b][4 * g + 3] * mul)};
      bstore8(dst, (uint32_t)((row * D + col) * 2), v);
    }
}

// The same rows kept in float32 (partial sums that a later pass adds up).
template <int D>
__device__ __forceinline__ void store_rows_f32(__amdgpu_buffer_rsrc_t dst, int row, const f32x16* acc, int lane) {
  const int h = lane >> 5;
  // The element is taken by value first: a bit cast applied directly to a
  // vector-element expression reads the vector's first element.
  auto bits = [](float x) { return __builtin_bit_cast(uint32_t, x); };
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * b + 8 * g + 4 * h;
      const u32x4 v = {bits(acc[b][4 * g + 0]), bits(acc[b][4 * g + 1]), bits(acc[b][4 * g + 2]),
                       bits(acc[b][4 * g + 3])};
      bstore16(dst, (uint32_t)((row * D + col) * 4), v);
    }
}

}  // namespace fa
