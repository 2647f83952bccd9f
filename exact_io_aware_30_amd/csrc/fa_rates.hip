// Instruction-rate loops behind the benchmark's measured ceilings (see
// fa_rates.h).  One workgroup of 512 lanes per compute unit, each loop
// writing one float per lane so that nothing is optimised away.
#include "fa_rates.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;  // 8 waves: 2 per SIMD
constexpr int kRegs = 16;      // independent chains per lane in the VALU loops

enum Kind { kMfma = 0, kExp = 1, kFma = 2, kSoftmax = 3, kPairMfma = 4, kPairValu = 5, kPair = 6 };

// One score of the forward's per-score vector sequence on chain x; every
// second score also a max3 and a bf16 pack of the pair.
__device__ __forceinline__ void score_step(float* x, int j, float c, float& sum, float& mx, unsigned& pk) {
  x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], c, -c));
  sum += x[j];
  if (j & 1) {
    mx = fmaxf(mx, fmaxf(x[j - 1], x[j]));
    pk ^= __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x[j - 1], x[j]}, bf16x2));
  }
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void probe_kernel(float* out, int iters, float c) {
  const int tid = threadIdx.x;
  float r = 0.f;
  if constexpr (KIND >= kPairMfma) {
    // The interleaved pair: per step one MFMA (on one of four accumulators)
    // and the per-score sequence of two scores, in issue order; kPairMfma
    // and kPairValu run one half of it alone.
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(1e-3f * (tid + i));
      b[i] = (__bf16)(1e-3f * (tid - i));
    }
    f32x16 acc[4] = {};
    float x[kRegs];
#pragma unroll
    for (int j = 0; j < kRegs; ++j) x[j] = -1e-3f * (tid + j);
    float sum = 0.f, mx = -1e30f;
    unsigned pk = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < kRegs / 2; ++k) {
        if constexpr (KIND != kPairValu)
          acc[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k & 3], 0, 0, 0);
        if constexpr (KIND != kPairMfma) {
          score_step(x, 2 * k, c, sum, mx, pk);
          score_step(x, 2 * k + 1, c, sum, mx, pk);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int j = 0; j < kRegs; ++j) r += x[j];
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[0][i] + acc[1][i] + acc[2][i] + acc[3][i];
    r += sum + mx + (float)(pk & 0xff);
  } else if constexpr (KIND == kMfma) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(1e-3f * (tid + i));
      b[i] = (__bf16)(1e-3f * (tid - i));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
  } else {
    float x[kRegs];
#pragma unroll
    for (int j = 0; j < kRegs; ++j) x[j] = -1e-3f * (tid + j);
    float sum = 0.f, mx = -1e30f;
    unsigned pk = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kRegs; ++j) {
        if constexpr (KIND == kExp) {
          x[j] = __builtin_amdgcn_exp2f(-__builtin_fabsf(x[j]));  // stays in (0, 1]
        } else if constexpr (KIND == kFma) {
          x[j] = __builtin_fmaf(x[j], c, -c);
        } else {
          score_step(x, j, c, sum, mx, pk);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kRegs; ++j) r += x[j];
    r += sum + mx + (float)(pk & 0xff);
  }
  out[blockIdx.x * kThreads + tid] = r;
}

template <int KIND>
hipError_t time_kernel(float* out, int grid, int iters, hipStream_t st, float* best_ms) {
  hipEvent_t e0, e1;
  hipError_t err = hipEventCreate(&e0);
  if (err != hipSuccess) return err;
  if ((err = hipEventCreate(&e1)) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return err;
  }
  hipLaunchKernelGGL((probe_kernel<KIND>), dim3(grid), dim3(kThreads), 0, st, out, iters, 0.5f);  // warm-up
  float best = 1e30f;
  for (int rep = 0; rep < 3 && err == hipSuccess; ++rep) {
    err = hipEventRecord(e0, st);
    if (err == hipSuccess) {
      hipLaunchKernelGGL((probe_kernel<KIND>), dim3(grid), dim3(kThreads), 0, st, out, iters, 0.5f);
      err = hipGetLastError();
    }
    if (err == hipSuccess) err = hipEventRecord(e1, st);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    if (err == hipSuccess) best = std::min(best, ms);
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  *best_ms = best;
  return err;
}

// ---------------------------------------------------------------------------
// LDS loops.  Every kernel of the library feeds each 32x32x16 MFMA one
// 1 KiB operand from LDS (a K, V, Q or dO tile read by the 64 lanes of a
// wave); these loops measure how fast LDS delivers such reads, alone and as
// MFMA operands, with the same 8 waves per CU.
constexpr int kLdsBytes = 32768;  // one 32 KiB buffer; lanes read 16-byte chunks, consecutive lanes adjacent
constexpr int kLdsSteps = 8;      // reads (and MFMAs) per loop iteration

enum LdsKind { kLdsRead = 0, kLdsMfma1 = 1, kLdsMfma2 = 2 };

typedef unsigned u32x4p __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ __launch_bounds__(kThreads) void lds_probe_kernel(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned char buf[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kLdsBytes / 4; i += kThreads)
    reinterpret_cast<unsigned*>(buf)[i] = 0x3c003c00u ^ (unsigned)(i * 2654435761u >> 20);
  __syncthreads();
  // Step k of wave w reads 1 KiB block (w + k) mod 32: 64 lanes x 16 bytes,
  // contiguous, so every read is free of bank conflicts.
  const unsigned base = (unsigned)(lane * 16);
  float r = 0.f;
  f32x16 acc[4] = {};
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (__bf16)(1e-3f * (tid - i));
  // The same 8 blocks every iteration (LDS has no cache, so repeated reads
  // cost the same), which keeps address arithmetic out of the loop.
  auto addr = [&](int, int k) { return base + (unsigned)(((w + k) & 31) * 1024); };
  if constexpr (KIND == kLdsRead) {
    for (int it = 0; it < iters; ++it) {
      u32x4p x[kLdsSteps];
#pragma unroll
      for (int k = 0; k < kLdsSteps; ++k) x[k] = *reinterpret_cast<const u32x4p*>(buf + addr(it, k));
      // All 8 reads in flight, then one wait: keeps every byte of each read.
      asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
    }
  } else {
    // Per iteration the 8 operand reads are issued kPre MFMAs ahead of
    // their use (scheduling groups: kPre reads, then MFMA and read pairs,
    // then the last MFMAs), the pattern of the attention kernels' MFMA runs.
    constexpr int kPre = 4;
    for (int it = 0; it < iters; ++it) {
      u32x4p x[kLdsSteps], y[kLdsSteps];
#pragma unroll
      for (int k = 0; k < kLdsSteps; ++k) {
        x[k] = *reinterpret_cast<const u32x4p*>(buf + addr(it, k));
        // kLdsMfma2: the B operand from LDS too (a second 1 KiB per MFMA).
        if constexpr (KIND == kLdsMfma2) y[k] = *reinterpret_cast<const u32x4p*>(buf + (addr(it, k) ^ 16384u));
      }
#pragma unroll
      for (int k = 0; k < kLdsSteps; ++k) {
        const bf16x8 bk = KIND == kLdsMfma2 ? __builtin_bit_cast(bf16x8, y[k]) : b;
        acc[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x[k]), bk, acc[k & 3], 0, 0, 0);
      }
      constexpr int R = KIND == kLdsMfma2 ? 2 : 1;  // reads per MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, kPre * R, 0);
#pragma unroll
      for (int k = 0; k < kLdsSteps - kPre; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kPre, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) r += acc[0][i] + acc[1][i] + acc[2][i] + acc[3][i];
  out[blockIdx.x * kThreads + tid] = r;
}

template <int KIND>
hipError_t time_lds(float* out, int grid, int iters, hipStream_t st, float* best_ms) {
  hipEvent_t e0, e1;
  hipError_t err = hipEventCreate(&e0);
  if (err != hipSuccess) return err;
  if ((err = hipEventCreate(&e1)) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return err;
  }
  hipLaunchKernelGGL((lds_probe_kernel<KIND>), dim3(grid), dim3(kThreads), 0, st, out, iters);  // warm-up
  float best = 1e30f;
  for (int rep = 0; rep < 3 && err == hipSuccess; ++rep) {
    err = hipEventRecord(e0, st);
    if (err == hipSuccess) {
      hipLaunchKernelGGL((lds_probe_kernel<KIND>), dim3(grid), dim3(kThreads), 0, st, out, iters);
      err = hipGetLastError();
    }
    if (err == hipSuccess) err = hipEventRecord(e1, st);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    if (err == hipSuccess) best = std::min(best, ms);
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  *best_ms = best;
  return err;
}

// ---------------------------------------------------------------------------
// fp32 atomic adds in the pattern a backward that accumulated dQ with
// atomics inside the dK/dV kernel would issue: one workgroup of 256 lanes
// per (128-key block, head), walking the 32-row query tiles its block sees
// under the causal mask and adding a 32 x 128 float32 tile (16 values per
// lane) into acc[head][row][128] for each.  ORDER 0: head index fastest in
// the grid (a head's blocks share an XCD under round-robin dispatch); 1: key
// block fastest (a head's blocks spread over every XCD); 2: the same
// traffic as plain load-add-store (wrong sums: the memory-only reference).
// ---------------------------------------------------------------------------
template <int ORDER>
__global__ __launch_bounds__(256) void atomic_tile_kernel(float* acc, int N, int BH, int nkb) {
  const int x = blockIdx.x;
  const int kb = ORDER == 1 ? x % nkb : x / BH, bh = ORDER == 1 ? x / nkb : x % BH;
  float* head = acc + (size_t)bh * N * 128;
  const int nt = N / 32, tid = threadIdx.x;
  for (int t = kb * 4; t < nt; ++t) {
    float* tile = head + (size_t)t * 32 * 128;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float* p = tile + i * 256 + tid;
      if constexpr (ORDER <= 1)
        unsafeAtomicAdd(p, 1.0f);
      else
        *p += 1.0f;
    }
  }
}

template <int ORDER>
hipError_t time_atomic(float* acc, int N, int BH, hipStream_t st, float* best_ms) {
  hipEvent_t e0, e1;
  hipError_t err = hipEventCreate(&e0);
  if (err != hipSuccess) return err;
  if ((err = hipEventCreate(&e1)) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return err;
  }
  const int nkb = N / 128;
  float best = 1e30f;
  for (int rep = 0; rep < 3 && err == hipSuccess; ++rep) {
    err = hipMemsetAsync(acc, 0, (size_t)BH * N * 128 * sizeof(float), st);
    if (err == hipSuccess) err = hipEventRecord(e0, st);
    if (err == hipSuccess) {
      hipLaunchKernelGGL((atomic_tile_kernel<ORDER>), dim3(nkb * BH), dim3(256), 0, st, acc, N, BH, nkb);
      err = hipGetLastError();
    }
    if (err == hipSuccess) err = hipEventRecord(e1, st);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    if (err == hipSuccess) best = std::min(best, ms);
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  *best_ms = best;
  return err;
}

// Rows whose count differs from the number of key blocks that see them
// (row r is seen by blocks 0 .. r / 128).
long count_wrong(const float* h, int N, int BH) {
  long bad = 0;
  for (long i = 0; i < (long)BH * N * 128; ++i) {
    const long row = (i / 128) % N;
    if (h[i] != (float)(row / 128 + 1)) ++bad;
  }
  return bad;
}

}  // namespace

extern "C" int fa_rates_atomic(double* out, int n, int N, int BH, void* stream) {
  if (!out || n < 8 || N < 128 || N % 128 != 0 || BH < 1 || (long)BH * N * 128 > (1L << 30)) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t count = (size_t)BH * N * 128;
  float* acc = nullptr;
  if (hipMalloc(&acc, count * sizeof(float)) != hipSuccess) return -4;
  float* host = static_cast<float*>(malloc(count * sizeof(float)));
  if (!host) {
    (void)hipFree(acc);
    return -4;
  }
  float ms[3] = {0, 0, 0};
  long bad[2] = {0, 0};
  hipError_t err = time_atomic<0>(acc, N, BH, st, &ms[0]);
  if (err == hipSuccess) err = hipMemcpyAsync(host, acc, count * sizeof(float), hipMemcpyDeviceToHost, st);
  if (err == hipSuccess) err = hipStreamSynchronize(st);
  if (err == hipSuccess) bad[0] = count_wrong(host, N, BH);
  if (err == hipSuccess) err = time_atomic<1>(acc, N, BH, st, &ms[1]);
  if (err == hipSuccess) err = hipMemcpyAsync(host, acc, count * sizeof(float), hipMemcpyDeviceToHost, st);
  if (err == hipSuccess) err = hipStreamSynchronize(st);
  if (err == hipSuccess) bad[1] = count_wrong(host, N, BH);
  if (err == hipSuccess) err = time_atomic<2>(acc, N, BH, st, &ms[2]);
  free(host);
  (void)hipFree(acc);
  if (err != hipSuccess) return -4;
  double tiles = 0;
  for (int kb = 0; kb < N / 128; ++kb) tiles += N / 32 - 4 * kb;
  const double bytes = tiles * BH * 4096.0 * 4.0;
  out[0] = bytes;            // bytes of float32 added
  out[1] = ms[0];            // atomics, a head's blocks on one XCD, ms
  out[2] = ms[1];            // atomics, a head's blocks over every XCD, ms
  out[3] = ms[2];            // the same traffic as plain read-add-write, ms
  out[4] = bytes / (ms[0] * 1e-3) / 1e12;  // TB/s of atomic adds (first ordering)
  out[5] = (double)bad[0];   // wrong sums, first ordering
  out[6] = (double)bad[1];   // wrong sums, second ordering
  out[7] = bytes / (ms[2] * 1e-3) / 1e12;  // TB/s of the plain reference
  return 0;
}

extern "C" int fa_rates_lds(double* out, int n, void* stream) {
  if (!out || n < 6) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -4;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return -4;
  float* buf = nullptr;
  if (hipMalloc(&buf, (size_t)cus * kThreads * sizeof(float)) != hipSuccess) return -4;
  const int iters = 4000;
  float ms[4] = {0, 0, 0, 0};
  hipError_t err = time_lds<kLdsRead>(buf, cus, iters, st, &ms[0]);
  if (err == hipSuccess) err = time_lds<kLdsMfma1>(buf, cus, iters, st, &ms[1]);
  if (err == hipSuccess) err = time_lds<kLdsMfma2>(buf, cus, iters, st, &ms[2]);
  if (err == hipSuccess) err = time_kernel<kMfma>(buf, cus, iters * kLdsSteps / 4, st, &ms[3]);
  (void)hipFree(buf);
  if (err != hipSuccess) return -4;
  const double waves = (double)cus * (kThreads / 64), steps = waves * iters * kLdsSteps;
  out[0] = steps * 1024.0 / (ms[0] * 1e-3) / 1e12;            // LDS reads alone, TB/s (whole chip)
  out[1] = steps * 32768.0 / (ms[1] * 1e-3) / 1e12;           // MFMA with one 1 KiB LDS operand each, TFLOP/s
  out[2] = steps * 32768.0 / (ms[2] * 1e-3) / 1e12;           // the same with a second 1 KiB read per MFMA
  out[3] = steps * 32768.0 / (ms[3] * 1e-3) / 1e12;           // the same number of MFMAs from registers, TFLOP/s
  out[4] = cus;
  out[5] = ms[0];
  return 0;
}

extern "C" int fa_rates_valu(double* out, int n, void* stream) {
  if (!out || n < 8) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -4;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return -4;
  float* buf = nullptr;
  if (hipMalloc(&buf, (size_t)cus * kThreads * sizeof(float)) != hipSuccess) return -4;
  // Iteration counts give each loop a few milliseconds.
  const int it_mfma = 20000, it_valu = 4000;
  float ms[7] = {0, 0, 0, 0, 0, 0, 0};
  hipError_t err = time_kernel<kMfma>(buf, cus, it_mfma, st, &ms[0]);
  if (err == hipSuccess) err = time_kernel<kExp>(buf, cus, it_valu, st, &ms[1]);
  if (err == hipSuccess) err = time_kernel<kFma>(buf, cus, it_valu, st, &ms[2]);
  if (err == hipSuccess) err = time_kernel<kSoftmax>(buf, cus, it_valu, st, &ms[3]);
  if (err == hipSuccess) err = time_kernel<kPairMfma>(buf, cus, it_valu, st, &ms[4]);
  if (err == hipSuccess) err = time_kernel<kPairValu>(buf, cus, it_valu, st, &ms[5]);
  if (err == hipSuccess) err = time_kernel<kPair>(buf, cus, it_valu, st, &ms[6]);
  (void)hipFree(buf);
  if (err != hipSuccess) return -4;
  const double waves = (double)cus * (kThreads / 64), lanes = (double)cus * kThreads;
  out[0] = waves * it_mfma * 4 * 32768.0 / (ms[0] * 1e-3) / 1e12;
  out[1] = lanes * it_valu * kRegs / (ms[1] * 1e-3) / 1e12;
  out[2] = lanes * it_valu * kRegs / (ms[2] * 1e-3) / 1e12;
  out[3] = lanes * it_valu * kRegs / (ms[3] * 1e-3) / 1e12;
  out[4] = cus;
  out[5] = ms[4];  // the interleaved pair: MFMA half alone, ms
  out[6] = ms[5];  //                       vector half alone, ms
  out[7] = ms[6];  //                       both, ms
  return 0;
}
