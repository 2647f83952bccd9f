// Instruction-rate microbenchmarks (see include/fa_probe.h).  Four loops,
// one workgroup of 512 lanes per compute unit, each writing one float per
// lane so that nothing is optimised away.
#include "../../include/fa_probe.h"

#include <hip/hip_runtime.h>

#include <algorithm>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;  // 8 waves: 2 per SIMD
constexpr int kRegs = 16;      // independent chains per lane in the VALU loops

enum Kind { kMfma = 0, kExp = 1, kFma = 2, kSoftmax = 3, kPairMfma = 4, kPairValu = 5, kPair = 6, kPairAgprMfma = 7,
            kPairAgpr = 8 };

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
        if constexpr (KIND == kPairAgprMfma || KIND == kPairAgpr)
          // The accumulator in AGPRs (the MFMA-only register file).
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[k & 3]) : "v"(a), "v"(b));
        else if constexpr (KIND != kPairValu)
          acc[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k & 3], 0, 0, 0);
        if constexpr (KIND != kPairMfma && KIND != kPairAgprMfma) {
          score_step(x, 2 * k, c, sum, mx, pk);
          score_step(x, 2 * k + 1, c, sum, mx, pk);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (KIND == kPairAgprMfma || KIND == kPairAgpr) {
      // The compiler does not see the assembly MFMAs: wait states between
      // their last result and the reads below, with every accumulator tied
      // to the statement.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
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
// LDS probes.  Every kernel of the library feeds each 32x32x16 MFMA one
// 1 KiB operand from LDS (a K, V, Q or dO tile read by the 64 lanes of a
// wave); these loops measure how fast LDS delivers such reads, alone and as
// MFMA operands, with the same 8 waves per CU.
constexpr int kLdsBytes = 32768;  // one 32 KiB buffer; lanes read 16-byte chunks, consecutive lanes adjacent
constexpr int kLdsSteps = 8;      // reads (and MFMAs) per loop iteration

enum LdsKind { kLdsRead = 0, kLdsMfma1 = 1, kLdsMfma2 = 2 };

// MFMAs from registers on CHAINS accumulators in rotation: with one, each
// MFMA takes the previous one's result as its accumulator input.
template <int CHAINS>
__global__ __launch_bounds__(kThreads) void chain_kernel(float* out, int iters) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (tid + i));
    b[i] = (__bf16)(1e-3f * (tid - i));
  }
  f32x16 acc[CHAINS] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k % CHAINS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k % CHAINS], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[c][i];
  out[blockIdx.x * kThreads + tid] = r;
}

template <int CHAINS>
hipError_t time_chain(float* out, int grid, int iters, hipStream_t st, float* best_ms) {
  hipEvent_t e0, e1;
  hipError_t err = hipEventCreate(&e0);
  if (err != hipSuccess) return err;
  if ((err = hipEventCreate(&e1)) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return err;
  }
  hipLaunchKernelGGL((chain_kernel<CHAINS>), dim3(grid), dim3(kThreads), 0, st, out, iters);  // warm-up
  float best = 1e30f;
  for (int rep = 0; rep < 3 && err == hipSuccess; ++rep) {
    err = hipEventRecord(e0, st);
    if (err == hipSuccess) {
      hipLaunchKernelGGL((chain_kernel<CHAINS>), dim3(grid), dim3(kThreads), 0, st, out, iters);
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

// Which SIMD each wave of a 512-lane workgroup runs on: the SIMD_ID field
// (bits 5:4) of the HW_ID hardware register, the CU_ID field (11:8), and the
// XCD (accelerator complex die) from the XCC_ID register (bits 3:0).
__global__ __launch_bounds__(kThreads) void wave_simd_kernel(int* out) {
  const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);  // HW_ID, all 32 bits
  unsigned xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  const int tid = threadIdx.x;
  if ((tid & 63) == 0)
    out[blockIdx.x * (kThreads / 64) + (tid >> 6)] =
        (int)((xcc & 15u) << 8 | ((hw >> 8) & 15u) << 4 | ((hw >> 4) & 3u));
}

}  // namespace

extern "C" int fa_probe_lds(double* out, int n, void* stream) {
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
  float chain_ms[2] = {0, 0};
  if (n >= 8 && err == hipSuccess) err = time_chain<1>(buf, cus, iters, st, &chain_ms[0]);
  if (n >= 8 && err == hipSuccess) err = time_chain<2>(buf, cus, iters, st, &chain_ms[1]);
  (void)hipFree(buf);
  if (err != hipSuccess) return -4;
  const double waves = (double)cus * (kThreads / 64), steps = waves * iters * kLdsSteps;
  out[0] = steps * 1024.0 / (ms[0] * 1e-3) / 1e12;            // LDS reads alone, TB/s (whole chip)
  out[1] = steps * 32768.0 / (ms[1] * 1e-3) / 1e12;           // MFMA with one 1 KiB LDS operand each, TFLOP/s
  out[2] = steps * 32768.0 / (ms[2] * 1e-3) / 1e12;           // the same with a second 1 KiB read per MFMA
  out[3] = steps * 32768.0 / (ms[3] * 1e-3) / 1e12;           // the same number of MFMAs from registers, TFLOP/s
  out[4] = cus;
  out[5] = ms[0];
  if (n >= 8) {
    out[6] = steps * 32768.0 / (chain_ms[0] * 1e-3) / 1e12;  // one dependent accumulator chain, TFLOP/s
    out[7] = steps * 32768.0 / (chain_ms[1] * 1e-3) / 1e12;  // two chains
  }
  return 0;
}

extern "C" int fa_probe_wave_simd(int* out, int n, void* stream) {
  if (!out || n < 1) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -4;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return -4;
  const int total = cus * (kThreads / 64);
  int* buf = nullptr;
  if (hipMalloc(&buf, (size_t)total * sizeof(int)) != hipSuccess) return -4;
  hipLaunchKernelGGL(wave_simd_kernel, dim3(cus), dim3(kThreads), 0, st, buf);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = hipMemcpyAsync(out, buf, (size_t)std::min(n, total) * sizeof(int), hipMemcpyDeviceToHost, st);
  if (err == hipSuccess) err = hipStreamSynchronize(st);
  (void)hipFree(buf);
  return err == hipSuccess ? std::min(n, total) : -4;
}

extern "C" int fa_probe_rates(double* out, int n, void* stream) {
  if (!out || n < 8) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -4;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return -4;
  float* buf = nullptr;
  if (hipMalloc(&buf, (size_t)cus * kThreads * sizeof(float)) != hipSuccess) return -4;
  // Iteration counts give each loop a few milliseconds.
  const int it_mfma = 20000, it_valu = 4000;
  float ms[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
  hipError_t err = time_kernel<kMfma>(buf, cus, it_mfma, st, &ms[0]);
  if (err == hipSuccess) err = time_kernel<kExp>(buf, cus, it_valu, st, &ms[1]);
  if (err == hipSuccess) err = time_kernel<kFma>(buf, cus, it_valu, st, &ms[2]);
  if (err == hipSuccess) err = time_kernel<kSoftmax>(buf, cus, it_valu, st, &ms[3]);
  if (err == hipSuccess) err = time_kernel<kPairMfma>(buf, cus, it_valu, st, &ms[4]);
  if (err == hipSuccess) err = time_kernel<kPairValu>(buf, cus, it_valu, st, &ms[5]);
  if (err == hipSuccess) err = time_kernel<kPair>(buf, cus, it_valu, st, &ms[6]);
  if (n >= 10 && err == hipSuccess) err = time_kernel<kPairAgprMfma>(buf, cus, it_valu, st, &ms[7]);
  if (n >= 10 && err == hipSuccess) err = time_kernel<kPairAgpr>(buf, cus, it_valu, st, &ms[8]);
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
  if (n >= 10) {
    out[8] = ms[7];  // the pair with AGPR accumulators: MFMA half alone, ms
    out[9] = ms[8];  //                                  both, ms
  }
  return 0;
}
