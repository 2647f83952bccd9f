// Host-side launch descriptors shared by the C-ABI layer and the kernel files.
// Arguments arrive here already validated (fa_api.cpp).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct FwdArgs {
  const void *q, *k, *v;
  void* o;
  float* lse;
  int B, H, N, d;
  int Hkv;  // key/value heads; H is a multiple of Hkv
  float scale;
  int wl, wr;  // window: key j visible to query i iff i - wl <= j <= i + wr (negative: unbounded)
  bool bf16;
  const int* cu = nullptr;  // packed variable-length: B + 1 device row offsets (N = longest sequence)
  int T = 0;                // packed: total rows
};

struct PreArgs {
  const void *o, *dO;
  float* delta;
  int B, H, N, d;
  bool bf16;
};

struct BwdArgs {
  const void *q, *k, *v, *dO;
  const float *lse, *delta;
  void *dq, *dk, *dv;
  int B, H, N, d;
  int Hkv;  // key/value heads; H is a multiple of Hkv
  float scale;
  int wl, wr;  // window, as in FwdArgs
  bool bf16;
  const int* cu = nullptr;  // packed variable-length, as in FwdArgs
  int T = 0;
  // Query heads of a key/value head's group split over `splits` dK/dV
  // workgroups (splits divides H / Hkv), their float32 partial sums in
  // `part` (2 * splits * R * d floats, R = rows of the K tensor); null: no
  // split.
  float* part = nullptr;
  int splits = 1;
};

// Bytes of the static scratch array that holds the head-split partial sums
// for the backward entry point that allocates nothing: 2 * 2048 * 128 rows
// of d = 128 float32 values, the partials of a split that brings the dK/dV
// grid to its 2048-workgroup target at d = 128.
constexpr size_t kScratchBytes = size_t(256) << 20;
// Device address of the scratch array on the current device (looked up on
// the first call per device, then cached).
hipError_t scratch_region(void** base);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st);
hipError_t launch_preprocess(const PreArgs& a, hipStream_t st);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st);

}  // namespace fa
