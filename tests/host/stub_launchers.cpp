// Stand-ins for the kernel launchers behind the C ABI, for a host-only build
// of fa_api.cpp (no HIP runtime, no GPU) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every launch is recorded instead of run, so
// the driver can check that rejected calls launch nothing and that accepted
// calls pass the right arguments down.
#include "stub_launchers.h"

namespace fa {

Record g_last;
int g_launches = 0;

namespace {
alignas(256) unsigned char g_scratch_standin[64];
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t) {
  g_last = Record{};
  g_last.kind = 'F';
  g_last.fwd = a;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_preprocess(const PreArgs& a, hipStream_t) {
  g_last = Record{};
  g_last.kind = 'P';
  g_last.pre = a;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t) {
  g_last = Record{};
  g_last.kind = 'K';
  g_last.bwd = a;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t) {
  // the dQ launch follows dK/dV in the full backward: keep both
  if (g_last.kind != 'K') g_last = Record{};
  g_last.kind2 = 'Q';
  g_last.bwd_dq = a;
  ++g_launches;
  return hipSuccess;
}
hipError_t scratch_region(void** base) {
  *base = g_scratch_standin;
  return hipSuccess;
}

}  // namespace fa
