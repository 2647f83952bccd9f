// Host-only check of the C ABI's validation and dispatch (fa_api.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer: every rejection path
// returns its status and launches nothing; accepted calls hand the
// launchers the arguments the caller gave (masks as windows, grouped heads,
// packed offsets, head splits and their workspace); extreme sizes go through
// the size arithmetic without overflow.  Pointers are fake, disjoint device
// addresses that are never dereferenced (the launchers are stubs).
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/fa.h"
#include "stub_launchers.h"

namespace {

int g_fails = 0;
int g_checks = 0;

#define EXPECT(cond)                                                    \
  do {                                                                  \
    ++g_checks;                                                         \
    if (!(cond)) {                                                      \
      std::printf("FAIL line %d: %s\n", __LINE__, #cond);               \
      ++g_fails;                                                        \
    }                                                                   \
  } while (0)

// Fake device addresses: 1 GiB apart, 256-byte aligned.
void* P(int i) { return reinterpret_cast<void*>(static_cast<uintptr_t>(0x100000000ULL + 0x40000000ULL * i)); }
float* F(int i) { return static_cast<float*>(P(i)); }
void* off(void* p, long long bytes) { return static_cast<char*>(p) + bytes; }

// A call that must be refused with `want` and launch nothing.
#define REJECT(call, want)                  \
  do {                                      \
    const int n0 = fa::g_launches;          \
    const int rc = (call);                  \
    EXPECT(rc == (want));                   \
    EXPECT(fa::g_launches == n0);           \
  } while (0)

// A call that must be accepted and launch `n` kernels.
#define ACCEPT(call, n)                     \
  do {                                      \
    const int n0 = fa::g_launches;          \
    fa::g_last = fa::Record{};              \
    const int rc = (call);                  \
    EXPECT(rc == FA_OK);                    \
    EXPECT(fa::g_launches == n0 + (n));     \
  } while (0)

void forward() {
  // fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dt, stream)
  ACCEPT(fa_fwd(P(0), P(1), P(2), P(3), F(4), 2, 3, 100, 64, 0.125f, 1, FA_BF16, nullptr), 1);
  const fa::FwdArgs& a = fa::g_last.fwd;
  EXPECT(fa::g_last.kind == 'F' && a.q == P(0) && a.k == P(1) && a.v == P(2) && a.o == P(3) && a.lse == F(4));
  EXPECT(a.B == 2 && a.H == 3 && a.Hkv == 3 && a.N == 100 && a.d == 64 && a.scale == 0.125f && a.bf16);
  EXPECT(a.wl == -1 && a.wr == 0 && a.cu == nullptr);
  ACCEPT(fa_fwd(P(0), P(1), P(2), P(3), F(4), 1, 1, 1, 32, 0.5f, 0, FA_F16, nullptr), 1);
  EXPECT(fa::g_last.fwd.wl == -1 && fa::g_last.fwd.wr == -1 && !fa::g_last.fwd.bf16);

  REJECT(fa_fwd(nullptr, P(1), P(2), P(3), F(4), 1, 1, 64, 64, 0.125f, 0, FA_BF16, nullptr), FA_ERR_INVALID_ARG);
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), nullptr, 1, 1, 64, 64, 0.125f, 0, FA_BF16, nullptr), FA_ERR_INVALID_ARG);
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), F(4), 0, 1, 64, 64, 0.125f, 0, FA_BF16, nullptr), FA_ERR_INVALID_ARG);
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), F(4), 1, -3, 64, 64, 0.125f, 0, FA_BF16, nullptr), FA_ERR_INVALID_ARG);
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), F(4), 1, 1, 0, 64, 0.125f, 0, FA_BF16, nullptr), FA_ERR_INVALID_ARG);
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 48, 0.125f, 0, FA_BF16, nullptr), FA_ERR_UNSUPPORTED);
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 64, 0.125f, 0, static_cast<fa_dtype>(7), nullptr),
         FA_ERR_INVALID_ARG);
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 64, 0.125f, 2, FA_BF16, nullptr), FA_ERR_INVALID_ARG);
  for (float bad : {0.f, -1.f, NAN, INFINITY})
    REJECT(fa_fwd(P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 64, bad, 0, FA_BF16, nullptr), FA_ERR_INVALID_ARG);
  REJECT(fa_fwd(off(P(0), 8), P(1), P(2), P(3), F(4), 1, 1, 64, 64, 0.125f, 0, FA_BF16, nullptr),
         FA_ERR_ALIGNMENT);
  REJECT(fa_fwd(P(0), P(1), P(2), P(0), F(4), 1, 1, 64, 64, 0.125f, 0, FA_BF16, nullptr), FA_ERR_ALIAS);
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), static_cast<float*>(off(P(2), 4096)), 1, 1, 64, 64, 0.125f, 0, FA_BF16,
                nullptr),
         FA_ERR_ALIAS);
  // o and lse overlapping each other
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), static_cast<float*>(off(P(3), 16)), 1, 1, 64, 64, 0.125f, 0, FA_BF16,
                nullptr),
         FA_ERR_ALIAS);
  // sizes beyond the limits: a head over the 32-bit buffer range, a grid too large, extreme ints
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), F(4), 1, 1, 1 << 24, 128, 0.125f, 0, FA_BF16, nullptr), FA_ERR_UNSUPPORTED);
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), F(4), 1 << 16, 1 << 10, 4096, 64, 0.125f, 0, FA_BF16, nullptr),
         FA_ERR_UNSUPPORTED);
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), F(4), INT_MAX, INT_MAX, INT_MAX, 128, 0.125f, 0, FA_BF16, nullptr),
         FA_ERR_UNSUPPORTED);
  REJECT(fa_fwd(P(0), P(1), P(2), P(3), F(4), INT_MIN, 1, 64, 64, 0.125f, 0, FA_BF16, nullptr), FA_ERR_INVALID_ARG);

  // grouped heads and windows
  ACCEPT(fa_fwd_gqa(P(0), P(1), P(2), P(3), F(4), 2, 8, 2, 64, 128, 0.1f, 1, FA_F16, nullptr), 1);
  EXPECT(fa::g_last.fwd.H == 8 && fa::g_last.fwd.Hkv == 2 && fa::g_last.fwd.wr == 0);
  REJECT(fa_fwd_gqa(P(0), P(1), P(2), P(3), F(4), 2, 8, 3, 64, 128, 0.1f, 1, FA_F16, nullptr), FA_ERR_INVALID_ARG);
  REJECT(fa_fwd_gqa(P(0), P(1), P(2), P(3), F(4), 2, 8, 0, 64, 128, 0.1f, 1, FA_F16, nullptr), FA_ERR_INVALID_ARG);
  ACCEPT(fa_fwd_ex(P(0), P(1), P(2), P(3), F(4), 1, 4, 4, 64, 64, 0.1f, 5, 3, FA_BF16, nullptr), 1);
  EXPECT(fa::g_last.fwd.wl == 5 && fa::g_last.fwd.wr == 3);
  REJECT(fa_fwd_ex(P(0), P(1), P(2), P(3), F(4), 1, 4, 4, 64, 64, 0.1f, -2, 0, FA_BF16, nullptr),
         FA_ERR_INVALID_ARG);
}

void varlen() {
  const int* cu = static_cast<const int*>(P(10));
  // fa_fwd_varlen(q, k, v, o, lse, cu, B, max_seqlen, T, H, Hkv, d, scale, wl, wr, dt, stream)
  ACCEPT(fa_fwd_varlen(P(0), P(1), P(2), P(3), F(4), cu, 3, 40, 100, 4, 2, 64, 0.125f, -1, 0, FA_BF16, nullptr), 1);
  EXPECT(fa::g_last.fwd.cu == cu && fa::g_last.fwd.T == 100 && fa::g_last.fwd.N == 40 && fa::g_last.fwd.B == 3);
  REJECT(fa_fwd_varlen(P(0), P(1), P(2), P(3), F(4), nullptr, 3, 40, 100, 4, 2, 64, 0.125f, -1, 0, FA_BF16,
                       nullptr),
         FA_ERR_INVALID_ARG);
  REJECT(fa_fwd_varlen(P(0), P(1), P(2), P(3), F(4), static_cast<const int*>(off(P(10), 2)), 3, 40, 100, 4, 2, 64,
                       0.125f, -1, 0, FA_BF16, nullptr),
         FA_ERR_ALIGNMENT);
  // an output over the offsets
  REJECT(fa_fwd_varlen(P(0), P(1), P(2), P(10), F(4), cu, 3, 40, 100, 4, 2, 64, 0.125f, -1, 0, FA_BF16, nullptr),
         FA_ERR_ALIAS);
  REJECT(fa_fwd_varlen(P(0), P(1), P(2), P(3), static_cast<float*>(off(P(10), -64)), cu, 3, 40, 100, 4, 2, 64,
                       0.125f, -1, 0, FA_BF16, nullptr),
         FA_ERR_ALIAS);
  // fa_bwd_varlen(q, k, v, dO, lse, delta, dq, dk, dv, cu, B, max_seqlen, T, H, Hkv, d, scale, wl, wr, dt, stream)
  ACCEPT(fa_bwd_varlen(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), cu, 3, 40, 100, 4, 2, 64, 0.125f, -1,
                       0, FA_BF16, nullptr),
         2);
  EXPECT(fa::g_last.kind == 'K' && fa::g_last.kind2 == 'Q' && fa::g_last.bwd.cu == cu && fa::g_last.bwd.T == 100);
  REJECT(fa_bwd_varlen(P(0), P(1), P(2), P(3), F(4), F(5), P(10), P(7), P(8), cu, 3, 40, 100, 4, 2, 64, 0.125f, -1,
                       0, FA_BF16, nullptr),
         FA_ERR_ALIAS);
  // workspace over the offsets (16 query heads on one key/value head: a split)
  const size_t need = fa_bwd_varlen_workspace_size(3, 40, 100, 16, 1, 64);
  EXPECT(need > 0);
  REJECT(fa_bwd_varlen_ws(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), cu, 3, 40, 100, 16, 1, 64, 0.125f,
                          -1, 0, FA_BF16, off(P(10), -4096), need, nullptr),
         FA_ERR_ALIAS);
  ACCEPT(fa_bwd_varlen_ws(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), cu, 3, 40, 100, 16, 1, 64, 0.125f,
                          -1, 0, FA_BF16, P(11), need, nullptr),
         2);
  EXPECT(fa::g_last.bwd.part == F(11) && fa::g_last.bwd.splits > 1);
}

void backward() {
  // fa_bwd_preprocess(o, dO, delta, B, H, N, d, dt, stream)
  ACCEPT(fa_bwd_preprocess(P(0), P(1), F(2), 2, 3, 50, 32, FA_F16, nullptr), 1);
  EXPECT(fa::g_last.kind == 'P' && fa::g_last.pre.B == 2 && fa::g_last.pre.H == 3 && fa::g_last.pre.N == 50 &&
         fa::g_last.pre.d == 32 && !fa::g_last.pre.bf16);
  REJECT(fa_bwd_preprocess(P(0), P(1), static_cast<float*>(off(P(1), 64)), 2, 3, 50, 32, FA_F16, nullptr),
         FA_ERR_ALIAS);
  REJECT(fa_bwd_preprocess(P(0), nullptr, F(2), 2, 3, 50, 32, FA_F16, nullptr), FA_ERR_INVALID_ARG);

  // fa_bwd(q, k, v, dO, lse, delta, dq, dk, dv, B, H, N, d, scale, causal, dt, stream)
  ACCEPT(fa_bwd(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), 2, 2, 300, 128, 0.09f, 1, FA_BF16, nullptr), 2);
  const fa::BwdArgs& b = fa::g_last.bwd;
  EXPECT(fa::g_last.kind == 'K' && fa::g_last.kind2 == 'Q');
  EXPECT(b.q == P(0) && b.dq == P(6) && b.dk == P(7) && b.dv == P(8) && b.part == nullptr && b.splits == 1);
  EXPECT(b.B == 2 && b.H == 2 && b.Hkv == 2 && b.N == 300 && b.d == 128 && b.wl == -1 && b.wr == 0 && b.bf16);
  REJECT(fa_bwd(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(6), P(8), 2, 2, 300, 128, 0.09f, 1, FA_BF16, nullptr),
         FA_ERR_ALIAS);
  REJECT(fa_bwd(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(3), 2, 2, 300, 128, 0.09f, 1, FA_BF16, nullptr),
         FA_ERR_ALIAS);
  REJECT(fa_bwd(P(0), P(1), P(2), P(3), F(4), nullptr, P(6), P(7), P(8), 2, 2, 300, 128, 0.09f, 1, FA_BF16,
                nullptr),
         FA_ERR_INVALID_ARG);
  ACCEPT(fa_bwd_dkdv(P(0), P(1), P(2), P(3), F(4), F(5), P(7), P(8), 1, 1, 64, 64, 0.125f, 0, FA_F16, nullptr), 1);
  EXPECT(fa::g_last.kind == 'K' && fa::g_last.kind2 == 0 && fa::g_last.bwd.dq == nullptr);
  ACCEPT(fa_bwd_dq(P(0), P(1), P(2), P(3), F(4), F(5), P(6), 1, 1, 64, 64, 0.125f, 0, FA_F16, nullptr), 1);
  EXPECT(fa::g_last.kind2 == 'Q' && fa::g_last.bwd_dq.dk == nullptr);

  // head-split workspace: the rule's size, a smaller one (fewer splits), none
  const size_t need = fa_bwd_workspace_size(1, 16, 1, 1000, 128);
  EXPECT(need == 2ULL * 16 * 1000 * 128 * 4);
  ACCEPT(fa_bwd_ex_ws(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), 1, 16, 1, 1000, 128, 0.09f, -1, 0,
                      FA_BF16, P(9), need, nullptr),
         2);
  EXPECT(fa::g_last.bwd.part == F(9) && fa::g_last.bwd.splits == 16);
  ACCEPT(fa_bwd_ex_ws(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), 1, 16, 1, 1000, 128, 0.09f, -1, 0,
                      FA_BF16, P(9), need / 3, nullptr),
         2);
  EXPECT(fa::g_last.bwd.splits == 4);  // the largest divisor of 16 whose partials fit a third of the rule's size
  ACCEPT(fa_bwd_ex_ws(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), 1, 16, 1, 1000, 128, 0.09f, -1, 0,
                      FA_BF16, nullptr, 0, nullptr),
         2);
  EXPECT(fa::g_last.bwd.part == nullptr && fa::g_last.bwd.splits == 1);
  REJECT(fa_bwd_ex_ws(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), 1, 16, 1, 1000, 128, 0.09f, -1, 0,
                      FA_BF16, nullptr, 16, nullptr),
         FA_ERR_INVALID_ARG);
  REJECT(fa_bwd_ex_ws(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), 1, 16, 1, 1000, 128, 0.09f, -1, 0,
                      FA_BF16, off(P(0), 1024), need, nullptr),
         FA_ERR_ALIAS);

  // the static-scratch form: the rule's split into the library's array, or FA_ERR_SCRATCH
  ACCEPT(fa_bwd_ex_scratch(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), 1, 16, 1, 1000, 128, 0.09f, -1, 0,
                           FA_BF16, nullptr),
         2);
  EXPECT(fa::g_last.bwd.part != nullptr && fa::g_last.bwd.splits == 16);
  REJECT(fa_bwd_ex_scratch(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), 1, 16, 1, 25600, 128, 0.09f, -1,
                           0, FA_BF16, nullptr),
         FA_ERR_SCRATCH);
  ACCEPT(fa_bwd_ex_scratch(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), 2, 4, 4, 1000, 64, 0.125f, -1, 0,
                           FA_F16, nullptr),
         2);
  EXPECT(fa::g_last.bwd.part == nullptr && fa::g_last.bwd.splits == 1);  // no grouping: no split, no scratch
}

void sizes_and_strings() {
  // extreme arguments go through the size rules without overflow
  EXPECT(fa_bwd_workspace_size(1, 1, 1, INT_MAX, 128) == 0);
  EXPECT(fa_bwd_workspace_size(INT_MAX, INT_MAX, 1, INT_MAX, 128) == 0 ||
         fa_bwd_workspace_size(INT_MAX, INT_MAX, 1, INT_MAX, 128) > 0);
  EXPECT(fa_bwd_varlen_workspace_size(INT_MAX, INT_MAX, INT_MAX, 16, 1, 128) == 0 ||
         fa_bwd_varlen_workspace_size(INT_MAX, INT_MAX, INT_MAX, 16, 1, 128) > 0);
  EXPECT(fa_bwd_workspace_size(0, 1, 1, 64, 64) == 0 && fa_bwd_workspace_size(1, 3, 2, 64, 64) == 0);
  EXPECT(fa_bwd_workspace_size(1, 8, 8, 64, 64) == 0);
  for (int code = -8; code <= 1; ++code) {
    const char* s = fa_status_string(code);
    EXPECT(s != nullptr && std::strlen(s) > 0);
  }
  EXPECT(fa_version() > 0);
}

}  // namespace

int main() {
  forward();
  varlen();
  backward();
  sizes_and_strings();
  std::printf("%d checks, %d failed\n", g_checks, g_fails);
  if (g_fails == 0) std::printf("ALL OK\n");
  return g_fails == 0 ? 0 : 1;
}
