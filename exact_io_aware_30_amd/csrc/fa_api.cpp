// C ABI of the attention library: argument checks, then kernel launches on
// the caller's stream.  Every check runs before anything is enqueued, so a
// rejected call has no effect.  See include/fa.h for the contract.
#include "../../include/fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "fa_launch.h"

static_assert(FA_SCRATCH_BYTES == fa::kScratchBytes, "the header's scratch size is the array's");

namespace {

// One head slice is addressed with 32-bit byte offsets; the margin keeps the
// offsets of the zero-filled rows past N (at most 255 rows) below 2^31 too.
constexpr long long kMaxHeadBytes = (1LL << 31) - (1LL << 20);
constexpr long long kMaxBlocks = 1LL << 24;           // workgroups of 256 lanes per launch

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

Range range_of(const void* p, long long bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + static_cast<uintptr_t>(bytes)};
}

int check_common(int B, int H, int N, int d, fa_dtype dt) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (dt != FA_F16 && dt != FA_BF16) return FA_ERR_INVALID_ARG;
  if (d != 32 && d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (static_cast<long long>(N) * d * 2 > kMaxHeadBytes) return FA_ERR_UNSUPPORTED;
  const long long bh = static_cast<long long>(B) * H;
  if (bh * ((N + 63) / 64) >= kMaxBlocks) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int check_scale_window(float scale, int wl, int wr) {
  if (!(std::isfinite(scale) && scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (wl < -1 || wr < -1) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// The causal flag as a window: (unbounded, 0); the full mask: (unbounded, unbounded).
bool causal_window(int causal, int* wl, int* wr) {
  if (causal != 0 && causal != 1) return false;
  *wl = -1;
  *wr = causal ? 0 : -1;
  return true;
}

// outs must not overlap each other or any of ins.
int check_alias(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

int check_heads(int H, int Hkv) {
  if (Hkv < 1 || H % Hkv != 0) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// dK/dV workgroups per launch below which the query heads that share a
// key/value head are split over several workgroups, whose float32 partial
// sums a second pass adds up: with few key/value heads the grid of key
// blocks x key/value heads alone leaves compute units idle.  Measured on
// bf16 causal backwards (d = 64, 128; Hkv = 1 .. 8): grids of about 2048
// (eight workgroups per compute unit) are within 1% of the fastest split,
// 1024 up to 3% slower, 512 up to 15%.
#ifndef FA_DKDV_SPLIT_TARGET
#define FA_DKDV_SPLIT_TARGET 2048
#endif
constexpr int kDkdvKeys = 128;  // keys per dK/dV workgroup

// Largest divisor of G below gs (1 at least).
int smaller_divisor(int G, int gs) {
  for (int x = gs - 1; x > 1; --x)
    if (G % x == 0) return x;
  return 1;
}

// Head splits for a dK/dV grid of ceil(n / 128) key blocks x B x Hkv with G
// query heads per key/value head: the smallest divisor of G that brings the
// grid to the target, G at most.
int head_splits(int B, int Hkv, int G, int n) {
  const long long base = (static_cast<long long>(n) + kDkdvKeys - 1) / kDkdvKeys * B * Hkv;
  int gs = 1;
  while (gs < G && base * gs < FA_DKDV_SPLIT_TARGET) {
    int next = gs + 1;
    while (G % next != 0) ++next;
    gs = next;
  }
  return gs;
}

// Workspace bytes of `gs` splits over R key rows of width d (dK and dV).
long long split_bytes(int gs, long long R, int d) { return gs > 1 ? 2LL * gs * R * d * 4 : 0; }

// The splits a call runs with: the rule's, reduced until its partials fit.
int fitted_splits(int B, int Hkv, int G, int n, long long R, int d, size_t workspace_bytes) {
  int gs = head_splits(B, Hkv, G, n);
  while (gs > 1 && split_bytes(gs, R, d) > static_cast<long long>(workspace_bytes)) gs = smaller_divisor(G, gs);
  return gs;
}

int check_bwd(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
              const void* dq, const void* dk, const void* dv, int B, int H, int Hkv, int N, int d, float scale,
              int wl, int wr, fa_dtype dt, bool want_dq, bool want_dkdv, const void* ws = nullptr,
              long long ws_bytes = 0) {
  if (!q || !k || !v || !dO || !lse || !delta) return FA_ERR_INVALID_ARG;
  if ((want_dq && !dq) || (want_dkdv && (!dk || !dv))) return FA_ERR_INVALID_ARG;
  int rc = check_common(B, H, N, d, dt);
  if (rc) return rc;
  if ((rc = check_heads(H, Hkv))) return rc;
  if ((rc = check_scale_window(scale, wl, wr))) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(lse) || !aligned16(delta))
    return FA_ERR_ALIGNMENT;
  if ((want_dq && !aligned16(dq)) || (want_dkdv && (!aligned16(dk) || !aligned16(dv)))) return FA_ERR_ALIGNMENT;
  const long long tb = static_cast<long long>(B) * H * N * d * 2, rb = static_cast<long long>(B) * H * N * 4;
  const long long kvb = static_cast<long long>(B) * Hkv * N * d * 2;
  const Range ins[6] = {range_of(q, tb), range_of(k, kvb), range_of(v, kvb), range_of(dO, tb), range_of(lse, rb),
                        range_of(delta, rb)};
  Range outs[4];
  int n = 0;
  if (want_dq) outs[n++] = range_of(dq, tb);
  if (want_dkdv) {
    outs[n++] = range_of(dk, kvb);
    outs[n++] = range_of(dv, kvb);
  }
  if (ws_bytes > 0) {
    if (!aligned16(ws)) return FA_ERR_ALIGNMENT;
    outs[n++] = range_of(ws, ws_bytes);
  }
  return check_alias(outs, n, ins, 6);
}

fa::BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                     const float* delta, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                     float scale, int wl, int wr, fa_dtype dt) {
  return fa::BwdArgs{q, k, v, dO, lse, delta, dq, dk, dv, B, H, N, d, Hkv, scale, wl, wr, dt == FA_BF16};
}

// Packed variable-length batches: q, o, dO, dq [H, T, d]; k, v, dk, dv
// [Hkv, T, d]; lse, delta [H, T]; sequence b at rows cu[b] .. cu[b+1] - 1.
int check_varlen(const int* cu, int B, int max_seqlen, int T, int H, int Hkv, int d, fa_dtype dt, float scale,
                 int wl, int wr) {
  if (!cu || B < 1 || max_seqlen < 1 || T < 1) return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(cu) & 3u) != 0) return FA_ERR_ALIGNMENT;
  int rc = check_common(B, H, max_seqlen, d, dt);  // per-sequence limits as for a batch of max_seqlen
  if (rc) return rc;
  if ((rc = check_heads(H, Hkv))) return rc;
  return check_scale_window(scale, wl, wr);
}

}  // namespace

extern "C" {

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens, int B,
                  int max_seqlen, int T, int H, int Hkv, int d, float scale, int window_left, int window_right,
                  fa_dtype dt, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  int rc = check_varlen(cu_seqlens, B, max_seqlen, T, H, Hkv, d, dt, scale, window_left, window_right);
  if (rc) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGNMENT;
  const long long tb = static_cast<long long>(H) * T * d * 2, rb = static_cast<long long>(H) * T * 4;
  const long long kvb = static_cast<long long>(Hkv) * T * d * 2;
  // The offsets are an input too: an output over them would be read by some
  // workgroups while others write it.
  const Range ins[4] = {range_of(q, tb), range_of(k, kvb), range_of(v, kvb),
                        range_of(cu_seqlens, (static_cast<long long>(B) + 1) * 4)};
  const Range outs[2] = {range_of(o, tb), range_of(lse, rb)};
  if ((rc = check_alias(outs, 2, ins, 4))) return rc;
  fa::FwdArgs a{q, k, v, o, lse, B, H, max_seqlen, d, Hkv, scale, window_left, window_right, dt == FA_BF16};
  a.cu = cu_seqlens;
  a.T = T;
  return hip_status(fa::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd_varlen_ws(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                     const float* delta, void* dq, void* dk, void* dv, const int* cu_seqlens, int B, int max_seqlen,
                     int T, int H, int Hkv, int d, float scale, int window_left, int window_right, fa_dtype dt,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !dO || !lse || !delta || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!workspace && workspace_bytes > 0) return FA_ERR_INVALID_ARG;
  int rc = check_varlen(cu_seqlens, B, max_seqlen, T, H, Hkv, d, dt, scale, window_left, window_right);
  if (rc) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(lse) || !aligned16(delta) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGNMENT;
  const long long tb = static_cast<long long>(H) * T * d * 2, rb = static_cast<long long>(H) * T * 4;
  const long long kvb = static_cast<long long>(Hkv) * T * d * 2;
  const int gs = fitted_splits(B, Hkv, H / Hkv, max_seqlen, static_cast<long long>(Hkv) * T, d, workspace_bytes);
  const long long used = split_bytes(gs, static_cast<long long>(Hkv) * T, d);
  if (used > 0 && !aligned16(workspace)) return FA_ERR_ALIGNMENT;
  const Range ins[7] = {range_of(q, tb), range_of(k, kvb), range_of(v, kvb), range_of(dO, tb), range_of(lse, rb),
                        range_of(delta, rb), range_of(cu_seqlens, (static_cast<long long>(B) + 1) * 4)};
  const Range outs[4] = {range_of(dq, tb), range_of(dk, kvb), range_of(dv, kvb), range_of(workspace, used)};
  if ((rc = check_alias(outs, used > 0 ? 4 : 3, ins, 7))) return rc;
  fa::BwdArgs a = bwd_args(q, k, v, dO, lse, delta, dq, dk, dv, B, H, Hkv, max_seqlen, d, scale, window_left,
                           window_right, dt);
  a.cu = cu_seqlens;
  a.T = T;
  if (gs > 1) {
    a.part = static_cast<float*>(workspace);
    a.splits = gs;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = hip_status(fa::launch_bwd_dkdv(a, st)))) return rc;
  return hip_status(fa::launch_bwd_dq(a, st));
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
                  void* dq, void* dk, void* dv, const int* cu_seqlens, int B, int max_seqlen, int T, int H, int Hkv,
                  int d, float scale, int window_left, int window_right, fa_dtype dt, void* stream) {
  return fa_bwd_varlen_ws(q, k, v, dO, lse, delta, dq, dk, dv, cu_seqlens, B, max_seqlen, T, H, Hkv, d, scale,
                          window_left, window_right, dt, nullptr, 0, stream);
}

size_t fa_bwd_workspace_size(int B, int H, int Hkv, int N, int d) {
  // 0 for any size the backward entry points refuse
  if (check_common(B, H, N, d, FA_BF16) || check_heads(H, Hkv)) return 0;
  return static_cast<size_t>(split_bytes(head_splits(B, Hkv, H / Hkv, N), static_cast<long long>(B) * Hkv * N, d));
}

size_t fa_bwd_varlen_workspace_size(int B, int max_seqlen, int T, int H, int Hkv, int d) {
  // 0 for any size the packed backward refuses
  if (T < 1 || check_common(B, H, max_seqlen, d, FA_BF16) || check_heads(H, Hkv)) return 0;
  return static_cast<size_t>(
      split_bytes(head_splits(B, Hkv, H / Hkv, max_seqlen), static_cast<long long>(Hkv) * T, d));
}


int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int d,
              float scale, int window_left, int window_right, fa_dtype dt, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  int rc = check_common(B, H, N, d, dt);
  if (rc) return rc;
  if ((rc = check_heads(H, Hkv))) return rc;
  if ((rc = check_scale_window(scale, window_left, window_right))) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGNMENT;
  const long long tb = static_cast<long long>(B) * H * N * d * 2, rb = static_cast<long long>(B) * H * N * 4;
  const long long kvb = static_cast<long long>(B) * Hkv * N * d * 2;
  const Range ins[3] = {range_of(q, tb), range_of(k, kvb), range_of(v, kvb)};
  const Range outs[2] = {range_of(o, tb), range_of(lse, rb)};
  if ((rc = check_alias(outs, 2, ins, 3))) return rc;
  const fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, Hkv, scale, window_left, window_right, dt == FA_BF16};
  return hip_status(fa::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd_dkdv_ex(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
                   void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int window_left,
                   int window_right, fa_dtype dt, void* stream) {
  const int rc = check_bwd(q, k, v, dO, lse, delta, nullptr, dk, dv, B, H, Hkv, N, d, scale, window_left,
                           window_right, dt, false, true);
  if (rc) return rc;
  const fa::BwdArgs a =
      bwd_args(q, k, v, dO, lse, delta, nullptr, dk, dv, B, H, Hkv, N, d, scale, window_left, window_right, dt);
  return hip_status(fa::launch_bwd_dkdv(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd_dq_ex(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
                 void* dq, int B, int H, int Hkv, int N, int d, float scale, int window_left, int window_right,
                 fa_dtype dt, void* stream) {
  const int rc = check_bwd(q, k, v, dO, lse, delta, dq, nullptr, nullptr, B, H, Hkv, N, d, scale, window_left,
                           window_right, dt, true, false);
  if (rc) return rc;
  const fa::BwdArgs a =
      bwd_args(q, k, v, dO, lse, delta, dq, nullptr, nullptr, B, H, Hkv, N, d, scale, window_left, window_right, dt);
  return hip_status(fa::launch_bwd_dq(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd_ex_ws(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
                 void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int window_left,
                 int window_right, fa_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace && workspace_bytes > 0) return FA_ERR_INVALID_ARG;
  int rc = check_bwd(q, k, v, dO, lse, delta, dq, dk, dv, B, H, Hkv, N, d, scale, window_left, window_right, dt,
                     true, true);
  if (rc) return rc;
  const long long R = static_cast<long long>(B) * Hkv * N;
  const int gs = fitted_splits(B, Hkv, H / Hkv, N, R, d, workspace_bytes);
  const long long used = split_bytes(gs, R, d);
  if (used > 0 && (rc = check_bwd(q, k, v, dO, lse, delta, dq, dk, dv, B, H, Hkv, N, d, scale, window_left,
                                  window_right, dt, true, true, workspace, used)))
    return rc;
  fa::BwdArgs a =
      bwd_args(q, k, v, dO, lse, delta, dq, dk, dv, B, H, Hkv, N, d, scale, window_left, window_right, dt);
  if (gs > 1) {
    a.part = static_cast<float*>(workspace);
    a.splits = gs;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = hip_status(fa::launch_bwd_dkdv(a, st)))) return rc;
  return hip_status(fa::launch_bwd_dq(a, st));
}

int fa_bwd_ex_scratch(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                      const float* delta, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                      float scale, int window_left, int window_right, fa_dtype dt, void* stream) {
  int rc = check_bwd(q, k, v, dO, lse, delta, dq, dk, dv, B, H, Hkv, N, d, scale, window_left, window_right, dt,
                     true, true);
  if (rc) return rc;
  // The split the rule asks for, as fa_bwd_ex_ws runs it with
  // fa_bwd_workspace_size bytes; rejected before anything is looked up or
  // launched when its partials exceed the static array.
  const long long R = static_cast<long long>(B) * Hkv * N;
  const int gs = head_splits(B, Hkv, H / Hkv, N);
  const long long used = split_bytes(gs, R, d);
  if (used > static_cast<long long>(fa::kScratchBytes)) return FA_ERR_SCRATCH;
  fa::BwdArgs a =
      bwd_args(q, k, v, dO, lse, delta, dq, dk, dv, B, H, Hkv, N, d, scale, window_left, window_right, dt);
  if (gs > 1) {
    void* base = nullptr;
    if ((rc = hip_status(fa::scratch_region(&base)))) return rc;
    a.part = static_cast<float*>(base);
    a.splits = gs;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = hip_status(fa::launch_bwd_dkdv(a, st)))) return rc;
  return hip_status(fa::launch_bwd_dq(a, st));
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
              void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int window_left,
              int window_right, fa_dtype dt, void* stream) {
  return fa_bwd_ex_ws(q, k, v, dO, lse, delta, dq, dk, dv, B, H, Hkv, N, d, scale, window_left, window_right, dt,
                      nullptr, 0, stream);
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
               int d, float scale, int causal, fa_dtype dt, void* stream) {
  int wl, wr;
  if (!causal_window(causal, &wl, &wr)) return FA_ERR_INVALID_ARG;
  return fa_fwd_ex(q, k, v, o, lse, B, H, Hkv, N, d, scale, wl, wr, dt, stream);
}

int fa_bwd_dkdv_gqa(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                    const float* delta, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale,
                    int causal, fa_dtype dt, void* stream) {
  int wl, wr;
  if (!causal_window(causal, &wl, &wr)) return FA_ERR_INVALID_ARG;
  return fa_bwd_dkdv_ex(q, k, v, dO, lse, delta, dk, dv, B, H, Hkv, N, d, scale, wl, wr, dt, stream);
}

int fa_bwd_dq_gqa(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
                  void* dq, int B, int H, int Hkv, int N, int d, float scale, int causal, fa_dtype dt,
                  void* stream) {
  int wl, wr;
  if (!causal_window(causal, &wl, &wr)) return FA_ERR_INVALID_ARG;
  return fa_bwd_dq_ex(q, k, v, dO, lse, delta, dq, B, H, Hkv, N, d, scale, wl, wr, dt, stream);
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
               void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
               fa_dtype dt, void* stream) {
  int wl, wr;
  if (!causal_window(causal, &wl, &wr)) return FA_ERR_INVALID_ARG;
  return fa_bwd_ex(q, k, v, dO, lse, delta, dq, dk, dv, B, H, Hkv, N, d, scale, wl, wr, dt, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, fa_dtype dt, void* stream) {
  return fa_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, scale, causal, dt, stream);
}

int fa_bwd_preprocess(const void* o, const void* dO, float* delta, int B, int H, int N, int d, fa_dtype dt,
                      void* stream) {
  if (!o || !dO || !delta) return FA_ERR_INVALID_ARG;
  int rc = check_common(B, H, N, d, dt);
  if (rc) return rc;
  if (!aligned16(o) || !aligned16(dO) || !aligned16(delta)) return FA_ERR_ALIGNMENT;
  const long long tb = static_cast<long long>(B) * H * N * d * 2, rb = static_cast<long long>(B) * H * N * 4;
  const Range ins[2] = {range_of(o, tb), range_of(dO, tb)};
  const Range outs[1] = {range_of(delta, rb)};
  if ((rc = check_alias(outs, 1, ins, 2))) return rc;
  const fa::PreArgs a{o, dO, delta, B, H, N, d, dt == FA_BF16};
  return hip_status(fa::launch_preprocess(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
                void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, fa_dtype dt, void* stream) {
  return fa_bwd_dkdv_gqa(q, k, v, dO, lse, delta, dk, dv, B, H, H, N, d, scale, causal, dt, stream);
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
              void* dq, int B, int H, int N, int d, float scale, int causal, fa_dtype dt, void* stream) {
  return fa_bwd_dq_gqa(q, k, v, dO, lse, delta, dq, B, H, H, N, d, scale, causal, dt, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, fa_dtype dt,
           void* stream) {
  return fa_bwd_gqa(q, k, v, dO, lse, delta, dq, dk, dv, B, H, H, N, d, scale, causal, dt, stream);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG:
      return "invalid argument (null pointer, size < 1, bad dtype, mask, window or scale, or H not a multiple of Hkv)";
    case FA_ERR_UNSUPPORTED: return "unsupported (head dim not 32/64/128, or sizes beyond the library limits)";
    case FA_ERR_ALIGNMENT: return "a pointer is not 16-byte aligned";
    case FA_ERR_HIP: return "the HIP runtime refused a kernel launch";
    case FA_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA_ERR_SCRATCH:
      return "the call needs more head-split scratch than the library's static array holds (pass a workspace to "
             "fa_bwd_ex_ws instead)";
    default: return "unknown status";
  }
}

int fa_version(void) { return 400; }

}  // extern "C"
