/*
 * fa.h -- C ABI of the MI355X (gfx950) exact FlashAttention-2 library.
 *
 * The operation is exact softmax attention O = softmax(scale * Q K^T [+ causal
 * mask]) V and its gradient, computed tile by tile without the N x N score
 * matrix ever reaching device memory ("flash-attn-triton" docs, spec sheet and
 * "Tiling softmax is exact algebra"; "flash attention" note, "Key
 * Mechanisms").
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * Tensors      Q, K, V, O, dO, dQ, dK, dV: device pointers to contiguous
 *              [B, H, N, d] arrays (d fastest, then N, then H, then B) of the
 *              element type `dt`.  L (lse) and D (delta): device pointers to
 *              contiguous [B, H, N] float32 arrays.
 * Sizes        B, H, N >= 1; d in {32, 64, 128}; N * d * 2 <= 2^31 - 2^20
 *              (one head slice is addressed with 32-bit byte offsets);
 *              B * H * ceil(N / 64) < 2^24.  N need not be a multiple of any
 *              tile size.  Larger sizes return FA_ERR_UNSUPPORTED.
 * Mask         causal = 0: every key is visible to every query.  causal = 1:
 *              key j is visible to query i iff j <= i ("flash attention"
 *              note, "Key Mechanisms": lower-triangular causal mask).
 * Scale        scale > 0 and finite; the caller passes 1/sqrt(d) for the
 *              usual attention ("flash-attn-triton" docs, "The argument").
 * Alignment    every pointer 16-byte aligned.
 * Ownership    the caller allocates and owns every buffer, workspaces
 *              included.  The library allocates no device memory, keeps no
 *              mutable global state and may be called from several host
 *              threads.
 * Streams      `stream` is a hipStream_t (NULL = the default stream).  Every
 *              call only enqueues kernels on that stream and returns; nothing
 *              synchronises.  Outputs are valid once the stream reaches them.
 * Errors       arguments are checked before anything is enqueued; a failed
 *              check returns a negative FA_ERR_* code and enqueues nothing.
 *              FA_ERR_HIP means a kernel launch was refused by the runtime.
 *              Faults during execution surface at the caller's next
 *              synchronisation as HIP errors.  Outputs must not overlap
 *              inputs or each other (FA_ERR_ALIAS).
 * Determinism  no atomics: repeated calls on the same inputs give the same bits
 *              (the workspace forms: with the same workspace size).
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad mask/window/scale/dtype, bad Hkv */
  FA_ERR_UNSUPPORTED = -2, /* head dim not in {32,64,128}, or sizes beyond the limits above */
  FA_ERR_ALIGNMENT = -3,   /* a pointer is not 16-byte aligned */
  FA_ERR_HIP = -4,         /* the HIP runtime refused a launch */
  FA_ERR_ALIAS = -5,       /* an output overlaps an input or another output */
  FA_ERR_SCRATCH = -6      /* fa_bwd_ex_scratch: the split needs more than FA_SCRATCH_BYTES */
};

/*
 * fa_fwd -- forward pass ("flash-attn-triton" docs, Fig. 3 "the update, per
 * tile", and "Tiling softmax is exact algebra").
 *   in : q, k, v  [B,H,N,d] of dt
 *   out: o        [B,H,N,d] of dt, o = softmax(scale*q k^T, masked) v,
 *                 rounded to nearest even
 *        lse      [B,H,N] float32, lse_i = log(sum_j exp(scale*q_i.k_j)) over
 *                 the keys visible to query i (natural logarithm).  This is
 *                 the only state the backward needs besides the inputs.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, fa_dtype dt,
           void* stream);

/*
 * fa_bwd_preprocess -- the delta pre-pass of the backward ("flash-attn-triton"
 * docs, "Where things live": delta pre-pass, then dK/dV and dQ).
 *   in : o, dO    [B,H,N,d] of dt (o as written by fa_fwd)
 *   out: delta    [B,H,N] float32, delta_i = sum_k dO_ik * o_ik (fp32 sum)
 */
int fa_bwd_preprocess(const void* o, const void* dO, float* delta,
                      int B, int H, int N, int d, fa_dtype dt, void* stream);

/*
 * fa_bwd -- backward pass: rebuilds P from lse and produces dQ, dK, dV
 * ("flash-attn-triton" docs, "Scope": backward kernels for dQ, dK, dV
 * rebuilding P from the saved L; "flash attention" note, "Key Mechanisms":
 * backward recomputation).  Enqueues fa_bwd_dkdv then fa_bwd_dq.
 *   in : q, k, v, dO   [B,H,N,d] of dt
 *        lse           [B,H,N] float32 from fa_fwd (same q, k, scale, causal)
 *        delta         [B,H,N] float32 from fa_bwd_preprocess
 *   out: dq, dk, dv    [B,H,N,d] of dt, the gradients of sum(dO * o) with
 *                      respect to q, k, v:
 *                        P = exp(scale*q k^T - lse), masked entries 0
 *                        dv = P^T dO;  dP = dO v^T;  dS = P * (dP - delta)
 *                        dq = scale * dS k;  dk = scale * dS^T q
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* dO,
           const float* lse, const float* delta, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal, fa_dtype dt,
           void* stream);

/* fa_bwd_dkdv -- the first half of fa_bwd: dk and dv only (key-block outer
 * loop over query blocks).  Same arguments and rules as fa_bwd. */
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                const float* lse, const float* delta, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal,
                fa_dtype dt, void* stream);

/* fa_bwd_dq -- the second half of fa_bwd: dq only (query-block outer loop
 * over key blocks).  Same arguments and rules as fa_bwd. */
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
              const float* lse, const float* delta, void* dq,
              int B, int H, int N, int d, float scale, int causal,
              fa_dtype dt, void* stream);

/*
 * Grouped-query forms ("flash attention" note, "Versions and Evolution":
 * FlashAttention-2 added multi-query and grouped-query attention;
 * "flash-attn-triton" docs, "Scope", lists MQA/GQA as not yet done there).
 * Hkv key/value heads serve H query heads, H a multiple of Hkv: query head h
 * of a batch attends with key/value head h / (H / Hkv) of the same batch.
 *   q, o, dO, dq   [B,H,N,d] of dt;    k, v, dk, dv   [B,Hkv,N,d] of dt;
 *   lse, delta     [B,H,N] float32.
 * The operation is that of the plain entry points with k and v repeated
 * H / Hkv times along the head axis; dk and dv are the sums of the
 * gradients over the query heads that share them.  Hkv = H is exactly
 * fa_fwd / fa_bwd*; Hkv = 1 is multi-query attention.  Hkv < 1 or H not a
 * multiple of Hkv returns FA_ERR_INVALID_ARG.  Everything else (sizes,
 * masks, alignment, aliasing, streams, errors, determinism) is as above;
 * the pre-pass is fa_bwd_preprocess on the query heads.
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Hkv, int N, int d, float scale, int causal,
               fa_dtype dt, void* stream);
int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* dO,
               const float* lse, const float* delta, void* dq, void* dk,
               void* dv, int B, int H, int Hkv, int N, int d, float scale,
               int causal, fa_dtype dt, void* stream);
int fa_bwd_dkdv_gqa(const void* q, const void* k, const void* v,
                    const void* dO, const float* lse, const float* delta,
                    void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                    float scale, int causal, fa_dtype dt, void* stream);
int fa_bwd_dq_gqa(const void* q, const void* k, const void* v, const void* dO,
                  const float* lse, const float* delta, void* dq, int B,
                  int H, int Hkv, int N, int d, float scale, int causal,
                  fa_dtype dt, void* stream);

/*
 * Windowed forms (sliding-window or local attention; "flash-attn-triton"
 * docs, "Scope", lists sliding windows as not yet done there): key j is
 * visible to query i iff i - window_left <= j <= i + window_right, -1 meaning
 * no bound on that side.  (-1, 0) is the causal mask, (-1, -1) the full one;
 * every window contains the diagonal, so no row is ever fully masked.
 * Grouped heads as in the _gqa forms (Hkv = H for plain attention).
 * window_left or window_right below -1 returns FA_ERR_INVALID_ARG; everything
 * else as above.  lse and delta are over each query's visible keys.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Hkv, int N, int d, float scale,
              int window_left, int window_right, fa_dtype dt, void* stream);
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* dO,
              const float* lse, const float* delta, void* dq, void* dk,
              void* dv, int B, int H, int Hkv, int N, int d, float scale,
              int window_left, int window_right, fa_dtype dt, void* stream);
int fa_bwd_dkdv_ex(const void* q, const void* k, const void* v,
                   const void* dO, const float* lse, const float* delta,
                   void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                   float scale, int window_left, int window_right,
                   fa_dtype dt, void* stream);
int fa_bwd_dq_ex(const void* q, const void* k, const void* v, const void* dO,
                 const float* lse, const float* delta, void* dq, int B, int H,
                 int Hkv, int N, int d, float scale, int window_left,
                 int window_right, fa_dtype dt, void* stream);

/*
 * Variable-length batches (packed sequences; "flash-attn-triton" docs,
 * "Scope", lists variable-length batches as not yet done there).  The B
 * sequences are packed along the row axis of head-major tensors:
 *   q, o, dO, dq   [H, T, d] of dt;  k, v, dk, dv  [Hkv, T, d] of dt;
 *   lse, delta     [H, T] float32;
 *   cu_seqlens     device pointer to B + 1 int32 row offsets: sequence b is
 *                  rows cu_seqlens[b] .. cu_seqlens[b+1] - 1 of every head,
 *                  cu_seqlens[0] = 0, nondecreasing, cu_seqlens[B] = T, every
 *                  length <= max_seqlen.
 * Each sequence is attended on its own (positions, windows and the causal
 * mask are relative to its first row); the result equals the batched entry
 * points applied to every sequence separately.  Offsets are read on the
 * device and clamped to [0, T], so malformed offsets never address rows
 * outside the tensors, but give unspecified results (so do lengths above
 * max_seqlen); empty sequences are allowed.  Per-sequence size limits are
 * those of a batch of max_seqlen rows.  The pre-pass is fa_bwd_preprocess
 * with B = 1, H, N = T.  Null cu_seqlens, B, max_seqlen or T below 1 return
 * FA_ERR_INVALID_ARG; a cu_seqlens not 4-byte aligned FA_ERR_ALIGNMENT.
 * cu_seqlens is an input: an output or workspace that overlaps its B + 1
 * offsets returns FA_ERR_ALIAS.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                  float* lse, const int* cu_seqlens, int B, int max_seqlen,
                  int T, int H, int Hkv, int d, float scale, int window_left,
                  int window_right, fa_dtype dt, void* stream);
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* dO,
                  const float* lse, const float* delta, void* dq, void* dk,
                  void* dv, const int* cu_seqlens, int B, int max_seqlen,
                  int T, int H, int Hkv, int d, float scale, int window_left,
                  int window_right, fa_dtype dt, void* stream);

/*
 * Workspace forms of the backward, for few key/value heads (multi-query and
 * grouped-query attention with small Hkv).  The dK/dV kernel runs one
 * workgroup per block of 128 keys of each key/value head, which loops over
 * the H / Hkv query heads that share it; with few key/value heads that grid
 * leaves compute units idle.  With a workspace the query heads of a group
 * are split over S workgroups (S divides H / Hkv), each of which writes
 * float32 partial sums of dK and dV into the workspace; a second kernel adds
 * the S partials in a fixed order (split 0 first) and rounds them to dt.
 * The operation and every rule are those of fa_bwd_ex and fa_bwd_varlen
 * (the head axis of the gradient sums is the grouped-query form's, "flash
 * attention" note, "Versions and Evolution"), plus:
 *   workspace        device pointer, 16-byte aligned when used, owned by the
 *                    caller; nothing in it is read before this call writes
 *                    it (no clearing needed); it must not overlap any
 *                    argument (FA_ERR_ALIAS).  Calls that share a workspace
 *                    must be ordered on one stream.
 *   workspace_bytes  its size.  The library takes S from its own rule (the
 *                    smallest divisor of H / Hkv that brings the dK/dV grid
 *                    to 2048 workgroups), then lowers S to the largest
 *                    divisor that fits 2 * S * R * d * 4 bytes, R being the
 *                    rows of the K tensor (B * Hkv * N batched, Hkv * T
 *                    packed); S = 1 uses no workspace and gives the bits of
 *                    the form without it.  NULL with workspace_bytes > 0 is
 *                    FA_ERR_INVALID_ARG.
 * dQ does not depend on S; dK and dV are deterministic for a given S.
 *
 * fa_bwd_workspace_size / fa_bwd_varlen_workspace_size return the bytes the
 * rule asks for (0 when no split applies, including H = Hkv, or when the
 * sizes are invalid); they touch no device.
 */
int fa_bwd_ex_ws(const void* q, const void* k, const void* v, const void* dO,
                 const float* lse, const float* delta, void* dq, void* dk,
                 void* dv, int B, int H, int Hkv, int N, int d, float scale,
                 int window_left, int window_right, fa_dtype dt,
                 void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_varlen_ws(const void* q, const void* k, const void* v,
                     const void* dO, const float* lse, const float* delta,
                     void* dq, void* dk, void* dv, const int* cu_seqlens,
                     int B, int max_seqlen, int T, int H, int Hkv, int d,
                     float scale, int window_left, int window_right,
                     fa_dtype dt, void* workspace, size_t workspace_bytes,
                     void* stream);
size_t fa_bwd_workspace_size(int B, int H, int Hkv, int N, int d);
size_t fa_bwd_varlen_workspace_size(int B, int max_seqlen, int T, int H,
                                    int Hkv, int d);

/*
 * fa_bwd_ex_scratch -- fa_bwd_ex_ws without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The head-split partial
 * sums go to a static device array of FA_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends; no call
 * allocates or frees anything.  Arguments, operation and results are those
 * of fa_bwd_ex_ws given fa_bwd_workspace_size(B, H, Hkv, N, d) bytes (the
 * same split, the same bits); when that size exceeds FA_SCRATCH_BYTES the
 * call returns FA_ERR_SCRATCH before launching anything.  The array needs
 * no clearing (nothing in it is read before a call writes it), but every
 * call on a device uses the same array: calls that overlap in time on one
 * device (different streams, or host threads without ordering) race on it
 * and must be ordered by the caller, for example on one stream.  The first
 * call on a device looks the array's address up with that device current;
 * a failure there returns FA_ERR_HIP.
 */
#define FA_SCRATCH_BYTES (256u << 20)
int fa_bwd_ex_scratch(const void* q, const void* k, const void* v,
                      const void* dO, const float* lse, const float* delta,
                      void* dq, void* dk, void* dv, int B, int H, int Hkv,
                      int N, int d, float scale, int window_left,
                      int window_right, fa_dtype dt, void* stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char* fa_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
