"""Exact softmax attention and its analytic gradient, in fp64 on the CPU.

TEST INFRASTRUCTURE (see the package docstring).

Layout: every tensor is a NumPy array [B, H, N, d] (float64); L and D are
[B, H, N].  Heads are independent (flash attention note, "Key Mechanisms",
multi-head support), so each function loops over (b, h) and works on one
head's [N, d] matrices.

Forward (flash-attn-triton docs, "The argument"; tensortonic "What is
FlashAttention?"):
    S = scale * Q K^T                       (scale = 1/sqrt(d) by default)
    S_ij = -inf for j > i under the causal mask (flash attention note, "Key
           Mechanisms", causal masking: lower-triangular)
    P = safe softmax of S by rows           (tensortonic, "Start with a safe
                                             softmax")
    O = P V
    L_i = log sum_j exp(S_ij), natural log  (the one float per row that
          flash-attn-triton docs, Fig. 3, keeps after the loop; Fig. 3 writes
          it as m + log l with m in base-2 units -- read here as the natural
          logsumexp of the scaled scores)

Backward (the pages only say the backward rebuilds P from L -- flash-attn-
triton docs, "Scope" and the note under "The argument"; the equations are the
gradient of the forward above, derived by the chain rule):
    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij  ( = sum_k dO_ik O_ik )
    dS = P o (dP - D 1^T)                   (softmax Jacobian-vector product)
    dQ = scale * dS K,  dK = scale * dS^T Q

A row with no visible key (cannot arise for causal with equal query and key
lengths, for the full mask or for a window that contains the diagonal, but
handled) has P = 0, O = 0, L = -inf and contributes nothing to any gradient.

Sliding windows (flash-attn-triton docs, "Scope", lists them as not yet done
there): ``window=(left, right)`` keeps key j for query i iff
i - left <= j <= i + right, a bound of -1 meaning none on that side; it
applies on top of ``causal``.

Row blocking (``row_block``) only bounds memory: each block of query rows sees
its full key range, so every row's softmax is still one-shot.  Under the
causal mask keys after a block's last row are all masked and are skipped.
"""

from __future__ import annotations

import numpy as np


def _as64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _check_shapes(*ts):
    s = ts[0].shape
    if len(s) != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    for t in ts[1:]:
        if t.shape != s:
            raise ValueError("shape mismatch")


def _scores(qh, kh, scale, causal, r0, r1, nk, window=None):
    """Scaled scores of query rows [r0, r1) against keys [0, nk), masked."""
    s = scale * (qh[r0:r1] @ kh[:nk].T)
    if causal:
        i = np.arange(r0, r1)[:, None]
        j = np.arange(nk)[None, :]
        s = np.where(j > i, -np.inf, s)
    if window is not None:
        # key j visible to query i iff i - left <= j <= i + right (-1: no bound)
        left, right = window
        i = np.arange(r0, r1)[:, None]
        j = np.arange(nk)[None, :]
        if left >= 0:
            s = np.where(j < i - left, -np.inf, s)
        if right >= 0:
            s = np.where(j > i + right, -np.inf, s)
    return s


def _probs(s):
    """Safe softmax of score rows plus their natural-log logsumexp."""
    m = np.max(s, axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    live = np.isfinite(m)
    e = np.where(live[:, None], np.exp(s - np.where(live, m, 0.0)[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.where(live[:, None], e / np.where(live, l, 1.0)[:, None], 0.0)
    L = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return p, L


def _key_extent(causal, r1, n, window=None):
    """Keys past this one are masked for every row before r1."""
    nk = min(r1, n) if causal else n
    if window is not None and window[1] >= 0:
        nk = min(nk, r1 + window[1])
    return nk


def attention_forward(q, k, v, scale, causal, row_block=None, window=None):
    """O [B,H,N,d] and L [B,H,N] of exact softmax attention.  ``window``
    (left, right) further restricts query i to keys i - left .. i + right
    (-1: no bound on that side)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    _check_shapes(q, k, v)
    B, H, N, _ = q.shape
    rb = N if row_block is None else max(1, int(row_block))
    o = np.zeros_like(q)
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, rb):
                r1 = min(N, r0 + rb)
                nk = _key_extent(causal, r1, N, window)
                p, L[b, h, r0:r1] = _probs(_scores(q[b, h], k[b, h], scale, causal, r0, r1, nk, window))
                o[b, h, r0:r1] = p @ v[b, h, :nk]
    return o, L


def delta_rowsum(o, do):
    """D_i = sum_k dO_ik O_ik for every row, [B,H,N] (the backward pre-pass)."""
    return np.sum(_as64(o) * _as64(do), axis=-1)


def attention_backward(q, k, v, do, scale, causal, row_block=None, window=None):
    """Gradients of sum(dO o O) with respect to Q, K, V.

    Returns a dict with dq, dk, dv ([B,H,N,d]), and the forward quantities the
    backward uses: o, lse (natural log, [B,H,N]), delta (sum_j P_ij dP_ij) and
    delta_o (sum_k dO_ik O_ik); the last two are equal up to rounding.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    _check_shapes(q, k, v, do)
    B, H, N, _ = q.shape
    rb = N if row_block is None else max(1, int(row_block))
    out = {name: np.zeros_like(q) for name in ("dq", "dk", "dv", "o")}
    for name in ("lse", "delta", "delta_o"):
        out[name] = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = q[b, h], k[b, h], v[b, h], do[b, h]
            for r0 in range(0, N, rb):
                r1 = min(N, r0 + rb)
                nk = _key_extent(causal, r1, N, window)
                p, lse = _probs(_scores(qh, kh, scale, causal, r0, r1, nk, window))
                ob = p @ vh[:nk]
                dob = doh[r0:r1]
                out["dv"][b, h, :nk] += p.T @ dob
                dp = dob @ vh[:nk].T
                dsum = np.sum(p * dp, axis=1)
                ds = p * (dp - dsum[:, None])
                out["dq"][b, h, r0:r1] = scale * (ds @ kh[:nk])
                out["dk"][b, h, :nk] += scale * (ds.T @ qh[r0:r1])
                out["o"][b, h, r0:r1] = ob
                out["lse"][b, h, r0:r1] = lse
                out["delta"][b, h, r0:r1] = dsum
                out["delta_o"][b, h, r0:r1] = np.sum(dob * ob, axis=1)
    return out


# ---------------------------------------------------------------------------
# Grouped-query attention (flash attention note, "Versions and Evolution":
# multi-query and grouped-query attention).  H query heads share Hkv key/value
# heads, H a multiple of Hkv; query head h reads key/value head h // G,
# G = H / Hkv.  By definition that is plain attention with every key/value
# head repeated G times along the head axis, and the gradient of a shared key
# or value head is the sum of the gradients of its G copies.
# ---------------------------------------------------------------------------
def _group(q, k):
    H, Hkv = q.shape[1], k.shape[1]
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"query heads {H} must be a multiple of key/value heads {Hkv}")
    return H // Hkv


def attention_forward_gqa(q, k, v, scale, causal, row_block=None, window=None):
    """(O [B,H,N,d], L [B,H,N]) for q [B,H,N,d] and k, v [B,Hkv,N,d]."""
    G = _group(q, k)
    return attention_forward(q, np.repeat(_as64(k), G, axis=1), np.repeat(_as64(v), G, axis=1), scale, causal,
                             row_block, window)


def attention_backward_gqa(q, k, v, do, scale, causal, row_block=None, window=None):
    """attention_backward for grouped heads: dk and dv [B,Hkv,N,d] sum the
    gradients of the G query heads that read each key/value head."""
    G = _group(q, k)
    out = attention_backward(q, np.repeat(_as64(k), G, axis=1), np.repeat(_as64(v), G, axis=1), do, scale,
                             causal, row_block, window)
    B, Hkv, N, d = k.shape
    for name in ("dk", "dv"):
        out[name] = out[name].reshape(B, Hkv, G, N, d).sum(axis=2)
    return out


# ---------------------------------------------------------------------------
# Packed variable-length batches (flash-attn-triton docs, "Scope", lists
# variable-length batches as not yet done there): the B sequences sit along
# the row axis of [H, T, d] tensors, sequence b at rows cu[b] .. cu[b+1] - 1,
# and each is attended on its own -- by definition the plain attention of
# every sequence separately.
# ---------------------------------------------------------------------------
def attention_backward_varlen(q, k, v, do, cu, scale, causal, window=None):
    """Forward and backward quantities for packed sequences: q, do [H,T,d],
    k, v [Hkv,T,d], cu the B + 1 row offsets.  Returns o, dq [H,T,d], dk, dv
    [Hkv,T,d], lse, delta [H,T]."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    H, T, d = q.shape
    out = {"o": np.zeros_like(q), "dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "lse": np.zeros((H, T)), "delta": np.zeros((H, T))}
    for s0, s1 in zip(cu[:-1], cu[1:]):
        if s1 <= s0:
            continue
        r = attention_backward_gqa(q[None, :, s0:s1], k[None, :, s0:s1], v[None, :, s0:s1], do[None, :, s0:s1],
                                   scale, causal, window=window)
        for name in ("o", "dq", "dk", "dv", "lse", "delta"):
            out[name][:, s0:s1] = r[name][0]
    return out


# ---------------------------------------------------------------------------
# Samplers: the same definitions restricted to chosen rows or key columns of
# one head, for sizes where the whole N x N matrix is too costly on the CPU.
# ---------------------------------------------------------------------------

def forward_rows(qh, kh, vh, scale, causal, rows):
    """O and L of the given query rows of one head ([N, d] inputs)."""
    qh, kh, vh = _as64(qh), _as64(kh), _as64(vh)
    N = qh.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, qh.shape[1]))
    L = np.zeros(rows.size)
    for t, i in enumerate(rows):
        nk = _key_extent(causal, i + 1, N)
        p, L[t:t + 1] = _probs(_scores(qh, kh, scale, causal, i, i + 1, nk))
        o[t] = (p @ vh[:nk])[0]
    return o, L


def dq_rows(qh, kh, vh, doh, scale, causal, rows):
    """dQ of the given query rows of one head.

    Row i of dQ needs only row i of P and dP: D_i = sum_j P_ij dP_ij.
    """
    qh, kh, vh, doh = _as64(qh), _as64(kh), _as64(vh), _as64(doh)
    N = qh.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((rows.size, qh.shape[1]))
    for t, i in enumerate(rows):
        nk = _key_extent(causal, i + 1, N)
        p, _ = _probs(_scores(qh, kh, scale, causal, i, i + 1, nk))
        dp = doh[i:i + 1] @ vh[:nk].T
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        dq[t] = scale * (ds @ kh[:nk])[0]
    return dq


def dkdv_cols(qh, kh, vh, doh, scale, causal, cols, row_block=2048, rows=None):
    """dK and dV of the given key rows (columns of P) of one head.

    Column j of P involves every query row i that sees key j (i >= j under
    the causal mask), and each such row needs its own full softmax, so this
    walks those rows in blocks of ``row_block`` with their full key range.

    ``rows`` = (r_lo, r_hi) restricts the walk to query rows [r_lo, r_hi):
    the result is then those rows' share of the sums dV_j = sum_i P_ij dO_i
    and dK_j = scale sum_i dS_ij Q_i, so the shares of disjoint ranges that
    cover [0, N) add up to the whole gradient.
    """
    qh, kh, vh, doh = _as64(qh), _as64(kh), _as64(vh), _as64(doh)
    N, d = qh.shape
    cols = np.asarray(cols, dtype=np.int64)
    dk = np.zeros((cols.size, d))
    dv = np.zeros((cols.size, d))
    if cols.size == 0:
        return dk, dv
    lo, hi = (0, N) if rows is None else (max(0, int(rows[0])), min(N, int(rows[1])))
    first = max(lo, int(cols.min())) if causal else lo
    for r0 in range(first, hi, row_block):
        r1 = min(hi, r0 + row_block)
        nk = _key_extent(causal, r1, N)
        p, _ = _probs(_scores(qh, kh, scale, causal, r0, r1, nk))
        dob = doh[r0:r1]
        dp = dob @ vh[:nk].T
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        sel = cols < nk
        c = cols[sel]
        dv[sel] += p[:, c].T @ dob
        dk[sel] += scale * (ds[:, c].T @ qh[r0:r1])
    return dk, dv
