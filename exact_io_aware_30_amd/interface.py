"""User-facing attention API over the C ABI.

The "flash-attn-triton" docs ("Scope", "Where things live", "using it") give
the method a Python surface: ``flash_attn(q, k, v, causal=True)`` returning
the output for (B, H, N, D) fp16/bf16 inputs, an ``autograd.Function`` behind
it, and a drop-in ``FlashSelfAttention(embed_dim, num_heads, causal)``
module.  This module provides the same three names on top of
``libfa_mi355x.so``:

* ``FlashAttnFunction`` -- forward calls ``fa_fwd`` and saves q, k, v, o and
  the row log-sum-exp L; backward calls ``fa_bwd_preprocess`` then
  ``fa_bwd`` (P is rebuilt from L, never stored).
* ``flash_attn(q, k, v, causal=False, softmax_scale=None, window_size=(-1, -1))``
  -- the function
  form; inputs are made contiguous, the scale defaults to 1/sqrt(D).  k and
  v may carry fewer heads than q (Hkv dividing H): grouped-query attention,
  query head h reading key/value head h / (H / Hkv).
* ``flash_attn_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False,
  softmax_scale=None, window_size=(-1, -1))`` -- packed sequences: q (H, T, D),
  k, v (Hkv, T, D), sequence b at rows cu_seqlens[b] .. cu_seqlens[b+1] - 1,
  each attended on its own.
* ``FlashSelfAttention(embed_dim, num_heads, causal=False, bias=True)`` --
  x (B, N, E) -> (B, N, E): one input projection to Q, K, V, attention
  through the kernels, one output projection.  The two projections are
  plain library GEMMs (torch.nn.Linear); the attention itself runs only in
  the HIP kernels.

There is no fallback: the binding refuses to import without the built
library, and the kernels reject CPU tensors.
"""

from __future__ import annotations

import math

import torch

from . import binding

_DTYPES = (torch.float16, torch.bfloat16)
HEAD_DIMS = (32, 64, 128)


def _check_inputs(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be (B, H, N, D) and k, v (B, Hkv, N, D)")
    B, H, N, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != q.shape[2:] or k.shape[1] < 1 \
            or H % k.shape[1]:
        raise ValueError(f"k and v must be (B, Hkv, N, D) with H a multiple of Hkv, got q {tuple(q.shape)}, "
                         f"k {tuple(k.shape)}, v {tuple(v.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be float16 or all bfloat16")
    if q.shape[-1] not in HEAD_DIMS:
        raise ValueError(f"head dimension must be one of {HEAD_DIMS}, got {q.shape[-1]}")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors: the attention runs only in the HIP kernels")


class FlashAttnFunction(torch.autograd.Function):
    """Exact attention whose backward rebuilds P from the saved L."""

    @staticmethod
    def forward(ctx, q, k, v, causal: bool, scale: float, window=None):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = binding.attention_forward(q, k, v, scale, causal, window)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale, ctx.window = bool(causal), float(scale), window
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv, _ = binding.attention_backward(q, k, v, o, do.contiguous().to(o.dtype), lse, ctx.scale,
                                                   ctx.causal, ctx.window)
        return dq, dk, dv, None, None, None


def flash_attn(q, k, v, causal: bool = False, softmax_scale: float | None = None, window_size=(-1, -1)):
    """softmax(q k^T * scale [+ mask]) v for q (B, H, N, D) and k, v
    (B, Hkv, N, D), Hkv dividing H.  window_size = (left, right) keeps keys
    i - left .. i + right for query i (-1: no bound), on top of `causal`."""
    _check_inputs(q, k, v)
    scale = 1.0 / math.sqrt(q.shape[-1]) if softmax_scale is None else float(softmax_scale)
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("softmax_scale must be finite and positive")
    left, right = (int(window_size[0]), int(window_size[1]))
    if left < -1 or right < -1:
        raise ValueError("window_size bounds must be >= -1 (-1: no bound)")
    window = None if (left, right) == (-1, -1) else (left, right)
    return FlashAttnFunction.apply(q, k, v, bool(causal), scale, window)


class FlashAttnVarlenFunction(torch.autograd.Function):
    """Exact attention over packed variable-length sequences."""

    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, max_seqlen: int, causal: bool, scale: float, window=None):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = binding.attention_forward_varlen(q, k, v, cu_seqlens, max_seqlen, scale, causal, window)
        ctx.save_for_backward(q, k, v, o, lse, cu_seqlens)
        ctx.args = (int(max_seqlen), bool(causal), float(scale), window)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, cu = ctx.saved_tensors
        max_seqlen, causal, scale, window = ctx.args
        dq, dk, dv, _ = binding.attention_backward_varlen(q, k, v, o, do.contiguous().to(o.dtype), lse, cu,
                                                          max_seqlen, scale, causal, window)
        return dq, dk, dv, None, None, None, None, None


def flash_attn_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False,
                      softmax_scale: float | None = None, window_size=(-1, -1)):
    """Attention over packed sequences: q (H, T, D), k and v (Hkv, T, D),
    cu_seqlens int32 (B + 1,) on the GPU; every sequence attends on its own."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be (H, T, D) and k, v (Hkv, T, D)")
    if q.shape[-1] not in HEAD_DIMS:
        raise ValueError(f"head dimension must be one of {HEAD_DIMS}, got {q.shape[-1]}")
    if not (q.is_cuda and k.is_cuda and v.is_cuda and cu_seqlens.is_cuda):
        raise ValueError("q, k, v and cu_seqlens must be GPU tensors: the attention runs only in the HIP kernels")
    scale = 1.0 / math.sqrt(q.shape[-1]) if softmax_scale is None else float(softmax_scale)
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("softmax_scale must be finite and positive")
    left, right = (int(window_size[0]), int(window_size[1]))
    if left < -1 or right < -1:
        raise ValueError("window_size bounds must be >= -1 (-1: no bound)")
    window = None if (left, right) == (-1, -1) else (left, right)
    return FlashAttnVarlenFunction.apply(q, k, v, cu_seqlens.to(torch.int32).contiguous(), int(max_seqlen),
                                         bool(causal), scale, window)


class FlashSelfAttention(torch.nn.Module):
    """Multi-head self-attention: x (B, N, E) -> (B, N, E)."""

    def __init__(self, embed_dim: int, num_heads: int, causal: bool = False, bias: bool = True,
                 device=None, dtype=None):
        super().__init__()
        if embed_dim % num_heads:
            raise ValueError("embed_dim must be a multiple of num_heads")
        self.embed_dim, self.num_heads, self.causal = embed_dim, num_heads, bool(causal)
        self.head_dim = embed_dim // num_heads
        if self.head_dim not in HEAD_DIMS:
            raise ValueError(f"embed_dim / num_heads must be one of {HEAD_DIMS}, got {self.head_dim}")
        kw = {"device": device, "dtype": dtype}
        self.in_proj = torch.nn.Linear(embed_dim, 3 * embed_dim, bias=bias, **kw)
        self.out_proj = torch.nn.Linear(embed_dim, embed_dim, bias=bias, **kw)

    def forward(self, x):
        B, N, E = x.shape
        if E != self.embed_dim:
            raise ValueError(f"expected last dimension {self.embed_dim}, got {E}")
        qkv = self.in_proj(x).view(B, N, 3, self.num_heads, self.head_dim).permute(2, 0, 3, 1, 4)
        o = flash_attn(qkv[0], qkv[1], qkv[2], causal=self.causal)  # (B, H, N, D)
        return self.out_proj(o.transpose(1, 2).reshape(B, N, E))
