"""ctypes binding of ``libfa_mi355x.so`` (C ABI in include/fa.h).

Argument marshalling only: each function checks that the torch tensors are
contiguous GPU tensors of the expected shape and dtype, then passes their
``data_ptr()``, the sizes and torch's current HIP stream to the C function of
the same name.  All arithmetic runs in the library's HIP kernels; there is no
fallback path, and importing this module fails if the library is not built.

``attention_forward`` / ``attention_backward`` allocate the outputs with
torch and call the C functions.
"""

from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

FA_F16, FA_BF16 = 0, 1
FA_OK = 0
_DT = {torch.float16: FA_F16, torch.bfloat16: FA_BF16}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m exact_io_aware_30_amd.build` "
        "(hipcc, gfx950) first -- there is no non-HIP fallback")

_lib = ctypes.CDLL(LIB_PATH)

_p, _i, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_SIG = {
    "fa_fwd": [_p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _i, _i, _p],
    "fa_bwd_preprocess": [_p, _p, _p, _i, _i, _i, _i, _i, _p],
    "fa_bwd": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _i, _i, _p],
    "fa_bwd_dkdv": [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _i, _i, _p],
    "fa_bwd_dq": [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _i, _i, _p],
    "fa_fwd_gqa": [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _p],
    "fa_bwd_gqa": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _p],
    "fa_bwd_dkdv_gqa": [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _p],
    "fa_bwd_dq_gqa": [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _p],
    "fa_fwd_ex": [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _i, _p],
    "fa_bwd_ex": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _i, _p],
    "fa_bwd_dkdv_ex": [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _i, _p],
    "fa_bwd_dq_ex": [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _i, _p],
    "fa_fwd_varlen": [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _p],
    "fa_bwd_varlen": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _p],
    "fa_bwd_ex_ws": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _i, _p, ctypes.c_size_t,
                     _p],
    "fa_bwd_varlen_ws": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _p,
                         ctypes.c_size_t, _p],
    "fa_bwd_ex_scratch": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _i, _p],
    "fa_bwd_workspace_size": [_i, _i, _i, _i, _i],
    "fa_bwd_varlen_workspace_size": [_i, _i, _i, _i, _i, _i],
    "fa_status_string": [_i],
    "fa_version": [],
}
for _name, _args in _SIG.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = ctypes.c_char_p if _name == "fa_status_string" else \
        ctypes.c_size_t if _name.endswith("_workspace_size") else _i

EXPORTED = tuple(_SIG)


class FAError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {fa_status_string(code)} (status {code})")
        self.code = code


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(int(status)).decode()


def fa_version() -> int:
    return _lib.fa_version()


def _check(code: int, where: str):
    if code != FA_OK:
        raise FAError(code, where)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _bhnd(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d]")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if t.dtype not in _DT:
        raise ValueError(f"{name} must be float16 or bfloat16")
    return t.shape


def _same(ref: torch.Tensor, *pairs):
    for t, name in pairs:
        if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_cuda or not t.is_contiguous() \
                or t.device != ref.device:
            raise ValueError(f"{name} must match q in shape, dtype and device and be contiguous")


def _rows(ref: torch.Tensor, *pairs):
    B, H, N, _ = ref.shape
    for t, name in pairs:
        if t.shape != (B, H, N) or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 [B, H, N] GPU tensor")


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool) -> None:
    B, H, N, d = _bhnd(q, "q")
    _same(q, (k, "k"), (v, "v"), (o, "o"))
    _rows(q, (lse, "lse"))
    _check(_lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, H, N, d, float(scale), int(bool(causal)), _DT[q.dtype], _stream(q)), "fa_fwd")


def fa_bwd_preprocess(o, do, delta) -> None:
    B, H, N, d = _bhnd(o, "o")
    _same(o, (do, "do"))
    _rows(o, (delta, "delta"))
    _check(_lib.fa_bwd_preprocess(o.data_ptr(), do.data_ptr(), delta.data_ptr(), B, H, N, d,
                                  _DT[o.dtype], _stream(o)), "fa_bwd_preprocess")


def fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, scale: float, causal: bool) -> None:
    B, H, N, d = _bhnd(q, "q")
    _same(q, (k, "k"), (v, "v"), (do, "do"), (dq, "dq"), (dk, "dk"), (dv, "dv"))
    _rows(q, (lse, "lse"), (delta, "delta"))
    _check(_lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                       delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                       float(scale), int(bool(causal)), _DT[q.dtype], _stream(q)), "fa_bwd")


def fa_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, scale: float, causal: bool) -> None:
    B, H, N, d = _bhnd(q, "q")
    _same(q, (k, "k"), (v, "v"), (do, "do"), (dk, "dk"), (dv, "dv"))
    _rows(q, (lse, "lse"), (delta, "delta"))
    _check(_lib.fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                            delta.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale),
                            int(bool(causal)), _DT[q.dtype], _stream(q)), "fa_bwd_dkdv")


def fa_bwd_dq(q, k, v, do, lse, delta, dq, scale: float, causal: bool) -> None:
    B, H, N, d = _bhnd(q, "q")
    _same(q, (k, "k"), (v, "v"), (do, "do"), (dq, "dq"))
    _rows(q, (lse, "lse"), (delta, "delta"))
    _check(_lib.fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                          delta.data_ptr(), dq.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                          _DT[q.dtype], _stream(q)), "fa_bwd_dq")


def _kv(q, pairs):
    """Hkv of k-shaped tensors [B, Hkv, N, d] that go with q [B, H, N, d]."""
    B, H, N, d = q.shape
    Hkv = pairs[0][0].shape[1] if pairs[0][0].dim() == 4 else -1
    for t, name in pairs:
        if t.dim() != 4 or t.shape != (B, Hkv, N, d) or t.dtype != q.dtype or not t.is_cuda \
                or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous [B, Hkv, N, d] GPU tensor of q's dtype")
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"the query heads ({H}) must be a multiple of the key/value heads ({Hkv})")
    return Hkv


def fa_fwd_gqa(q, k, v, o, lse, scale: float, causal: bool) -> None:
    B, H, N, d = _bhnd(q, "q")
    Hkv = _kv(q, ((k, "k"), (v, "v")))
    _same(q, (o, "o"))
    _rows(q, (lse, "lse"))
    _check(_lib.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           B, H, Hkv, N, d, float(scale), int(bool(causal)), _DT[q.dtype], _stream(q)),
           "fa_fwd_gqa")


def fa_bwd_gqa(q, k, v, do, lse, delta, dq, dk, dv, scale: float, causal: bool) -> None:
    B, H, N, d = _bhnd(q, "q")
    Hkv = _kv(q, ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")))
    _same(q, (do, "do"), (dq, "dq"))
    _rows(q, (lse, "lse"), (delta, "delta"))
    _check(_lib.fa_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                           delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d,
                           float(scale), int(bool(causal)), _DT[q.dtype], _stream(q)), "fa_bwd_gqa")


def fa_bwd_dkdv_gqa(q, k, v, do, lse, delta, dk, dv, scale: float, causal: bool) -> None:
    B, H, N, d = _bhnd(q, "q")
    Hkv = _kv(q, ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")))
    _same(q, (do, "do"))
    _rows(q, (lse, "lse"), (delta, "delta"))
    _check(_lib.fa_bwd_dkdv_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                                delta.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d, float(scale),
                                int(bool(causal)), _DT[q.dtype], _stream(q)), "fa_bwd_dkdv_gqa")


def fa_bwd_dq_gqa(q, k, v, do, lse, delta, dq, scale: float, causal: bool) -> None:
    B, H, N, d = _bhnd(q, "q")
    Hkv = _kv(q, ((k, "k"), (v, "v")))
    _same(q, (do, "do"), (dq, "dq"))
    _rows(q, (lse, "lse"), (delta, "delta"))
    _check(_lib.fa_bwd_dq_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                              delta.data_ptr(), dq.data_ptr(), B, H, Hkv, N, d, float(scale), int(bool(causal)),
                              _DT[q.dtype], _stream(q)), "fa_bwd_dq_gqa")


def _window(window, causal):
    """(left, right) for fa_*_ex: `window` on top of the causal flag."""
    left, right = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    if left < -1 or right < -1:
        raise ValueError("window bounds must be >= -1 (-1: no bound)")
    if causal:
        right = 0 if right < 0 else min(right, 0)
    return left, right


def fa_fwd_ex(q, k, v, o, lse, scale: float, window) -> None:
    B, H, N, d = _bhnd(q, "q")
    Hkv = _kv(q, ((k, "k"), (v, "v")))
    _same(q, (o, "o"))
    _rows(q, (lse, "lse"))
    wl, wr = window
    _check(_lib.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Hkv, N, d,
                          float(scale), int(wl), int(wr), _DT[q.dtype], _stream(q)), "fa_fwd_ex")


def fa_bwd_ex(q, k, v, do, lse, delta, dq, dk, dv, scale: float, window) -> None:
    B, H, N, d = _bhnd(q, "q")
    Hkv = _kv(q, ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")))
    _same(q, (do, "do"), (dq, "dq"))
    _rows(q, (lse, "lse"), (delta, "delta"))
    wl, wr = window
    _check(_lib.fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                          delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d,
                          float(scale), int(wl), int(wr), _DT[q.dtype], _stream(q)), "fa_bwd_ex")


def fa_bwd_dkdv_ex(q, k, v, do, lse, delta, dk, dv, scale: float, window) -> None:
    B, H, N, d = _bhnd(q, "q")
    Hkv = _kv(q, ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")))
    _same(q, (do, "do"))
    _rows(q, (lse, "lse"), (delta, "delta"))
    wl, wr = window
    _check(_lib.fa_bwd_dkdv_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                               delta.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d, float(scale),
                               int(wl), int(wr), _DT[q.dtype], _stream(q)), "fa_bwd_dkdv_ex")


def fa_bwd_dq_ex(q, k, v, do, lse, delta, dq, scale: float, window) -> None:
    B, H, N, d = _bhnd(q, "q")
    Hkv = _kv(q, ((k, "k"), (v, "v")))
    _same(q, (do, "do"), (dq, "dq"))
    _rows(q, (lse, "lse"), (delta, "delta"))
    wl, wr = window
    _check(_lib.fa_bwd_dq_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                             delta.data_ptr(), dq.data_ptr(), B, H, Hkv, N, d, float(scale), int(wl), int(wr),
                             _DT[q.dtype], _stream(q)), "fa_bwd_dq_ex")


def fa_bwd_workspace_size(B: int, H: int, Hkv: int, N: int, d: int) -> int:
    """Bytes of workspace with which fa_bwd_ex_ws splits the query heads of a
    key/value head over several dK/dV workgroups (0: no split pays)."""
    return int(_lib.fa_bwd_workspace_size(int(B), int(H), int(Hkv), int(N), int(d)))


def fa_bwd_varlen_workspace_size(B: int, max_seqlen: int, T: int, H: int, Hkv: int, d: int) -> int:
    return int(_lib.fa_bwd_varlen_workspace_size(int(B), int(max_seqlen), int(T), int(H), int(Hkv), int(d)))


def _workspace(ws, device):
    """(pointer, bytes) of an optional uint8 workspace tensor on `device`."""
    if ws is None:
        return None, 0
    if ws.dtype != torch.uint8 or not ws.is_cuda or not ws.is_contiguous() or ws.device != device:
        raise ValueError("workspace must be a contiguous uint8 GPU tensor on q's device")
    return ws.data_ptr(), ws.numel()


def fa_bwd_ex_ws(q, k, v, do, lse, delta, dq, dk, dv, scale: float, window, workspace) -> None:
    B, H, N, d = _bhnd(q, "q")
    Hkv = _kv(q, ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")))
    _same(q, (do, "do"), (dq, "dq"))
    _rows(q, (lse, "lse"), (delta, "delta"))
    wl, wr = window
    wp, wb = _workspace(workspace, q.device)
    _check(_lib.fa_bwd_ex_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                             delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d,
                             float(scale), int(wl), int(wr), _DT[q.dtype], wp, wb, _stream(q)), "fa_bwd_ex_ws")


# Bytes of the library's static scratch array (FA_SCRATCH_BYTES).
SCRATCH_BYTES = 256 << 20


def fa_bwd_ex_scratch(q, k, v, do, lse, delta, dq, dk, dv, scale: float, window) -> None:
    """fa_bwd_ex_ws with the head-split partials in the library's static
    scratch array instead of a workspace: nothing is allocated."""
    B, H, N, d = _bhnd(q, "q")
    Hkv = _kv(q, ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")))
    _same(q, (do, "do"), (dq, "dq"))
    _rows(q, (lse, "lse"), (delta, "delta"))
    wl, wr = window
    _check(_lib.fa_bwd_ex_scratch(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                                  delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d,
                                  float(scale), int(wl), int(wr), _DT[q.dtype], _stream(q)), "fa_bwd_ex_scratch")


def attention_forward(q, k, v, scale: float, causal: bool, window=None):
    """(o, lse) with o like q and lse float32 [B, H, N]; k and v may have
    fewer heads than q (grouped-query attention); window = (left, right)
    keeps keys i - left .. i + right for query i (-1: no bound)."""
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if window is not None:
        fa_fwd_ex(q, k, v, o, lse, scale, _window(window, causal))
    elif k.dim() == 4 and k.shape[1] != q.shape[1]:
        fa_fwd_gqa(q, k, v, o, lse, scale, causal)
    else:
        fa_fwd(q, k, v, o, lse, scale, causal)
    return o, lse


def attention_backward(q, k, v, o, do, lse, scale: float, causal: bool, window=None):
    """(dq, dk, dv, delta): the pre-pass then the two backward kernels; dk and
    dv are shaped like k and v."""
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa_bwd_preprocess(o, do, delta)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, H, N, d = q.shape
    nbytes = fa_bwd_workspace_size(B, H, k.shape[1], N, d) if k.dim() == 4 else 0
    if nbytes:
        # few key/value heads: split their query heads over more workgroups
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        fa_bwd_ex_ws(q, k, v, do, lse, delta, dq, dk, dv, scale, _window(window, causal), ws)
    elif window is not None:
        fa_bwd_ex(q, k, v, do, lse, delta, dq, dk, dv, scale, _window(window, causal))
    elif k.dim() == 4 and k.shape[1] != q.shape[1]:
        fa_bwd_gqa(q, k, v, do, lse, delta, dq, dk, dv, scale, causal)
    else:
        fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, scale, causal)
    return dq, dk, dv, delta


# ---------------------------------------------------------------------------
# Packed variable-length batches: q, o, do, dq [H, T, d]; k, v, dk, dv
# [Hkv, T, d]; lse, delta [H, T]; cu_seqlens int32 [B + 1] on the GPU.
# ---------------------------------------------------------------------------
def _packed(q, kv_pairs, q_pairs, rows, cu_seqlens):
    if q.dim() != 3 or not q.is_cuda or not q.is_contiguous() or q.dtype not in _DT:
        raise ValueError("q must be a contiguous [H, T, d] float16/bfloat16 GPU tensor")
    H, T, d = q.shape
    Hkv = kv_pairs[0][0].shape[0] if kv_pairs[0][0].dim() == 3 else -1
    for t, name in kv_pairs:
        if t.dim() != 3 or t.shape != (Hkv, T, d) or t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [Hkv, T, d] GPU tensor of q's dtype")
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"the query heads ({H}) must be a multiple of the key/value heads ({Hkv})")
    for t, name in q_pairs:
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must match q")
    for t, name in rows:
        if t.shape != (H, T) or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 [H, T] GPU tensor")
    if (cu_seqlens.dim() != 1 or cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda
            or not cu_seqlens.is_contiguous() or cu_seqlens.numel() < 2):
        raise ValueError("cu_seqlens must be a contiguous int32 [B + 1] GPU tensor")
    return H, Hkv, T, d, cu_seqlens.numel() - 1


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen: int, scale: float, window) -> None:
    H, Hkv, T, d, B = _packed(q, ((k, "k"), (v, "v")), ((o, "o"),), ((lse, "lse"),), cu_seqlens)
    wl, wr = window
    _check(_lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              cu_seqlens.data_ptr(), B, int(max_seqlen), T, H, Hkv, d, float(scale), int(wl), int(wr),
                              _DT[q.dtype], _stream(q)), "fa_fwd_varlen")


def fa_bwd_varlen(q, k, v, do, lse, delta, dq, dk, dv, cu_seqlens, max_seqlen: int, scale: float, window) -> None:
    H, Hkv, T, d, B = _packed(q, ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")), ((do, "do"), (dq, "dq")),
                              ((lse, "lse"), (delta, "delta")), cu_seqlens)
    wl, wr = window
    _check(_lib.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                              delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens.data_ptr(), B,
                              int(max_seqlen), T, H, Hkv, d, float(scale), int(wl), int(wr), _DT[q.dtype],
                              _stream(q)), "fa_bwd_varlen")


def fa_bwd_varlen_ws(q, k, v, do, lse, delta, dq, dk, dv, cu_seqlens, max_seqlen: int, scale: float, window,
                     workspace) -> None:
    H, Hkv, T, d, B = _packed(q, ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")), ((do, "do"), (dq, "dq")),
                              ((lse, "lse"), (delta, "delta")), cu_seqlens)
    wl, wr = window
    wp, wb = _workspace(workspace, q.device)
    _check(_lib.fa_bwd_varlen_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                                 delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens.data_ptr(),
                                 B, int(max_seqlen), T, H, Hkv, d, float(scale), int(wl), int(wr), _DT[q.dtype], wp,
                                 wb, _stream(q)), "fa_bwd_varlen_ws")


def attention_forward_varlen(q, k, v, cu_seqlens, max_seqlen: int, scale: float, causal: bool, window=None):
    """(o [H, T, d], lse [H, T]) for packed sequences."""
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen, scale, _window(window, causal))
    return o, lse


def attention_backward_varlen(q, k, v, o, do, lse, cu_seqlens, max_seqlen: int, scale: float, causal: bool,
                              window=None):
    """(dq, dk, dv, delta) for packed sequences: the pre-pass over [1, H, T, d]
    views, then the two backward kernels."""
    H, T, d = q.shape
    delta = torch.empty((H, T), dtype=torch.float32, device=q.device)
    fa_bwd_preprocess(o.view(1, H, T, d), do.view(1, H, T, d), delta.view(1, H, T))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = fa_bwd_varlen_workspace_size(cu_seqlens.numel() - 1, max_seqlen, T, H, k.shape[0], d) \
        if k.dim() == 3 else 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    fa_bwd_varlen_ws(q, k, v, do, lse, delta, dq, dk, dv, cu_seqlens, max_seqlen, scale, _window(window, causal), ws)
    return dq, dk, dv, delta
