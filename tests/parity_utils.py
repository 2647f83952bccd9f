"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the CPU fp64 oracle on the same seeded inputs.

Tolerances (written here, used by every parity test):
  O      max |O_gpu - O_ref|                 <= 4e-3 (fp16), 3e-2 (bf16)
  L      max |L_gpu - L_ref|                 <= 1e-4
  dQ, dK, dV, each: max |g_gpu - g_ref| / max |g_ref| <= 1e-2 (fp16), 5e-2 (bf16)
  D (pre-pass on given O, dO): |D_gpu - D_ref| <= 1e-5 * sum_k |dO_ik O_ik| + 1e-6
Any NaN or Inf in an output fails.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

TOL_O = {"fp16": 4e-3, "bf16": 3e-2}
TOL_L = 1e-4
TOL_G = {"fp16": 1e-2, "bf16": 5e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def run_gpu(q, k, v, do, scale, causal):
    """fwd -> preprocess -> bwd on the GPU; returns CPU fp64 numpy arrays."""
    from exact_io_aware_30_amd import binding

    dev = "cuda"
    qg, kg, vg, dog = (x.to(dev) for x in (q, k, v, do))
    o, lse = binding.attention_forward(qg, kg, vg, scale, causal)
    dq, dk, dv, delta = binding.attention_backward(qg, kg, vg, o, dog, lse, scale, causal)
    torch.cuda.synchronize()
    return {"o": to64(o), "lse": to64(lse), "dq": to64(dq), "dk": to64(dk), "dv": to64(dv),
            "delta": to64(delta)}


def check_finite(out):
    for name, a in out.items():
        assert np.all(np.isfinite(a)), f"{name} has NaN/Inf"


def err_abs(a, b):
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def err_rel(a, b):
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def assert_fwd(dtype, o, o_ref, L, L_ref, what=""):
    eo, el = err_abs(o, o_ref), err_abs(L, L_ref)
    say(f"  {what} O max-abs {eo:.3e} (tol {TOL_O[dtype]:g})  L max-abs {el:.3e} (tol {TOL_L:g})")
    assert eo <= TOL_O[dtype], f"O error {eo}"
    assert el <= TOL_L, f"L error {el}"


def assert_grad(dtype, name, g, g_ref, what=""):
    e = err_rel(g, g_ref)
    say(f"  {what} {name} max-abs/max-ref {e:.3e} (tol {TOL_G[dtype]:g})")
    assert e <= TOL_G[dtype], f"{name} error {e}"


def host_threads() -> int:
    """Host threads for oracle work: the CPUs this process may use, at most 16."""
    import os

    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def dkdv_cols_split(qh, kh, vh, doh, scale, causal, cols, row_block=512, workers=None):
    """oracle.dkdv_cols over [0, N), the query rows split into contiguous
    ranges evaluated on host threads and their shares added in range order
    (the sampler's ``rows`` option; NumPy releases the GIL in its kernels)."""
    import concurrent.futures

    import oracle

    N = qh.shape[0]
    n = workers or host_threads()
    lo = int(np.min(cols)) if causal else 0
    # causal: rows i carry about i - lo keys each, so cut the range where the
    # running work (a triangle) reaches equal shares
    if causal:
        cuts = [lo + int(round((N - lo) * np.sqrt(t / (4 * n)))) for t in range(4 * n + 1)]
    else:
        cuts = [int(round(N * t / (4 * n))) for t in range(4 * n + 1)]
    ranges = [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    with concurrent.futures.ThreadPoolExecutor(max_workers=n) as ex:
        parts = list(ex.map(lambda r: oracle.dkdv_cols(qh, kh, vh, doh, scale, causal, cols, row_block, rows=r),
                            ranges))
    dk = np.zeros((len(cols), qh.shape[1]))
    dv = np.zeros_like(dk)
    for pk, pv in parts:
        dk += pk
        dv += pv
    return dk, dv
