"""GPU parity of the windowed entry points (fa_fwd_ex, fa_bwd_ex and its
halves) against the oracle's window masks, on seeded inputs, at the parity
tolerances: left-only, right-only and two-sided windows, the window that
keeps only the diagonal, windows on top of the causal mask and of grouped
heads, and a window wider than the sequence (the full mask)."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_30_amd import workloads as wl
from parity_utils import TOL_G, TOL_L, TOL_O, err_abs, err_rel, say, to64

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, H, Hkv, N, d, (left, right)  -- causal is right = 0
    ("bf16", 2, 4, 4, 1000, 128, (256, 0)),
    ("fp16", 1, 3, 3, 777, 64, (100, 50)),
    ("bf16", 2, 2, 2, 600, 128, (-1, 37)),
    ("fp16", 1, 2, 2, 300, 64, (5, 5)),
    ("bf16", 1, 2, 1, 2048, 128, (1024, 0)),
    ("fp16", 2, 4, 2, 513, 32, (70, -1)),
    ("bf16", 1, 2, 2, 450, 32, (33, 0)),
    ("fp16", 1, 2, 2, 257, 128, (5000, 5000)),
    # sequences past the short-sequence cut (2048).  Windows bounded on both
    # sides and at most 4096 keys wide take the 4-wave forward at any N:
    ("bf16", 1, 2, 2, 3000, 128, (700, 0)),
    ("fp16", 1, 2, 1, 2600, 64, (300, 200)),
    ("bf16", 1, 2, 2, 5000, 128, (2047, 2048)),
    ("fp16", 1, 2, 1, 3300, 64, (1500, 0)),
    # the others take the long-sequence forwards (pipelined at d = 128): a
    # window unbounded on the left, and one key wider than 4096
    ("bf16", 1, 2, 2, 2300, 128, (-1, 100)),
    ("fp16", 1, 2, 2, 4500, 128, (2048, 2048)),
]


def _inputs(dtype, B, H, Hkv, N, d, seed):
    q = wl.make_tensor((B, H, N, d), dtype, seed)
    k = wl.make_tensor((B, Hkv, N, d), dtype, seed + 1)
    v = wl.make_tensor((B, Hkv, N, d), dtype, seed + 2)
    do = wl.make_tensor((B, H, N, d), dtype, seed + 3)
    return q, k, v, do


@pytest.mark.parametrize("dtype,B,H,Hkv,N,d,window", CASES)
def test_window_matches_oracle(dtype, B, H, Hkv, N, d, window):
    from exact_io_aware_30_amd import binding

    say(f"[window] {dtype} B={B} H={H} Hkv={Hkv} N={N} d={d} window={window}")
    q, k, v, do = _inputs(dtype, B, H, Hkv, N, d, 11000 + N + d + window[0])
    scale = 1.0 / math.sqrt(d)
    qg, kg, vg, dog = (x.cuda() for x in (q, k, v, do))
    o = torch.empty_like(qg)
    lse = torch.empty(qg.shape[:3], dtype=torch.float32, device="cuda")
    binding.fa_fwd_ex(qg, kg, vg, o, lse, scale, window)
    delta = torch.empty_like(lse)
    binding.fa_bwd_preprocess(o, dog, delta)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    binding.fa_bwd_ex(qg, kg, vg, dog, lse, delta, dq, dk, dv, scale, window)
    dq2, dk2, dv2 = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    binding.fa_bwd_dkdv_ex(qg, kg, vg, dog, lse, delta, dk2, dv2, scale, window)
    binding.fa_bwd_dq_ex(qg, kg, vg, dog, lse, delta, dq2, scale, window)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    ref = oracle.attention_backward_gqa(*(x.double().numpy() for x in (q, k, v, do)), scale, False,
                                        row_block=512, window=window)
    eo, el = err_abs(to64(o), ref["o"]), err_abs(to64(lse), ref["lse"])
    say(f"  O {eo:.3e}  L {el:.3e}")
    assert eo <= TOL_O[dtype] and el <= TOL_L
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        g = to64(t)
        assert np.all(np.isfinite(g)), name
        e = err_rel(g, ref[name])
        say(f"  {name} {e:.3e}")
        assert e <= TOL_G[dtype], name


@pytest.mark.parametrize("d", [32, 64, 128])
def test_diagonal_window_gives_v_and_do(d):
    # window (0, 0): every query sees only its own key, so O = V and dV = dO
    # exactly (P = 1, l = 1); dS = dP_ii - D_i is zero up to the rounding of
    # two fp32 dot products summed in different orders (MFMA vs the pre-pass)
    from exact_io_aware_30_amd import binding

    q, k, v, do = _inputs("bf16", 1, 2, 2, 333, d, 11500 + d)
    qg, kg, vg, dog = (x.cuda() for x in (q, k, v, do))
    o, lse = binding.attention_forward(qg, kg, vg, 0.125, False, window=(0, 0))
    dq, dk, dv, _ = binding.attention_backward(qg, kg, vg, o, dog, lse, 0.125, False, window=(0, 0))
    torch.cuda.synchronize()
    assert torch.equal(o, vg) and torch.equal(dv, dog)
    assert dq.abs().max().item() <= 1e-5 and dk.abs().max().item() <= 1e-5


def test_causal_window_equals_causal_flag():
    from exact_io_aware_30_amd import binding

    q, k, v, do = _inputs("fp16", 2, 3, 3, 700, 64, 11600)
    qg, kg, vg, dog = (x.cuda() for x in (q, k, v, do))
    o1, l1 = binding.attention_forward(qg, kg, vg, 0.125, True)
    o2, l2 = binding.attention_forward(qg, kg, vg, 0.125, False, window=(-1, 0))
    g1 = binding.attention_backward(qg, kg, vg, o1, dog, l1, 0.125, True)
    g2 = binding.attention_backward(qg, kg, vg, o2, dog, l2, 0.125, False, window=(-1, 0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_flash_attn_window_size_autograd():
    from exact_io_aware_30_amd import interface

    B, H, N, d = 1, 4, 640, 128
    q, k, v, do = _inputs("bf16", B, H, H, N, d, 11700)
    qg, kg, vg = (x.cuda().requires_grad_(True) for x in (q, k, v))
    o = interface.flash_attn(qg, kg, vg, causal=True, window_size=(128, -1))
    o.backward(do.cuda())
    torch.cuda.synchronize()
    ref = oracle.attention_backward(*(x.double().numpy() for x in (q, k, v, do)), 1 / math.sqrt(d), True,
                                    window=(128, -1))
    assert err_abs(to64(o), ref["o"]) <= TOL_O["bf16"]
    for name, t in (("dq", qg), ("dk", kg), ("dv", vg)):
        assert err_rel(to64(t.grad), ref[name]) <= TOL_G["bf16"], name
