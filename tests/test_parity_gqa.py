"""GPU parity of the grouped-query entry points (fa_fwd_gqa, fa_bwd_gqa and
its halves) against the oracle's grouped-query forms, on seeded inputs, at
the parity tolerances; plus the Python API with fewer key/value heads.
Shapes span several tiles with ragged tails; group sizes 1 (the plain path),
2, 4 and H (multi-query)."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_30_amd import workloads as wl
from parity_utils import TOL_G, TOL_L, TOL_O, err_abs, err_rel, say, to64

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, H, Hkv, N, d, causal
    ("bf16", 2, 8, 2, 300, 128, True),
    ("fp16", 1, 6, 1, 257, 64, False),
    ("bf16", 2, 4, 2, 129, 32, True),
    ("fp16", 1, 4, 4, 200, 128, False),
    ("bf16", 1, 8, 1, 1000, 64, True),
    # past the short-sequence cut (2048)
    ("bf16", 1, 4, 2, 2200, 128, True),
    ("fp16", 1, 4, 1, 2300, 64, False),
]


def _inputs(dtype, B, H, Hkv, N, d, seed):
    q = wl.make_tensor((B, H, N, d), dtype, seed)
    k = wl.make_tensor((B, Hkv, N, d), dtype, seed + 1)
    v = wl.make_tensor((B, Hkv, N, d), dtype, seed + 2)
    do = wl.make_tensor((B, H, N, d), dtype, seed + 3)
    return q, k, v, do


@pytest.mark.parametrize("dtype,B,H,Hkv,N,d,causal", CASES)
def test_gqa_matches_oracle(dtype, B, H, Hkv, N, d, causal):
    from exact_io_aware_30_amd import binding

    say(f"[gqa] {dtype} B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v, do = _inputs(dtype, B, H, Hkv, N, d, 9000 + H + 10 * Hkv + N)
    scale = 1.0 / math.sqrt(d)
    qg, kg, vg, dog = (x.cuda() for x in (q, k, v, do))
    o = torch.empty_like(qg)
    lse = torch.empty(qg.shape[:3], dtype=torch.float32, device="cuda")
    binding.fa_fwd_gqa(qg, kg, vg, o, lse, scale, causal)
    delta = torch.empty_like(lse)
    binding.fa_bwd_preprocess(o, dog, delta)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    binding.fa_bwd_gqa(qg, kg, vg, dog, lse, delta, dq, dk, dv, scale, causal)
    # the two halves on their own give the same bits
    dq2, dk2, dv2 = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    binding.fa_bwd_dkdv_gqa(qg, kg, vg, dog, lse, delta, dk2, dv2, scale, causal)
    binding.fa_bwd_dq_gqa(qg, kg, vg, dog, lse, delta, dq2, scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    ref = oracle.attention_backward_gqa(*(x.double().numpy() for x in (q, k, v, do)), scale, causal)
    eo, el = err_abs(to64(o), ref["o"]), err_abs(to64(lse), ref["lse"])
    say(f"  O {eo:.3e}  L {el:.3e}")
    assert eo <= TOL_O[dtype] and el <= TOL_L
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        g = to64(t)
        assert np.all(np.isfinite(g)), name
        e = err_rel(g, ref[name])
        say(f"  {name} {e:.3e}")
        assert e <= TOL_G[dtype], name


def test_gqa_with_one_group_equals_plain_entry_points():
    from exact_io_aware_30_amd import binding

    dtype, B, H, N, d = "bf16", 2, 3, 333, 64
    q, k, v, do = _inputs(dtype, B, H, H, N, d, 9500)
    qg, kg, vg, dog = (x.cuda() for x in (q, k, v, do))
    o1, l1 = binding.attention_forward(qg, kg, vg, 0.125, True)
    o2 = torch.empty_like(qg)
    l2 = torch.empty_like(l1)
    binding.fa_fwd_gqa(qg, kg, vg, o2, l2, 0.125, True)
    g1 = binding.attention_backward(qg, kg, vg, o1, dog, l1, 0.125, True)
    delta = torch.empty_like(l1)
    binding.fa_bwd_preprocess(o1, dog, delta)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    binding.fa_bwd_gqa(qg, kg, vg, dog, l1, delta, dq, dk, dv, 0.125, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(g1[0], dq) and torch.equal(g1[1], dk) and torch.equal(g1[2], dv)


def test_flash_attn_with_fewer_kv_heads():
    from exact_io_aware_30_amd import interface

    B, H, Hkv, N, d = 2, 8, 2, 150, 128
    q, k, v, do = _inputs("bf16", B, H, Hkv, N, d, 9600)
    qg, kg, vg = (x.cuda().requires_grad_(True) for x in (q, k, v))
    o = interface.flash_attn(qg, kg, vg, causal=True)
    o.backward(do.cuda())
    torch.cuda.synchronize()
    assert kg.grad.shape == kg.shape and vg.grad.shape == vg.shape
    ref = oracle.attention_backward_gqa(*(x.double().numpy() for x in (q, k, v, do)), 1 / math.sqrt(d), True)
    assert err_abs(to64(o), ref["o"]) <= TOL_O["bf16"]
    for name, t in (("dq", qg), ("dk", kg), ("dv", vg)):
        assert err_rel(to64(t.grad), ref[name]) <= TOL_G["bf16"], name
