"""GPU parity of the workspace forms of the backward (fa_bwd_ex_ws,
fa_bwd_varlen_ws), in which the query heads that share a key/value head are
split over several dK/dV workgroups and their float32 partial sums added up
by a second pass.  Checked against the oracle's grouped-query and packed
forms at the parity tolerances, on shapes with ragged tails, windows and
both masks; with workspaces of every size from none to more than enough
(fewer splits, same tolerances; none: the bits of fa_bwd_ex); dQ is the
unsplit kernel's, bit for bit; repeated calls give the same bits."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_30_amd import workloads as wl
from parity_utils import TOL_G, TOL_L, TOL_O, err_abs, err_rel, say, to64

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, H, Hkv, N, d, window (None: full mask; (-1, 0): causal)
    ("bf16", 1, 8, 1, 1000, 64, (-1, 0)),
    ("fp16", 2, 6, 2, 257, 128, None),
    ("bf16", 1, 16, 1, 300, 32, (50, 10)),
    ("fp16", 1, 12, 3, 513, 128, (-1, 0)),
    ("bf16", 2, 4, 1, 129, 128, (64, 0)),
    ("bf16", 1, 8, 1, 2500, 128, (-1, 0)),  # past the short-sequence cut (2048)
]


def _inputs(dtype, B, H, Hkv, N, d, seed):
    q = wl.make_tensor((B, H, N, d), dtype, seed)
    k = wl.make_tensor((B, Hkv, N, d), dtype, seed + 1)
    v = wl.make_tensor((B, Hkv, N, d), dtype, seed + 2)
    do = wl.make_tensor((B, H, N, d), dtype, seed + 3)
    return q, k, v, do


def _forward(qg, kg, vg, dog, scale, win):
    from exact_io_aware_30_amd import binding

    o = torch.empty_like(qg)
    lse = torch.empty(qg.shape[:3], dtype=torch.float32, device="cuda")
    binding.fa_fwd_ex(qg, kg, vg, o, lse, scale, win)
    delta = torch.empty_like(lse)
    binding.fa_bwd_preprocess(o, dog, delta)
    return o, lse, delta


def _backward_ws(qg, kg, vg, dog, lse, delta, scale, win, nbytes):
    from exact_io_aware_30_amd import binding

    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    binding.fa_bwd_ex_ws(qg, kg, vg, dog, lse, delta, dq, dk, dv, scale, win, ws)
    return dq, dk, dv


@pytest.mark.parametrize("dtype,B,H,Hkv,N,d,window", CASES)
def test_split_backward_matches_oracle(dtype, B, H, Hkv, N, d, window):
    from exact_io_aware_30_amd import binding

    say(f"[gqa-split] {dtype} B={B} H={H} Hkv={Hkv} N={N} d={d} window={window}")
    nbytes = binding.fa_bwd_workspace_size(B, H, Hkv, N, d)
    assert nbytes > 0  # every case is small enough for the split to apply
    q, k, v, do = _inputs(dtype, B, H, Hkv, N, d, 14000 + H + 10 * Hkv + N + d)
    scale = 1.0 / math.sqrt(d)
    win = (-1, -1) if window is None else window
    qg, kg, vg, dog = (x.cuda() for x in (q, k, v, do))
    o, lse, delta = _forward(qg, kg, vg, dog, scale, win)
    dq, dk, dv = _backward_ws(qg, kg, vg, dog, lse, delta, scale, win, nbytes)
    dq0, dk0, dv0 = _backward_ws(qg, kg, vg, dog, lse, delta, scale, win, 0)  # no workspace: fa_bwd_ex
    dq1, dk1, dv1 = _backward_ws(qg, kg, vg, dog, lse, delta, scale, win, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq0)  # the dQ kernel does not depend on the split
    assert torch.equal(dk, dk1) and torch.equal(dv, dv1)  # same workspace, same bits
    causal = window == (-1, 0)
    ref = oracle.attention_backward_gqa(*(x.double().numpy() for x in (q, k, v, do)), scale, causal,
                                        window=None if (window is None or causal) else window)
    eo, el = err_abs(to64(o), ref["o"]), err_abs(to64(lse), ref["lse"])
    say(f"  O {eo:.3e}  L {el:.3e}")
    assert eo <= TOL_O[dtype] and el <= TOL_L
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dk unsplit", dk0), ("dv unsplit", dv0)):
        g = to64(t)
        assert np.all(np.isfinite(g)), name
        e = err_rel(g, ref[name.split()[0]])
        say(f"  {name} {e:.3e}")
        assert e <= TOL_G[dtype], name


def test_every_workspace_size_gives_a_correct_split():
    """Workspaces too small for the chosen split run with fewer splits (the
    largest divisor of the group size that fits); below the smallest split,
    with none.  Every size is checked against the oracle."""
    from exact_io_aware_30_amd import binding

    dtype, B, H, Hkv, N, d = "fp16", 1, 12, 1, 300, 64
    q, k, v, do = _inputs(dtype, B, H, Hkv, N, d, 14500)
    scale = 1.0 / math.sqrt(d)
    qg, kg, vg, dog = (x.cuda() for x in (q, k, v, do))
    o, lse, delta = _forward(qg, kg, vg, dog, scale, (-1, 0))
    full = binding.fa_bwd_workspace_size(B, H, Hkv, N, d)
    per_split = 2 * B * Hkv * N * d * 4  # float32 dK and dV partials of one split
    assert full % per_split == 0 and full // per_split == 12  # 3 key blocks: every head its own split
    ref = oracle.attention_backward_gqa(*(x.double().numpy() for x in (q, k, v, do)), scale, True)
    results = {}
    for nbytes in (0, per_split, 2 * per_split, 5 * per_split, 6 * per_split, full, full + 4096):
        dq, dk, dv = _backward_ws(qg, kg, vg, dog, lse, delta, scale, (-1, 0), nbytes)
        torch.cuda.synchronize()
        for name, t in (("dk", dk), ("dv", dv)):
            e = err_rel(to64(t), ref[name])
            say(f"  workspace {nbytes // per_split} splits' worth: {name} {e:.3e}")
            assert e <= TOL_G[dtype], (nbytes, name)
        results[nbytes] = (dk, dv)
    # room for one split runs unsplit: the bits of no workspace
    assert torch.equal(results[0][0], results[per_split][0]) and torch.equal(results[0][1], results[per_split][1])
    # more room than the rule asks for changes nothing
    assert torch.equal(results[full][0], results[full + 4096][0])


def test_interface_gradients_with_split():
    """flash_attn's backward takes the split path by itself for few
    key/value heads (the binding allocates the workspace)."""
    from exact_io_aware_30_amd import binding, interface

    B, H, Hkv, N, d = 1, 16, 1, 400, 128
    assert binding.fa_bwd_workspace_size(B, H, Hkv, N, d) > 0
    q, k, v, do = _inputs("bf16", B, H, Hkv, N, d, 14700)
    qg, kg, vg = (x.cuda().requires_grad_(True) for x in (q, k, v))
    o = interface.flash_attn(qg, kg, vg, causal=True)
    o.backward(do.cuda())
    torch.cuda.synchronize()
    ref = oracle.attention_backward_gqa(*(x.double().numpy() for x in (q, k, v, do)), 1 / math.sqrt(d), True)
    for name, t in (("dq", qg), ("dk", kg), ("dv", vg)):
        e = err_rel(to64(t.grad), ref[name])
        say(f"  {name} {e:.3e}")
        assert e <= TOL_G["bf16"], name


@pytest.mark.parametrize("dtype,H,Hkv,d,lens,causal,window", [
    ("bf16", 8, 1, 128, [300, 1, 0, 517, 64, 1000], True, None),
    ("fp16", 6, 2, 64, [129, 700, 33], False, (40, 40)),
])
def test_varlen_split_matches_oracle(dtype, H, Hkv, d, lens, causal, window):
    from exact_io_aware_30_amd import binding

    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, mx, B = int(cu[-1]), max(lens), len(lens)
    say(f"[varlen-split] {dtype} H={H} Hkv={Hkv} d={d} lens={lens} causal={causal} window={window}")
    nbytes = binding.fa_bwd_varlen_workspace_size(B, mx, T, H, Hkv, d)
    assert nbytes > 0
    q = wl.make_tensor((H, T, d), dtype, 15000 + T)
    k = wl.make_tensor((Hkv, T, d), dtype, 15001 + T)
    v = wl.make_tensor((Hkv, T, d), dtype, 15002 + T)
    do = wl.make_tensor((H, T, d), dtype, 15003 + T)
    scale = 1.0 / math.sqrt(d)
    qg, kg, vg, dog = (x.cuda() for x in (q, k, v, do))
    cug = torch.tensor(cu, device="cuda")
    o, lse = binding.attention_forward_varlen(qg, kg, vg, cug, mx, scale, causal, window)
    delta = torch.empty_like(lse)
    binding.fa_bwd_preprocess(o.view(1, H, T, d), dog.view(1, H, T, d), delta.view(1, H, T))
    win = binding._window(window, causal)
    outs = []
    for ws_bytes in (nbytes, 0):
        dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
        binding.fa_bwd_varlen_ws(qg, kg, vg, dog, lse, delta, dq, dk, dv, cug, mx, scale, win, ws)
        outs.append((dq, dk, dv))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    ref = oracle.attention_backward_varlen(*(x.double().numpy() for x in (q, k, v, do)), cu, scale, causal, window)
    for (dq, dk, dv), label in zip(outs, ("split", "unsplit")):
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            g = to64(t)
            assert np.all(np.isfinite(g)), name
            e = err_rel(g, ref[name])
            say(f"  {label} {name} {e:.3e}")
            assert e <= TOL_G[dtype], (label, name)
