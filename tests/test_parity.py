"""GPU parity: the HIP path through the C ABI against the CPU fp64 oracle.

Every input comes from the seeded generator in exact_io_aware_30_amd.workloads;
every expected value comes from oracle/.  Tolerances are in parity_utils.
Small workloads are compared element by element over every output; the two
large ones (bf16 [2,16,8192,128] causal and bf16 [1,8,65536,64] causal) on
sampled rows of O, L, dQ and sampled key rows of dK, dV, which the oracle
evaluates one by one, plus invariants that hold at any size.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_30_amd import workloads as wl
from parity_utils import (TOL_G, TOL_L, TOL_O, assert_fwd, assert_grad, check_finite, dkdv_cols_split, err_abs,
                          run_gpu, say, to64)

pytestmark = pytest.mark.gpu


def _binding():
    from exact_io_aware_30_amd import binding
    return binding


def _np(x):
    return x.to(torch.float64).numpy()


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "gpt2_medium", "ragged"])
def test_workload_full(name):
    w = wl.WORKLOADS[name]
    say(f"[parity] {w.describe()}")
    q, k, v, do = wl.make_inputs(w)
    out = run_gpu(q, k, v, do, w.scale, w.causal)
    check_finite(out)
    ref = oracle.attention_backward(_np(q), _np(k), _np(v), _np(do), w.scale, w.causal, row_block=1024)
    assert_fwd(w.dtype, out["o"], ref["o"], out["lse"], ref["lse"], name)
    for g in ("dq", "dk", "dv"):
        assert_grad(w.dtype, g, out[g], ref[g], name)


def _rows_every_block(N, rng, block):
    """The edge rows of the tiles, plus one random row in every ``block`` rows."""
    base = [0, 1, 31, 32, 63, 64, 127, 128, 129, N // 2 - 1, N // 2, N - 2, N - 1]
    per = np.arange(0, N, block) + rng.integers(0, block, (N + block - 1) // block)
    return np.unique(np.clip(np.concatenate([base, per]), 0, N - 1))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,heads", [
    ("long", [(0, 0), (1, 15), (0, 9)]),
    ("batch1_64k", [(0, 0), (0, 5)]),
])
def test_workload_sampled(name, heads):
    """The two large workloads on sampled outputs of whole heads: O, L and dQ
    of the tile-edge rows plus one random row in every 256-row forward block
    (every forward workgroup's rows are checked), dK and dV of keys 0, 1,
    127, 128, N - 1 plus one random key in every 32-key group (every wave of
    every dK/dV workgroup, the first key block's long accumulation loops
    included).  The oracle walks all query rows for the columns, split over
    host threads."""
    w = wl.WORKLOADS[name]
    say(f"[parity] {w.describe()} (sampled)")
    q, k, v, do = wl.make_inputs(w)
    out = run_gpu(q, k, v, do, w.scale, w.causal)
    check_finite(out)
    rng = np.random.default_rng(7)
    for (b, h) in heads:
        qh, kh, vh, doh = (_np(x[b, h]) for x in (q, k, v, do))
        rows = _rows_every_block(w.N, rng, 256)
        o_ref, L_ref = oracle.forward_rows(qh, kh, vh, w.scale, w.causal, rows)
        assert_fwd(w.dtype, out["o"][b, h, rows], o_ref, out["lse"][b, h, rows], L_ref, f"{name} head {b},{h}")
        dq_ref = oracle.dq_rows(qh, kh, vh, doh, w.scale, w.causal, rows)
        cols = np.unique(np.concatenate([[0, 1, 127, 128, w.N - 1],
                                         np.arange(0, w.N, 32) + rng.integers(0, 32, w.N // 32)]))
        dk_ref, dv_ref = dkdv_cols_split(qh, kh, vh, doh, w.scale, w.causal, cols)
        say(f"  head {b},{h}: {rows.size} rows, {cols.size} key columns")
        # Relative errors are normalised by the largest reference value over
        # the sampled rows of this head.
        assert_grad(w.dtype, "dq", out["dq"][b, h, rows], dq_ref, f"{name} head {b},{h}")
        assert_grad(w.dtype, "dk", out["dk"][b, h, cols], dk_ref, f"{name} head {b},{h}")
        assert_grad(w.dtype, "dv", out["dv"][b, h, cols], dv_ref, f"{name} head {b},{h}")
        # The first key block on its own: its workgroup runs the longest
        # query loop (every row of the head under the causal mask).
        first = cols < 128
        assert_grad(w.dtype, "dk", out["dk"][b, h, cols[first]], dk_ref[first], f"{name} head {b},{h} keys < 128")
        assert_grad(w.dtype, "dv", out["dv"][b, h, cols[first]], dv_ref[first], f"{name} head {b},{h} keys < 128")
    # Whole-tensor sums, printed as a diagnostic only (not a parity bar):
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i hold exactly for the true
    # gradient; on the GPU they carry the accumulated rounding of N rows.
    dk_sum = np.abs(out["dk"].sum(axis=2)).max()
    dv_gap = np.abs(out["dv"].sum(axis=2) - _np(do).sum(axis=2)).max()
    say(f"  diagnostic: max |sum_j dK_j| {dk_sum:.3e}, max |sum_j dV_j - sum_i dO_i| {dv_gap:.3e}")


# --------------------------------------------------------------------------
# Ragged lengths, every head dim, dtype and mask
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_sweep(dtype, d, causal):
    # 2500: past the short-sequence cut (2048), the pipelined d = 128 and 8-wave d = 64 forwards
    for N in (1, 17, 127, 129, 1999, 2500):
        seed = 20000 + N * 7 + d + (1 if causal else 0) + (2 if dtype == "bf16" else 0)
        w = wl.Workload(f"sweep_N{N}", dtype, 1, 2, N, d, causal, 2.0 if N == 129 else 1.0, seed)
        say(f"[parity] {w.describe()}")
        q, k, v, do = wl.make_inputs(w)
        out = run_gpu(q, k, v, do, w.scale, w.causal)
        check_finite(out)
        ref = oracle.attention_backward(_np(q), _np(k), _np(v), _np(do), w.scale, w.causal)
        assert_fwd(dtype, out["o"], ref["o"], out["lse"], ref["lse"], f"N={N}")
        for g in ("dq", "dk", "dv"):
            if N == 1 and g in ("dq", "dk"):
                # one key: P = 1 and dS = dP - D vanishes up to the two fp32
                # summation orders of dO.v (the reference is exactly 0)
                assert np.max(np.abs(out[g])) <= 1e-3, g
                continue
            assert_grad(dtype, g, out[g], ref[g], f"N={N}")


# --------------------------------------------------------------------------
# The pre-pass on its own (same O and dO on both sides)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64), ("bf16", 32)])
def test_preprocess(dtype, d):
    B, H, N = 2, 3, 777
    say(f"[parity] preprocess {dtype} d={d}")
    o = wl.make_tensor((B, H, N, d), dtype, 31 + d)
    do = wl.make_tensor((B, H, N, d), dtype, 32 + d)
    delta = torch.full((B, H, N), float("nan"), device="cuda")
    _binding().fa_bwd_preprocess(o.cuda(), do.cuda(), delta)
    torch.cuda.synchronize()
    got = to64(delta)
    ref = oracle.delta_rowsum(_np(o), _np(do))
    bound = 1e-5 * np.sum(np.abs(_np(o) * _np(do)), axis=-1) + 1e-6
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))


# --------------------------------------------------------------------------
# Special cases, guard bands, determinism, streams
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64), ("bf16", 32)])
def test_causal_row0_is_v0(dtype, d):
    w = wl.Workload("row0", dtype, 2, 3, 300, d, True, 1.0, 555 + d)
    say(f"[parity] {w.describe()}")
    q, k, v, do = wl.make_inputs(w)
    o, lse = _binding().attention_forward(q.cuda(), k.cuda(), v.cuda(), w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])
    l0 = w.scale * (_np(q)[:, :, 0] * _np(k)[:, :, 0]).sum(-1)
    assert np.max(np.abs(to64(lse)[:, :, 0] - l0)) <= TOL_L


def _guarded(shape, dtype, guard=64, fill=float("nan")):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * guard,), 7.0, dtype=dtype, device="cuda")
    buf[guard:guard + n] = fill
    return buf, buf[guard:guard + n].view(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_guard_bands_and_poisoned_outputs(causal):
    w = wl.Workload("guards", "bf16", 1, 3, 200, 64, causal, 1.0, 777)
    say(f"[parity] {w.describe()}")
    b = _binding()
    q, k, v, do = (x.cuda() for x in wl.make_inputs(w))
    shp, rows = tuple(q.shape), tuple(q.shape[:3])
    ob, o = _guarded(shp, q.dtype)
    lb, lse = _guarded(rows, torch.float32)
    b.fa_fwd(q, k, v, o, lse, w.scale, causal)
    db, delta = _guarded(rows, torch.float32)
    b.fa_bwd_preprocess(o, do, delta)
    gb = [_guarded(shp, q.dtype) for _ in range(3)]
    b.fa_bwd(q, k, v, do, lse, delta, gb[0][1], gb[1][1], gb[2][1], w.scale, causal)
    torch.cuda.synchronize()
    for buf, view in [(ob, o), (lb, lse), (db, delta)] + gb:
        guard = 64
        assert torch.all(buf[:guard] == 7.0) and torch.all(buf[-guard:] == 7.0), "guard band overwritten"
        assert torch.all(torch.isfinite(view.float())), "an output element was never written"


def test_deterministic_and_split_calls_match():
    w = wl.Workload("determinism", "bf16", 2, 4, 1000, 128, True, 1.0, 999)
    say(f"[parity] {w.describe()}")
    b = _binding()
    q, k, v, do = (x.cuda() for x in wl.make_inputs(w))
    res = []
    for _ in range(2):
        o, lse = b.attention_forward(q, k, v, w.scale, True)
        dq, dk, dv, delta = b.attention_backward(q, k, v, o, do, lse, w.scale, True)
        res.append((o, lse, dq, dk, dv, delta))
    dk2, dv2, dq2 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    o, lse, dq, dk, dv, delta = res[0]
    b.fa_bwd_dkdv(q, k, v, do, lse, delta, dk2, dv2, w.scale, True)
    b.fa_bwd_dq(q, k, v, do, lse, delta, dq2, w.scale, True)
    torch.cuda.synchronize()
    for a, c in zip(res[0], res[1]):
        assert torch.equal(a, c), "run-to-run difference"
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2) and torch.equal(dq, dq2)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_inputs_are_read_only(d):
    """No entry point writes to its inputs: the dK/dV kernel works on a copy
    of V with its signs flipped in LDS (or in registers), never on V itself;
    the grouped-query split path and the packed form included."""
    w = wl.Workload("readonly", "bf16", 2, 4, 333, d, True, 1.0, 4100 + d)
    say(f"[parity] {w.describe()}: inputs unchanged")
    b = _binding()
    q, k, v, do = (x.cuda() for x in wl.make_inputs(w))
    kg, vg = k[:, :1].contiguous(), v[:, :1].contiguous()  # one key/value head: the head split
    snap = [x.clone() for x in (q, k, v, do, kg, vg)]
    o, lse = b.attention_forward(q, k, v, w.scale, True)
    lse_s, o_s = lse.clone(), o.clone()
    dq, dk, dv, delta = b.attention_backward(q, k, v, o, do, lse, w.scale, True)
    delta_s = delta.clone()
    b.fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, w.scale, True)
    og, lg = b.attention_forward(q, kg, vg, w.scale, True)
    assert b.fa_bwd_workspace_size(2, 4, 1, 333, d) > 0
    b.attention_backward(q, kg, vg, og, do, lg, w.scale, True)
    T = 2 * 333
    cu = torch.tensor([0, 333, T], dtype=torch.int32, device="cuda")
    qp, kp, vp, dop = (x.transpose(0, 1).reshape(4, T, d).contiguous() for x in (q, k, v, do))
    snap_p = [x.clone() for x in (qp, kp, vp, dop, cu)]
    op, lp = b.attention_forward_varlen(qp, kp, vp, cu, 333, w.scale, True)
    b.attention_backward_varlen(qp, kp, vp, op, dop, lp, cu, 333, w.scale, True)
    torch.cuda.synchronize()
    for before, after in zip(snap, (q, k, v, do, kg, vg)):
        assert torch.equal(before, after), "an input was modified"
    for before, after in zip(snap_p, (qp, kp, vp, dop, cu)):
        assert torch.equal(before, after), "a packed input was modified"
    assert torch.equal(lse, lse_s) and torch.equal(o, o_s) and torch.equal(delta, delta_s)


def test_side_stream():
    w = wl.Workload("stream", "fp16", 1, 4, 640, 64, False, 1.0, 4242)
    say(f"[parity] {w.describe()} on a side stream")
    b = _binding()
    q, k, v, do = (x.cuda() for x in wl.make_inputs(w))
    o_ref, lse_ref = b.attention_forward(q, k, v, w.scale, False)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = b.attention_forward(q, k, v, w.scale, False)
    s.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_tolerances_written_down():
    # the bars the parity tests apply
    assert TOL_O == {"fp16": 4e-3, "bf16": 3e-2} and TOL_L == 1e-4 and TOL_G == {"fp16": 1e-2, "bf16": 5e-2}
    assert err_abs(np.zeros(0), np.zeros(0)) == 0.0
