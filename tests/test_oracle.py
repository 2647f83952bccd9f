"""Pins of the CPU fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a closed form, a
hand-derived example, an invariant, finite differences, a textbook/library
routine, or a size the pages print.  The mutation tests in
test_oracle_mutants.py show that plausible mistakes fail at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle.attention import attention_backward, attention_forward
from exact_io_aware_30_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def head(x):
    return x[None, None]


# --------------------------------------------------------------------------
# Safe softmax ("What is FlashAttention?", "Start with a safe softmax")
# --------------------------------------------------------------------------

def test_safe_softmax_rows_sum_to_one():
    s = rand((64, 37), 1, 3.0)
    for shift in (0.0, 1e4, -1e4):
        p = oracle.safe_softmax(s + shift)
        assert np.all(np.isfinite(p))
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
    # causal rows: row i sees keys 0..i
    sc = np.where(np.arange(37)[None, :] > np.arange(37)[:, None], -np.inf, rand((37, 37), 2))
    p = oracle.safe_softmax(sc)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
    assert np.all(p[np.triu_indices(37, 1)] == 0.0)


def test_safe_softmax_matches_library_and_masked_rows():
    s = rand((16, 50), 3, 2.0)
    np.testing.assert_allclose(oracle.safe_softmax(s), scipy.special.softmax(s, axis=1), rtol=1e-13, atol=0)
    s[3] = -np.inf
    p = oracle.safe_softmax(s)
    assert np.all(p[3] == 0.0) and not np.any(np.isnan(p))


# --------------------------------------------------------------------------
# Online softmax and the merge (flash-attn-triton docs, Fig. 3; tensortonic
# "What you will build", item 01)
# --------------------------------------------------------------------------

def _one_shot(s, v):
    p = oracle.safe_softmax(s)
    m = np.max(s, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        L = np.where(np.isfinite(m), m + np.log(np.sum(np.exp(s - np.where(np.isfinite(m), m, 0)[:, None]), axis=1)), -np.inf)
    return p @ v, L


@pytest.mark.parametrize("seed", range(6))
def test_merge_of_two_partials_equals_one_shot(seed):
    rng = np.random.default_rng(100 + seed)
    n = 41
    s = rng.standard_normal((9, n)) * (1 + 4 * seed)
    v = rng.standard_normal((n, 5))
    if seed == 4:
        s[:, :20] = -np.inf          # first half fully masked
    splits = [0, n, int(rng.integers(1, n))]  # empty halves and a random cut
    o_ref, L_ref = _one_shot(s, v)
    for c in splits:
        a = oracle.partial_softmax_state(s[:, :c], v[:c])
        b = oracle.partial_softmax_state(s[:, c:], v[c:])
        o, L = oracle.softmax.finish_state(oracle.merge_partials(a, b))
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(L, L_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tile", [1, 7, 16, 64, 100])
@pytest.mark.parametrize("q_scale", [1.0, 4.0])
def test_fig3_recurrence_equals_one_shot(tile, q_scale):
    rng = np.random.default_rng(7)
    q = rng.standard_normal((20, 8)) * q_scale
    k = rng.standard_normal((75, 8))
    v = rng.standard_normal((75, 8))
    s = (q @ k.T) / math.sqrt(8)
    o, L = oracle.online_softmax_tiles(s, v, tile)
    o_ref, L_ref = _one_shot(s, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, L_ref, rtol=1e-12, atol=1e-12)
    # and through the oracle's forward (rows of one head, full mask)
    o2, L2 = attention_forward(head(q), head(k[:20]), head(v[:20]), 1 / math.sqrt(8), False)
    o3, L3 = oracle.online_softmax_tiles((q @ k[:20].T) / math.sqrt(8), v[:20], tile)
    np.testing.assert_allclose(o2[0, 0], o3, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L2[0, 0], L3, rtol=1e-12, atol=1e-12)


def test_fig3_recurrence_with_masked_leading_tiles():
    rng = np.random.default_rng(8)
    s = rng.standard_normal((5, 30))
    s[:, :12] = -np.inf
    s[2, :] = -np.inf
    v = rng.standard_normal((30, 3))
    o, L = oracle.online_softmax_tiles(s, v, 8)
    o_ref, L_ref = _one_shot(s, v)
    assert not np.any(np.isnan(o))
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    assert L[2] == -np.inf and np.all(o[2] == 0)


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_values(causal):
    rng = np.random.default_rng(11)
    N, d = 13, 6
    q = rng.standard_normal((N, d))
    k = np.tile(rng.standard_normal((1, d)), (N, 1))
    v = rng.standard_normal((N, d))
    do = rng.standard_normal((N, d))
    out = attention_backward(head(q), head(k), head(v), head(do), 0.4, causal)
    if causal:
        mean = np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None]
    else:
        mean = np.tile(v.mean(axis=0), (N, 1))
    np.testing.assert_allclose(out["o"][0, 0], mean, rtol=1e-12, atol=1e-12)
    # every row's scores are constant, so sum_j dS_ij = 0 and dQ = dS K = 0
    assert np.max(np.abs(out["dq"])) <= 1e-12


@pytest.mark.parametrize("N", [1, 2, 9])
def test_causal_first_row_and_last_key(N):
    rng = np.random.default_rng(12 + N)
    d, scale = 5, 0.7
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    out = attention_backward(head(q), head(k), head(v), head(do), scale, True)
    np.testing.assert_array_equal(out["o"][0, 0, 0], v[0])
    assert abs(out["lse"][0, 0, 0] - scale * q[0] @ k[0]) <= 1e-13
    assert np.all(out["dq"][0, 0, 0] == 0.0)
    # key N-1 is seen only by query N-1 with weight P[N-1,N-1]
    s_last = scale * (q[N - 1] @ k.T)
    p_last = np.exp(s_last - s_last.max())
    p_last /= p_last.sum()
    np.testing.assert_allclose(out["dv"][0, 0, N - 1], p_last[N - 1] * do[N - 1], rtol=1e-12, atol=1e-14)
    if N == 1:
        np.testing.assert_array_equal(out["o"][0, 0], v)
        assert np.all(out["dq"] == 0) and np.all(out["dk"] == 0)
        np.testing.assert_array_equal(out["dv"][0, 0], do)


def test_hand_worked_two_by_two():
    """Two examples derived by hand from the definition (scale = 1).

    Example A (d = 1): q = [1, 1], k = [0, ln 3], v = [4, 8], dO = [1, 2].
      Full mask: both rows have P = [1/4, 3/4], O = 7, L = ln 4;
        dV = [3/4, 9/4]; dP rows [4, 8] and [8, 16]; D = [7, 14];
        dS rows [-3/4, 3/4] and [-3/2, 3/2]; dQ = [3/4 ln 3, 3/2 ln 3];
        dK = [-9/4, 9/4].
      Causal: row 0 has P = [1, 0], O = 4, L = 0; row 1 as above;
        dV = [3/2, 3/2]; dQ = [0, 3/2 ln 3]; dK = [-3/2, 3/2].
    Example B (d = 2, full): q = [[1,0],[0,1]], k = [[0,0],[ln 3, ln 2]],
      v = [[4,0],[8,3]], dO = identity.
      P rows [1/4, 3/4] and [1/3, 2/3]; O = [[7, 9/4], [20/3, 2]];
      L = [ln 4, ln 3]; dV = [[1/4, 1/3], [3/4, 2/3]];
      dQ = [3/4 (ln 3, ln 2), 2/3 (ln 3, ln 2)]; dK = [[-3/4, -2/3], [3/4, 2/3]].
    """
    l3, l2 = math.log(3), math.log(2)
    q = np.array([[1.0], [1.0]])
    k = np.array([[0.0], [l3]])
    v = np.array([[4.0], [8.0]])
    do = np.array([[1.0], [2.0]])
    full = attention_backward(head(q), head(k), head(v), head(do), 1.0, False)
    np.testing.assert_allclose(full["o"][0, 0, :, 0], [7, 7], rtol=1e-14)
    np.testing.assert_allclose(full["lse"][0, 0], [math.log(4)] * 2, rtol=1e-14)
    np.testing.assert_allclose(full["dv"][0, 0, :, 0], [0.75, 2.25], rtol=1e-14)
    np.testing.assert_allclose(full["delta"][0, 0], [7, 14], rtol=1e-14)
    np.testing.assert_allclose(full["dq"][0, 0, :, 0], [0.75 * l3, 1.5 * l3], rtol=1e-14)
    np.testing.assert_allclose(full["dk"][0, 0, :, 0], [-2.25, 2.25], rtol=1e-14)
    cau = attention_backward(head(q), head(k), head(v), head(do), 1.0, True)
    np.testing.assert_allclose(cau["o"][0, 0, :, 0], [4, 7], rtol=1e-14)
    np.testing.assert_allclose(cau["lse"][0, 0], [0.0, math.log(4)], atol=1e-15)
    np.testing.assert_allclose(cau["dv"][0, 0, :, 0], [1.5, 1.5], rtol=1e-14)
    np.testing.assert_allclose(cau["dq"][0, 0, :, 0], [0.0, 1.5 * l3], atol=1e-15)
    np.testing.assert_allclose(cau["dk"][0, 0, :, 0], [-1.5, 1.5], rtol=1e-14)

    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    k = np.array([[0.0, 0.0], [l3, l2]])
    v = np.array([[4.0, 0.0], [8.0, 3.0]])
    do = np.eye(2)
    b = attention_backward(head(q), head(k), head(v), head(do), 1.0, False)
    np.testing.assert_allclose(b["o"][0, 0], [[7, 2.25], [20 / 3, 2]], rtol=1e-14)
    np.testing.assert_allclose(b["lse"][0, 0], [math.log(4), math.log(3)], rtol=1e-14)
    np.testing.assert_allclose(b["dv"][0, 0], [[0.25, 1 / 3], [0.75, 2 / 3]], rtol=1e-14)
    np.testing.assert_allclose(b["dq"][0, 0], [[0.75 * l3, 0.75 * l2], [2 / 3 * l3, 2 / 3 * l2]], rtol=1e-14)
    np.testing.assert_allclose(b["dk"][0, 0], [[-0.75, -2 / 3], [0.75, 2 / 3]], rtol=1e-14)


# --------------------------------------------------------------------------
# Finite differences of f = sum(dO o O)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 1), (3, 2), (5, 4), (8, 3)])
def test_gradients_match_central_differences(causal, N, d):
    rng = np.random.default_rng(1000 * N + d + int(causal))
    q, k, v, do = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
    scale = 0.8
    out = attention_backward(q, k, v, do, scale, causal)
    h = 1e-6

    def f(qq, kk, vv):
        o, _ = attention_forward(qq, kk, vv, scale, causal)
        return float(np.sum(do * o))

    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if x is t else t for t in (q, k, v)]
            args_m = [xm if x is t else t for t in (q, k, v)]
            g[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        err = np.max(np.abs(g - out[name])) / max(np.max(np.abs(g)), 1e-3)
        assert err <= 1e-7, (name, err)


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    B, H, N, d = 2, 3, 40, 8
    q, k, v, do = (rand((B, H, N, d), 20 + i) for i in range(4))
    out = attention_backward(q, k, v, do, 0.35, causal)
    # softmax is shift invariant along each row: sum_j dS_ij = 0, so sum_j dK_j = 0
    assert np.max(np.abs(out["dk"].sum(axis=2))) <= 1e-10
    # rows of P sum to 1: sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(out["dv"].sum(axis=2), do.sum(axis=2), rtol=1e-10, atol=1e-10)
    # D = rowsum(P o dP) = rowsum(dO o O)
    np.testing.assert_allclose(out["delta"], out["delta_o"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.delta_rowsum(out["o"], do), out["delta_o"], rtol=1e-14, atol=1e-14)
    # adding a constant vector c to every value row adds c to every output row
    c = rand((1, 1, 1, d), 99)
    o2, _ = attention_forward(q, k, v + c, 0.35, causal)
    np.testing.assert_allclose(o2, out["o"] + c, rtol=1e-12, atol=1e-12)
    # outputs and L from the forward agree with the backward's own recompute
    o, L = attention_forward(q, k, v, 0.35, causal)
    np.testing.assert_allclose(o, out["o"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(L, out["lse"], rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------
# Library routine: torch fp64 on the CPU (explicit softmax + autograd, SDPA)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(17, 8), (64, 32)])
def test_against_torch_fp64(causal, N, d):
    B, H = 2, 2
    q, k, v, do = (rand((B, H, N, d), 40 + i) for i in range(4))
    scale = 1 / math.sqrt(d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = (tq @ tk.transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    lse_t = torch.logsumexp(s, dim=-1)
    o_t = torch.softmax(s, dim=-1) @ tv
    o_t.backward(torch.tensor(do))
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), is_causal=causal, scale=scale)
    out = attention_backward(q, k, v, do, scale, causal)
    o, L = attention_forward(q, k, v, scale, causal)

    def rel(a, b):
        return np.max(np.abs(a - b)) / np.max(np.abs(b))

    assert rel(o, o_t.detach().numpy()) <= 1e-12
    assert rel(o, sdpa.numpy()) <= 1e-12
    assert rel(L, lse_t.detach().numpy()) <= 1e-12
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert rel(out[name], t.grad.numpy()) <= 1e-12, name


# --------------------------------------------------------------------------
# Row blocking and the samplers compute the same definition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_row_blocking_and_samplers(causal):
    B, H, N, d = 1, 2, 77, 16
    q, k, v, do = (rand((B, H, N, d), 60 + i, 2.0 if i == 0 else 1.0) for i in range(4))
    scale = 0.25
    ref = attention_backward(q, k, v, do, scale, causal)
    for rb in (1, 10, 32, 77, 500):
        blk = attention_backward(q, k, v, do, scale, causal, row_block=rb)
        for name in ("o", "lse", "dq", "dk", "dv"):
            np.testing.assert_allclose(blk[name], ref[name], rtol=1e-12, atol=1e-12, err_msg=f"{name} rb={rb}")
        o, L = attention_forward(q, k, v, scale, causal, row_block=rb)
        np.testing.assert_allclose(o, ref["o"], rtol=1e-12, atol=1e-12)
    rows = np.array([0, 1, 31, 32, 76])
    for h in range(H):
        o, L = oracle.forward_rows(q[0, h], k[0, h], v[0, h], scale, causal, rows)
        np.testing.assert_allclose(o, ref["o"][0, h, rows], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(L, ref["lse"][0, h, rows], rtol=1e-12, atol=1e-12)
        dq = oracle.dq_rows(q[0, h], k[0, h], v[0, h], do[0, h], scale, causal, rows)
        np.testing.assert_allclose(dq, ref["dq"][0, h, rows], rtol=1e-12, atol=1e-12)
        dk, dv = oracle.dkdv_cols(q[0, h], k[0, h], v[0, h], do[0, h], scale, causal, rows, row_block=13)
        np.testing.assert_allclose(dk, ref["dk"][0, h, rows], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dv, ref["dv"][0, h, rows], rtol=1e-12, atol=1e-12)
        # Shares of disjoint query-row ranges covering [0, N) add up to the
        # whole gradient; a range before every sampled key's first visible
        # row (causal) contributes nothing.
        cuts = [0, 5, 31, 32, 60, N]
        parts = [oracle.dkdv_cols(q[0, h], k[0, h], v[0, h], do[0, h], scale, causal, rows, row_block=7,
                                  rows=(a, b)) for a, b in zip(cuts[:-1], cuts[1:])]
        np.testing.assert_allclose(sum(p[0] for p in parts), ref["dk"][0, h, rows], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sum(p[1] for p in parts), ref["dv"][0, h, rows], rtol=1e-12, atol=1e-12)
        first = oracle.dkdv_cols(q[0, h], k[0, h], v[0, h], do[0, h], scale, causal, rows[1:], rows=(0, 1))
        assert (np.all(first[0] == 0) and np.all(first[1] == 0)) if causal else np.any(first[1] != 0)


# --------------------------------------------------------------------------
# Sizes the pages print (footprint calculator and the IO model's constants)
# --------------------------------------------------------------------------

def test_page_sizes():
    g = json.load(open(os.path.join(GOLDEN, "page_sizes.json")))
    e = g["score_matrix_8k_fp16_per_head"]
    fp = workloads.footprint(1, 1, 8192, 64, 2)
    assert fp["score"] == e["value_bytes"] == 128 * 2**20
    e = g["score_table_entries_4096"]
    assert workloads.footprint(1, 1, 4096, 64, 1)["score"] == e["value_entries"]
    assert round(e["value_entries"] / 1e6, 1) == 16.8
    e = g["tile_bytes_128x128_fp16"]
    assert e["inputs"]["BLOCK_M"] * e["inputs"]["BLOCK_N"] * e["inputs"]["elem_bytes"] == e["value_bytes"] == 32 * 1024
    e = g["d2_over_M"]
    r = e["inputs"]["d"] ** 2 / e["inputs"]["M"]
    assert abs(r - 1 / 25) / (1 / 25) <= e["tolerance_relative"]
    # the linear part is Q, K, V, O plus one fp32 L per row
    fp = workloads.footprint(2, 16, 8192, 128, 2, capacity_bytes=288e9)
    assert fp["linear"] == 4 * 2 * 16 * 8192 * 128 * 2 + 4 * 2 * 16 * 8192
    assert fp["n_max"] ** 2 * 2 * 16 * 2 <= 288e9 < (fp["n_max"] + 1) ** 2 * 2 * 16 * 2


def test_workload_counts():
    w = workloads.WORKLOADS["long"]
    f, b, fb = workloads.flops(w)
    assert f == 2 * 16 * 8192**2 * 128 * 2 and b == 2 * 16 * 8192**2 * 128 * 5 and fb == f + b
    kf = workloads.kernel_flops(w)
    assert kf["fwd"] == f and kf["bwd_dkdv"] + kf["bwd_dq"] == b
    by = workloads.algorithmic_bytes(w)
    T = w.elems
    assert sum(by.values()) == 17 * T * 2 + 24 * w.B * w.H * w.N
    q, k, v, do = workloads.make_inputs(workloads.WORKLOADS["tiny"])
    assert q.dtype == torch.float16 and q.shape == (1, 2, 256, 64)
    q2, *_ = workloads.make_inputs(workloads.WORKLOADS["tiny"])
    assert torch.equal(q, q2)
    qr, *_ = workloads.make_inputs(workloads.WORKLOADS["ragged"])
    g = torch.Generator().manual_seed(1003)
    assert torch.equal(qr, (torch.randn((3, 12, 2000, 32), generator=g) * 4).half())


# --------------------------------------------------------------------------
# Grouped-query attention (flash attention note, "Versions and Evolution")
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 1), (3, 3)])
def test_gqa_against_torch_fp64(causal, H, Hkv):
    # torch autograd through repeat_interleave sums the gradients of the
    # repeated key/value heads by itself; SDPA gives the forward.
    B, N, d = 2, 23, 8
    q, do = (rand((B, H, N, d), 60 + i) for i in range(2))
    k, v = (rand((B, Hkv, N, d), 70 + i) for i in range(2))
    scale = 0.4
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    G = H // Hkv
    s = (tq @ tk.repeat_interleave(G, dim=1).transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o_t = torch.softmax(s, dim=-1) @ tv.repeat_interleave(G, dim=1)
    o_t.backward(torch.tensor(do))
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k).repeat_interleave(G, dim=1), torch.tensor(v).repeat_interleave(G, dim=1),
        is_causal=causal, scale=scale)
    out = oracle.attention_backward_gqa(q, k, v, do, scale, causal)
    o, _ = oracle.attention_forward_gqa(q, k, v, scale, causal)
    assert out["dk"].shape == k.shape and out["dv"].shape == v.shape and out["dq"].shape == q.shape

    def rel(a, b):
        return np.max(np.abs(a - b)) / np.max(np.abs(b))

    assert rel(o, sdpa.numpy()) <= 1e-12
    assert rel(out["o"], o_t.detach().numpy()) <= 1e-12
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert rel(out[name], t.grad.numpy()) <= 1e-12, name


def test_gqa_one_group_is_plain_attention_and_mqa_sums_heads():
    B, H, N, d = 1, 4, 19, 6
    q, k, v, do = (rand((B, H, N, d), 80 + i) for i in range(4))
    plain = attention_backward(q, k, v, do, 0.5, True)
    grouped = oracle.attention_backward_gqa(q, k, v, do, 0.5, True)
    for name in ("o", "dq", "dk", "dv", "lse"):
        np.testing.assert_array_equal(grouped[name], plain[name])
    # multi-query: one key/value head read by every query head; its gradient
    # is the sum of what each head alone would give it
    k1, v1 = k[:, :1], v[:, :1]
    mqa = oracle.attention_backward_gqa(q, k1, v1, do, 0.5, False)
    dk = sum(attention_backward(q[:, h:h + 1], k1, v1, do[:, h:h + 1], 0.5, False)["dk"] for h in range(H))
    dv = sum(attention_backward(q[:, h:h + 1], k1, v1, do[:, h:h + 1], 0.5, False)["dv"] for h in range(H))
    np.testing.assert_allclose(mqa["dk"], dk, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(mqa["dv"], dv, rtol=1e-13, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.attention_forward_gqa(q, k[:, :3], v[:, :3], 0.5, False)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_gradients_match_central_differences(causal):
    rng = np.random.default_rng(515 + int(causal))
    H, Hkv, N, d = 4, 2, 5, 3
    q, do = (rng.standard_normal((1, H, N, d)) for _ in range(2))
    k, v = (rng.standard_normal((1, Hkv, N, d)) for _ in range(2))
    out = oracle.attention_backward_gqa(q, k, v, do, 0.7, causal)
    h = 1e-6

    def f(kk, vv):
        o, _ = oracle.attention_forward_gqa(q, kk, vv, 0.7, causal)
        return float(np.sum(do * o))

    for name, x in (("dk", k), ("dv", v)):
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            g[idx] = (f(*[xp if x is t else t for t in (k, v)]) - f(*[xm if x is t else t for t in (k, v)])) / (2 * h)
        assert np.max(np.abs(g - out[name])) / np.max(np.abs(g)) <= 1e-7, name


# --------------------------------------------------------------------------
# Sliding windows (flash-attn-triton docs, "Scope")
# --------------------------------------------------------------------------

def _torch_window_mask(N, window, causal):
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    ok = torch.ones(N, N, dtype=torch.bool)
    if causal:
        ok &= j <= i
    left, right = window
    if left >= 0:
        ok &= j >= i - left
    if right >= 0:
        ok &= j <= i + right
    return ok


@pytest.mark.parametrize("window,causal", [((3, 2), False), ((5, -1), False), ((-1, 4), False), ((7, 0), False),
                                           ((4, -1), True), ((0, 6), False)])
def test_window_against_torch_fp64(window, causal):
    B, H, N, d = 2, 2, 29, 8
    q, k, v, do = (rand((B, H, N, d), 120 + i) for i in range(4))
    scale = 0.45
    ok = _torch_window_mask(N, window, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = ((tq @ tk.transpose(-1, -2)) * scale).masked_fill(~ok, float("-inf"))
    lse_t = torch.logsumexp(s, dim=-1)
    o_t = torch.softmax(s, dim=-1) @ tv
    o_t.backward(torch.tensor(do))
    sdpa = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k), torch.tensor(v),
                                                            attn_mask=ok, scale=scale)
    out = attention_backward(q, k, v, do, scale, causal, window=window)
    o, L = attention_forward(q, k, v, scale, causal, window=window, row_block=7)

    def rel(a, b):
        return np.max(np.abs(a - b)) / np.max(np.abs(b))

    assert rel(o, sdpa.numpy()) <= 1e-12
    assert rel(out["o"], o_t.detach().numpy()) <= 1e-12
    assert rel(L, lse_t.detach().numpy()) <= 1e-12
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert rel(out[name], t.grad.numpy()) <= 1e-12, name


def test_window_special_cases():
    B, H, N, d = 1, 2, 17, 5
    q, k, v, do = (rand((B, H, N, d), 140 + i) for i in range(4))
    plain_c = attention_backward(q, k, v, do, 0.6, True)
    plain_f = attention_backward(q, k, v, do, 0.6, False)
    # (-1, 0) is the causal mask and (-1, -1) the full one, bit for bit
    for ref, window in ((plain_c, (-1, 0)), (plain_f, (-1, -1)), (plain_f, (N - 1, N - 1))):
        got = attention_backward(q, k, v, do, 0.6, False, window=window)
        for name in ("o", "lse", "dq", "dk", "dv"):
            np.testing.assert_allclose(got[name], ref[name], rtol=1e-14, atol=1e-14)
    # (0, 0): each query sees only its own key, so O = V, L = scale q.k,
    # dV = dO and dQ = dK = 0 (a softmax over one element is constant)
    one = attention_backward(q, k, v, do, 0.6, False, window=(0, 0))
    np.testing.assert_allclose(one["o"], v, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(one["lse"], 0.6 * np.sum(q * k, axis=-1), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(one["dv"], do, rtol=1e-14, atol=1e-14)
    assert np.max(np.abs(one["dq"])) == 0 and np.max(np.abs(one["dk"])) == 0


@pytest.mark.parametrize("window", [(2, 1), (1, -1)])
def test_window_gradients_match_central_differences(window):
    rng = np.random.default_rng(77 + window[0])
    q, k, v, do = (rng.standard_normal((1, 1, 6, 3)) for _ in range(4))
    out = attention_backward(q, k, v, do, 0.9, False, window=window)
    h = 1e-6

    def f(qq, kk, vv):
        o, _ = attention_forward(qq, kk, vv, 0.9, False, window=window)
        return float(np.sum(do * o))

    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            g[idx] = (f(*[xp if x is t else t for t in (q, k, v)]) - f(*[xm if x is t else t for t in (q, k, v)])) / (2 * h)
        assert np.max(np.abs(g - out[name])) / np.max(np.abs(g)) <= 1e-7, name


# --------------------------------------------------------------------------
# Packed variable-length batches (flash-attn-triton docs, "Scope")
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (False, (3, 2)), (True, (4, -1))])
def test_varlen_against_torch_block_diagonal(causal, window):
    # the packed sequences attended as one long sequence under a
    # block-diagonal mask (plus the causal mask / window within each block)
    lens = [5, 1, 0, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    T, H, Hkv, d = int(cu[-1]), 4, 2, 6
    q, do = (rand((H, T, d), 160 + i) for i in range(2))
    k, v = (rand((Hkv, T, d), 170 + i) for i in range(2))
    seq = np.repeat(np.arange(len(lens)), lens)
    pos = np.concatenate([np.arange(n) for n in lens])
    i_, j_ = pos[:, None], pos[None, :]
    ok = seq[:, None] == seq[None, :]
    if causal:
        ok &= j_ <= i_
    if window is not None:
        if window[0] >= 0:
            ok &= j_ >= i_ - window[0]
        if window[1] >= 0:
            ok &= j_ <= i_ + window[1]
    okt = torch.tensor(ok)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = ((tq @ tk.repeat_interleave(2, dim=0).transpose(-1, -2)) * 0.5).masked_fill(~okt, float("-inf"))
    o_t = torch.softmax(s, dim=-1) @ tv.repeat_interleave(2, dim=0)
    o_t.backward(torch.tensor(do))
    out = oracle.attention_backward_varlen(q, k, v, do, cu, 0.5, causal, window)

    def rel(a, b):
        return np.max(np.abs(a - b)) / np.max(np.abs(b))

    assert rel(out["o"], o_t.detach().numpy()) <= 1e-12
    assert rel(out["lse"], torch.logsumexp(s, -1).detach().numpy()) <= 1e-12
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert rel(out[name], t.grad.numpy()) <= 1e-12, name


def test_varlen_equal_lengths_is_the_batched_layout():
    B, H, N, d = 3, 2, 11, 4
    q, k, v, do = (rand((B, H, N, d), 180 + i) for i in range(4))
    packed = [x.transpose(1, 0, 2, 3).reshape(H, B * N, d) for x in (q, k, v, do)]
    out = oracle.attention_backward_varlen(*packed, np.arange(0, B * N + 1, N), 0.7, True)
    ref = attention_backward(q, k, v, do, 0.7, True)
    for name in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(out[name], ref[name].transpose(1, 0, 2, 3).reshape(H, B * N, d),
                                   rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(out["lse"], ref["lse"].transpose(1, 0, 2).reshape(H, B * N), rtol=1e-14,
                               atol=1e-14)
