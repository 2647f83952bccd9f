"""Planted mistakes in a copy of the oracle must fail its pins.

Each mutant is the oracle's attention module with one plausible error
inserted (a dropped term, a wrong sign, index or operand, a mask off by one),
loaded from source into a private namespace.  The real oracle is untouched.
The pin battery below is the same kind of check test_oracle.py makes: a
hand-derived example, central differences, invariants and torch fp64.
"""

import math
import os
import types

import numpy as np
import pytest
import torch

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = {
    "dropped_delta_term": ("ds = p * (dp - dsum[:, None])", "ds = p * dp"),
    "delta_sign": ("ds = p * (dp - dsum[:, None])", "ds = p * (dp + dsum[:, None])"),
    "dq_uses_v": ('out["dq"][b, h, r0:r1] = scale * (ds @ kh[:nk])', 'out["dq"][b, h, r0:r1] = scale * (ds @ vh[:nk])'),
    "dk_missing_scale": ('out["dk"][b, h, :nk] += scale * (ds.T @ qh[r0:r1])', 'out["dk"][b, h, :nk] += (ds.T @ qh[r0:r1])'),
    "dv_uses_q_rows": ('out["dv"][b, h, :nk] += p.T @ dob', 'out["dv"][b, h, :nk] += p.T @ qh[r0:r1]'),
    "causal_excludes_diagonal": ("s = np.where(j > i, -np.inf, s)", "s = np.where(j >= i, -np.inf, s)"),
    "scale_twice": ("s = scale * (qh[r0:r1] @ kh[:nk].T)", "s = scale * scale * (qh[r0:r1] @ kh[:nk].T)"),
    "lse_without_log": ("L = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)",
                        "L = np.where(live, m + np.where(live, l, 1.0), -np.inf)"),
    "no_max_subtraction": ("e = np.where(live[:, None], np.exp(s - np.where(live, m, 0.0)[:, None]), 0.0)",
                           "e = np.where(live[:, None], np.exp(s), 0.0)\n    m = np.zeros_like(m)"),
    "transposed_p_in_bwd_pv": ("ob = p @ vh[:nk]", "ob = p.T @ vh[:nk]"),
    "transposed_p_in_fwd_pv": ("o[b, h, r0:r1] = p @ v[b, h, :nk]", "o[b, h, r0:r1] = p.T @ v[b, h, :nk]"),
    "delta_wrong_axis": ("dsum = np.sum(p * dp, axis=1)", "dsum = np.sum(p * dp, axis=0)"),
    # sliding window: the left bound must keep key i - left
    "window_left_off_by_one": ("s = np.where(j < i - left, -np.inf, s)", "s = np.where(j <= i - left, -np.inf, s)"),
    "window_extent_too_short": ("nk = min(nk, r1 + window[1])", "nk = min(nk, r1 + window[1] - 1)"),
    # grouped-query attention: query head h must read key/value head h // G
    "gqa_heads_interleaved": ("return attention_forward(q, np.repeat(_as64(k), G, axis=1), np.repeat(_as64(v), G, axis=1)",
                              "return attention_forward(q, np.tile(_as64(k), (1, G, 1, 1)), "
                              "np.tile(_as64(v), (1, G, 1, 1))"),
    "gqa_grad_not_summed": ('out[name] = out[name].reshape(B, Hkv, G, N, d).sum(axis=2)',
                            'out[name] = out[name].reshape(B, Hkv, G, N, d)[:, :, 0]'),
    "gqa_grad_wrong_group_axis": ('out[name] = out[name].reshape(B, Hkv, G, N, d).sum(axis=2)',
                                  'out[name] = out[name].reshape(B, G, Hkv, N, d).sum(axis=1)'),
}


def load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def pin_battery(m):
    """Raises AssertionError if the module fails any pin."""
    rng = np.random.default_rng(5)
    # hand example A (see test_oracle.test_hand_worked_two_by_two)
    l3 = math.log(3)
    q = np.array([[[[1.0], [1.0]]]])
    k = np.array([[[[0.0], [l3]]]])
    v = np.array([[[[4.0], [8.0]]]])
    do = np.array([[[[1.0], [2.0]]]])
    for causal, o_ref, L_ref, dq_ref, dk_ref, dv_ref in (
        (False, [7, 7], [math.log(4)] * 2, [0.75 * l3, 1.5 * l3], [-2.25, 2.25], [0.75, 2.25]),
        (True, [4, 7], [0.0, math.log(4)], [0.0, 1.5 * l3], [-1.5, 1.5], [1.5, 1.5]),
    ):
        out = m.attention_backward(q, k, v, do, 1.0, causal)
        o, L = m.attention_forward(q, k, v, 1.0, causal)
        np.testing.assert_allclose(o[0, 0, :, 0], o_ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(L[0, 0], L_ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(out["dq"][0, 0, :, 0], dq_ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(out["dk"][0, 0, :, 0], dk_ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(out["dv"][0, 0, :, 0], dv_ref, rtol=1e-12, atol=1e-14)
    # torch fp64 on small random heads, one with scores in the thousands
    # (safe softmax: no overflow when the row maximum is subtracted)
    for causal, qs in ((False, 1.0), (True, 1.0), (False, 300.0)):
        N, d = 5, 3
        q, k, v, do = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
        q = q * qs
        out = m.attention_backward(q, k, v, do, 0.8, causal)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = (tq @ tk.transpose(-1, -2)) * 0.8
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        ot = torch.softmax(s, -1) @ tv
        ot.backward(torch.tensor(do))
        o, L = m.attention_forward(q, k, v, 0.8, causal)
        np.testing.assert_allclose(o, ot.detach().numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(L, torch.logsumexp(s, -1).detach().numpy(), rtol=1e-10, atol=1e-12)
        for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
            np.testing.assert_allclose(out[name], t.grad.numpy(), rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(out["o"], ot.detach().numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(out["delta"], out["delta_o"], rtol=1e-10, atol=1e-12)
        assert np.max(np.abs(out["dk"].sum(axis=2))) <= 1e-10
    # a sliding window against torch fp64 with the same boolean mask
    N, d = 9, 3
    q, k, v, do = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
    i_, j_ = torch.arange(N)[:, None], torch.arange(N)[None, :]
    ok = (j_ >= i_ - 2) & (j_ <= i_ + 1)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = ((tq @ tk.transpose(-1, -2)) * 0.7).masked_fill(~ok, float("-inf"))
    ot = torch.softmax(s, -1) @ tv
    ot.backward(torch.tensor(do))
    out = m.attention_backward(q, k, v, do, 0.7, False, window=(2, 1), row_block=3)
    o, L = m.attention_forward(q, k, v, 0.7, False, window=(2, 1), row_block=2)
    np.testing.assert_allclose(o, ot.detach().numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(L, torch.logsumexp(s, -1).detach().numpy(), rtol=1e-10, atol=1e-12)
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(out[name], t.grad.numpy(), rtol=1e-9, atol=1e-11)
    # grouped-query forms against torch fp64 through repeat_interleave
    for causal in (False, True):
        H, Hkv, N, d = 4, 2, 5, 3
        q, do = (rng.standard_normal((1, H, N, d)) for _ in range(2))
        k, v = (rng.standard_normal((1, Hkv, N, d)) for _ in range(2))
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = (tq @ tk.repeat_interleave(2, dim=1).transpose(-1, -2)) * 0.8
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        ot = torch.softmax(s, -1) @ tv.repeat_interleave(2, dim=1)
        ot.backward(torch.tensor(do))
        o, _ = m.attention_forward_gqa(q, k, v, 0.8, causal)
        out = m.attention_backward_gqa(q, k, v, do, 0.8, causal)
        np.testing.assert_allclose(o, ot.detach().numpy(), rtol=1e-10, atol=1e-12)
        for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
            np.testing.assert_allclose(out[name], t.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_real_oracle_passes_battery():
    import oracle.attention as real
    pin_battery(real)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    mut = load_mutant(old, new)
    with pytest.raises(Exception):
        pin_battery(mut)
