"""Parity where every row's running maximum moves after its first key tile.

The forward keeps a reference maximum per row and moves it (rescaling the row
sum and the accumulator by alpha = 2^(m_old - m_new)) only when a tile's row
maximum exceeds it by more than 8 base-2 units ("flash-attn-triton" docs,
Fig. 3, the update per tile, and "Tiling softmax is exact algebra": alpha is
the correction that keeps the tiled result exact).  With i.i.d. N(0, 1)
inputs that almost never happens after the first tile, so these inputs are
built to climb: make_rising_inputs adds a staircase to the scores along the
key axis (steps of 12 base-2 units at key blocks 1, 2, the middle one and
the last one).  The host checks on the very inputs the GPU gets that the
move rule fires after the first tile in every row that sees a whole step
block, at least twice in rows that see every step (three times or more in
nine rows out of ten); then the HIP path is
compared with the oracle element by element at the parity tolerances, for
every forward form (the short-sequence 4-wave kernel at N = 1500; at
N = 2500 the pipelined kernel at d = 128 and the 8-wave plain one at d = 64),
fp16 and bf16, causal and full.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_30_amd import workloads as wl
from parity_utils import assert_fwd, assert_grad, check_finite, run_gpu, say

# 1500: 24 key tiles of 64, the reference moves at tiles 1, 2, 12, 23 (the
# short-sequence forward); 2500: 40 tiles, moves at 1, 2, 20, 39 (the long
# forwards: at d = 128 the pipelined kernel, whose four unrolled steps each
# see a move).
N_RISE = (1500, 2500)
TILE = 64       # the forward's key tile at every head dimension
SLACK = 8.0     # base-2 units a tile's row maximum must exceed the reference by

CASES = [(n, dt, d, causal) for n in N_RISE for dt in ("fp16", "bf16") for d in (32, 64, 128)
         for causal in (False, True)]


def _workload(n, dt, d, causal):
    return wl.Workload(f"rising_{dt}_d{d}_{'causal' if causal else 'full'}_N{n}", dt, 1, 2, n, d, causal, 1.0,
                       7100 + n + d + (1 if causal else 0) + (2 if dt == "bf16" else 0))


def move_counts(qh, kh, scale, causal):
    """Per query row: how often the reference maximum moves after the first
    key tile under the rule above (tiles of TILE keys, scores in base-2
    units, every lane on its own), and the row maximum's total rise over the
    first tile's maximum.  fp64 on the rounded inputs."""
    n = qh.shape[0]
    s = (qh @ kh.T) * (scale * math.log2(math.e))
    if causal:
        s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    nt = (n + TILE - 1) // TILE
    tmax = np.stack([s[:, t * TILE:(t + 1) * TILE].max(axis=1) for t in range(nt)], axis=1)
    ref = tmax[:, 0].copy()
    moves = np.zeros(n, dtype=np.int64)
    for t in range(1, nt):
        mv = tmax[:, t] > ref + SLACK
        ref = np.where(mv, tmax[:, t], ref)
        moves += mv
    return moves, tmax.max(axis=1) - tmax[:, 0]


def check_rising(q, k, w):
    """Assert the move rule fires as designed on every head of (q, k)."""
    steps = wl.rise_steps(w.N)
    nt = (w.N + TILE - 1) // TILE
    assert steps == [1, 2, nt // 2, nt - 1], steps
    rows = np.arange(w.N)
    # rows that see all of key block 1, and rows that see all of every step
    # block (the last block is the ragged tail: rows that see its first key)
    see_one = rows >= (2 * TILE - 1 if w.causal else 0)
    see_all = rows >= (steps[-1] * TILE if w.causal else 0)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            qh, kh = (x[b, h].to(torch.float64).numpy() for x in (q, k))
            moves, rise = move_counts(qh, kh, w.scale, w.causal)
            assert np.all(moves[see_one] >= 1), f"head {b},{h}: a row never moves after its first tile"
            assert np.all(rise[see_one] > SLACK)
            assert np.all(moves[see_all] >= 2), f"head {b},{h}: a row moves fewer than 2 times"
            assert np.mean(moves[see_all] >= 3) >= 0.9, f"head {b},{h}: under 90% of rows move 3 times"
            assert see_all.sum() > 0 and see_one.sum() > w.N // 2


@pytest.mark.parametrize("n,dt,d,causal", CASES)
def test_rising_inputs_move_the_reference(n, dt, d, causal):
    """Host logic: the planted inputs fire the move rule (no GPU)."""
    w = _workload(n, dt, d, causal)
    q, k, _, _ = wl.make_rising_inputs(w)
    check_rising(q, k, w)


@pytest.mark.gpu
@pytest.mark.parametrize("n,dt,d,causal", CASES)
def test_parity_running_max_moves(n, dt, d, causal):
    w = _workload(n, dt, d, causal)
    say(f"[parity] {w.describe()} rising scores (reference moves after tile 0)")
    q, k, v, do = wl.make_rising_inputs(w)
    check_rising(q, k, w)
    out = run_gpu(q, k, v, do, w.scale, w.causal)
    check_finite(out)
    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    ref = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), w.scale, w.causal)
    assert_fwd(dt, out["o"], ref["o"], out["lse"], ref["lse"], w.name)
    for g in ("dq", "dk", "dv"):
        assert_grad(dt, g, out[g], ref[g], w.name)
