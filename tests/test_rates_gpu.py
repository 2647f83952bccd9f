"""The instruction-rate loops behind the benchmark's ceilings, on the GPU:
every rate positive and in a range the MI355X can reach (dense bf16 MFMA
under the published 2.5 PFLOP/s; an exponential no faster than an FMA; the
per-score sequence, which holds an exponential and several other vector
instructions, slower than either; the interleaved MFMA + vector loop no
faster than its longer half and no slower than both halves; LDS-fed MFMA
loops no faster than the register-fed one; the atomic dQ accumulation
giving every sum exactly, in both grid orders)."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.gpu


def test_rates_are_plausible():
    r = bench.probe_rates()
    print(r, flush=True)
    assert r["compute_units"] >= 1
    assert 200.0 < r["mfma_bf16_tflops"] < 2600.0
    assert 0 < r["exp_tlanes_per_s"] <= r["fma_tlanes_per_s"] * 1.05
    assert 0 < r["softmax_tscores_per_s"] < r["exp_tlanes_per_s"]
    # the interleaved pair takes at least as long as its longer half, at most both halves (5% timing slack)
    longer = max(r["pair_mfma_ms"], r["pair_valu_ms"])
    assert 0.95 * longer <= r["pair_both_ms"] <= 1.05 * (r["pair_mfma_ms"] + r["pair_valu_ms"])


def test_lds_rates_are_plausible():
    r = bench.probe_lds()
    print(r, flush=True)
    assert r["compute_units"] >= 1
    assert r["lds_read_tbs"] > 0
    assert 200.0 < r["mfma_regs_tflops"] < 2600.0
    # an operand read from LDS cannot make the matrix core faster (5% timing slack)
    assert 0 < r["mfma_lds2_tflops"] <= 1.05 * r["mfma_lds1_tflops"] <= 1.05 * 1.05 * r["mfma_regs_tflops"]


def test_atomic_accumulation_is_exact_and_timed():
    r = bench.probe_atomic(N=2048, BH=8)
    print(r, flush=True)
    assert r["wrong_sums"] == 0
    assert r["atomic_ms_head_per_xcd"] > 0 and r["atomic_ms_head_spread"] > 0 and r["plain_rmw_ms"] > 0
    assert 0 < r["atomic_tbs"] < 100 and r["plain_tbs"] > 0
