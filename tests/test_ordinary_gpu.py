"""The ordinary-attention comparator the benchmark times beside the tiled
kernels (library GEMMs, softmax and elementwise kernels with S and P in
device memory) computes the same attention: checked against the oracle to
the same tolerances as the HIP path."""

import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_30_amd import workloads as wl
from parity_utils import TOL_G, TOL_L, TOL_O, err_abs, err_rel, say, to64

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,B,H,N,d,causal", [
    ("bf16", 2, 3, 300, 64, True),
    ("fp16", 1, 2, 257, 128, False),
    ("fp16", 2, 2, 100, 32, True),
])
def test_ordinary_comparator_matches_oracle(dtype, B, H, N, d, causal):
    say(f"[ordinary] {dtype} B={B} H={H} N={N} d={d} causal={causal}")
    w = wl.Workload("cmp", dtype, B, H, N, d, causal, 1.0, 13000 + N)
    q, k, v, do = wl.make_inputs(w)
    mask = bench.causal_mask(N, "cuda") if causal else None
    o, dq, dk, dv = bench.ordinary_attention(*(x.cuda() for x in (q, k, v, do)), w.scale, causal, mask)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(*(x.double().numpy() for x in (q, k, v, do)), w.scale, causal)
    assert err_abs(to64(o), ref["o"]) <= TOL_O[dtype]
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert err_rel(to64(g), ref[name]) <= TOL_G[dtype], name


def test_peak_growth_of_the_tiled_step_is_zero():
    w = wl.WORKLOADS["gpt2_medium"]
    args = bench._inputs(w, torch.device("cuda:0"))
    grown = bench._peak_growth(lambda: bench._flash_step(*args, w.scale, w.causal))
    assert grown == 0
