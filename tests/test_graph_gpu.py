"""The hot path under HIP graph capture: one forward + backward step (fa_fwd,
fa_bwd_preprocess, fa_bwd) captured into a graph and replayed several times,
with eager work and synchronisation between the replays, gives the eager
step's outputs bit for bit on every replay (the kernels are deterministic,
allocate nothing and enqueue no memset)."""

import pytest
import torch

from exact_io_aware_30_amd import workloads as wl
from parity_utils import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("fp16", 64, False)])
def test_step_replays_in_a_graph(dtype, d, causal):
    from exact_io_aware_30_amd import binding

    say(f"[graph] {dtype} d={d} causal={causal}")
    w = wl.Workload("graph", dtype, 2, 4, 1000, d, causal, 1.0, 14000 + d)
    q, k, v, do = (x.cuda() for x in wl.make_inputs(w))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    outs = (o, lse, delta, dq, dk, dv)

    def step():
        binding.fa_fwd(q, k, v, o, lse, w.scale, causal)
        binding.fa_bwd_preprocess(o, do, delta)
        binding.fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, w.scale, causal)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        x = torch.randn(256, 256, device="cuda")
        (x @ x).sum().item()  # eager work and a synchronisation between replays
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {rep}"
