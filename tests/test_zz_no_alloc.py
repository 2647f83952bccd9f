"""fa_bwd_ex_scratch, the backward that allocates nothing, against
fa_bwd_ex_ws with a caller workspace of the rule's size: the same split,
so dQ, dK and dV must be the same bits.  Two calls in a row on the shared
static array, the second on a smaller input (its partials overwrite only
part of what the first left), then the first shape again; workspaces and
outputs are poisoned with NaN beforehand, so a read of a partial row that
the call did not write, or an output element left unwritten, shows."""

import pytest
import torch

from exact_io_aware_30_amd import binding
from exact_io_aware_30_amd import workloads as wl
from parity_utils import say

pytestmark = pytest.mark.gpu

# (dtype, B, H, Hkv, N, d, causal): both split the query heads of a group
SHAPES = [("bf16", 2, 8, 1, 1000, 128, True), ("fp16", 1, 4, 2, 300, 64, False)]


def _inputs(dt, B, H, Hkv, N, d, seed):
    dev = torch.device("cuda")
    q = wl.make_tensor((B, H, N, d), dt, seed, dev)
    k = wl.make_tensor((B, Hkv, N, d), dt, seed + 1, dev)
    v = wl.make_tensor((B, Hkv, N, d), dt, seed + 2, dev)
    do = wl.make_tensor((B, H, N, d), dt, seed + 3, dev)
    return q, k, v, do


def _poisoned(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def _run(shape, seed):
    dt, B, H, Hkv, N, d, causal = shape
    say(f"[no-alloc] {dt} [B={B},H={H},Hkv={Hkv},N={N},d={d}] {'causal' if causal else 'full'} seed={seed}")
    scale = d ** -0.5
    window = (-1, 0) if causal else (-1, -1)
    q, k, v, do = _inputs(dt, B, H, Hkv, N, d, seed)
    o, lse = binding.attention_forward(q, k, v, scale, causal)
    delta = torch.empty(B, H, N, device="cuda")
    binding.fa_bwd_preprocess(o, do, delta)
    need = binding.fa_bwd_workspace_size(B, H, Hkv, N, d)
    assert 0 < need <= binding.SCRATCH_BYTES, need  # the call takes the split path and fits the array
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN float32 partials
    ref = [_poisoned(x.shape, x.dtype) for x in (q, k, v)]
    binding.fa_bwd_ex_ws(q, k, v, do, lse, delta, ref[0], ref[1], ref[2], scale, window, ws)
    got = [_poisoned(x.shape, x.dtype) for x in (q, k, v)]
    binding.fa_bwd_ex_scratch(q, k, v, do, lse, delta, got[0], got[1], got[2], scale, window)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(b.float()).all(), f"{name}: the workspace form left NaN"
        assert torch.equal(a, b), f"{name}: the scratch form differs from the workspace form"
    return got


def test_scratch_form_matches_workspace_form():
    first = _run(SHAPES[0], 8100)
    _run(SHAPES[1], 8200)          # smaller: part of the array still holds the first call's partials
    again = _run(SHAPES[0], 8100)  # the first shape again, after the smaller call
    for a, b in zip(first, again):
        assert torch.equal(a, b)
