"""The Python API over the C ABI: flash_attn, its autograd.Function and the
FlashSelfAttention module ("flash-attn-triton" docs, "Scope" and "using it").

GPU tests compare autograd's gradients with the oracle's (same seeded inputs,
the parity tolerances), and the module with an fp64 CPU reference whose
attention step is the oracle.  The CPU test checks that the API refuses CPU
tensors instead of computing anything itself.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_30_amd import workloads as wl
from parity_utils import TOL_G, TOL_O, err_abs, err_rel, say, to64


def test_cpu_tensors_are_refused():
    from exact_io_aware_30_amd import interface

    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        interface.flash_attn(q, q, q)
    with pytest.raises(ValueError, match="head dimension"):
        interface.flash_attn(*(torch.zeros(1, 1, 8, 48, dtype=torch.float16),) * 3)
    with pytest.raises(ValueError, match="one of"):
        interface.FlashSelfAttention(embed_dim=96, num_heads=2)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_flash_attn_autograd_matches_oracle(dtype, causal, d):
    from exact_io_aware_30_amd import interface

    B, H, N = 2, 3, 131
    say(f"[interface] flash_attn autograd {dtype} d={d} causal={causal}")
    q, k, v, do = (wl.make_tensor((B, H, N, d), dtype, 7000 + 10 * d + i + 5 * causal) for i in range(4))
    qg, kg, vg = (x.cuda().requires_grad_(True) for x in (q, k, v))
    o = interface.flash_attn(qg, kg, vg, causal=causal)
    o.backward(do.cuda())
    torch.cuda.synchronize()
    ref = oracle.attention_backward(*(x.double().numpy() for x in (q, k, v, do)), 1.0 / math.sqrt(d), causal)
    eo = err_abs(to64(o), ref["o"])
    say(f"  O {eo:.3e}")
    assert eo <= TOL_O[dtype]
    for name, t in (("dq", qg), ("dk", kg), ("dv", vg)):
        e = err_rel(to64(t.grad), ref[name])
        say(f"  {name} {e:.3e}")
        assert np.all(np.isfinite(to64(t.grad))) and e <= TOL_G[dtype]


@pytest.mark.gpu
def test_noncontiguous_inputs_and_explicit_scale():
    from exact_io_aware_30_amd import interface

    B, H, N, d = 1, 2, 70, 64
    base = wl.make_tensor((B, N, H, d), "fp16", 7100)
    q = base.transpose(1, 2)  # (B, H, N, d), not contiguous
    k, v = (wl.make_tensor((B, H, N, d), "fp16", 7101 + i) for i in range(2))
    o = interface.flash_attn(q.cuda(), k.cuda(), v.cuda(), causal=True, softmax_scale=0.3)
    ref_o, _ = oracle.attention_forward(*(x.double().numpy() for x in (q, k, v)), 0.3, True)
    assert err_abs(to64(o), ref_o) <= TOL_O["fp16"]


class _OracleAttention(torch.autograd.Function):
    """fp64 CPU attention through the oracle, for the module reference."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal):
        ctx.save_for_backward(q, k, v)
        ctx.scale, ctx.causal = scale, causal
        return torch.from_numpy(oracle.attention_forward(q.numpy(), k.numpy(), v.numpy(), scale, causal)[0])

    @staticmethod
    def backward(ctx, do):
        q, k, v = ctx.saved_tensors
        r = oracle.attention_backward(q.numpy(), k.numpy(), v.numpy(), do.numpy(), ctx.scale, ctx.causal)
        return torch.from_numpy(r["dq"]), torch.from_numpy(r["dk"]), torch.from_numpy(r["dv"]), None, None


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [False, True])
def test_flash_self_attention_module(causal):
    from exact_io_aware_30_amd import interface

    torch.manual_seed(11)
    B, N, E, H = 2, 97, 256, 4
    say(f"[interface] FlashSelfAttention E={E} H={H} causal={causal}")
    mod = interface.FlashSelfAttention(E, H, causal=causal).to("cuda", torch.bfloat16)
    x = wl.make_tensor((B, N, E), "bf16", 7200 + causal).cuda().requires_grad_(True)
    dy = wl.make_tensor((B, N, E), "bf16", 7210 + causal).cuda()
    y = mod(x)
    y.backward(dy)
    torch.cuda.synchronize()
    # fp64 reference: the same bf16 parameters and input, the oracle for attention.
    W1, b1 = (p.detach().double().cpu() for p in (mod.in_proj.weight, mod.in_proj.bias))
    W2, b2 = (p.detach().double().cpu() for p in (mod.out_proj.weight, mod.out_proj.bias))
    W1, b1, W2, b2 = (p.requires_grad_(True) for p in (W1, b1, W2, b2))
    xr = x.detach().double().cpu().requires_grad_(True)
    qkv = (xr @ W1.T + b1).view(B, N, 3, H, E // H).permute(2, 0, 3, 1, 4)
    o = _OracleAttention.apply(qkv[0].contiguous(), qkv[1].contiguous(), qkv[2].contiguous(),
                               1.0 / math.sqrt(E // H), causal)
    yr = o.transpose(1, 2).reshape(B, N, E) @ W2.T + b2
    yr.backward(dy.double().cpu())
    ey = err_rel(to64(y), yr.detach().numpy())
    ex = err_rel(to64(x.grad), xr.grad.numpy())
    ew = err_rel(to64(mod.in_proj.weight.grad), W1.grad.numpy())
    say(f"  y {ey:.3e}  dx {ex:.3e}  dW_in {ew:.3e}")
    # bf16 storage of the projections' outputs adds rounding on both sides of
    # the attention; the gradient tolerance of the parity tests covers it.
    assert ey <= TOL_G["bf16"] and ex <= TOL_G["bf16"] and ew <= TOL_G["bf16"]
