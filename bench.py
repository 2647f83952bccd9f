"""Throughput of exact attention forward + backward on one MI355X.

One step = the whole hot path on one batch of synthetic input already resident
in device memory: fa_fwd, fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq (the last
two are what fa_bwd enqueues).  The workload is bf16 [B=2, H=16, N=8192,
d=128] with the causal mask.  FLOPs: forward 4 B H N^2 d, backward 10 B H N^2 d,
both halved under the causal mask.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --report    every workload: forward, backward and
                                forward+backward TFLOP/s (median of 30 timed
                                calls after 10 warm-up calls, min and max),
                                device-memory growth, and the oracle on one
                                head of each (a markdown table, then one JSON
                                line per workload), then the forward's MFMA
                                and vector-ALU ceilings per head dimension
                                from rates measured by libfa_rates.so
    python bench.py --sweep     bf16 causal d=128, B=1, H=16, N = 1K .. 64K:
                                one pass of each kernel per N (for hardware
                                counters) and its time
    python bench.py --compare   ordinary attention (library GEMMs, softmax,
                                S and P in device memory) beside the tiled
                                kernels on every workload: forward+backward
                                time, peak device memory, exact traffic
                                counts of both and, from the committed
                                counter summary, the measured bytes
    python bench.py --oom       bf16 causal d=128, B=1, H=16, N = 4K .. 128K:
                                peak memory and time of both versions until
                                ordinary attention runs out of memory
    python bench.py --variants  grouped-query heads, sliding windows, a packed
                                variable-length batch and the autograd
                                interface, forward+backward TFLOP/s over the
                                exact visible query-key pairs
    python bench.py --compare-step flash|ordinary --workload W
                                one forward+backward step of one version
                                (for hardware byte counters)
    --results PATH              also write every JSON record the run prints
                                to PATH as one JSON list (a results file)
    --graph                     also time the step captured once in a HIP
                                graph and replayed (graph_ms_per_step,
                                graph_tflops); `value` stays the eager rate

Without a mode option it prints one JSON line.  Besides the contract fields it carries
  roofline      the dominant kernel (longest average launch, timed with HIP
                events on the launch stream over the timed region) against
                the dense bf16 MFMA peak, plus its HBM traffic per launch
                from the committed rocprofv3 counter summary when that was
                taken on the current kernel sources (else null);
  cpu_baseline  the CPU fp64 oracle timed on 24 of the 32 heads of the same
                workload (a bounded sample), in the same unit;
  kernels       average duration, TFLOP/s and fraction of peak per kernel.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
METRIC = "attention fwd+bwd TFLOP/s (bf16 causal N=8192 d=128) + % of MFMA peak"
WORKLOAD = "long"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_traffic_long.txt")
LIBRARY = os.path.join(ROOT, "exact_io_aware_30_amd", "libfa_mi355x.so")


RECORDS = []  # every JSON record printed, for --results


def emit(record):
    """Print one JSON record on its own line and keep it for --results."""
    RECORDS.append(record)
    print(json.dumps(record), flush=True)


def library_hash():
    """First 16 hex digits of the SHA-256 of the built library: it changes
    exactly when the compiled kernels do (the build is byte-reproducible and
    comments do not reach it)."""
    try:
        with open(LIBRARY, "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()[:16]
    except OSError:
        return None


def traffic_from_summary(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if
    it was measured on the library that is built now."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    m = re.search(r"^library_hash:\s*(\S+)", text, re.M)
    if not m or m.group(1) != library_hash():
        return None
    m = re.search(rf"^traffic_bytes\s+{re.escape(kernel)}:\s*([0-9.eE+]+)", text, re.M)
    return float(m.group(1)) if m else None


def host_cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, heads: int = 24):
    """The oracle, as it stands, on the first `heads` of the B*H heads."""
    import numpy as np

    import oracle
    from exact_io_aware_30_amd import workloads

    q, k, v, do = workloads.make_inputs(w)
    one = [x.reshape(1, w.B * w.H, w.N, w.d)[:, :heads].to("cpu").double().numpy() for x in (q, k, v, do)]
    cores = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=cores)
    except Exception:
        pass
    t0 = time.perf_counter()
    oracle.attention_backward(*one, w.scale, w.causal, row_block=1024)
    dt = time.perf_counter() - t0
    sample = workloads.Workload("sample", w.dtype, 1, heads, w.N, w.d, w.causal, w.q_scale, w.seed)
    fb = workloads.flops(sample)[2]
    return {"value": fb / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"the first {heads} of {w.B * w.H} heads of {w.describe()}: fwd+bwd, {dt:.1f} s wall, "
                      f"numpy fp64",
            "seconds": round(dt, 3), "cpu_model": host_cpu_model()}


def _inputs(w, dev):
    import torch

    from exact_io_aware_30_amd import workloads

    q, k, v, do = (x.to(dev) for x in workloads.make_inputs(w))
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    return q, k, v, do, o, dq, dk, dv, lse, delta


def _median_ms(fn, warmup=10, reps=30):
    """Median, min and max of `reps` calls of fn timed with HIP events on the current stream."""
    import torch

    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2], t[0], t[-1]


def calib_copy(mib: int):
    """One device-to-device copy of `mib` MiB: a kernel of known traffic for
    scaling hardware byte counters."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def report():
    """Every workload: forward, backward, forward+backward; oracle on one head."""
    import torch

    from exact_io_aware_30_amd import binding, workloads

    dev = torch.device("cuda:0")
    rows = []
    for name, w in workloads.WORKLOADS.items():
        q, k, v, do, o, dq, dk, dv, lse, delta = _inputs(w, dev)
        torch.cuda.synchronize()
        fwd = lambda: binding.fa_fwd(q, k, v, o, lse, w.scale, w.causal)

        def bwd():
            binding.fa_bwd_preprocess(o, do, delta)
            binding.fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, w.scale, w.causal)

        def both():
            fwd()
            bwd()

        torch.cuda.reset_peak_memory_stats()
        before = torch.cuda.max_memory_allocated()
        both()
        torch.cuda.synchronize()
        grown = torch.cuda.max_memory_allocated() - before
        tf, tb, tfb = _median_ms(fwd), _median_ms(bwd), _median_ms(both)
        f, b, fb = workloads.flops(w)
        cb = cpu_baseline(w, heads=1)  # the oracle on the first head (heads are independent)
        r = {"workload": w.describe(), "fwd_ms": [round(x, 4) for x in tf], "bwd_ms": [round(x, 4) for x in tb],
             "fwd_bwd_ms": [round(x, 4) for x in tfb], "fwd_tflops": round(f / tf[0] / 1e9, 1),
             "bwd_tflops": round(b / tb[0] / 1e9, 1), "fwd_bwd_tflops": round(fb / tfb[0] / 1e9, 1),
             "frac_mfma_peak": round(fb / tfb[0] / 1e9 / PEAK_BF16_TFLOPS, 4),
             "device_memory_growth_bytes": int(grown),
             "oracle_one_head_s": cb["seconds"], "oracle_tflops": round(cb["value"], 4),
             "oracle_threads": cb["cores"]}
        rows.append(r)
        del q, k, v, do, o, dq, dk, dv, lse, delta
        torch.cuda.empty_cache()
    print("| workload | fwd ms (min-max) | bwd ms (min-max) | fwd+bwd ms | fwd TF/s | bwd TF/s | fwd+bwd TF/s "
          "| % of 2.5 PF | memory growth | oracle, one head |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['workload']} | {r['fwd_ms'][0]:.4f} ({r['fwd_ms'][1]:.4f}-{r['fwd_ms'][2]:.4f}) "
              f"| {r['bwd_ms'][0]:.4f} ({r['bwd_ms'][1]:.4f}-{r['bwd_ms'][2]:.4f}) | {r['fwd_bwd_ms'][0]:.4f} "
              f"| {r['fwd_tflops']} | {r['bwd_tflops']} | {r['fwd_bwd_tflops']} | {100 * r['frac_mfma_peak']:.1f} "
              f"| {r['device_memory_growth_bytes']} B | {r['oracle_one_head_s']} s ({r['oracle_tflops']} TF/s) |")
    for r in rows:
        emit(r)
    ceilings(rows)


RATES_LIBRARY = os.path.join(ROOT, "exact_io_aware_30_amd", "libfa_rates.so")


def probe_rates():
    """Instruction rates measured on the GPU by libfa_rates.so: dense bf16
    MFMA TFLOP/s, v_exp_f32 and v_fma_f32 lane-results per second, the
    forward's per-score vector sequence in scores per second (1e12 units),
    and the interleaved MFMA + vector loop's three timings."""
    import ctypes

    import torch

    lib = ctypes.CDLL(RATES_LIBRARY)
    lib.fa_rates_valu.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int, ctypes.c_void_p]
    lib.fa_rates_valu.restype = ctypes.c_int
    out = (ctypes.c_double * 8)()
    rc = lib.fa_rates_valu(out, 8, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"fa_rates_valu failed (status {rc})")
    return {"mfma_bf16_tflops": out[0], "exp_tlanes_per_s": out[1], "fma_tlanes_per_s": out[2],
            "softmax_tscores_per_s": out[3], "compute_units": int(out[4]),
            "pair_mfma_ms": out[5], "pair_valu_ms": out[6], "pair_both_ms": out[7],
            "pair_overlap": overlap_fraction(out[5], out[6], out[7])}


def probe_lds():
    """LDS rates measured by libfa_rates.so: ds_read_b128 alone (TB/s over
    the chip), and dense bf16 MFMA TFLOP/s with one, two or no 1 KiB operands
    read from LDS per MFMA."""
    import ctypes

    import torch

    lib = ctypes.CDLL(RATES_LIBRARY)
    lib.fa_rates_lds.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int, ctypes.c_void_p]
    lib.fa_rates_lds.restype = ctypes.c_int
    out = (ctypes.c_double * 6)()
    rc = lib.fa_rates_lds(out, 6, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"fa_rates_lds failed (status {rc})")
    return {"lds_read_tbs": out[0], "mfma_lds1_tflops": out[1], "mfma_lds2_tflops": out[2],
            "mfma_regs_tflops": out[3], "compute_units": int(out[4]), "lds_read_ms": out[5]}


def probe_atomic(N: int = 8192, BH: int = 32):
    """The atomic-dQ accumulation measured alone by libfa_rates.so (float32
    atomic adds of 32 x 128 tiles, one workgroup per 128-key block and head,
    causal, d = 128), beside the same traffic as plain read-add-write."""
    import ctypes

    import torch

    lib = ctypes.CDLL(RATES_LIBRARY)
    lib.fa_rates_atomic.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    lib.fa_rates_atomic.restype = ctypes.c_int
    out = (ctypes.c_double * 8)()
    rc = lib.fa_rates_atomic(out, 8, N, BH, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"fa_rates_atomic failed (status {rc})")
    return {"N": N, "BH": BH, "bytes": out[0], "atomic_ms_head_per_xcd": out[1], "atomic_ms_head_spread": out[2],
            "plain_rmw_ms": out[3], "atomic_tbs": out[4], "wrong_sums": int(out[5] + out[6]), "plain_tbs": out[7]}


def overlap_fraction(t_mfma: float, t_valu: float, t_both: float) -> float:
    """Share of the shorter half's time hidden under the longer one when both
    run interleaved: 0 = executed one after the other, 1 = fully hidden."""
    return (t_mfma + t_valu - t_both) / min(t_mfma, t_valu)


def forward_ceilings(rates, d: int):
    """Forward TFLOP/s ceilings at head dimension d from measured rates: the
    matrix core alone; the vector ALU alone (each score carries 4 d counted
    FLOPs and needs the per-score sequence: scale-and-subtract, exponential,
    row-sum add, half a max3, half a pack; the kernel adds address and mask
    work, so this bound is optimistic); and both executed one after the
    other, which is how the kernels' counters show them running."""
    mfma = float(rates["mfma_bf16_tflops"])
    valu = 4.0 * d * float(rates["softmax_tscores_per_s"])
    return {"d": d, "mfma_tflops": mfma, "valu_tflops": valu, "serial_tflops": 1.0 / (1.0 / mfma + 1.0 / valu)}


def ceilings(rows=()):
    """Measured ceilings beside the measured forward of each workload."""
    rates = probe_rates()
    print(f"\nceilings (measured on this GPU, {rates['compute_units']} CUs): dense bf16 MFMA "
          f"{rates['mfma_bf16_tflops']:.0f} TFLOP/s; v_exp_f32 {rates['exp_tlanes_per_s']:.1f}e12/s; "
          f"v_fma_f32 {rates['fma_tlanes_per_s']:.1f}e12/s; forward per-score sequence "
          f"{rates['softmax_tscores_per_s']:.2f}e12 scores/s; an interleaved loop of one MFMA per two scores' "
          f"vector work runs in {rates['pair_both_ms']:.3f} ms against {rates['pair_mfma_ms']:.3f} (MFMAs alone) and "
          f"{rates['pair_valu_ms']:.3f} (vector work alone): {100 * rates['pair_overlap']:.0f}% of the shorter half "
          f"hidden")
    print("| d | MFMA ceiling TF/s | VALU ceiling TF/s | both in series TF/s | measured forward TF/s |")
    print("|---|---|---|---|---|")
    out = []
    for d in (32, 64, 128):
        c = forward_ceilings(rates, d)
        meas = ", ".join(f"{r['fwd_tflops']} ({r['workload'].split(':')[0]})" for r in rows
                         if f",d={d}]" in r["workload"])
        print(f"| {d} | {c['mfma_tflops']:.0f} | {c['valu_tflops']:.0f} | {c['serial_tflops']:.0f} | {meas or '-'} |")
        out.append({k: (round(v, 1) if isinstance(v, float) else v) for k, v in c.items()})
    lds = probe_lds()
    print(f"LDS: ds_read_b128 alone {lds['lds_read_tbs']:.1f} TB/s over {lds['compute_units']} CUs; dense bf16 MFMA "
          f"{lds['mfma_regs_tflops']:.0f} TFLOP/s with operands in registers, {lds['mfma_lds1_tflops']:.0f} with one "
          f"1 KiB LDS operand per MFMA, {lds['mfma_lds2_tflops']:.0f} with two")
    at = probe_atomic()
    print(f"atomic dQ accumulation alone (bf16 [{at['BH']} heads, N={at['N']}, d=128] causal, 128-key blocks): "
          f"{at['bytes'] / 1e9:.2f} GB of float32 atomic adds in {at['atomic_ms_head_per_xcd']:.3f} ms "
          f"({at['atomic_tbs']:.2f} TB/s; {at['atomic_ms_head_spread']:.3f} ms with a head's blocks spread over "
          f"the XCDs; {at['wrong_sums']} wrong sums), against {at['plain_rmw_ms']:.3f} ms for the same traffic "
          f"as plain read-add-write")
    emit({"probe_rates": {k: (round(v, 3) if isinstance(v, float) else v) for k, v in rates.items()},
          "probe_lds": {k: (round(v, 3) if isinstance(v, float) else v) for k, v in lds.items()},
          "probe_atomic": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in at.items()},
          "forward_ceilings": out})


SWEEP_N = (1024, 2048, 4096, 8192, 16384, 32768, 65536)


def sweep():
    """bf16 causal d=128, B=1, H=16: one pass of each kernel per N, then its time."""
    import torch

    from exact_io_aware_30_amd import binding, workloads

    dev = torch.device("cuda:0")
    for n in SWEEP_N:
        w = workloads.Workload(f"sweep{n}", "bf16", 1, 16, n, 128, True, 1.0, 2000 + n // 1024)
        q, k, v, do, o, dq, dk, dv, lse, delta = _inputs(w, dev)
        torch.cuda.synchronize()
        binding.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
        binding.fa_bwd_preprocess(o, do, delta)
        binding.fa_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, w.scale, w.causal)
        binding.fa_bwd_dq(q, k, v, do, lse, delta, dq, w.scale, w.causal)
        torch.cuda.synchronize()
        fb = workloads.flops(w)[2]
        t = _median_ms(lambda: (binding.fa_fwd(q, k, v, o, lse, w.scale, w.causal),
                                binding.fa_bwd_preprocess(o, do, delta),
                                binding.fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, w.scale, w.causal)),
                       warmup=2, reps=5)
        emit({"N": n, "B": 1, "H": 16, "d": 128, "fwd_bwd_ms": round(t[0], 4),
              "fwd_bwd_tflops": round(fb / t[0] / 1e9, 1), "algorithmic_bytes": workloads.algorithmic_bytes(w)})
        del q, k, v, do, o, dq, dk, dv, lse, delta
        torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# Ordinary attention beside the tiled kernels: time, peak memory, the point
# where it runs out of memory, and the exact traffic of both versions
# ("flash-attn-triton" docs, "The argument", Table 2, "Work it out" / Fig. 2,
# "Scope"; "What is FlashAttention?", "Why is it faster if it does the same
# math?" and "What you will build")
# --------------------------------------------------------------------------

def ordinary_attention(q, k, v, do, scale, causal, mask=None):
    """Ordinary attention forward and backward on the GPU from library GEMMs,
    softmax and elementwise kernels: S = scale QK^T, the causal mask and
    P = softmax(S) go through device memory, then O = PV; backward dV = P^T dO,
    dP = dO V^T, dS = P o (dP - rowsum(P o dP)), dQ = scale dS K,
    dK = scale dS^T Q.  q, k, v, do: contiguous (B, H, N, d).  Every batched
    product takes contiguous operands (transposed N x d copies are made
    explicitly).  ``mask``: the (N, N) bool array of hidden entries (key
    after query), built by the caller.  Returns (o, dq, dk, dv)."""
    import torch

    B, H, N, d = q.shape
    q3, k3, v3, do3 = (x.reshape(B * H, N, d) for x in (q, k, v, do))
    kt = k3.transpose(1, 2).contiguous()
    s = torch.empty(B * H, N, N, dtype=q.dtype, device=q.device).baddbmm_(q3, kt, beta=0.0, alpha=scale)
    del kt
    if causal:
        s.masked_fill_(mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    del s
    o = torch.bmm(p, v3)
    dot = do3.transpose(1, 2).contiguous()
    dv = torch.bmm(dot, p).transpose(1, 2).contiguous()
    del dot
    vt = v3.transpose(1, 2).contiguous()
    dp = torch.bmm(do3, vt)
    del vt
    ds = torch.ops.aten._softmax_backward_data(dp, p, -1, p.dtype)
    del dp, p
    dq = torch.empty(B * H, N, d, dtype=q.dtype, device=q.device).baddbmm_(ds, k3, beta=0.0, alpha=scale)
    qt = q3.transpose(1, 2).contiguous()
    dk = torch.empty(B * H, d, N, dtype=q.dtype, device=q.device).baddbmm_(qt, ds, beta=0.0, alpha=scale)
    dk = dk.transpose(1, 2).contiguous()
    shape = (B, H, N, d)
    return o.view(shape), dq.view(shape), dk.view(shape), dv.view(shape)


def causal_mask(n, device):
    """(N, N) bool, True where the key comes after the query; built on the
    host and copied, so that building it launches no kernel."""
    import torch

    return torch.ones(n, n, dtype=torch.bool).triu_(1).to(device)


def _flash_step(q, k, v, do, o, dq, dk, dv, lse, delta, scale, causal):
    from exact_io_aware_30_amd import binding

    binding.fa_fwd(q, k, v, o, lse, scale, causal)
    binding.fa_bwd_preprocess(o, do, delta)
    binding.fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, scale, causal)


def _peak_growth(fn):
    """Device memory fn allocates at its peak beyond what was allocated before."""
    import torch

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    fn()
    torch.cuda.synchronize()
    return torch.cuda.max_memory_allocated() - base


def io_summary_bytes(path=os.path.join(ROOT, "profiles", "io_compare_counters.txt")):
    """{(workload, version): (read bytes, written bytes)} measured by the
    committed counter summary of one forward+backward step, or {}."""
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        m = re.match(r"^measured (\w+) (\w+): read (\d+) written (\d+)", line)
        if m:
            out[(m.group(1), m.group(2))] = (int(m.group(3)), int(m.group(4)))
    return out


COMPARE_WORKLOADS = ("tiny", "gpt2_medium", "ragged", "long", "batch1_64k")


def compare():
    """Both versions on every workload: forward+backward time, peak device
    memory beyond inputs and outputs, and the exact traffic counts."""
    import torch

    from exact_io_aware_30_amd import workloads

    dev = torch.device("cuda:0")
    measured = io_summary_bytes()
    rows = []
    for name in COMPARE_WORKLOADS:
        w = workloads.WORKLOADS[name]
        q, k, v, do, o, dq, dk, dv, lse, delta = _inputs(w, dev)
        e = q.element_size()
        flash = lambda: _flash_step(q, k, v, do, o, dq, dk, dv, lse, delta, w.scale, w.causal)  # noqa: E731
        reps = 5 if w.N * w.N * w.B * w.H > 1 << 33 else 20
        mem_f = _peak_growth(flash)
        t_f = _median_ms(flash, warmup=3, reps=reps)
        run_ordinary = w.N * w.N <= ORDINARY_MAX_SLICE
        if run_ordinary:
            mask = causal_mask(w.N, dev) if w.causal else None
            ordinary = lambda: ordinary_attention(q, k, v, do, w.scale, w.causal, mask)  # noqa: E731
            # the comparator's peak includes the four outputs it returns, not its mask
            mem_o = _peak_growth(ordinary) - 4 * w.elems * e + (mask.numel() if w.causal else 0)
            t_o = _median_ms(ordinary, warmup=2, reps=reps)
            od = ordinary()
            torch.cuda.synchronize()
            diff = max((a.float() - b.float()).abs().max().item() / max(b.float().abs().max().item(), 1e-30)
                       for a, b in zip(od, (o, dq, dk, dv)))
            del od, mask, ordinary
        cnt_t = sum(r + x for r, x in workloads.io_count_tiled(w.B, w.H, w.N, w.d, e, w.causal).values())
        cnt_o = sum(r + x for _, r, x in workloads.io_count_ordinary(w.B, w.H, w.N, w.d, e, w.causal))
        alg = sum(workloads.algorithmic_bytes(w).values())
        r = {"workload": w.describe(), "flash_fwd_bwd_ms": round(t_f[0], 4), "flash_peak_extra_bytes": int(mem_f),
             "flash_count_bytes": cnt_t, "ordinary_count_bytes": cnt_o, "algorithmic_bytes": alg}
        if run_ordinary:
            r.update({"ordinary_fwd_bwd_ms": round(t_o[0], 4), "speedup": round(t_o[0] / t_f[0], 2),
                      "ordinary_peak_extra_bytes": int(mem_o), "max_rel_diff_outputs": round(diff, 5)})
        else:
            r["ordinary"] = "not run: score matrix above 2^31 elements per slice"
        for ver in ("flash", "ordinary"):
            if (name, ver) in measured:
                r[f"{ver}_measured_bytes"] = sum(measured[(name, ver)])
        rows.append(r)
        del q, k, v, do, o, dq, dk, dv, lse, delta
        torch.cuda.empty_cache()
    print("| workload | ordinary ms | tiled ms | speed-up | ordinary peak extra | tiled peak extra "
          "| ordinary count | tiled count | ordinary measured | tiled measured |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    gib = lambda x: f"{x / 2**30:.3f} GiB" if x is not None else "-"  # noqa: E731
    for r in rows:
        t_o = f"{r['ordinary_fwd_bwd_ms']:.3f}" if "ordinary_fwd_bwd_ms" in r else "not run"
        sp = f"{r['speedup']}x" if "speedup" in r else "-"
        print(f"| {r['workload'].split(':')[0]} | {t_o} | {r['flash_fwd_bwd_ms']:.3f} "
              f"| {sp} | {gib(r.get('ordinary_peak_extra_bytes'))} | {gib(r['flash_peak_extra_bytes'])} "
              f"| {gib(r['ordinary_count_bytes'])} | {gib(r['flash_count_bytes'])} "
              f"| {gib(r.get('ordinary_measured_bytes'))} | {gib(r.get('flash_measured_bytes'))} |")
    for r in rows:
        emit(r)


OOM_N = (4096, 8192, 16384, 32768, 65536, 131072)
# Library GEMM and softmax calls are only made on score matrices of at most
# 2^31 elements per (batch, head) slice.
ORDINARY_MAX_SLICE = 1 << 31


def _ordinary_fits(bh, n, dtype, device):
    """Try to allocate what ordinary attention holds at its peak (four
    N x N matrices per slice: P, dP, dS and the P o dP product torch's
    softmax backward forms, plus the N x N mask) without launching anything.
    Returns None if it fits, else the allocator's message."""
    import torch

    held = []
    try:
        for _ in range(4):
            held.append(torch.empty(bh, n, n, dtype=dtype, device=device))
        held.append(torch.empty(n, n, dtype=torch.bool, device=device))
        return None
    except torch.cuda.OutOfMemoryError as err:
        return str(err).split("\n")[0][:200]
    finally:
        del held
        torch.cuda.empty_cache()


def oom():
    """bf16 causal d=128, B=1, H=16, N doubling: peak device memory and time of
    both versions until ordinary attention runs out of device memory (found by
    allocating its peak working set, which launches nothing)."""
    import torch

    from exact_io_aware_30_amd import workloads

    dev = torch.device("cuda:0")
    total = torch.cuda.get_device_properties(0).total_memory
    ordinary_ok = True
    for n in OOM_N:
        w = workloads.Workload(f"oom{n}", "bf16", 1, 16, n, 128, True, 1.0, 3000 + n // 1024)
        q, k, v, do, o, dq, dk, dv, lse, delta = _inputs(w, dev)
        e = q.element_size()
        fp = workloads.footprint(w.B, w.H, n, w.d, e, total)
        r = {"N": n, "B": 1, "H": 16, "d": 128, "device_bytes": total, "score_matrix_bytes": fp["score"],
             "score_matrix_alone_runs_out_at_N": fp["n_max"]}
        flash = lambda: _flash_step(q, k, v, do, o, dq, dk, dv, lse, delta, w.scale, w.causal)  # noqa: E731
        r["flash_peak_extra_bytes"] = int(_peak_growth(flash))
        r["flash_fwd_bwd_ms"] = round(_median_ms(flash, warmup=1, reps=3)[0], 3)
        if not ordinary_ok:
            r["ordinary"] = "not run (out of memory at a smaller N)"
        elif n * n > ORDINARY_MAX_SLICE:
            msg = _ordinary_fits(w.B * w.H, n, q.dtype, dev)
            if msg is None:
                r["ordinary"] = "fits, not run (score matrix above 2^31 elements per slice)"
            else:
                ordinary_ok = False
                r["ordinary"] = "out of memory: " + msg
        else:
            mask = causal_mask(n, dev)
            run = lambda: ordinary_attention(q, k, v, do, w.scale, True, mask)  # noqa: E731
            try:
                r["ordinary_peak_extra_bytes"] = int(_peak_growth(run) - 4 * w.elems * e + mask.numel())
                r["ordinary_fwd_bwd_ms"] = round(_median_ms(run, warmup=1, reps=3)[0], 3)
            except torch.cuda.OutOfMemoryError as err:
                ordinary_ok = False
                r["ordinary"] = "out of memory: " + str(err).split("\n")[0][:200]
            del mask, run
        emit(r)
        del q, k, v, do, o, dq, dk, dv, lse, delta
        torch.cuda.empty_cache()


def variants():
    """Throughput of the wider forms: grouped-query heads, sliding windows,
    packed variable-length batches, and the autograd interface beside raw
    ABI calls.  FLOPs: 4 d (forward) + 10 d (backward) per visible
    query-key pair and query head, counted exactly (for the plain causal
    mask this is N(N+1)/2 pairs, not the N^2/2 of the headline convention)."""
    import torch

    from exact_io_aware_30_amd import binding, interface, workloads

    dev = torch.device("cuda:0")
    B, H, N, d = 2, 16, 8192, 128
    scale = d ** -0.5
    rows = []

    def put(kind, desc, ms, pairs_heads, extra=None):
        fl = 14.0 * d * pairs_heads
        r = {"form": kind, "case": desc, "fwd_bwd_ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
             "frac_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        r.update(extra or {})
        rows.append(r)

    def bufs(shape_q, shape_kv, seed):
        q = workloads.make_tensor(shape_q, "bf16", seed, dev)
        do = workloads.make_tensor(shape_q, "bf16", seed + 1, dev)
        k = workloads.make_tensor(shape_kv, "bf16", seed + 2, dev)
        v = workloads.make_tensor(shape_kv, "bf16", seed + 3, dev)
        o, dq = torch.empty_like(q), torch.empty_like(q)
        dk, dv = torch.empty_like(k), torch.empty_like(k)
        return q, k, v, do, o, dq, dk, dv

    # grouped-query heads: 16 query heads over 16, 4, 1 key/value heads
    for hkv in (16, 4, 1):
        q, k, v, do, o, dq, dk, dv = bufs((B, H, N, d), (B, hkv, N, d), 5000 + hkv)
        lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
        delta = torch.empty_like(lse)
        nbytes = binding.fa_bwd_workspace_size(B, H, hkv, N, d)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None

        def step(ws=ws):
            binding.fa_fwd_gqa(q, k, v, o, lse, scale, True)
            binding.fa_bwd_preprocess(o, do, delta)
            binding.fa_bwd_ex_ws(q, k, v, do, lse, delta, dq, dk, dv, scale, (-1, 0), ws)

        extra = {"workspace_mib": round(nbytes / 2 ** 20, 1)}
        if nbytes:  # the same step without the head split, for comparison
            extra["unsplit_ms"] = round(_median_ms(lambda: step(None), warmup=3, reps=10)[0], 4)
        put("gqa", f"bf16 [2,16,8192,128] causal, Hkv={hkv}", _median_ms(step, warmup=3, reps=10)[0],
            B * H * workloads.visible_pairs(N, True), extra)
        del q, k, v, do, o, dq, dk, dv, lse, delta, ws

    # sliding windows on the headline shape
    q, k, v, do, o, dq, dk, dv = bufs((B, H, N, d), (B, H, N, d), 5100)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    for win in ((-1, 0), (1024, 0), (256, 0), (512, 512)):
        def step(win=win):
            binding.fa_fwd_ex(q, k, v, o, lse, scale, win)
            binding.fa_bwd_preprocess(o, do, delta)
            binding.fa_bwd_ex(q, k, v, do, lse, delta, dq, dk, dv, scale, win)

        put("window", f"bf16 [2,16,8192,128] window (left, right) = {win}",
            _median_ms(step, warmup=3, reps=10)[0], B * H * workloads.visible_pairs(N, False, win))

    # autograd interface beside the raw calls (same inputs, causal)
    def raw():
        binding.fa_fwd(q, k, v, o, lse, scale, True)
        binding.fa_bwd_preprocess(o, do, delta)
        binding.fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, scale, True)

    qa, ka, va = (x.detach().clone().requires_grad_(True) for x in (q, k, v))

    def auto():
        qa.grad = ka.grad = va.grad = None
        out = interface.flash_attn(qa, ka, va, causal=True, softmax_scale=scale)
        out.backward(do)

    t_raw, t_auto = _median_ms(raw, warmup=3, reps=10)[0], _median_ms(auto, warmup=3, reps=10)[0]
    put("interface", "flash_attn + backward (autograd), bf16 [2,16,8192,128] causal", t_auto,
        B * H * workloads.visible_pairs(N, True), {"raw_abi_ms": round(t_raw, 4), "overhead_ms": round(t_auto - t_raw, 4)})
    del q, k, v, do, o, dq, dk, dv, lse, delta, qa, ka, va

    # packed variable-length batch: 24 sequences of seeded lengths 256 .. 4096
    g = torch.Generator().manual_seed(5200)
    lens = torch.randint(256, 4097, (24,), generator=g).tolist()
    T, mx = sum(lens), max(lens)
    cu = torch.tensor([0] + torch.tensor(lens).cumsum(0).tolist(), dtype=torch.int32, device=dev)
    q, k, v, do, o, dq, dk, dv = bufs((H, T, d), (H, T, d), 5300)
    lse = torch.empty(H, T, dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)

    def step():
        binding.fa_fwd_varlen(q, k, v, o, lse, cu, mx, scale, (-1, 0))
        binding.fa_bwd_preprocess(o.view(1, H, T, d), do.view(1, H, T, d), delta.view(1, H, T))
        binding.fa_bwd_varlen(q, k, v, do, lse, delta, dq, dk, dv, cu, mx, scale, (-1, 0))

    put("varlen", f"bf16 H=16 d=128 causal, 24 packed sequences, T={T}, lengths {min(lens)}..{mx}",
        _median_ms(step, warmup=3, reps=10)[0], H * sum(workloads.visible_pairs(n, True) for n in lens))
    del q, k, v, do, o, dq, dk, dv, lse, delta

    # the same packed batch with one key/value head (multi-query), head split on
    q, k, v, do, o, dq, dk, dv = bufs((H, T, d), (1, T, d), 5400)
    lse = torch.empty(H, T, dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    nbytes = binding.fa_bwd_varlen_workspace_size(len(lens), mx, T, H, 1, d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None

    def step(ws=ws):
        binding.fa_fwd_varlen(q, k, v, o, lse, cu, mx, scale, (-1, 0))
        binding.fa_bwd_preprocess(o.view(1, H, T, d), do.view(1, H, T, d), delta.view(1, H, T))
        binding.fa_bwd_varlen_ws(q, k, v, do, lse, delta, dq, dk, dv, cu, mx, scale, (-1, 0), ws)

    extra = {"workspace_mib": round(nbytes / 2 ** 20, 1)}
    if nbytes:
        extra["unsplit_ms"] = round(_median_ms(lambda: step(None), warmup=3, reps=10)[0], 4)
    put("varlen", f"bf16 H=16 Hkv=1 d=128 causal, the same 24 packed sequences", _median_ms(step, warmup=3, reps=10)[0],
        H * sum(workloads.visible_pairs(n, True) for n in lens), extra)

    print("| form | case | fwd+bwd ms | TFLOP/s (exact visible pairs) | % of 2.5 PF | notes |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        note = f"raw ABI {r['raw_abi_ms']} ms, overhead {r['overhead_ms']} ms" if "raw_abi_ms" in r else \
            f"head split: {r['workspace_mib']} MiB workspace; unsplit {r['unsplit_ms']} ms" if "unsplit_ms" in r \
            else ""
        print(f"| {r['form']} | {r['case']} | {r['fwd_bwd_ms']} | {r['tflops']} | {100 * r['frac_mfma_peak']:.1f} "
              f"| {note} |")
    for r in rows:
        emit(r)


def compare_step(version, name):
    """One forward+backward step of one version on one workload, nothing else
    launched on the device (for hardware byte counters)."""
    import torch

    from exact_io_aware_30_amd import workloads

    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    q, k, v, do, o, dq, dk, dv, lse, delta = _inputs(w, dev)
    mask = causal_mask(w.N, dev) if w.causal else None
    torch.cuda.synchronize()
    if version == "flash":
        _flash_step(q, k, v, do, o, dq, dk, dv, lse, delta, w.scale, w.causal)
    else:
        ordinary_attention(q, k, v, do, w.scale, w.causal, mask)
    torch.cuda.synchronize()
    emit({"compare_step": version, "workload": w.describe()})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--report", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--compare", action="store_true")
    ap.add_argument("--oom", action="store_true")
    ap.add_argument("--variants", action="store_true")
    ap.add_argument("--compare-step", choices=("flash", "ordinary"), default=None)
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph (replays; reported as graph_* fields)")
    ap.add_argument("--results", default=None, help="also write every JSON record printed to this file "
                                                    "(a JSON list)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, copy a buffer of this many MiB once (a kernel of known "
                         "traffic for scaling hardware byte counters)")
    args = ap.parse_args()
    try:
        run(args)
    finally:
        if args.results and RECORDS:
            with open(args.results, "w") as f:
                json.dump(RECORDS, f, indent=1)


def run(args):
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.compare_step:
        compare_step(args.compare_step, args.workload)
        if args.calib_copy_mib:
            calib_copy(args.calib_copy_mib)
        return
    if args.report or args.sweep or args.compare or args.oom or args.variants:
        (report if args.report else sweep if args.sweep else compare if args.compare else oom if args.oom
         else variants)()
        if args.calib_copy_mib:
            calib_copy(args.calib_copy_mib)
        return

    import torch

    from exact_io_aware_30_amd import binding, workloads

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in workloads.make_inputs(w))
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    torch.cuda.synchronize()

    phases = ("fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        binding.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
        if ev is not None:
            ev[1].record()
        binding.fa_bwd_preprocess(o, do, delta)
        if ev is not None:
            ev[2].record()
        binding.fa_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, w.scale, w.causal)
        if ev is not None:
            ev[3].record()
        binding.fa_bwd_dq(q, k, v, do, lse, delta, dq, w.scale, w.causal)
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {p: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / args.steps for j, p in enumerate(phases)}
    assert torch.isfinite(o).all() and torch.isfinite(dq).all(), "non-finite output"
    graph_ms = None
    if args.graph:
        # The same step captured once and replayed: no per-launch host cost.
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    if args.calib_copy_mib:
        calib_copy(args.calib_copy_mib)

    f, b, fb = workloads.flops(w)
    ms = wall * 1e3 / args.steps
    kf = workloads.kernel_flops(w)
    kx = workloads.kernel_flops(w, executed=True)
    kb = workloads.algorithmic_bytes(w)
    kernels = {}
    for p in phases:
        t = per[p] * 1e-3
        ent = {"ms": round(per[p], 4)}
        if kf[p] > 0:
            ent["tflops"] = round(kf[p] / t / 1e12, 1)
            ent["frac_mfma_peak"] = round(kf[p] / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        if kx[p] != kf[p]:
            # the MFMA work the kernel executes, recomputation included
            ent["executed_tflops"] = round(kx[p] / t / 1e12, 1)
            ent["executed_frac_mfma_peak"] = round(kx[p] / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        ent["gbs_algorithmic"] = round(kb[p] / t / 1e9, 1)
        kernels[p] = ent
    dom = max(("fwd", "bwd_dkdv", "bwd_dq"), key=lambda p: per[p])
    achieved = kf[dom] / (per[dom] * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_from_summary(dom), "algorithmic_bytes": kb[dom],
                "algorithmic_flops": kf[dom]}
    t_fwd = per["fwd"] * 1e-3
    t_bwd = (per["bwd_preprocess"] + per["bwd_dkdv"] + per["bwd_dq"]) * 1e-3
    value = fb / (ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp16",
        "data": "synthetic: seeded i.i.d. N(0,1) Q, K, V, dO",
        "config": {"workload": f"{w.name}: {w.dtype} [B={w.B},H={w.H},N={w.N},d={w.d}] "
                               f"{'causal' if w.causal else 'full'}",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal},
        "frac_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(f / t_fwd / 1e12, 1),
        "bwd_tflops": round(b / t_bwd / 1e12, 1),
        "fwd_plus_bwd_tflops_from_events": round(fb / (t_fwd + t_bwd) / 1e12, 1),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
        "library_hash": library_hash(),
    }
    if graph_ms is not None:
        line["graph_ms_per_step"] = round(graph_ms, 4)
        line["graph_tflops"] = round(fb / (graph_ms * 1e-3) / 1e12, 2)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    emit(line)


if __name__ == "__main__":
    main()
