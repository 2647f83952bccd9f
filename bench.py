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
                                line per workload)
    python bench.py --sweep     bf16 causal d=128, B=1, H=16, N = 1K .. 64K:
                                one pass of each kernel per N (for hardware
                                counters) and its time

Without --report or --sweep it prints one JSON line.  Besides the contract fields it carries
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
            "seconds": round(dt, 3)}


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
        print(json.dumps(r), flush=True)


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
        print(json.dumps({"N": n, "B": 1, "H": 16, "d": 128, "fwd_bwd_ms": round(t[0], 4),
                          "fwd_bwd_tflops": round(fb / t[0] / 1e9, 1),
                          "algorithmic_bytes": workloads.algorithmic_bytes(w)}), flush=True)
        del q, k, v, do, o, dq, dk, dv, lse, delta
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--report", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, copy a buffer of this many MiB once (a kernel of known "
                         "traffic for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.report or args.sweep:
        report() if args.report else sweep()
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
    if args.calib_copy_mib:
        calib_copy(args.calib_copy_mib)

    f, b, fb = workloads.flops(w)
    ms = wall * 1e3 / args.steps
    kf = workloads.kernel_flops(w)
    kb = workloads.algorithmic_bytes(w)
    kernels = {}
    for p in phases:
        t = per[p] * 1e-3
        ent = {"ms": round(per[p], 4)}
        if kf[p] > 0:
            ent["tflops"] = round(kf[p] / t / 1e12, 1)
            ent["frac_mfma_peak"] = round(kf[p] / t / 1e12 / PEAK_BF16_TFLOPS, 4)
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
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
