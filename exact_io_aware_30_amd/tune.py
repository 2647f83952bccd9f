"""Offline tuning sweep over the kernels' compile-time tile configurations.

The Triton implementation the pages describe autotunes BLOCK_M, BLOCK_N,
warps and stages at run time ("flash-attn-triton" docs, spec sheet and
"Scope").  Here the tile shapes are compile-time constants of the HIP
kernels (one table per head dimension: ``FwdCfg`` in fa_fwd.hip,
``DkdvCfg`` and the dQ settings in fa_bwd.hip), and this module is the sweep
that chooses them: it builds one library per candidate configuration,
rejects candidates whose device code spills registers to scratch memory (or
reads anything through flat addressing), runs the rest on the GPU against
the default library's outputs, and ranks them by time.

    python -m exact_io_aware_30_amd.tune --kernel fwd --build-only
    python -m exact_io_aware_30_amd.tune --kernel fwd --time-only --shape bf16,2,16,8192,64,causal

Building needs only hipcc (any machine); timing needs a GPU.  Candidates are
built under ``_build/tune/<kernel>/<name>/``; the in-tree library is the
reference and is not modified.  Each candidate is timed in alternating rounds
(every candidate once per round, the minimum kept) so that clock drift does
not favour the first one.
"""

from __future__ import annotations

import argparse
import concurrent.futures
import ctypes
import json
import os
import re
import shutil
import subprocess
import sys

from . import build as _build

LLVM_OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

# Candidate configurations per kernel: name -> preprocessor definitions.
# The macros override the per-head-dimension defaults for every head
# dimension of that kernel.
SPACES = {
    "fwd": {
        "default": [],
        "w8_k2_s2": ["-DFA_FWD_WAVES=8", "-DFA_FWD_KEYBLOCKS=2", "-DFA_FWD_STAGES=2"],
        "w8_k2_s3": ["-DFA_FWD_WAVES=8", "-DFA_FWD_KEYBLOCKS=2", "-DFA_FWD_STAGES=3"],
        "w8_k1_s3": ["-DFA_FWD_WAVES=8", "-DFA_FWD_KEYBLOCKS=1", "-DFA_FWD_STAGES=3"],
        "w4_k2_s2": ["-DFA_FWD_WAVES=4", "-DFA_FWD_KEYBLOCKS=2", "-DFA_FWD_STAGES=2"],
        "w4_k2_s3": ["-DFA_FWD_WAVES=4", "-DFA_FWD_KEYBLOCKS=2", "-DFA_FWD_STAGES=3"],
        "w4_k1_s2": ["-DFA_FWD_WAVES=4", "-DFA_FWD_KEYBLOCKS=1", "-DFA_FWD_STAGES=2"],
        "w4_k1_s3": ["-DFA_FWD_WAVES=4", "-DFA_FWD_KEYBLOCKS=1", "-DFA_FWD_STAGES=3"],
        "w2_k2_s2": ["-DFA_FWD_WAVES=2", "-DFA_FWD_KEYBLOCKS=2", "-DFA_FWD_STAGES=2"],
        "prio": ["-DFA_FWD_PRIO=1"],
        "pipe_pre_2_2": ["-DFA_FWD_PIPE_PRE1=2", "-DFA_FWD_PIPE_PRE2=2"],
        "pipe_pre_4_3": ["-DFA_FWD_PIPE_PRE1=4", "-DFA_FWD_PIPE_PRE2=3"],
        "sum_in_qk": ["-DFA_FWD_SUM_IN_PV=0"],
        "pipe_all": ["-DFA_FWD_PIPE=1"],
        "plain_sum_before_pv": ["-DFA_FWD_PLAIN_SUM_AFTER_PV=0"],
    },
    "dkdv": {
        "default": [],
        "occ1": ["-DFA_DKDV_OCC=1"],
        "occ2": ["-DFA_DKDV_OCC=2"],
        "pre1_3": ["-DFA_DKDV_PRE1=3"],
        "pre1_4": ["-DFA_DKDV_PRE1=4"],
        "pre1_5": ["-DFA_DKDV_PRE1=5"],
        "pre1_6": ["-DFA_DKDV_PRE1=6"],
        "pre1_4_occ1": ["-DFA_DKDV_PRE1=4", "-DFA_DKDV_OCC=1"],
        "pre1_4_pre2_2": ["-DFA_DKDV_PRE1=4", "-DFA_DKDV_PRE2=2"],
        "pre1_4_pre2_4": ["-DFA_DKDV_PRE1=4", "-DFA_DKDV_PRE2=4"],
        "pre2_2": ["-DFA_DKDV_PRE2=2"],
        "vlds": ["-DFA_DKDV_VLDS=1"],
        "pre1_3_vlds": ["-DFA_DKDV_PRE1=3", "-DFA_DKDV_VLDS=1"],
        "occ2_vlds": ["-DFA_DKDV_OCC=2", "-DFA_DKDV_VLDS=1"],
        "pre2_4": ["-DFA_DKDV_PRE2=4"],
        "tile64": ["-DFA_DKDV_TILE=64"],
        "vregs": ["-DFA_DKDV_VLDS=0"],
        "stages3": ["-DFA_DKDV_STAGES=3"],
        "dv_first": ["-DFA_DKDV_DV_FIRST=1"],
        "dv_first_off": ["-DFA_DKDV_DV_FIRST=0"],
    },
    "dq": {
        "default": [],
        "t32": ["-DFA_DQ_TILE=32"],
        "t32_s4": ["-DFA_DQ_TILE=32", "-DFA_DQ_STAGES=4"],
        "pipe": ["-DFA_DQ_PIPE=1"],
        "nopipe": ["-DFA_DQ_PIPE=0"],
        "t32_pipe": ["-DFA_DQ_TILE=32", "-DFA_DQ_PIPE=1"],
        "pre1_4": ["-DFA_DQ_PRE1=4"],
        "pre1_8": ["-DFA_DQ_PRE1=8"],
        "pre2_2": ["-DFA_DQ_PRE2=2"],
        "pre2_4": ["-DFA_DQ_PRE2=4"],
        "pre1_4_pre2_2": ["-DFA_DQ_PRE1=4", "-DFA_DQ_PRE2=2"],
        "stages3": ["-DFA_DQ_STAGES=3"],
        "stages4": ["-DFA_DQ_STAGES=4"],
        "pipe_pre1_3": ["-DFA_DQ_PIPE_PRE1=3"],
        "pipe_pre1_4": ["-DFA_DQ_PIPE_PRE1=4"],
        "pipe_pre3_2": ["-DFA_DQ_PIPE_PRE3=2"],
        "pipe_pre1_3_pre3_2": ["-DFA_DQ_PIPE_PRE1=3", "-DFA_DQ_PIPE_PRE3=2"],
    },
}
SOURCE = {"fwd": "fa_fwd.hip", "dkdv": "fa_bwd.hip", "dq": "fa_bwd.hip"}


def _objects_except(src: str):
    """The default build's objects other than the one built from `src`."""
    objs = []
    for s in _build.SOURCES:
        if s != src:
            objs.append(os.path.join(_build.BUILD_DIR, os.path.splitext(s)[0] + ".o"))
    return objs


def _device_memory_ops(lib: str, workdir: str):
    """Count scratch and flat instructions in the library's device code
    (a spill goes to scratch; LDS or global data read through a flat
    pointer means a wrong address space)."""
    for f in os.listdir(workdir):
        if f.startswith(os.path.basename(lib) + "."):
            os.remove(os.path.join(workdir, f))
    subprocess.run([LLVM_OBJDUMP, "--offloading", os.path.basename(lib)], cwd=workdir, capture_output=True)
    n = 0
    for f in os.listdir(workdir):
        if f.startswith(os.path.basename(lib) + ".") and "amdgcn" in f:
            out = subprocess.run([LLVM_OBJDUMP, "-d", os.path.join(workdir, f)], capture_output=True, text=True)
            n += len(re.findall(r"\b(?:scratch|flat)_(?:load|store)\w*", out.stdout))
            os.remove(os.path.join(workdir, f))
    for f in os.listdir(workdir):
        if f.startswith(os.path.basename(lib) + "."):
            os.remove(os.path.join(workdir, f))
    return n


def build_candidates(kernel: str, names=None, jobs: int = 4):
    """Build every candidate of `kernel`; returns {name: (library path or
    None, note)}.  The default in-tree build runs first (its objects are
    linked into every candidate)."""
    _build.build()
    space = SPACES[kernel]
    names = list(space) if names is None else names
    src = SOURCE[kernel]
    root = os.path.join(_build.BUILD_DIR, "tune", kernel)

    def one(name):
        d = os.path.join(root, name)
        os.makedirs(d, exist_ok=True)
        obj = os.path.join(d, os.path.splitext(src)[0] + ".o")
        r = subprocess.run([_build.HIPCC, *_build.FLAGS, *space[name], "-c", os.path.join(_build.CSRC, src), "-o",
                            obj], capture_output=True, text=True)
        if r.returncode:
            return name, (None, "does not compile: " + r.stderr.strip().splitlines()[-1][:160])
        lib = os.path.join(d, _build.LIB_NAME)
        r = subprocess.run([_build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", obj, *_objects_except(src),
                            "-o", lib], capture_output=True, text=True)
        os.remove(obj)
        if r.returncode:
            return name, (None, "does not link")
        n = _device_memory_ops(lib, d)
        if n:
            os.remove(lib)
            return name, (None, f"rejected: {n} scratch/flat instructions (register spills)")
        return name, (lib, "built")

    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        return dict(ex.map(one, names))


def built_candidates(kernel: str, names=None):
    """The candidates of `kernel` built by an earlier build_candidates call:
    {name: (library path or None, note)}."""
    root = os.path.join(_build.BUILD_DIR, "tune", kernel)
    out = {}
    for name in (list(SPACES[kernel]) if names is None else names):
        lib = os.path.join(root, name, _build.LIB_NAME)
        out[name] = (lib, "built earlier") if os.path.exists(lib) else (None, "not built (rejected or missing)")
    return out


def _parse_shape(text: str):
    dt, B, H, N, d, mask = text.split(",")
    return dt, int(B), int(H), int(N), int(d), mask == "causal"


def time_candidates(kernel: str, libs: dict, shape, rounds: int = 3, reps: int = 10):
    """Run every built candidate on `shape` and rank them.  Outputs are
    compared with the in-tree library's; a candidate whose outputs differ by
    more than the parity tolerances is marked wrong and not ranked."""
    import torch

    from . import binding, workloads

    dt, B, H, N, d, causal = shape
    w = workloads.Workload("tune", dt, B, H, N, d, causal, 1.0, 4242)
    q, k, v, do = (x.cuda() for x in workloads.make_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    binding.fa_fwd(q, k, v, o, lse, w.scale, causal)
    binding.fa_bwd_preprocess(o, do, delta)
    ref = torch.empty_like(q)
    ref2 = torch.empty_like(q)
    if kernel == "fwd":
        ref.copy_(o)
    elif kernel == "dkdv":
        binding.fa_bwd_dkdv(q, k, v, do, lse, delta, ref, ref2, w.scale, causal)
    else:
        binding.fa_bwd_dq(q, k, v, do, lse, delta, ref, w.scale, causal)
    torch.cuda.synchronize()
    tol = {"fwd": {"fp16": 4e-3, "bf16": 3e-2}, "dkdv": {"fp16": 1e-2, "bf16": 5e-2},
           "dq": {"fp16": 1e-2, "bf16": 5e-2}}[kernel][dt]
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    dtc = 1 if dt == "bf16" else 0
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)  # noqa: E731
    sc = ctypes.c_float(w.scale)
    loaded = {n: ctypes.CDLL(p) for n, (p, _) in libs.items() if p}
    out, out2, lse2 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(lse)

    def call(lib):
        if kernel == "fwd":
            return lib.fa_fwd(P(q), P(k), P(v), P(out), P(lse2), B, H, N, d, sc, int(causal), dtc, st())
        if kernel == "dkdv":
            return lib.fa_bwd_dkdv(P(q), P(k), P(v), P(do), P(lse), P(delta), P(out), P(out2), B, H, N, d, sc,
                                   int(causal), dtc, st())
        return lib.fa_bwd_dq(P(q), P(k), P(v), P(do), P(lse), P(delta), P(out), B, H, N, d, sc, int(causal), dtc,
                             st())

    best, err = {}, {}
    for _ in range(rounds):
        for name, lib in loaded.items():
            if call(lib) != 0:
                err[name] = float("inf")
                continue
            torch.cuda.synchronize()
            pairs = [(out, ref)] + ([(out2, ref2)] if kernel == "dkdv" else [])
            e = max(((a.float() - b_.float()).abs().max() / b_.float().abs().max().clamp_min(1e-30)).item()
                    for a, b_ in pairs)
            err[name] = max(err.get(name, 0.0), e)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            call(lib)
            ev[0].record()
            for _ in range(reps):
                call(lib)
            ev[1].record()
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1]) / reps
            best[name] = min(best.get(name, float("inf")), ms)
    rows = []
    for name in libs:
        p, note = libs[name]
        if not p:
            rows.append({"candidate": name, "note": note})
        elif err.get(name, 0.0) > tol:
            rows.append({"candidate": name, "note": f"wrong output (max rel diff {err[name]:.2e})"})
        else:
            rows.append({"candidate": name, "ms": round(best[name], 4), "max_rel_diff": err[name]})
    rows.sort(key=lambda r: r.get("ms", float("inf")))
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--kernel", choices=sorted(SPACES), required=True)
    ap.add_argument("--candidates", default=None, help="comma-separated subset of the kernel's candidates")
    ap.add_argument("--shape", default="bf16,2,16,8192,128,causal",
                    help="dtype,B,H,N,d,causal|full of the workload to time on")
    ap.add_argument("--build-only", action="store_true")
    ap.add_argument("--time-only", action="store_true",
                    help="time the candidates built earlier (no compiler is run)")
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--json", default=None, help="also write the ranking to this file")
    args = ap.parse_args(argv)
    names = args.candidates.split(",") if args.candidates else None
    libs = built_candidates(args.kernel, names) if args.time_only else build_candidates(args.kernel, names)
    for n, (p, note) in libs.items():
        print(f"{args.kernel}/{n}: {note}", flush=True)
    if args.build_only:
        return
    rows = time_candidates(args.kernel, libs, _parse_shape(args.shape), rounds=args.rounds)
    print(f"kernel {args.kernel}, shape {args.shape}")
    for r in rows:
        print("  " + json.dumps(r), flush=True)
    if args.json:
        with open(args.json, "w") as f:
            json.dump({"kernel": args.kernel, "shape": args.shape, "ranking": rows}, f, indent=1)


def clean():
    """Remove every built candidate."""
    shutil.rmtree(os.path.join(_build.BUILD_DIR, "tune"), ignore_errors=True)


if __name__ == "__main__":
    main(sys.argv[1:])
