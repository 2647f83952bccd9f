"""Seeded synthetic attention inputs, and the FLOP / byte counts of a workload.

This module holds no attention arithmetic: it draws inputs and counts work.
Both the HIP path's tests and the CPU oracle's tests take their inputs from
here, so the two sides see the same bits.

Inputs: one CPU ``torch.Generator`` per workload, seeded, drawing float32
N(0, 1) tensors in the order Q, K, V, dO, each [B, H, N, d]; Q is multiplied
by ``q_scale`` (exact for a power of two) and every tensor is then rounded to
the workload dtype (round-to-nearest-even).

Counting conventions (the pages give "TFLOP/s" without a formula):
  forward  = 4 B H N^2 d      (QK^T and PV, 2 N^2 d each)
  backward = 10 B H N^2 d     (QK^T recompute, dO V^T, P^T dO, dS K, dS^T Q)
  both halved exactly under the causal mask.
Algorithmic bytes read or written once each, with T = B H N d elements of
e bytes: forward 4Te + 4BHN, preprocess 2Te + 4BHN, dK/dV 6Te + 8BHN,
dQ 5Te + 8BHN.
"""

from __future__ import annotations

import dataclasses
import math

import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "fp16" | "bf16"
    B: int
    H: int
    N: int
    d: int
    causal: bool
    q_scale: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    @property
    def elems(self) -> int:
        return self.B * self.H * self.N * self.d

    def describe(self) -> str:
        mask = "causal" if self.causal else "full"
        return (f"{self.name}: {self.dtype} [B={self.B},H={self.H},N={self.N},d={self.d}] "
                f"{mask} q_scale={self.q_scale:g} seed={self.seed}")


# The five workloads the method is checked and measured on.
WORKLOADS = {
    "tiny": Workload("tiny", "fp16", 1, 2, 256, 64, False, 1.0, 1001),
    "gpt2_medium": Workload("gpt2_medium", "bf16", 8, 16, 1024, 64, True, 1.0, 1002),
    "ragged": Workload("ragged", "fp16", 3, 12, 2000, 32, False, 4.0, 1003),
    "long": Workload("long", "bf16", 2, 16, 8192, 128, True, 1.0, 1004),
    "batch1_64k": Workload("batch1_64k", "bf16", 1, 8, 65536, 64, True, 1.0, 1005),
}


def make_inputs(w: Workload, device="cpu"):
    """(q, k, v, do) for workload ``w``: seeded N(0,1) fp32 draws, rounded."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    out = []
    for name in ("q", "k", "v", "do"):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if name == "q" and w.q_scale != 1.0:
            x = x * w.q_scale
        out.append(x.to(w.torch_dtype).to(device))
    return tuple(out)


RISE_TILE = 64      # keys per block of the staircase below
RISE_STEP = 12.0    # base-2 units the scores rise at each step block
RISE_QCOORD = 32.0  # value of every query's last coordinate


def rise_steps(n: int):
    """Key blocks (of RISE_TILE keys) at which the staircase of
    make_rising_inputs steps up: 1, 2, the middle one and the last one."""
    nt = (n + RISE_TILE - 1) // RISE_TILE
    return sorted({t for t in (1, 2, nt // 2, nt - 1) if 1 <= t <= nt - 1})


def make_rising_inputs(w: Workload, device="cpu"):
    """Inputs whose scores climb in steps along the key axis, so that every
    query row's running maximum moves several times after its first key
    block.  Start from make_inputs(w); set every query's last coordinate to
    RISE_QCOORD and the last coordinate of key j to RISE_STEP * s(j) /
    (RISE_QCOORD * scale * log2 e), s(j) the number of steps at or before
    key block j // RISE_TILE; round to the dtype.  The last coordinate then
    adds about RISE_STEP * s(j) base-2 units to every score of key j, on top
    of the N(0, 1) part of the other d - 1 coordinates (keys of block 0 add
    nothing).  The shift sits mostly on the query side (keys' last
    coordinate at most 12): the backward forms D from the rounded O, and
    dQ = scale dS K then carries D's rounding times the keys' shared
    component, which a large key coordinate would magnify."""
    q, k, v, do = make_inputs(w)
    q, k = q.float(), k.float()
    c = w.scale * math.log2(math.e)
    steps = rise_steps(w.N)
    blk = torch.arange(w.N) // RISE_TILE
    s = torch.zeros(w.N)
    for t in steps:
        s += (blk >= t).float()
    q[..., -1] = RISE_QCOORD
    k[..., -1] = (RISE_STEP * s / (RISE_QCOORD * c)).view(1, 1, w.N)
    dt = w.torch_dtype
    return q.to(dt).to(device), k.to(dt).to(device), v.to(device), do.to(device)


def make_tensor(shape, dtype: str, seed: int, device="cpu", scale: float = 1.0):
    """One seeded N(0,1)*scale fp32 draw rounded to ``dtype``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32) * scale
    return x.to(DTYPES[dtype]).to(device)


def flops(w: Workload):
    """(forward, backward, forward+backward) counted FLOPs."""
    base = w.B * w.H * w.N * w.N * w.d
    f, b = 4 * base, 10 * base
    if w.causal:
        f, b = f / 2, b / 2
    return float(f), float(b), float(f + b)


def visible_pairs(n: int, causal: bool, window=None) -> int:
    """Query-key pairs a length-n sequence attends: key j visible to query i
    iff i - left <= j <= i + right (-1: no bound), right capped at 0 by the
    causal flag."""
    import numpy as np

    left, right = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    if causal:
        right = 0 if right < 0 else min(right, 0)
    i = np.arange(n, dtype=np.int64)
    lo = np.zeros(n, dtype=np.int64) if left < 0 else np.maximum(0, i - left)
    hi = np.full(n, n - 1, dtype=np.int64) if right < 0 else np.minimum(n - 1, i + right)
    return int(np.maximum(hi - lo + 1, 0).sum())


def kernel_flops(w: Workload, executed: bool = False):
    """Counted FLOPs attributed to each kernel (causal halved).

    The dK/dV kernel carries the QK^T recompute, dO V^T, P^T dO and dS^T Q
    (8 B H N^2 d); the dQ kernel carries dS K (2 B H N^2 d).  The dQ
    kernel's own recomputation of S and dP is work the deterministic layout
    adds, not counted; with ``executed`` it is included (6 B H N^2 d).
    """
    base = w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
    return {"fwd": 4 * base, "bwd_dkdv": 8 * base, "bwd_dq": (6 if executed else 2) * base, "bwd_preprocess": 0.0}


def algorithmic_bytes(w: Workload):
    """Bytes each kernel must move at least once (inputs read, outputs written)."""
    e = torch.finfo(w.torch_dtype).bits // 8
    T = w.elems
    rows = w.B * w.H * w.N
    return {
        "fwd": 4 * T * e + 4 * rows,
        "bwd_preprocess": 2 * T * e + 4 * rows,
        "bwd_dkdv": 6 * T * e + 8 * rows,
        "bwd_dq": 5 * T * e + 8 * rows,
    }


def footprint(B: int, H: int, N: int, d: int, elem_bytes: int, capacity_bytes: float | None = None):
    """The footprint calculator: score matrix versus what the tiled kernel holds.

    score   -- B*H*N*N elements of the score matrix, in bytes
    linear  -- Q, K, V, O (B*H*N*d each) plus one fp32 L per row, in bytes
    ratio   -- score / linear
    n_max   -- largest N whose score matrix alone fits ``capacity_bytes``
    """
    score = B * H * N * N * elem_bytes
    linear = 4 * B * H * N * d * elem_bytes + 4 * B * H * N
    res = {"score": score, "linear": linear, "ratio": score / linear}
    if capacity_bytes is not None:
        res["n_max"] = int(math.isqrt(int(capacity_bytes // (B * H * elem_bytes))))
    return res


# --------------------------------------------------------------------------
# Exact memory-traffic counts of the two versions
# ("flash-attn-triton" docs, "The argument" and Table 2; "What is
# FlashAttention?", "What you will build", step 03)
# --------------------------------------------------------------------------

# Tile geometry of the HIP kernels, as they request rows from device memory:
# forward: query blocks of 256 rows, key tiles of 64; dK/dV: key blocks of 128
# rows, query tiles of 32 (64 at d = 32) with the L and D vectors fetched 64
# entries per tile; dQ: query blocks of 128 rows, key tiles of 64.
def kernel_tiles(d: int) -> dict:
    return {"fwd_bm": 256, "fwd_bn": 64, "dkdv_bk": 128, "dkdv_bq": 64 if d == 32 else 32, "dkdv_stats": 64,
            "dq_bm": 128, "dq_bn": 64}


def _blocks(n: int, size: int):
    import numpy as np

    start = np.arange(0, n, size, dtype=np.int64)
    return start, np.minimum(size, n - start)


def _key_rows(n: int, q0, bm: int, bn: int, causal: bool):
    """Key rows a query block starting at q0 loads: whole key tiles up to its
    last visible key, the tile past row n - 1 clipped."""
    import numpy as np

    if not causal:
        return np.full_like(q0, n)
    kend = np.minimum(n, q0 + bm)
    return np.minimum(n, -(-kend // bn) * bn)


def io_count_tiled(B: int, H: int, N: int, d: int, e: int, causal: bool, tiles: dict | None = None) -> dict:
    """Bytes each tiled kernel reads from and writes to device memory, counting
    every tile load a workgroup issues (no cache): {kernel: (read, written)}.

    Per (batch, head) slice of N rows:
      fwd       Q, O and L once; K and V once per query block, up to the last
                key tile the block sees (all N keys without the causal mask).
      preprocess O and dO read, D written once.
      dK/dV     K, V, dK, dV once; per key block, Q and dO from its first
                visible query row to N, and L and D in 64-entry pieces, one
                per query tile.
      dQ        Q, dO, L, D and dQ once; K and V once per query block, as in
                the forward.
    Writes are linear in N: no N x N data is stored.
    """
    import numpy as np

    t = dict(kernel_tiles(d) if tiles is None else tiles)
    row = d * e
    q0, rq = _blocks(N, t["fwd_bm"])
    kv = _key_rows(N, q0, t["fwd_bm"], t["fwd_bn"], causal)
    fwd = (int(rq.sum()) * row + 2 * int(kv.sum()) * row, N * (row + 4))
    pre = (2 * N * row, 4 * N)
    k0, rk = _blocks(N, t["dkdv_bk"])
    i_start = k0 if causal else np.zeros_like(k0)
    stats = 0
    for s in i_start.tolist():
        i0 = np.arange(s, N, t["dkdv_bq"], dtype=np.int64)
        stats += int(np.minimum(t["dkdv_stats"], N - i0).sum())
    dkdv = (2 * int(rk.sum()) * row + 2 * int((N - i_start).sum()) * row + 2 * 4 * stats, 2 * N * row)
    q0, rq = _blocks(N, t["dq_bm"])
    kv = _key_rows(N, q0, t["dq_bm"], t["dq_bn"], causal)
    dq = (int(rq.sum()) * (2 * row + 8) + 2 * int(kv.sum()) * row, N * row)
    bh = B * H
    return {k: (bh * r, bh * w) for k, (r, w) in
            (("fwd", fwd), ("bwd_preprocess", pre), ("bwd_dkdv", dkdv), ("bwd_dq", dq))}


def io_count_ordinary(B: int, H: int, N: int, d: int, e: int, causal: bool, layout_copies: bool = True) -> list:
    """Bytes each step of ordinary attention reads and writes, each operand
    read once and each result written once: [(step, read, written)].

    The score matrix S, the probabilities P and, backward, dP and dS are
    N x N per (batch, head) and go through device memory.  With
    ``layout_copies`` the list also holds the N x d transposed copies and
    the causal mask pass the GPU comparator performs (the mask is one
    N x N byte array, read once per slice); without them it is the plain
    algorithm: S = scale QK^T written, read back by the softmax, P written
    and read by PV; backward dV = P^T dO, dP = dO V^T, dS = P o (dP - D),
    dQ = scale dS K, dK = scale dS^T Q.
    """
    nd, nn = N * d * e, N * N * e
    steps = []
    add = lambda name, r, w: steps.append((name, B * H * r, B * H * w))  # noqa: E731
    if layout_copies:
        add("K^T copy", nd, nd)
    add("S = scale Q K^T", 2 * nd, nn)
    if causal and layout_copies:
        add("mask S", nn + N * N, nn)
    add("P = softmax(S)", nn, nn)
    add("O = P V", nn + nd, nd)
    if layout_copies:
        add("dO^T copy", nd, nd)
    add("dV = P^T dO", nn + nd, nd)
    if layout_copies:
        add("dV transpose copy", nd, nd)
        add("V^T copy", nd, nd)
    add("dP = dO V^T", 2 * nd, nn)
    add("dS = P o (dP - D)", 2 * nn, nn)
    add("dQ = scale dS K", nn + nd, nd)
    if layout_copies:
        add("Q^T copy", nd, nd)
    add("dK = scale dS^T Q", nn + nd, nd)
    if layout_copies:
        add("dK transpose copy", nd, nd)
    return steps
