"""Memory-traffic simulator: both versions of attention executed over a
main memory that counts every byte read and written.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring).

The pages compare the two versions by the traffic they send over the slow
link ("flash-attn-triton" docs, "The argument" and Table 2; "What is
FlashAttention?", "What you will build", step 03, which asks for an exact
count of the reads and writes of both).  This module runs each version on
one (batch, head) slice in fp64, taking every operand from a
``CountingMemory`` and putting every result back into it, so that the count
is what the executed algorithm moved, and the results can be checked
against the plain definition:

* ``ordinary``  -- the materialising version: S = scale QK^T is written,
  read back by the softmax (which applies the causal mask), P is written and
  read again by PV; the backward writes dP and dS.  Optionally with the
  N x d transposed copies and the separate mask pass of a GPU comparator
  built from library GEMMs, softmax and elementwise kernels.
* ``tiled``     -- the tiled version: the forward of Fig. 3 (query blocks
  outer, key tiles inner, running max and sum, one divide at the end, L
  saved per row), the D = rowsum(dO o O) pass, a key-block-outer dK/dV pass
  and a query-block-outer dQ pass that rebuild P from L.  Only tiles are
  loaded; N x N data never reaches the memory.  Tile shapes are parameters;
  the L and D vectors are loaded ``stats`` entries per query tile in the
  dK/dV pass.
"""

from __future__ import annotations

import numpy as np


class CountingMemory:
    """Named row-major arrays; read and write count element size x elements."""

    def __init__(self):
        self.arrays, self.size = {}, {}
        self.read_bytes = 0
        self.write_bytes = 0

    def put(self, name, array, elem_bytes):
        """Initial contents (not counted)."""
        self.arrays[name] = np.array(array, dtype=np.float64)
        self.size[name] = elem_bytes

    def alloc(self, name, shape, elem_bytes):
        self.put(name, np.zeros(shape), elem_bytes)

    def read(self, name, r0=None, r1=None):
        a = self.arrays[name] if r0 is None else self.arrays[name][r0:r1]
        self.read_bytes += a.size * self.size[name]
        return a.copy()

    def write(self, name, value, r0=None, r1=None):
        value = np.asarray(value, dtype=np.float64)
        if r0 is None:
            self.arrays[name][...] = value
        else:
            self.arrays[name][r0:r1] = value
        self.write_bytes += value.size * self.size[name]

    def take(self, name):
        return self.arrays[name].copy()


def _inputs(q, k, v, do, e):
    mem = CountingMemory()
    for name, x in (("q", q), ("k", k), ("v", v), ("do", do)):
        mem.put(name, x, e)
    return mem


# ---------------------------------------------------------------------------
# ordinary attention
# ---------------------------------------------------------------------------

def ordinary(q, k, v, do, scale, causal, e, layout_copies=False):
    """Ordinary attention, forward and backward, on one slice (q, k, v, do:
    N x d).  Returns (outputs, [(step, read, written)]) with outputs o, lse,
    dq, dk, dv.  Every step reads its operands from memory once and writes
    its result once."""
    n, d = q.shape
    mem = _inputs(q, k, v, do, e)
    steps = []

    def step(name, fn):
        r0, w0 = mem.read_bytes, mem.write_bytes
        fn()
        steps.append((name, mem.read_bytes - r0, mem.write_bytes - w0))

    def transpose(src, dst):
        mem.alloc(dst, (mem.arrays[src].shape[1], mem.arrays[src].shape[0]), e)
        mem.write(dst, mem.read(src).T)

    future = np.triu(np.ones((n, n), dtype=bool), 1)  # key after query: not visible

    if layout_copies:
        step("K^T copy", lambda: transpose("k", "kt"))
    kname = "kt" if layout_copies else "k"
    mem.alloc("s", (n, n), e)
    step("S = scale Q K^T", lambda: mem.write(
        "s", scale * (mem.read("q") @ (mem.read(kname) if layout_copies else mem.read(kname).T))))
    if causal and layout_copies:
        mem.put("mask", future, 1)

        def mask():
            s, m = mem.read("s"), mem.read("mask").astype(bool)
            mem.write("s", np.where(m, -np.inf, s))

        step("mask S", mask)
    mem.alloc("p", (n, n), e)
    mem.alloc("lse", (n,), 4)

    def softmax():
        s = mem.read("s")
        if causal and not layout_copies:
            s = np.where(future, -np.inf, s)
        m = s.max(axis=1, keepdims=True)
        x = np.exp(s - m)
        mem.write("p", x / x.sum(axis=1, keepdims=True))
        mem.arrays["lse"][:] = (m + np.log(x.sum(axis=1, keepdims=True)))[:, 0]  # kept for the check only

    step("P = softmax(S)", softmax)
    mem.alloc("o", (n, d), e)
    step("O = P V", lambda: mem.write("o", mem.read("p") @ mem.read("v")))

    if layout_copies:
        step("dO^T copy", lambda: transpose("do", "dot"))
        mem.alloc("dvt", (d, n), e)
        step("dV = P^T dO", lambda: mem.write("dvt", mem.read("dot") @ mem.read("p")))
        step("dV transpose copy", lambda: transpose("dvt", "dv"))
        step("V^T copy", lambda: transpose("v", "vt"))
    else:
        mem.alloc("dv", (n, d), e)
        step("dV = P^T dO", lambda: mem.write("dv", mem.read("p").T @ mem.read("do")))
    mem.alloc("dp", (n, n), e)
    step("dP = dO V^T", lambda: mem.write(
        "dp", mem.read("do") @ (mem.read("vt") if layout_copies else mem.read("v").T)))
    mem.alloc("ds", (n, n), e)

    def dsoft():
        p, dp = mem.read("p"), mem.read("dp")
        mem.write("ds", p * (dp - (p * dp).sum(axis=1, keepdims=True)))

    step("dS = P o (dP - D)", dsoft)
    mem.alloc("dq", (n, d), e)
    step("dQ = scale dS K", lambda: mem.write("dq", scale * (mem.read("ds") @ mem.read("k"))))
    if layout_copies:
        step("Q^T copy", lambda: transpose("q", "qt"))
        mem.alloc("dkt", (d, n), e)
        step("dK = scale dS^T Q", lambda: mem.write("dkt", scale * (mem.read("qt") @ mem.read("ds"))))
        step("dK transpose copy", lambda: transpose("dkt", "dk"))
    else:
        mem.alloc("dk", (n, d), e)
        step("dK = scale dS^T Q", lambda: mem.write("dk", scale * (mem.read("ds").T @ mem.read("q"))))
    out = {name: mem.take(name) for name in ("o", "lse", "dq", "dk", "dv")}
    return out, steps


# ---------------------------------------------------------------------------
# tiled attention
# ---------------------------------------------------------------------------

def _visible(q_rows, k_rows, causal):
    return (k_rows[None, :] <= q_rows[:, None]) if causal else np.ones((len(q_rows), len(k_rows)), dtype=bool)


def _last_key_tile_end(n, q0, bm, bn, causal):
    """End row of the key tiles a query block loads: whole tiles up to its
    last visible key, clipped at n."""
    if not causal:
        return n
    last = min(n, q0 + bm)
    return min(n, -(-last // bn) * bn)


def tiled(q, k, v, do, scale, causal, e, fwd_bm, fwd_bn, dkdv_bk, dkdv_bq, dkdv_stats, dq_bm, dq_bn):
    """Tiled attention, forward and backward, on one slice.  Returns
    (outputs, {pass: (read, written)}) with outputs o, lse, dq, dk, dv."""
    n, d = q.shape
    mem = _inputs(q, k, v, do, e)
    for name in ("o", "dq", "dk", "dv"):
        mem.alloc(name, (n, d), e)
    for name in ("lse", "delta"):
        mem.alloc(name, (n,), 4)
    counts = {}

    def run(name, fn):
        r0, w0 = mem.read_bytes, mem.write_bytes
        fn()
        counts[name] = (mem.read_bytes - r0, mem.write_bytes - w0)

    def forward():
        # Fig. 3: one query block resident, key tiles streamed; running max m,
        # running sum l, accumulator rescaled by exp(m_old - m_new).
        for q0 in range(0, n, fwd_bm):
            q1 = min(n, q0 + fwd_bm)
            qi = mem.read("q", q0, q1)
            rows = np.arange(q0, q1)
            m = np.full(q1 - q0, -np.inf)
            l = np.zeros(q1 - q0)
            acc = np.zeros((q1 - q0, d))
            for j0 in range(0, _last_key_tile_end(n, q0, fwd_bm, fwd_bn, causal), fwd_bn):
                j1 = min(n, j0 + fwd_bn)
                kj, vj = mem.read("k", j0, j1), mem.read("v", j0, j1)
                s = np.where(_visible(rows, np.arange(j0, j1), causal), scale * (qi @ kj.T), -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                ref = np.where(np.isfinite(m_new), m_new, 0.0)
                p = np.exp(s - ref[:, None])
                alpha = np.exp(np.where(np.isfinite(m), m - ref, -np.inf))
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ vj
                m = m_new
            mem.write("o", acc / l[:, None], q0, q1)
            mem.write("lse", m + np.log(l), q0, q1)

    def preprocess():
        mem.write("delta", (mem.read("o") * mem.read("do")).sum(axis=1))

    def dkdv():
        for k0 in range(0, n, dkdv_bk):
            k1 = min(n, k0 + dkdv_bk)
            kj, vj = mem.read("k", k0, k1), mem.read("v", k0, k1)
            cols = np.arange(k0, k1)
            dk = np.zeros((k1 - k0, d))
            dv = np.zeros((k1 - k0, d))
            for i0 in range(k0 if causal else 0, n, dkdv_bq):  # queries before k0 see none of these keys
                i1 = min(n, i0 + dkdv_bq)
                qi, doi = mem.read("q", i0, i1), mem.read("do", i0, i1)
                s1 = min(n, i0 + dkdv_stats)
                li = mem.read("lse", i0, s1)[: i1 - i0]
                di = mem.read("delta", i0, s1)[: i1 - i0]
                vis = _visible(np.arange(i0, i1), cols, causal)
                p = np.where(vis, np.exp(scale * (qi @ kj.T) - li[:, None]), 0.0)
                dv += p.T @ doi
                ds = p * (doi @ vj.T - di[:, None])
                dk += scale * (ds.T @ qi)
            mem.write("dk", dk, k0, k1)
            mem.write("dv", dv, k0, k1)

    def dq():
        for q0 in range(0, n, dq_bm):
            q1 = min(n, q0 + dq_bm)
            qi, doi = mem.read("q", q0, q1), mem.read("do", q0, q1)
            li, di = mem.read("lse", q0, q1), mem.read("delta", q0, q1)
            rows = np.arange(q0, q1)
            acc = np.zeros((q1 - q0, d))
            for j0 in range(0, _last_key_tile_end(n, q0, dq_bm, dq_bn, causal), dq_bn):
                j1 = min(n, j0 + dq_bn)
                kj, vj = mem.read("k", j0, j1), mem.read("v", j0, j1)
                p = np.where(_visible(rows, np.arange(j0, j1), causal), np.exp(scale * (qi @ kj.T) - li[:, None]),
                             0.0)
                ds = p * (doi @ vj.T - di[:, None])
                acc += scale * (ds @ kj)
            mem.write("dq", acc, q0, q1)

    run("fwd", forward)
    run("bwd_preprocess", preprocess)
    run("bwd_dkdv", dkdv)
    run("bwd_dq", dq)
    out = {name: mem.take(name) for name in ("o", "lse", "dq", "dk", "dv")}
    return out, counts
