"""The C-ABI library loads, exports every function include/fa.h declares, and
rejects bad arguments before enqueuing anything (no GPU needed).

Where a GPU is visible the pointers handed to rejected calls are real device
buffers of the stated sizes, so that even a wrongly accepted call would stay
in bounds; without a GPU they are plain addresses that are never touched.
"""

import ctypes
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

from exact_io_aware_30_amd import binding  # noqa: E402

lib = binding._lib
OK, INVALID, UNSUPPORTED, ALIGN, HIPERR, ALIAS, SCRATCH = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_functions_are_exported():
    names = declared_functions()
    assert names == sorted(["fa_fwd", "fa_bwd_preprocess", "fa_bwd", "fa_bwd_dkdv", "fa_bwd_dq",
                            "fa_fwd_gqa", "fa_bwd_gqa", "fa_bwd_dkdv_gqa", "fa_bwd_dq_gqa",
                            "fa_fwd_ex", "fa_bwd_ex", "fa_bwd_dkdv_ex", "fa_bwd_dq_ex",
                            "fa_fwd_varlen", "fa_bwd_varlen",
                            "fa_bwd_ex_ws", "fa_bwd_varlen_ws", "fa_bwd_workspace_size", "fa_bwd_ex_scratch",
                            "fa_bwd_varlen_workspace_size",
                            "fa_status_string", "fa_version"])
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)$", out, flags=re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(binding.EXPORTED) == set(names)


def test_status_strings_and_version():
    for code in (OK, INVALID, UNSUPPORTED, ALIGN, HIPERR, ALIAS, SCRATCH):
        s = binding.fa_status_string(code)
        assert s and s != "unknown status"
    assert binding.fa_status_string(12345) == "unknown status"
    assert binding.fa_version() >= 100


class Ptrs:
    """Pointer values for argument checks: device buffers if a GPU exists."""

    def __init__(self, nbytes=1 << 16, count=12):
        self.keep = []
        if torch.cuda.is_available():
            for _ in range(count):
                t = torch.zeros(nbytes // 2, dtype=torch.float16, device="cuda")
                self.keep.append(t)
            self.p = [t.data_ptr() for t in self.keep]
        else:
            self.p = [0x10000000 * (i + 1) for i in range(count)]


SMALL = dict(B=1, H=1, N=64, d=64)  # 8 KiB per tensor, fits the 64 KiB buffers


def fwd(p, q=None, k=None, v=None, o=None, lse=None, B=1, H=1, N=64, d=64, scale=0.125, causal=0, dt=1):
    a = [p[0] if q is None else q, p[1] if k is None else k, p[2] if v is None else v,
         p[3] if o is None else o, p[4] if lse is None else lse]
    return lib.fa_fwd(*a, B, H, N, d, scale, causal, dt, None)


def bwd(p, fn="fa_bwd", B=1, H=1, N=64, d=64, scale=0.125, causal=0, dt=1, **over):
    names = ["q", "k", "v", "do", "lse", "delta", "dq", "dk", "dv"]
    vals = {n: p[i] for i, n in enumerate(names)}
    vals.update(over)
    if fn == "fa_bwd":
        args = [vals[n] for n in names]
    elif fn == "fa_bwd_dkdv":
        args = [vals[n] for n in names if n != "dq"]
    else:
        args = [vals[n] for n in names if n not in ("dk", "dv")]
    return getattr(lib, fn)(*args, B, H, N, d, scale, causal, dt, None)


@pytest.fixture(scope="module")
def p():
    return Ptrs().p


def test_fwd_rejects(p):
    for i in range(5):
        args = {k: None for k in ("q", "k", "v", "o", "lse")}
        key = list(args)[i]
        assert fwd(p, **{key: 0}) == INVALID
    assert fwd(p, B=0) == INVALID
    assert fwd(p, H=-1) == INVALID
    assert fwd(p, N=0) == INVALID
    for d in (0, 16, 48, 96, 256):
        assert fwd(p, d=d) == UNSUPPORTED
    for s in (0.0, -1.0, float("nan"), float("inf")):
        assert fwd(p, scale=s) == INVALID
    assert fwd(p, causal=2) == INVALID
    assert fwd(p, causal=-1) == INVALID
    assert fwd(p, dt=2) == INVALID
    assert fwd(p, q=p[0] + 8) == ALIGN
    assert fwd(p, lse=p[4] + 4) == ALIGN
    # one head slice must fit 32-bit byte offsets
    assert fwd(p, N=((1 << 31) - (1 << 20)) // 256 + 1, d=128) == UNSUPPORTED
    assert fwd(p, B=1 << 12, H=1 << 12, N=64) == UNSUPPORTED
    # outputs overlapping inputs or each other
    assert fwd(p, o=p[0]) == ALIAS
    assert fwd(p, lse=p[3] + 16) == ALIAS
    assert fwd(p, o=p[2] + 4096) == ALIAS


def test_preprocess_rejects(p):
    pre = lambda o=p[0], do=p[1], dl=p[2], B=1, H=1, N=64, d=64, dt=1: \
        lib.fa_bwd_preprocess(o, do, dl, B, H, N, d, dt, None)  # noqa: E731
    assert pre(o=0) == INVALID
    assert pre(dl=0) == INVALID
    assert pre(N=0) == INVALID
    assert pre(d=80) == UNSUPPORTED
    assert pre(dt=5) == INVALID
    assert pre(do=p[1] + 2) == ALIGN
    assert pre(dl=p[0] + 64) == ALIAS


@pytest.mark.parametrize("fn", ["fa_bwd", "fa_bwd_dkdv", "fa_bwd_dq"])
def test_bwd_rejects(p, fn):
    outs = {"fa_bwd": ["dq", "dk", "dv"], "fa_bwd_dkdv": ["dk", "dv"], "fa_bwd_dq": ["dq"]}[fn]
    for name in ["q", "k", "v", "do", "lse", "delta"] + outs:
        assert bwd(p, fn, **{name: 0}) == INVALID, name
    assert bwd(p, fn, N=0) == INVALID
    assert bwd(p, fn, d=100) == UNSUPPORTED
    assert bwd(p, fn, scale=float("nan")) == INVALID
    assert bwd(p, fn, causal=3) == INVALID
    assert bwd(p, fn, dt=9) == INVALID
    assert bwd(p, fn, delta=p[5] + 4) == ALIGN
    assert bwd(p, fn, **{outs[0]: p[0]}) == ALIAS
    assert bwd(p, fn, **{outs[-1]: p[4]}) == ALIAS
    if len(outs) > 1:
        assert bwd(p, fn, **{outs[0]: p[11], outs[1]: p[11] + 64}) == ALIAS


def test_gqa_rejects(p):
    # fa_fwd_gqa(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, dt, stream)
    f = lambda H=2, Hkv=1, **o: lib.fa_fwd_gqa(o.get("q", p[0]), o.get("k", p[1]), o.get("v", p[2]),  # noqa: E731
                                               o.get("o", p[3]), o.get("lse", p[4]), 1, H, Hkv, 64, 64, 0.125, 0,
                                               1, None)
    assert f(Hkv=0) == INVALID
    assert f(H=4, Hkv=3) == INVALID
    assert f(H=2, Hkv=4) == INVALID
    assert f(k=0) == INVALID
    # o [1,2,64,64] = 16 KiB from p[3]; with Hkv = 1, k is 8 KiB: o at k + 8 KiB is clear, at k + 4 KiB overlaps
    assert f(o=p[1] + 4096) == ALIAS
    names = ["q", "k", "v", "do", "lse", "delta", "dq", "dk", "dv"]

    def b(fn, H=2, Hkv=1, **over):
        vals = {n: p[i] for i, n in enumerate(names)}
        vals.update(over)
        keep = {"fa_bwd_gqa": names, "fa_bwd_dkdv_gqa": [n for n in names if n != "dq"],
                "fa_bwd_dq_gqa": [n for n in names if n not in ("dk", "dv")]}[fn]
        return getattr(lib, fn)(*[vals[n] for n in keep], 1, H, Hkv, 64, 64, 0.125, 0, 1, None)

    for fn in ("fa_bwd_gqa", "fa_bwd_dkdv_gqa", "fa_bwd_dq_gqa"):
        assert b(fn, Hkv=0) == INVALID
        assert b(fn, H=6, Hkv=4) == INVALID
        assert b(fn, q=0) == INVALID
    # dk [1,1,64,64] is 8 KiB: placed 4 KiB into v (8 KiB) it overlaps
    assert b("fa_bwd_dkdv_gqa", dk=p[2] + 4096) == ALIAS
    assert b("fa_bwd_gqa", dq=p[0] + 8192) == ALIAS  # q is 16 KiB with H = 2


def test_window_rejects(p):
    # fa_fwd_ex(q, k, v, o, lse, B, H, Hkv, N, d, scale, wl, wr, dt, stream)
    f = lambda wl, wr, Hkv=1: lib.fa_fwd_ex(p[0], p[1], p[2], p[3], p[4], 1, 1, Hkv, 64, 64, 0.125, wl, wr, 1,  # noqa
                                            None)
    assert f(-2, 0) == INVALID
    assert f(0, -5) == INVALID
    assert f(3, 3, Hkv=0) == INVALID
    g = lambda wl, wr: lib.fa_bwd_ex(*p[:9], 1, 1, 1, 64, 64, 0.125, wl, wr, 1, None)  # noqa: E731
    assert g(-3, 1) == INVALID
    assert lib.fa_bwd_dkdv_ex(*p[:6], p[7], p[8], 1, 1, 1, 64, 64, 0.125, 2, -9, 1, None) == INVALID
    assert lib.fa_bwd_dq_ex(*p[:7], 1, 1, 1, 64, 64, 0.125, -4, 0, 1, None) == INVALID
    # the causal flag of the older entry points must be 0 or 1
    assert lib.fa_fwd_gqa(*p[:5], 1, 1, 1, 64, 64, 0.125, 2, 1, None) == INVALID


def test_varlen_rejects(p):
    # fa_fwd_varlen(q, k, v, o, lse, cu, B, max_seqlen, T, H, Hkv, d, scale, wl, wr, dt, stream)
    def f(cu=None, B=2, mx=32, T=64, H=1, Hkv=1, d=64, wl=-1, wr=0):
        return lib.fa_fwd_varlen(p[0], p[1], p[2], p[3], p[4], p[5] if cu is None else cu, B, mx, T, H, Hkv, d,
                                 0.125, wl, wr, 1, None)
    assert f(cu=0) == INVALID
    assert f(B=0) == INVALID
    assert f(mx=0) == INVALID
    assert f(T=0) == INVALID
    assert f(Hkv=3, H=2) == INVALID
    assert f(d=48) == UNSUPPORTED
    assert f(wl=-7) == INVALID
    assert f(cu=p[5] + 2) == ALIGN
    assert lib.fa_bwd_varlen(*p[:9], 0, 2, 32, 64, 1, 1, 64, 0.125, -1, 0, 1, None) == INVALID
    # The offsets are an input: no output (nor the workspace) may cover them.
    assert f(cu=p[3]) == ALIAS                     # o over the offsets
    assert f(cu=p[4] + 64) == ALIAS                # lse over the offsets
    cu = p[10]
    assert lib.fa_bwd_varlen(*p[:6], cu, p[7], p[8], cu, 2, 32, 64, 1, 1, 64, 0.125, -1, 0, 1, None) == ALIAS  # dq
    assert lib.fa_bwd_varlen(*p[:7], cu - 16, p[8], cu, 2, 32, 64, 1, 1, 64, 0.125, -1, 0, 1, None) == ALIAS  # dk
    vneed = binding.fa_bwd_varlen_workspace_size(2, 32, 64, 8, 1, 32)
    assert vneed > 0
    assert lib.fa_bwd_varlen_ws(*p[:9], cu, 2, 32, 64, 8, 1, 32, 0.125, -1, 0, 1, cu - 4096, vneed,
                                None) == ALIAS  # workspace


def test_binding_rejects_host_tensors():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError):
        binding.fa_fwd(q, q, q, q.clone(), lse, 0.125, False)
    with pytest.raises(ValueError):
        binding.fa_bwd_preprocess(q.float(), q.float(), lse)


def test_every_kernel_launch_stub_is_defined():
    # A host pass that drops a kernel's launch stub leaves an undefined
    # symbol that only fails when the library is loaded.
    out = subprocess.run(["nm", "-D", binding.LIB_PATH], capture_output=True, text=True).stdout
    missing = [line for line in out.splitlines() if " U " in line and "device_stub" in line]
    assert not missing, missing[:3]


def test_workspace_forms_reject(p):
    # fa_bwd_ex_ws(q, k, v, dO, lse, delta, dq, dk, dv, B, H, Hkv, N, d, scale, wl, wr, dt, ws, ws_bytes, stream)
    def f(ws, nbytes, B=1, H=8, Hkv=1, N=64, d=32):
        return lib.fa_bwd_ex_ws(*p[:9], B, H, Hkv, N, d, 0.125, -1, 0, 1, ws, nbytes, None)

    need = binding.fa_bwd_workspace_size(1, 8, 1, 64, 32)
    assert need == 2 * 8 * 64 * 32 * 4  # one key block: all 8 heads split, dK and dV float32 partials
    assert f(None, 16) == INVALID  # bytes without a pointer
    assert f(p[9] + 8, need) == ALIGN  # a workspace the split would use must be 16-byte aligned
    assert f(p[0], need) == ALIAS  # over q
    assert f(p[9], need, Hkv=3) == INVALID  # 8 heads are not a multiple of 3
    assert f(p[9], need, d=48) == UNSUPPORTED
    # fa_bwd_varlen_ws(..., cu, B, max_seqlen, T, H, Hkv, d, scale, wl, wr, dt, ws, ws_bytes, stream)
    vneed = binding.fa_bwd_varlen_workspace_size(2, 32, 64, 8, 1, 32)
    assert vneed == 2 * 8 * 64 * 32 * 4
    assert lib.fa_bwd_varlen_ws(*p[:9], p[10], 2, 32, 64, 8, 1, 32, 0.125, -1, 0, 1, None, 16, None) == INVALID
    assert lib.fa_bwd_varlen_ws(*p[:9], p[10], 2, 32, 64, 8, 1, 32, 0.125, -1, 0, 1, p[3], vneed, None) == ALIAS


@pytest.mark.skipif(torch.cuda.is_available(), reason="fake pointers: run where no GPU is visible")
def test_scratch_form_rejects():
    """fa_bwd_ex_scratch checks like fa_bwd_ex_ws, then refuses a split whose
    partials exceed the static array, before any HIP call (fake, disjoint
    pointers: nothing may be launched)."""
    f = lib.fa_bwd_ex_scratch
    fake = [0x10000000 * (i + 1) for i in range(9)]
    args = lambda B, H, Hkv, N, d: (*fake, B, H, Hkv, N, d, 0.125, -1, 0, 1, None)  # noqa: E731
    # 16 query heads on one key/value head, 200 key blocks: the rule splits
    # 16 ways, 2 * 16 * 25600 * 128 * 4 bytes = 400 MiB > 256 MiB
    assert binding.fa_bwd_workspace_size(1, 16, 1, 25600, 128) == 2 * 16 * 25600 * 128 * 4
    assert f(*args(1, 16, 1, 25600, 128)) == SCRATCH
    assert binding.SCRATCH_BYTES == 256 << 20
    assert "static array" in binding.fa_status_string(SCRATCH)
    # the checks of the workspace form come first
    assert f(*args(1, 16, 3, 25600, 128)) == INVALID
    assert f(*args(1, 16, 1, 25600, 48)) == UNSUPPORTED
    a = list(args(1, 16, 1, 25600, 128))
    a[6] = a[0]  # dq over q
    assert f(*a) == ALIAS


def test_workspace_size_rule():
    ws = binding.fa_bwd_workspace_size
    assert ws(2, 16, 16, 8192, 128) == 0  # no grouping: nothing to split
    assert ws(1, 4, 3, 64, 64) == 0 and ws(0, 4, 1, 64, 64) == 0 and ws(1, 4, 1, 64, 48) == 0  # invalid
    # 64 key blocks x 2 batches x 4 kv heads = 512 workgroups: 4 splits reach 2048
    assert ws(2, 16, 4, 8192, 128) == 2 * 4 * (2 * 4 * 8192) * 128 * 4
    # 1024 workgroups: 2 splits
    assert ws(2, 16, 8, 8192, 128) == 2 * 2 * (2 * 8 * 8192) * 128 * 4
    # 128 workgroups: all 16 heads split, 2048
    assert ws(2, 16, 1, 8192, 128) == 2 * 16 * (2 * 8192) * 128 * 4
    # split counts are divisors of the group, at most the group: 12 heads, 100 workgroups -> 12
    assert ws(1, 12, 1, 12800, 64) == 2 * 12 * 12800 * 64 * 4
    # groups of 3 heads, 2 kv heads x 200 key blocks = 400 workgroups: at most 3 splits
    assert ws(1, 6, 2, 25600, 32) == 2 * 3 * (2 * 25600) * 32 * 4
    # enough workgroups already: no split
    assert ws(8, 32, 8, 8192, 128) == 0
    # 24 sequences x 32 key blocks of the longest = 768 workgroups: 4 splits
    assert binding.fa_bwd_varlen_workspace_size(24, 4077, 55662, 16, 1, 128) == 2 * 4 * 55662 * 128 * 4


def test_rates_library_exports_and_rejects():
    """libfa_rates.so (measurement support) exports what csrc/fa_rates.h
    declares, and rejects bad arguments before touching the GPU."""
    import ctypes

    from exact_io_aware_30_amd.build import CSRC, RATES_LIB_PATH

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(CSRC, "fa_rates.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))
    assert names == ["fa_rates_atomic", "fa_rates_lds", "fa_rates_valu"]
    out = subprocess.run(["nm", "-D", "--defined-only", RATES_LIB_PATH], capture_output=True, text=True).stdout
    assert set(names) <= set(re.findall(r"\bT (fa_\w+)$", out, flags=re.M))
    lib = ctypes.CDLL(RATES_LIB_PATH)
    lib.fa_rates_valu.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int, ctypes.c_void_p]
    lib.fa_rates_valu.restype = ctypes.c_int
    buf = (ctypes.c_double * 8)()
    assert lib.fa_rates_valu(None, 8, None) == -1
    assert lib.fa_rates_valu(buf, 7, None) == -1
    lib.fa_rates_lds.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int, ctypes.c_void_p]
    lib.fa_rates_lds.restype = ctypes.c_int
    assert lib.fa_rates_lds(None, 6, None) == -1
    assert lib.fa_rates_lds(buf, 5, None) == -1
    lib.fa_rates_atomic.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    lib.fa_rates_atomic.restype = ctypes.c_int
    assert lib.fa_rates_atomic(None, 8, 8192, 32, None) == -1
    assert lib.fa_rates_atomic(buf, 7, 8192, 32, None) == -1
    assert lib.fa_rates_atomic(buf, 8, 8190, 32, None) == -1   # N not a multiple of 128
    assert lib.fa_rates_atomic(buf, 8, 8192, 0, None) == -1
    assert lib.fa_rates_atomic(buf, 8, 65536, 1024, None) == -1  # over 2^30 floats
