"""Host-side logic of bench.py, on the CPU: the multi-GPU refusal, the
staleness rule for counter summaries, the summary parsers, the --results
file, the ordinary-attention footprint probe's size arithmetic, and the
exact visible-pair count the wider forms are priced with."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from exact_io_aware_30_amd import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_is_used_only_for_the_library_it_was_taken_on(tmp_path, monkeypatch):
    lib = tmp_path / "lib.so"
    lib.write_bytes(b"kernels v1")
    summary = tmp_path / "summary.txt"
    monkeypatch.setattr(bench, "LIBRARY", str(lib))
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    h = bench.library_hash()
    assert h is not None and len(h) == 16
    summary.write_text(f"header\nlibrary_hash: {h}\ntraffic_bytes bwd_dkdv: 682018949\ntraffic_bytes fwd: 5.5e8\n")
    assert bench.traffic_from_summary("bwd_dkdv") == 682018949.0
    assert bench.traffic_from_summary("fwd") == 5.5e8
    assert bench.traffic_from_summary("bwd_dq") is None
    lib.write_bytes(b"kernels v2")  # rebuilt: the counters no longer describe it
    assert bench.traffic_from_summary("bwd_dkdv") is None
    monkeypatch.setattr(bench, "LIBRARY", str(tmp_path / "missing.so"))
    assert bench.library_hash() is None and bench.traffic_from_summary("fwd") is None


def test_committed_summaries_parse():
    text = open(bench.TRAFFIC_SUMMARY).read()
    assert "library_hash:" in text
    for k in ("fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq"):
        assert f"traffic_bytes {k}:" in text
    measured = bench.io_summary_bytes()
    for key in (("gpt2_medium", "flash"), ("gpt2_medium", "ordinary"), ("long", "flash"), ("long", "ordinary")):
        r, w = measured[key]
        assert r > 0 and w > 0
    # the tiled step writes its outputs once; ordinary attention writes N x N matrices
    assert measured[("long", "ordinary")][1] > 20 * measured[("long", "flash")][1]


def test_io_summary_parser(tmp_path):
    p = tmp_path / "io.txt"
    p.write_text("junk\nmeasured long flash: read 10 written 20\nmeasured gpt2_medium ordinary: read 3 written 4\n")
    assert bench.io_summary_bytes(str(p)) == {("long", "flash"): (10, 20), ("gpt2_medium", "ordinary"): (3, 4)}
    assert bench.io_summary_bytes(str(tmp_path / "none.txt")) == {}


def test_results_file_collects_every_record(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "RECORDS", [])
    out = tmp_path / "results.json"

    def fake_run(args):
        bench.emit({"a": 1})
        bench.emit({"b": 2})

    monkeypatch.setattr(bench, "run", fake_run)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--results", str(out)])
    bench.main()
    assert json.loads(out.read_text()) == [{"a": 1}, {"b": 2}]


@pytest.mark.parametrize("n", [1, 7, 8192])
def test_causal_mask_helper_is_strict_upper_triangle(n):
    import torch

    m = bench.causal_mask(n, "cpu")
    assert m.dtype == torch.bool and m.shape == (n, n)
    assert int(m.sum()) == n * (n - 1) // 2
    assert not bool(m.diagonal().any())
    if n > 1:
        assert bool(m[0, 1]) and not bool(m[1, 0])


@pytest.mark.parametrize("causal", [False, True])
def test_ordinary_comparator_math_on_the_cpu(causal):
    # the comparator's steps (S, mask, softmax, PV; dV, dP, softmax backward,
    # dQ, dK) run on the CPU in float32 match the oracle
    import numpy as np
    import torch

    import oracle

    g = torch.Generator().manual_seed(11)
    B, H, N, d = 2, 3, 37, 16
    q, k, v, do = (torch.randn(B, H, N, d, generator=g) for _ in range(4))
    mask = bench.causal_mask(N, "cpu") if causal else None
    o, dq, dk, dv = bench.ordinary_attention(q, k, v, do, 0.25, causal, mask)
    ref = oracle.attention_backward(*(x.double().numpy() for x in (q, k, v, do)), 0.25, causal)
    for name, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(t.double().numpy(), ref[name], rtol=1e-4, atol=1e-5, err_msg=name)


def _pairs_brute(n, causal, window):
    left, right = (-1, -1) if window is None else window
    count = 0
    for i in range(n):
        for j in range(n):
            if causal and j > i:
                continue
            if left >= 0 and j < i - left:
                continue
            if right >= 0 and j > i + right:
                continue
            count += 1
    return count


@pytest.mark.parametrize("n", [1, 2, 7, 64, 133])
@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (False, (3, 0)), (True, (5, 9)),
                                           (False, (4, 4)), (False, (0, 0)), (True, (-1, 2)), (False, (200, -1))])
def test_visible_pairs_matches_brute_force(n, causal, window):
    assert workloads.visible_pairs(n, causal, window) == _pairs_brute(n, causal, window)


def test_visible_pairs_closed_forms():
    n = 8192
    assert workloads.visible_pairs(n, True) == n * (n + 1) // 2
    assert workloads.visible_pairs(n, False) == n * n
    w = 1024  # left window w, causal: row i sees min(i, w) + 1 keys
    assert workloads.visible_pairs(n, False, (w, 0)) == sum(min(i, w) + 1 for i in range(n))


def test_forward_ceilings_arithmetic():
    rates = {"mfma_bf16_tflops": 2000.0, "softmax_tscores_per_s": 4.0}
    c = bench.forward_ceilings(rates, 128)
    assert c["valu_tflops"] == pytest.approx(4 * 128 * 4.0)  # 4 d FLOPs per score
    assert c["serial_tflops"] == pytest.approx(1 / (1 / 2000.0 + 1 / 2048.0))
    assert bench.forward_ceilings(rates, 32)["valu_tflops"] == pytest.approx(c["valu_tflops"] / 4)
    # in series the pair is slower than either alone
    assert c["serial_tflops"] < min(c["mfma_tflops"], c["valu_tflops"])


def test_overlap_fraction():
    assert bench.overlap_fraction(1.0, 0.5, 1.5) == pytest.approx(0.0)  # one after the other
    assert bench.overlap_fraction(1.0, 0.5, 1.0) == pytest.approx(1.0)  # the shorter fully hidden
    assert bench.overlap_fraction(1.0, 0.8, 1.4) == pytest.approx(0.5)


def test_host_cpu_model_is_named():
    m = bench.host_cpu_model()
    assert isinstance(m, str) and len(m) > 0
