"""Host-side checks of the tuning sweep module (no compiler or GPU run)."""

import os
import re

from exact_io_aware_30_amd import build, tune


def test_every_swept_macro_is_read_by_its_kernel_source():
    for kernel, space in tune.SPACES.items():
        src = open(os.path.join(build.CSRC, tune.SOURCE[kernel])).read()
        assert "default" in space and space["default"] == []
        for name, flags in space.items():
            for f in flags:
                m = re.fullmatch(r"-D(FA_\w+)=(\d+)", f)
                assert m, (kernel, name, f)
                assert re.search(rf"#\s*if(n?def)?\s+{m.group(1)}\b", src), (kernel, m.group(1))


def test_candidates_not_built_are_reported(tmp_path, monkeypatch):
    monkeypatch.setattr(build, "BUILD_DIR", str(tmp_path))
    got = tune.built_candidates("dq")
    assert set(got) == set(tune.SPACES["dq"])
    assert all(p is None for p, _ in got.values())
    lib = tmp_path / "tune" / "dq" / "t32" / build.LIB_NAME
    lib.parent.mkdir(parents=True)
    lib.write_bytes(b"x")
    assert tune.built_candidates("dq", ["t32"])["t32"][0] == str(lib)


def test_shape_parser():
    assert tune._parse_shape("fp16,3,12,2000,32,full") == ("fp16", 3, 12, 2000, 32, False)
    assert tune._parse_shape("bf16,2,16,8192,128,causal") == ("bf16", 2, 16, 8192, 128, True)
