"""Host logic of bench.py, no GPU: the refusal of more than one GPU, the kernel hash that keys the
committed counter profiles (code only: comments and blank lines do not change it), and the
workloads the bench can build."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_kernel_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.hip"])
    src.write_text("int f(int x) {  // doubles\n  return 2 * x;\n}\n")
    h0 = bench.kernel_source_hash()
    src.write_text("// a new comment\nint f(int x) {  // twice x\n\n  return 2 * x;\n}\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f(int x) {\n  return 3 * x;\n}\n")
    assert bench.kernel_source_hash() != h0


@pytest.mark.parametrize("name", ["small_b1", "small_b1_v128256", "uniform_b64"])
def test_small_workloads_have_their_shapes(name):
    assert name in bench.WORKLOADS
    sets = [bench.make_workload(name, k) for k in range(2)]
    for b in sets:
        assert b.target.shape == (b.n_draft_rows + b.B, b.V)
        assert b.draft.shape == (b.n_draft_rows, b.V)
        assert b.cu[0] == 0 and b.cu[-1] == b.n_draft_rows and np.all(np.diff(b.cu) >= 0)
        assert np.all((b.tokens >= 0) & (b.tokens < b.V))
    assert not np.array_equal(sets[0].target, sets[1].target)  # rotated input sets differ


def test_unknown_workload_is_refused():
    with pytest.raises(SystemExit):
        bench.make_workload("no_such_workload", 0)
