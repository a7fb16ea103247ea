"""The 16-byte split plans (csrc/split.hpp) that let rows off the 16-byte grid use vector loads,
checked on the host: tests/split_bounds.cpp walks them over vocabularies 1..300 and sizes around
chunk boundaries, every element offset of the target base, draft and q bases, and several rows, and
checks that each chunk's head, vectors and tail cover it exactly, that the edges fit one element
per lane, and that every vector and every piece of the second row is aligned, lies inside its
chunk or row, and carries the bytes the kernels read under it.  No GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_split_plans_stay_inside_their_rows(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "split_bounds")
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-Werror", os.path.join(HERE, "split_bounds.cpp"), "-o", exe],
                   check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.startswith("ok "), out.stdout
    assert int(out.stdout.split()[1]) > 1_000_000
