"""Host-only check of the library's load indices and launch plans.

Compiles tests/index_check.cpp (g++, no GPU) against the constexpr index and
launch-geometry functions the kernels and launchers use
(stable_variance_amd/csrc/sv_index.hpp), runs it, and requires that every
load of every walked launch lies inside its array and every planned launch
stays within HIP's dispatch limits.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("index") / "index_check")
    res = subprocess.run([gxx, "-std=c++17", "-O2", "-Wall", "-Werror", os.path.join(HERE, "index_check.cpp"),
                          "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def test_every_load_and_launch_in_bounds(checker):
    res = subprocess.run([checker], capture_output=True, text=True, timeout=600)
    tail = res.stdout.strip().splitlines()[-1]
    assert res.returncode == 0 and tail.endswith(" 0 failures"), res.stdout[-4000:]
    loads = int(tail.split()[0])
    assert loads > 10**9  # the walk covered the shapes (not an empty loop)
