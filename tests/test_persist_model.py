"""The persistent kernel's scheduling protocol, run on the CPU: tests/persist_model.cpp
executes the kernel's control loop with one host thread per workgroup over the same
scheduling code the device compiles (csrc/persist_sched.hpp), with random timing, and
checks every ring-slot and task hazard, exactly-once execution, termination, and the
completion check's verdict for a pipeline that receives no workgroup."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "persist_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("persist_model") / "persist_model")
    r = subprocess.run([gxx, "-O2", "-std=c++17", "-pthread", "-Wall", "-Werror", SRC, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_protocol_random_layouts(model, seed):
    """Random expert loads (empty, one-row, partial and hot experts), ring sizes from one row
    tile up, 1..8 pipelines, uneven data-movement shares, dropped pipelines, and work stealing
    at the end of a launch on or off."""
    r = subprocess.run([model, str(seed), "150"], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("OK"), r.stdout
    assert int(r.stdout.split("stolen down tiles: ")[1].split(")")[0]) > 0, r.stdout   # stealing happened
