"""The C ABI used from C: tests/native/abi_c_test.c includes only
include/kvx.h (and the HIP runtime for the caller's own device memory) and
links libkvx.so. Its CPU mode runs here; its GPU mode moves pages on the
GPU and checks the round trip."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "native", "abi_c_test")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_without_gpu():
    from tests.native import build
    build.build()                      # host C only: seconds
    out = subprocess.run([EXE, "cpu"], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip().endswith("ok")


@pytest.mark.gpu
def test_c_program_round_trip_on_the_gpu():
    assert os.path.exists(EXE), "build the C test program first (__graft_entry__.build())"
    print("\n[c-abi] gpu round trip", flush=True)
    out = subprocess.run([EXE, "gpu"], capture_output=True, text=True, timeout=120)
    print(out.stdout, flush=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "round trip" in out.stdout and out.stdout.strip().endswith("ok")
