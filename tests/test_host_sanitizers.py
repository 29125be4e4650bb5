"""The host-only parts of the runtime (pool layout validator, page-list
checks, run planning, host-tier allocator, shared-memory rings) built with AddressSanitizer and
UndefinedBehaviorSanitizer by the host compiler and fuzzed (CPU only)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_offload_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_logic_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "geometry.cpp"), os.path.join(CSRC, "pages.cpp"),
           os.path.join(CSRC, "tier.cpp"), os.path.join(CSRC, "ring.cpp"),
           os.path.join(ROOT, "tests", "native", "host_fuzz.cpp"), "-o", exe, "-lpthread"]
    subprocess.run(cmd, check=True)
    # verify_asan_link_order=0: another preloaded library may come before the
    # ASan runtime in the process; the checks do not depend on the order
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "host fuzz ok" in out.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_rings_and_tier_under_tsan(tmp_path):
    """The rings and the host tier used from several threads at once, built
    with ThreadSanitizer: no data race, and every count adds up."""
    exe = str(tmp_path / "host_threads")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=thread",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "ring.cpp"), os.path.join(CSRC, "tier.cpp"),
           os.path.join(ROOT, "tests", "native", "host_threads.cpp"), "-o", exe, "-lpthread"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")
    out = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "host threads ok" in out.stdout
