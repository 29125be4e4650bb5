"""Builds tests/native/abi_c_test (a C11 program that uses kvx through
include/kvx.h alone) with the host C compiler, linked against the in-tree
libkvx.so and the HIP runtime."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "paged_kv_offload_amd")
EXE = os.path.join(HERE, "abi_c_test")


def build(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
           os.path.join(HERE, "abi_c_test.c"), "-o", EXE + ".tmp",
           "-L", PKG, "-lkvx", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
