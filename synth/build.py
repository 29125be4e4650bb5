"""Builds synth/libkvxsynth.so (the GPU fill/compare kernels of the input
generator) for gfx950."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fill.hip")
LIB = os.path.join(HERE, "libkvxsynth.so")


def _torch_lib_dir() -> str:
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        return ""
    return os.path.join(list(spec.submodule_search_locations)[0], "lib")


def build(verbose: bool = False) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    rp = [d for d in (_torch_lib_dir(), "/opt/rocm/lib") if d]
    cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-x", "hip", SRC, "-o", LIB + ".tmp"] + [f"-Wl,-rpath,{d}" for d in rp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
