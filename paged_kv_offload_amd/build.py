"""Builds libkvx.so (the HIP library behind include/kvx.h) for gfx950.

Every source is compiled with hipcc for gfx950 only. The library is linked so
that, inside a process that already imported torch, it binds to the same
HIP runtime instance as torch (both sonames are libamdhip64.so.7; the rpath
puts torch's copy first when kvx is loaded on its own).
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkvx.so")
SOURCES = ["api.cpp", "geometry.cpp", "pages.cpp", "ipc.cpp", "ready.cpp", "tier.cpp", "ring.cpp", "tier_policy.cpp", "ring_exec.cpp", "kernels.hip", "noalloc.hip"]
ARCH = "gfx950"
# packed-fp32 instructions are disabled for all device code
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wextra",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def torch_lib_dir() -> str:
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        return ""
    return os.path.join(list(spec.submodule_search_locations)[0], "lib")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, out_dir: str = None) -> str:
    out_dir = out_dir or HERE
    obj_dir = os.path.join(out_dir, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC] + lang +
                    ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # the sources compile independently: a few at a time
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
        for r in ex.map(lambda c: subprocess.run(c, check=True), cmds):
            pass
    rpaths = [d for d in (torch_lib_dir(), "/opt/rocm/lib") if d]
    lib = os.path.join(out_dir, "libkvx.so")
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", lib + ".tmp"] + objs + \
          [f"-Wl,-rpath,{d}" for d in rpaths] + ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx",
                                                 "-Wl,--no-undefined", "-Wl,-soname,libkvx.so"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
