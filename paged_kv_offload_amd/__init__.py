"""kvx: paged-KV backup/restore between an MI355X GPU KV pool and pinned host
memory, as hand-written HIP kernels behind a C ABI (include/kvx.h).

This package holds the HIP sources (csrc/), their build step (build.py) and a
ctypes binding (kvx.py) whose functions carry the C names.
"""
from .kvx import *  # noqa: F401,F403
from .kvx import KvxError, HostBuffer, lib, make_layout, register_tensor  # noqa: F401
