"""Exporting process of the device-memory IPC test (run by test_gpu_ipc.py,
not collected by pytest): allocates a pool with hipMalloc (so the
allocation is exactly the pool plus its padding), fills it from the seeded
generator, creates a ready object with device-memory counts, exports both
with kvx_ipc_export and serves commands read from stdin, one per line:
  arm <count>               - enqueues a bounded GPU wait for the last
                              layer's count to reach <count>
  check <params json file>  - waits for the GPU, then reports the armed
                              wait's status, the ready prefix, and the
                              whole allocation checked against the oracle's
                              closed form of BACKUP(src) -> RESTORE(dst)
                              done by the importer
  exit                      - frees everything and exits
Every reply is one JSON line on stdout. Stdin closing ends the process."""
import ctypes
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402
from paged_kv_offload_amd import kvx as K  # noqa: E402
from synth.workloads import Workload  # noqa: E402


def workload(p):
    wd = dict(p["workload"])
    wd["outer"] = tuple(wd["outer"])
    return Workload(**wd)


def oracle_layout(w):
    return oracle.Layout(outer=tuple({"page": oracle.PAGE, "layer": oracle.LAYER,
                                      "kv": oracle.KV}[a] for a in w.outer),
                         inner=oracle.NHD if w.inner == "NHD" else oracle.HND,
                         num_pages=w.num_pages, num_layers=w.num_layers, num_kv=w.num_kv,
                         page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
                         dtype_bytes=w.dtype_bytes, byte_offset=w.byte_offset)


def reply(obj):
    print(json.dumps(obj), flush=True)


def main():
    p = json.load(open(sys.argv[1]))
    w = workload(p)
    K.lib()
    paths = K.hip_runtimes_mapped()
    hip = ctypes.CDLL(paths[0])
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipFree.argtypes = [ctypes.c_void_p]
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    ptr = ctypes.c_void_p()
    if hip.hipMalloc(ctypes.byref(ptr), w.alloc_bytes) != 0:
        reply({"error": "hipMalloc failed"})
        return 1
    try:
        synth.fill_alloc_gpu(ptr.value, w, p["seed"])
        hip.hipDeviceSynchronize()
        handle = K.kvx_ipc_export(ptr.value + w.byte_offset)
        ready = K.kvx_ready_create_device(0, w.num_layers, p["generation"])
        ready_handle = K.kvx_ipc_export(K.kvx_ready_slot_ptr(ready, 0))
        status = ctypes.c_void_p()
        if hip.hipMalloc(ctypes.byref(status), 4096) != 0:
            reply({"error": "hipMalloc failed"})
            return 1
        reply({"handle": handle.hex(), "ready_handle": ready_handle.hex(), "pid": os.getpid()})
        for line in sys.stdin:
            cmd = line.split()
            if not cmd:
                continue
            if cmd[0] == "arm":
                # bounded: at most 10M polls (about 17 s), then status 0
                K.kvx_ready_wait_gpu(ready, w.num_layers - 1, int(cmd[1]), None, 10_000_000,
                                     status.value)
                reply({"armed": True})
            elif cmd[0] == "check":
                q = json.load(open(cmd[1]))
                img = np.empty(w.alloc_bytes, dtype=np.uint8)
                hip.hipDeviceSynchronize()
                st = np.zeros(1, dtype=np.int32)
                hip.hipMemcpy(st.ctypes.data, status.value, 4, 2)
                prefix = K.kvx_ready_prefix(ready)
                if hip.hipMemcpy(img.ctypes.data, ptr.value, w.alloc_bytes, 2) != 0:
                    reply({"error": "hipMemcpy failed"})
                    continue
                bad, first = oracle.check_alloc_roundtrip(
                    oracle_layout(w), p["seed"], p["seed"] + 1, np.array(q["src"], dtype=np.int32),
                    np.array(q["dst"], dtype=np.int32), 0, w.num_layers, img, 0)
                reply({"bad_bytes": int(bad), "first_bad": int(first), "wait_status": int(st[0]),
                       "prefix": int(prefix)})
            elif cmd[0] == "exit":
                break
    finally:
        hip.hipDeviceSynchronize()
        if "ready" in locals():
            K.kvx_ready_destroy(ready)
        if "status" in locals() and status.value:
            hip.hipFree(status)
        hip.hipFree(ptr)
    reply({"exited": True})
    return 0


if __name__ == "__main__":
    sys.exit(main())
