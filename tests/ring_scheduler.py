"""Scheduler process of the ring test (run by test_gpu_ring.py, not collected
by pytest): allocates a pool with hipMalloc, fills it from the seeded
generator, exports it with kvx_ipc_export, creates the ring and replies
with the handle. On "go" (stdin) it submits BACKUP_SLOTS of `src` into
the data plane's host tier and RESTORE_SLOTS of the same slots into `dst`,
reaps both completions, and replies with their statuses and the number of
allocation bytes that differ from the oracle's closed form of that round
trip. On "die" it submits two more descriptors and exits without reaping
or closing anything."""
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402
from paged_kv_offload_amd import kvx as K  # noqa: E402
from synth.workloads import Workload  # noqa: E402
from tests.ipc_exporter import oracle_layout, reply, workload  # noqa: E402


def main():
    p = json.load(open(sys.argv[1]))
    w = workload(p)
    K.lib()
    hip = ctypes.CDLL(K.hip_runtimes_mapped()[0])
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipFree.argtypes = [ctypes.c_void_p]
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    ptr = ctypes.c_void_p()
    if hip.hipMalloc(ctypes.byref(ptr), w.alloc_bytes) != 0:
        reply({"error": "hipMalloc failed"})
        return 1
    synth.fill_alloc_gpu(ptr.value, w, p["seed"])
    hip.hipDeviceSynchronize()
    handle = K.kvx_ipc_export(ptr.value + w.byte_offset)
    gen, n, S = p["generation"], p["n"], p["slots"]
    ring = K.kvx_ring_create(p["ring"], 8, gen)
    reply({"handle": handle.hex(), "pid": os.getpid()})
    src = np.array(p["src"], dtype=np.int32)
    dst = np.array(p["dst"], dtype=np.int32)
    slots = np.array(p["host_slots"], dtype=np.int32)
    nl = w.num_layers
    Z = K.KVX_PATH_ZEROCOPY
    for line in sys.stdin:
        cmd = line.strip()
        if cmd == "go":
            K.kvx_ring_submit(ring, K.make_sqe(K.KVX_OP_BACKUP_SLOTS, 1, gen, 0, 0, src, 0, nl, Z,
                                               host_slots=slots, num_host_slots=S))
            K.kvx_ring_submit(ring, K.make_sqe(K.KVX_OP_RESTORE_SLOTS, 2, gen, 0, 0, dst, 0, nl, Z,
                                               host_slots=slots, num_host_slots=S))
            got = []
            t0 = time.time()
            while len(got) < 2 and time.time() - t0 < 60:
                got += K.kvx_ring_reap(ring, 8)
                time.sleep(0.001)
            img = np.empty(w.alloc_bytes, dtype=np.uint8)
            if hip.hipMemcpy(img.ctypes.data, ptr.value, w.alloc_bytes, 2) != 0:
                reply({"error": "hipMemcpy failed"})
                continue
            bad, first = oracle.check_alloc_roundtrip(oracle_layout(w), p["seed"], p["seed"] + 1,
                                                      src, dst, 0, nl, img, 0)
            reply({"statuses": [g[2] for g in got], "op_ids": [g[0] for g in got],
                   "bad": int(bad), "first_bad": int(first)})
        elif cmd == "die":
            for k in (3, 4):
                K.kvx_ring_submit(ring, K.make_sqe(K.KVX_OP_BACKUP_SLOTS, k, gen, 0, 0, src, 0, nl,
                                                   Z, host_slots=slots, num_host_slots=S))
            sys.stdout.flush()
            os._exit(0)
    return 0


if __name__ == "__main__":
    sys.exit(main())
