"""Device-memory IPC across two processes on one GPU ([RFC] "Device IPC data
path"; [RAWIPC] "the full share/rebuild chain"). A second process allocates
a pool, fills it from the seeded generator and exports it; this process
imports it by handle bytes, checks a BACKUP of the shared pool
against the oracle, and RESTOREs into other pages of it. The exporting
process then checks its whole allocation against the oracle's closed form
of that round trip (the restored pages, every other page and the padding
around the pool at its byte offset).

The importer is the parent process. With ROCm 7's dmabuf-based IPC a child
importing its parent's allocation was refused (hipErrorInvalidValue from
hipIpcOpenMemHandle) where the parent importing its child's works: the
importer needs the rights to take the exporter's dmabuf file descriptor."""
import ctypes
import dataclasses
import json
import os
import select
import subprocess
import sys
import time

import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import WORKLOADS
from tests.gpu_util import kvx_layout, oracle_layout, torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CASES = {
    # head-major, pool at byte offset 12288 of its allocation
    "trtllm_small": (WORKLOADS["trtllm_hnd"].scaled(name="trtllm_small", num_pages=64, num_layers=3), 16),
    "llama_small": (WORKLOADS["llama8b"].scaled(name="llama_small", num_pages=96, num_layers=3), 24),
}


def read_reply(proc, timeout=120.0):
    """One JSON line from the exporting process, within `timeout` seconds."""
    deadline = time.monotonic() + timeout
    while True:
        left = deadline - time.monotonic()
        if left <= 0:
            raise TimeoutError("the exporting process did not answer")
        r, _, _ = select.select([proc.stdout], [], [], left)
        if r:
            line = proc.stdout.readline()
            if not line:
                raise RuntimeError(f"the exporting process ended ({proc.poll()})")
            line = line.strip()
            if line.startswith("{"):
                return json.loads(line)


def ptrace_scope():
    try:
        return open("/proc/sys/kernel/yama/ptrace_scope").read().strip()
    except OSError:
        return "n/a"


@pytest.mark.parametrize("case", list(CASES))
def test_pool_shared_with_a_second_process(case, tmp_path):
    w, n = CASES[case]
    torch()  # the GPU runtime of this process
    print(f"\n[ipc] case={case} alloc={w.alloc_bytes} offset={w.byte_offset} "
          f"ptrace_scope={ptrace_scope()} "
          f"HSA_ENABLE_IPC_MODE_LEGACY={os.environ.get('HSA_ENABLE_IPC_MODE_LEGACY')}", flush=True)
    perm = synth.page_perm(w.seed, w.num_pages)
    src, dst = perm[:n].copy(), perm[n:2 * n].copy()
    params = tmp_path / "params.json"
    params.write_text(json.dumps({"workload": dataclasses.asdict(w), "seed": w.seed, "generation": 11}))
    pages = tmp_path / "pages.json"
    pages.write_text(json.dumps({"src": src.tolist(), "dst": dst.tolist()}))
    proc = subprocess.Popen([sys.executable, os.path.join(ROOT, "tests", "ipc_exporter.py"),
                             str(params)], stdin=subprocess.PIPE, stdout=subprocess.PIPE,
                            stderr=subprocess.PIPE, text=True, env=dict(os.environ))
    pool = base = ready = rbase = None
    try:
        first = read_reply(proc)
        assert "handle" in first, first
        handle = bytes.fromhex(first["handle"])
        hs = K.ipc_handle_from_bytes(handle)
        assert hs.offset == w.byte_offset and hs.alloc_bytes >= w.alloc_bytes
        pool, base = K.register_imported(handle, kvx_layout(w), w.dtype_bytes, w.tensor_shape(), 11)
        # a second import of the same handle maps nothing new
        base2, _, off2, _ = K.kvx_ipc_import(handle)
        assert base2 == base and off2 == w.byte_offset
        K.kvx_ipc_close(base2)
        # the exporter's ready counts: this process publishes into them
        rbase, _, roff, _ = K.kvx_ipc_import(bytes.fromhex(first["ready_handle"]))
        ready = K.kvx_ready_attach_device(rbase + roff, w.num_layers, 11)
        assert K.kvx_ready_prefix(ready) == 0
        proc.stdin.write(f"arm {n}\n")
        proc.stdin.flush()
        assert read_reply(proc).get("armed")
        L = oracle_layout(w)
        P = w.payload_bytes(n)
        host = K.HostBuffer(P)
        try:
            K.kvx_backup(pool, src, host.ptr, P, 0, w.num_layers, None, K.KVX_PATH_ZEROCOPY)
            K.kvx_sync(None)
            bad, at = oracle.check_backup_gen(L, w.seed, src, 0, w.num_layers, host.numpy(), 0)
            assert bad == 0, f"backup of the imported pool: {bad} bytes differ, first at {at}"
            K.kvx_restore(pool, host.ptr, P, dst, 0, w.num_layers, ready, 0, None,
                          K.KVX_PATH_STAGED)
            K.kvx_sync(None)
            assert K.kvx_ready_prefix(ready) == n
        finally:
            host.free()
        K.kvx_unregister_pool(pool)
        pool = None
        K.kvx_ready_destroy(ready)
        ready = None
        K.kvx_ipc_close(rbase)
        rbase = None
        K.kvx_ipc_close(base)
        with pytest.raises(K.KvxError):
            K.kvx_ipc_close(base)          # the last open was closed
        base = None
        proc.stdin.write(f"check {pages}\n")
        proc.stdin.flush()
        res = read_reply(proc)
        assert res.get("bad_bytes") == 0, res
        # the exporter's GPU wait saw the count this process published, and
        # so does its host query
        assert res.get("wait_status") == 1 and res.get("prefix") == n, res
        proc.stdin.write("exit\n")
        proc.stdin.flush()
        assert read_reply(proc).get("exited")
        assert proc.wait(timeout=60) == 0
    finally:
        if pool:
            K.kvx_unregister_pool(pool)
        if ready:
            K.kvx_ready_destroy(ready)
        if rbase:
            K.kvx_ipc_close(rbase)
        if base:
            K.kvx_ipc_close(base)
        if proc.poll() is None:
            proc.kill()
            proc.wait(timeout=30)
        err = proc.stderr.read()
        if err:
            print(err[-2000:], flush=True)


def test_export_refuses_non_device_memory_and_large_allocations():
    t = torch()
    host = K.HostBuffer(1 << 20)
    try:
        with pytest.raises(K.KvxError) as e:
            K.kvx_ipc_export(host.ptr)
        assert e.value.code == K.KVX_E_INVAL
    finally:
        host.free()
    big = t.empty((2 << 30) + (2 << 20), dtype=t.uint8, device="cuda")
    with pytest.raises(K.KvxError) as e:
        K.kvx_ipc_export(big.data_ptr() + 4096)
    assert e.value.code == K.KVX_E_RANGE
    del big


def test_export_refuses_an_allocation_of_exactly_two_gib():
    """The IPC size bound is exclusive: an allocation of exactly
    KVX_IPC_MAX_BYTES (2 GiB) is refused with KVX_E_RANGE by the size check,
    before the runtime is asked for a handle, and one just below it is
    exported. The allocations come from hipMalloc itself (torch's caching
    allocator may hand out part of a larger segment)."""
    torch().cuda.init()
    hip = ctypes.CDLL(K.hip_runtimes_mapped()[0])
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipFree.argtypes = [ctypes.c_void_p]
    for size, ok in ((2 << 30, False), ((2 << 30) - (2 << 20), True)):
        p = ctypes.c_void_p()
        assert hip.hipMalloc(ctypes.byref(p), size) == 0
        try:
            base, got = K.kvx_alloc_range(p.value + 4096)
            assert (base, got) == (p.value, size)
            if ok:
                h = K.ipc_handle_from_bytes(K.kvx_ipc_export(p.value + 4096))
                assert (h.alloc_bytes, h.offset) == (size, 4096)
            else:
                with pytest.raises(K.KvxError) as e:
                    K.kvx_ipc_export(p.value + 4096)
                assert e.value.code == K.KVX_E_RANGE, e.value.message
        finally:
            assert hip.hipFree(p) == 0
