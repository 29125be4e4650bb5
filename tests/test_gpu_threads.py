"""Several host threads calling kvx at once, each with its own buffers and
ready object, on streams of their own or all on one shared stream (the
binding's ctypes calls release the interpreter lock, so the calls really
overlap): every backup, restore and exchange gives the oracle's bytes, and
each thread's restores publish into its own ready object."""
import threading

import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from tests.gpu_util import PATHS, DevicePool, Packed, oracle_layout, torch
from tests.test_gpu_parity import SMALL, diff_report

pytestmark = pytest.mark.gpu

# (path of the thread's backups and restores, whether it pairs them in kvx_exchange)
THREADS = [("staged", False), ("zerocopy", False), ("device", False), ("zerocopy", True),
           ("device", True), ("staged", False)]
ROUNDS = 6


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("case", ["llama_small", "trtllm_small", "ragged_hnd"])
def test_threads_calling_at_once(case, shared):
    t = torch()
    one = t.cuda.Stream() if shared else None
    w, _ = SMALL[case]
    n = min(w.num_pages // (len(THREADS) + 1), 64)
    print(f"\n[threads] case={case} shared={shared} threads={len(THREADS)} n={n} rounds={ROUNDS}",
          flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=w.seed + 50, generation=3)
    img = pool.host_image()
    perm = synth.page_perm(w.seed + 51, w.num_pages)
    src = perm[:n].copy()   # read by every thread, written by none
    dsts = [perm[n * (i + 1):n * (i + 2)].copy() for i in range(len(THREADS))]
    nb = w.host_bytes(n)
    errors, results = [], {}

    def worker(i):
        path, paired = THREADS[i]
        stream = one if shared else t.cuda.Stream()
        ready = K.kvx_ready_create(w.num_layers, 3)
        bufs = []
        try:
            got_b = []
            for r in range(ROUNDS):
                pb = Packed(w, n, path, fill_seed=1000 + 10 * i + r)
                pr = Packed(w, n, path, fill_seed=2000 + 10 * i + r)
                bufs += [pb, pr]
                K.kvx_ready_reset(ready)
                if paired:
                    K.kvx_exchange(pool.handle, src, pb.ptr, nb, (0, w.num_layers), pr.ptr, nb,
                                   dsts[i], (0, w.num_layers), ready, 0, stream, PATHS[path])
                else:
                    K.kvx_backup(pool.handle, src, pb.ptr, nb, 0, w.num_layers, stream, PATHS[path])
                    K.kvx_restore(pool.handle, pr.ptr, nb, dsts[i], 0, w.num_layers, ready, 0, stream,
                                  PATHS[path])
                K.kvx_sync(stream)
                got_b.append(pb.numpy())
                assert K.kvx_ready_prefix(ready) == n
            results[i] = got_b
        except Exception as e:   # reported by the main thread
            errors.append((i, repr(e)))
        finally:
            K.kvx_ready_destroy(ready)
            for b in bufs:
                b.close()

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(THREADS))]
    try:
        for th in threads:
            th.start()
        for th in threads:
            th.join(timeout=120)
        assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
        assert not errors, errors
        want_b = oracle.backup(L, img, src, 0, w.num_layers)
        want_alloc = img
        for i in range(len(THREADS)):
            for r, got in enumerate(results[i]):
                assert np.array_equal(got, want_b), f"thread {i} round {r} backup: " + \
                    diff_report(got, want_b)
            last = synth.gen_bytes(2000 + 10 * i + ROUNDS - 1, 0, nb)
            want_alloc = oracle.restore(L, want_alloc, last, dsts[i], 0, w.num_layers)
        after = pool.host_image()
        assert np.array_equal(after, want_alloc), "allocation: " + diff_report(after, want_alloc)
    finally:
        pool.close()
