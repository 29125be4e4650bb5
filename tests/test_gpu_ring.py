"""GPU tests of the ring executor: descriptors submitted on a ring are run by
kvx_ring_serve and their bytes equal the oracle's; completions arrive in
submission order only once the work has finished; a refused descriptor
does not hold up the others; and a data-plane process serves a scheduler
process that shares its pool through device-memory IPC, then releases
everything when that process dies."""
import dataclasses
import json
import os
import subprocess
import sys
import threading
import time

import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import Workload
from tests.gpu_util import DevicePool, Packed, oracle_layout, torch
from tests.test_gpu_parity import SMALL, diff_report

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def serve_until(ring, o, pools, bufs, sizes, want, ready=None, stream=None, limit=30.0):
    got = []
    t0 = time.time()
    while len(got) < want:
        K.kvx_ring_serve(o, pools, bufs, sizes, ready, stream)
        got += K.kvx_ring_reap(ring, 64)
        assert time.time() - t0 < limit, f"only {len(got)} of {want} completions"
    return got


@pytest.mark.parametrize("path", ["zerocopy", "device"])
@pytest.mark.parametrize("case", ["llama_small", "ragged_hnd"])
def test_ring_ops_match_the_oracle(case, path):
    """BACKUP, BACKUP_SLOTS, a descriptor of another generation, RESTORE
    with publish and RESTORE_SLOTS, served in one process: bytes, publish
    and completion order as the oracle and the calls say."""
    w, n = SMALL[case]
    n = min(n, K.KVX_RING_MAX_PAGES)
    print(f"\n[ring] case={case} path={path} n={n}", flush=True)
    t = torch()
    L = oracle_layout(w)
    pool = DevicePool(w, seed=w.seed + 80, generation=4)
    S = 2 * n + 1
    packed = Packed(w, n, path, fill_seed=w.seed + 81)
    tierbuf = Packed(w, S, path, fill_seed=w.seed + 82)
    ready = K.kvx_ready_create(w.num_layers, 4)
    stream = t.cuda.Stream()
    name = f"/kvx-gpu-{os.getpid()}-{case}-{path}"
    ring = K.kvx_ring_create(name, 8, 4)
    o = K.kvx_ring_open(name)
    P = K.PATHS[path]
    perm = synth.page_perm(w.seed + 83, w.num_pages)
    src, dst, dst2 = perm[:n], perm[n:2 * n], perm[2 * n:3 * n] if 3 * n <= w.num_pages else None
    slots = np.random.default_rng(w.seed + 84).permutation(S)[:n].astype(np.int32)
    try:
        img = pool.host_image()
        nl = w.num_layers
        ops = [K.make_sqe(K.KVX_OP_BACKUP, 1, 4, 0, 0, src, 0, nl, P),
               K.make_sqe(K.KVX_OP_BACKUP_SLOTS, 2, 4, 0, 1, src, 0, nl, P, host_slots=slots,
                          num_host_slots=S),
               K.make_sqe(K.KVX_OP_BACKUP, 3, 3, 0, 0, src, 0, nl, P),      # old generation
               K.make_sqe(K.KVX_OP_RESTORE, 4, 4, 0, 0, dst, 0, nl, P, ready_slot_base=0)]
        if dst2 is not None:
            ops.append(K.make_sqe(K.KVX_OP_RESTORE_SLOTS, 5, 4, 0, 1, dst2, 0, nl, P,
                                  host_slots=slots, num_host_slots=S))
        for q in ops:
            K.kvx_ring_submit(ring, q)
        got = serve_until(ring, o, [pool.handle], [packed.ptr, tierbuf.ptr],
                          [packed.nbytes, tierbuf.nbytes], len(ops), ready, stream)
        assert [(g[0], g[2]) for g in got] == \
            [(1, 0), (2, 0), (3, K.KVX_E_STALE), (4, 0)] + ([(5, 0)] if dst2 is not None else [])
        # completions only once the work is done: the bytes are there without a sync
        want_pk = oracle.backup(L, img, src, 0, nl)
        got_pk = packed.numpy()
        assert np.array_equal(got_pk, want_pk), "BACKUP " + diff_report(got_pk, want_pk)
        want_tier = oracle.backup_slots(L, img, src, slots, S, 0, nl,
                                        host=synth.gen_bytes(w.seed + 82, 0, tierbuf.nbytes))
        got_tier = tierbuf.numpy()
        assert np.array_equal(got_tier, want_tier), "BACKUP_SLOTS " + diff_report(got_tier, want_tier)
        want = oracle.restore(L, img, want_pk, dst, 0, nl)
        if dst2 is not None:
            want = oracle.restore_slots(L, want, want_tier, slots, dst2, S, 0, nl)
        after = pool.host_image()
        assert np.array_equal(after, want), "RESTORE " + diff_report(after, want)
        assert K.kvx_ready_prefix(ready) == n
        assert K.kvx_ring_drain(o) == 0
    finally:
        K.kvx_ring_close(o)
        K.kvx_ring_close(ring)
        K.kvx_ready_destroy(ready)
        packed.close()
        tierbuf.close()
        pool.close()


@pytest.mark.parametrize("pairing", [1, 0])
@pytest.mark.parametrize("path", ["zerocopy", "device"])
def test_ring_runs_backup_and_restore_together(path, pairing):
    """A BACKUP followed by a RESTORE of other pages runs as one exchange
    (or, with pairing off, one after the other) with the same bytes; a
    RESTORE followed by a BACKUP of the pages it writes is refused as a pair
    and runs in submission order, so the BACKUP reads the restored bytes."""
    t = torch()
    w, n = SMALL["llama_small"]
    print(f"\n[ring-pair] path={path} pairing={pairing} n={n}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=w.seed + 85, generation=4)
    nb = w.host_bytes(n)
    bufs = [Packed(w, n, path, fill_seed=w.seed + 86 + k) for k in range(3)]
    ready = K.kvx_ready_create(w.num_layers, 4)
    stream = t.cuda.Stream()
    name = f"/kvx-pair-{os.getpid()}-{path}-{pairing}"
    ring = K.kvx_ring_create(name, 8, 4)
    o = K.kvx_ring_open(name)
    P = K.PATHS[path]
    nl = w.num_layers
    perm = synth.page_perm(w.seed + 87, w.num_pages)
    src, dst, dst2 = perm[:n], perm[n:2 * n], perm[2 * n:3 * n]
    old = K.kvx_get_option(K.KVX_OPT_RING_PAIRING)
    try:
        K.kvx_set_option(K.KVX_OPT_RING_PAIRING, pairing)
        img = pool.host_image()
        h0 = synth.gen_bytes(w.seed + 86, 0, nb)
        ops = [K.make_sqe(K.KVX_OP_BACKUP, 1, 4, 0, 1, src, 0, nl, P),
               K.make_sqe(K.KVX_OP_RESTORE, 2, 4, 0, 0, dst, 0, nl, P, ready_slot_base=0),
               K.make_sqe(K.KVX_OP_RESTORE, 3, 4, 0, 1, dst2, 0, nl, P),
               K.make_sqe(K.KVX_OP_BACKUP, 4, 4, 0, 2, dst2, 0, nl, P)]
        for q in ops:
            K.kvx_ring_submit(ring, q)
        got = serve_until(ring, o, [pool.handle], [b.ptr for b in bufs], [b.nbytes for b in bufs],
                          len(ops), ready, stream)
        assert [(g[0], g[2]) for g in got] == [(1, 0), (2, 0), (3, 0), (4, 0)]
        b1 = oracle.backup(L, img, src, 0, nl)
        assert np.array_equal(bufs[1].numpy(), b1)
        want = oracle.restore(L, img, h0, dst, 0, nl)
        want = oracle.restore(L, want, b1, dst2, 0, nl)
        after = pool.host_image()
        assert np.array_equal(after, want), diff_report(after, want)
        # the BACKUP of dst2 ran after the RESTORE into it: it read b1
        assert np.array_equal(bufs[2].numpy(), b1), diff_report(bufs[2].numpy(), b1)
        assert K.kvx_ready_prefix(ready) == n
    finally:
        K.kvx_set_option(K.KVX_OPT_RING_PAIRING, old)
        K.kvx_ring_close(o)
        K.kvx_ring_close(ring)
        K.kvx_ready_destroy(ready)
        for b in bufs:
            b.close()
        pool.close()


@pytest.mark.parametrize("path", ["zerocopy", "device"])
def test_ring_pairs_slot_descriptors(path):
    """BACKUP_SLOTS followed by RESTORE_SLOTS of other slots and pages of one
    host tier run as one exchange: the tier and the pool hold the oracle's
    bytes, and the restore publishes."""
    t = torch()
    w, n = SMALL["ragged_hnd"]
    n = 300
    S = 2 * n + 8
    print(f"\n[ring-pair-slots] path={path} n={n} slots={S}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=w.seed + 95, generation=4)
    tier = Packed(w, S, path, fill_seed=w.seed + 96)
    ready = K.kvx_ready_create(w.num_layers, 4)
    stream = t.cuda.Stream()
    name = f"/kvx-pair-slots-{os.getpid()}-{path}"
    ring = K.kvx_ring_create(name, 8, 4)
    o = K.kvx_ring_open(name)
    P = K.PATHS[path]
    nl = w.num_layers
    perm = synth.page_perm(w.seed + 97, w.num_pages)
    src, dst = perm[:n], perm[n:2 * n]
    order = np.random.default_rng(w.seed + 98).permutation(S).astype(np.int32)
    bsl, rsl = order[:n], order[n:2 * n]
    try:
        img = pool.host_image()
        host0 = synth.gen_bytes(w.seed + 96, 0, tier.nbytes)
        K.kvx_ring_submit(ring, K.make_sqe(K.KVX_OP_BACKUP_SLOTS, 1, 4, 0, 0, src, 0, nl, P,
                                           host_slots=bsl, num_host_slots=S))
        K.kvx_ring_submit(ring, K.make_sqe(K.KVX_OP_RESTORE_SLOTS, 2, 4, 0, 0, dst, 0, nl, P,
                                           ready_slot_base=0, host_slots=rsl, num_host_slots=S))
        got = serve_until(ring, o, [pool.handle], [tier.ptr], [tier.nbytes], 2, ready, stream)
        assert [(g[0], g[2]) for g in got] == [(1, 0), (2, 0)]
        want_tier = oracle.backup_slots(L, img, src, bsl, S, 0, nl, host=host0.copy())
        assert np.array_equal(tier.numpy(), want_tier), diff_report(tier.numpy(), want_tier)
        want = oracle.restore_slots(L, img, host0, rsl, dst, S, 0, nl)
        after = pool.host_image()
        assert np.array_equal(after, want), diff_report(after, want)
        assert K.kvx_ready_prefix(ready) == n
    finally:
        K.kvx_ring_close(o)
        K.kvx_ring_close(ring)
        K.kvx_ready_destroy(ready)
        tier.close()
        pool.close()


IPC_CASE = Workload(name="ring_ipc", outer=("layer", "kv", "page"), inner="HND", num_pages=200,
                    num_layers=3, num_kv=2, page_size=16, num_heads=4, head_dim=64, dtype_bytes=2,
                    pages_per_request=40, seed=231, byte_offset=4096, alloc_tail=4096)


def test_data_plane_serves_a_scheduler_process_and_survives_its_death(tmp_path):
    """A scheduler process allocates and exports its pool, creates the ring
    and submits BACKUP_SLOTS then RESTORE_SLOTS of 40 pages; this process
    (the data plane) imports the pool, owns the host tier and serves. The
    scheduler checks its whole allocation against the oracle's closed form
    of the round trip. It then submits two more descriptors and dies
    without reaping; the data plane sees it gone, discards what it had not
    taken, drains, and releases the pool and the mapping without error."""
    t = torch()
    w = IPC_CASE
    n, S = w.pages_per_request, 64
    perm = synth.page_perm(w.seed, w.num_pages)
    slots = np.random.default_rng(w.seed + 1).permutation(S)[:n].astype(np.int32)
    params = {"workload": dataclasses.asdict(w),
              "seed": w.seed, "generation": 12, "n": n, "slots": S,
              "src": perm[:n].tolist(), "dst": perm[n:2 * n].tolist(),
              "host_slots": slots.tolist(), "ring": f"/kvx-ipc-{os.getpid()}"}
    pfile = tmp_path / "params.json"
    pfile.write_text(json.dumps(params))
    print(f"\n[ring-ipc] alloc={w.alloc_bytes} n={n} slots={S}", flush=True)
    child = subprocess.Popen([sys.executable, os.path.join(HERE, "ring_scheduler.py"), str(pfile)],
                             stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True)
    lines = []
    reader = threading.Thread(target=lambda: lines.extend(child.stdout), daemon=True)
    first = json.loads(child.stdout.readline())
    assert "error" not in first, first
    reader.start()
    base = pool = ring = None
    tier = K.HostBuffer(w.host_bytes(S))
    stream = t.cuda.Stream()
    try:
        lay = K.make_layout(w.outer, w.inner, w.num_pages, w.num_layers, w.num_kv, w.page_size,
                            w.num_heads, w.head_dim)
        pool, base = K.register_imported(bytes.fromhex(first["handle"]), lay, w.dtype_bytes,
                                         w.tensor_shape(), 12)
        ring = K.kvx_ring_open(params["ring"])
        child.stdin.write("go\n")
        child.stdin.flush()
        t0 = time.time()
        while not lines and time.time() - t0 < 60:
            K.kvx_ring_serve(ring, [pool], [tier.ptr], [tier.nbytes], None, stream)
            time.sleep(0.001)
        assert lines, "the scheduler process did not report"
        report = json.loads(lines[0])
        assert report.get("bad") == 0 and report.get("statuses") == [0, 0], report
        assert report.get("op_ids") == [1, 2], report
        # the scheduler submits two more descriptors and dies without reaping
        child.stdin.write("die\n")
        child.stdin.flush()
        assert child.wait(30) == 0
        assert not K.kvx_ring_peer_alive(ring)
        assert K.kvx_ring_discard(ring) == 2
        assert K.kvx_ring_drain(ring) == 0
        K.kvx_ring_close(ring)             # the dead creator's name is removed
        ring = None
        assert not os.path.exists("/dev/shm" + params["ring"])
    finally:
        if child.poll() is None:
            child.kill()
            child.wait()
        if ring:
            K.kvx_ring_close(ring)
        if pool:
            K.kvx_unregister_pool(pool)
        if base:
            K.kvx_ipc_close(base)
        tier.free()
