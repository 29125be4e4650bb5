"""GPU parity at full workload sizes, in the launch configuration the benchmark
times (default tuning; staged and zero-copy paths); also the llama8b shape at
one token per page, whose 16,384-page requests travel as device page lists
and whole 2 KiB pieces.

Pools are filled on the GPU from the seeded generator, so the oracle's
closed forms give every expected byte without a host copy of the input:
the whole packed buffer of every BACKUP and the whole allocation after every
RESTORE (pool, padding before the byte offset and after the pool) are
checked byte for byte, in parallel host threads."""
import os
import threading
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import WORKLOADS, request_pair
from tests.gpu_util import PATHS, DevicePool, oracle_layout, torch

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))
SPLIT = 64 << 20


def _ranges(total, step=SPLIT):
    return [(a, min(total, a + step)) for a in range(0, total, step)]


def check_packed(w, L, seed, ids, l0, l1, host: np.ndarray):
    """Whole packed buffer: the layers [l0, l1) against the closed form of
    BACKUP, the other layers against the prefill pattern (seed + 2)."""
    n = len(ids)
    lo, hi = l0 * w.num_kv * n * w.piece_bytes, l1 * w.num_kv * n * w.piece_bytes

    def one(r):
        a, b = r
        if a >= lo and b <= hi:
            return oracle.check_backup_gen(L, seed, ids, l0, l1, host[a:b], a)
        bad = np.flatnonzero(host[a:b] != synth.gen_bytes(w.seed + 2, a, b - a))
        return bad.size, (a + int(bad[0]) if bad.size else -1)

    rngs = [r for part in ((0, lo), (lo, hi), (hi, host.size)) for r in
            [(a + part[0], b + part[0]) for a, b in _ranges(part[1] - part[0])]]
    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(one, rngs))
    bad = sum(r[0] for r in res)
    first = min((r[1] for r in res if r[0]), default=-1)
    return bad, first


def check_alloc(w, L, seed, src, dst, l0, l1, alloc_dev):
    """Whole allocation after BACKUP(src) -> RESTORE(dst), copied to host one
    GiB at a time and checked against the oracle's closed form."""
    t = torch()
    t.cuda.synchronize()
    bad, first = 0, -1
    step = 1 << 30
    for a in range(0, w.alloc_bytes, step):
        b = min(w.alloc_bytes, a + step)
        buf = alloc_dev[a:b].cpu().numpy()

        def one(r, a=a, buf=buf):
            x, y = r
            return oracle.check_alloc_roundtrip(L, seed, seed + 1, src, dst, l0, l1, buf[x:y],
                                                a + x)

        with ThreadPoolExecutor(THREADS) as ex:
            res = list(ex.map(one, _ranges(b - a)))
        bad += sum(r[0] for r in res)
        fs = [r[1] for r in res if r[0]]
        if fs and first < 0:
            first = min(fs)
    return bad, first


@pytest.mark.parametrize("path", ["staged", "zerocopy"])
@pytest.mark.parametrize("name", ["llama8b", "mla_fp8", "trtllm_hnd", "token_pages"])
def test_full_size_backup_restore(name, path):
    t = torch()
    w = WORKLOADS[name]
    n = w.pages_per_request
    print(f"\n[full] {name} {path}: pool {w.pool_bytes / 2**30:.1f} GiB, n={n}", flush=True)
    L = oracle_layout(w)
    src, dst = request_pair(w)
    pool = DevicePool(w, generation=5)
    P = w.payload_bytes(n)
    host = K.HostBuffer(P)
    synth.fill_gpu(host.ptr, P, w.seed + 2, 0)
    t.cuda.synchronize()
    stream = t.cuda.Stream()
    ready = K.kvx_ready_create(w.num_layers, 5)
    try:
        K.kvx_backup(pool.handle, src, host.ptr, P, 0, w.num_layers, stream, PATHS[path])
        K.kvx_sync(stream)
        t0 = time.time()
        bad, first = check_packed(w, L, w.seed, src, 0, w.num_layers, host.numpy())
        print(f"[full] packed buffer checked in {time.time() - t0:.1f} s", flush=True)
        assert bad == 0, f"backup: {bad} bytes differ, first at packed offset {first}"
        K.kvx_restore(pool.handle, host.ptr, P, dst, 0, w.num_layers, ready, 0, stream,
                      PATHS[path])
        K.kvx_sync(stream)
        assert K.kvx_ready_prefix(ready) == n
        t0 = time.time()
        bad, first = check_alloc(w, L, w.seed, src, dst, 0, w.num_layers, pool.alloc)
        print(f"[full] allocation checked in {time.time() - t0:.1f} s", flush=True)
        assert bad == 0, f"restore: {bad} bytes differ, first at allocation byte {first}"
    finally:
        K.kvx_ready_destroy(ready)
        host.free()
        pool.close()


@pytest.mark.parametrize("name", ["llama8b", "mla_fp8", "token_pages"])
def test_full_size_device_path_as_benchmarked(name):
    """The benchmark's roofline calls at full size: the request packed into
    a device buffer in one call (the whole packed buffer checked against
    the closed form of BACKUP), unpacked into the destination pages without
    publish, then - after the pool is refilled - unpacked again publishing
    every layer (the queue-driven kernel drawing blocks of units); each time
    the whole allocation is checked against the closed form of the round
    trip."""
    t = torch()
    w = WORKLOADS[name]
    n = w.pages_per_request
    print(f"\n[full] {name} device path: pool {w.pool_bytes / 2**30:.1f} GiB, n={n}", flush=True)
    L = oracle_layout(w)
    src, dst = request_pair(w)
    pool = DevicePool(w, generation=5)
    P = w.payload_bytes(n)
    dev = t.empty(P, dtype=t.uint8, device="cuda")
    stream = t.cuda.Stream()
    ready = K.kvx_ready_create(w.num_layers, 5)
    D = K.KVX_PATH_DEVICE
    try:
        K.kvx_backup(pool.handle, src, dev.data_ptr(), P, 0, w.num_layers, stream, D)
        K.kvx_sync(stream)
        bad, first = check_packed(w, L, w.seed, src, 0, w.num_layers, dev.cpu().numpy())
        assert bad == 0, f"pack: {bad} bytes differ, first at packed offset {first}"
        for publish in (False, True):
            if publish:
                synth.fill_alloc_gpu(pool.alloc.data_ptr(), w, w.seed)
                t.cuda.synchronize()
            K.kvx_restore(pool.handle, dev.data_ptr(), P, dst, 0, w.num_layers,
                          ready if publish else None, 0, stream, D)
            K.kvx_sync(stream)
            if publish:
                assert [K.kvx_layer_ready(ready, l) for l in range(w.num_layers)] == [n] * w.num_layers
            t0 = time.time()
            bad, first = check_alloc(w, L, w.seed, src, dst, 0, w.num_layers, pool.alloc)
            print(f"[full] allocation (publish={publish}) checked in {time.time() - t0:.1f} s", flush=True)
            assert bad == 0, f"unpack (publish={publish}): {bad} bytes differ, first at allocation byte {first}"
    finally:
        K.kvx_ready_destroy(ready)
        del dev
        pool.close()


def test_full_size_mla_layerwise_ready():
    """The MLA fp8 pool: four 64-page requests, each backed up and restored
    layer by layer into its own pages; a CPU thread samples the published
    counts while the restore runs: they never decrease, never exceed n, and
    the prefix is their minimum; the first layer is published before the
    last one."""
    t = torch()
    w = WORKLOADS["mla_fp8"]
    n = w.pages_per_request
    L = oracle_layout(w)
    pool = DevicePool(w, generation=6)
    P = w.payload_bytes(n)
    host = K.HostBuffer(P)
    stream = t.cuda.Stream()
    ready = K.kvx_ready_create(w.num_layers, 6)
    srcs, dsts = [], []
    try:
        for r in range(4):
            src, dst = request_pair(w, r)
            srcs.append(src)
            dsts.append(dst)
            synth.fill_gpu(host.ptr, P, w.seed + 2, 0)
            t.cuda.synchronize()
            K.kvx_backup(pool.handle, src, host.ptr, P, 0, w.num_layers, stream,
                         K.KVX_PATH_STAGED)
            K.kvx_sync(stream)
            bad, first = check_packed(w, L, w.seed, src, 0, w.num_layers, host.numpy())
            assert bad == 0, f"request {r}: backup differs at {first}"

            K.kvx_ready_reset(ready)
            samples = []
            stop = threading.Event()

            def poll():
                # the prefix is read first: every count is monotonic, so the
                # counts read after it are each at least the prefix
                while not stop.is_set():
                    pfx = K.kvx_ready_prefix(ready)
                    c = [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)]
                    samples.append((time.perf_counter(), c, pfx))
                    if min(c) == n:
                        break

            th = threading.Thread(target=poll)
            th.start()
            K.kvx_restore(pool.handle, host.ptr, P, dst, 0, w.num_layers, ready, 0, stream,
                          K.KVX_PATH_STAGED)
            K.kvx_sync(stream)
            th.join(timeout=30)
            stop.set()
            final = [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)]
            assert final == [n] * w.num_layers
            assert K.kvx_ready_prefix(ready) == n
            prev = [0] * w.num_layers
            first_l0 = first_last = None
            for ts, c, pfx in samples:
                assert all(0 <= x <= n for x in c)
                assert all(x >= p for x, p in zip(c, prev)), "a published count decreased"
                assert pfx <= min(c)
                if first_l0 is None and c[0] == n:
                    first_l0 = ts
                if first_last is None and c[-1] == n:
                    first_last = ts
                prev = c
            if first_l0 is not None and first_last is not None:
                assert first_l0 <= first_last
        bad, first = check_alloc(w, L, w.seed, np.concatenate(srcs), np.concatenate(dsts), 0,
                                 w.num_layers, pool.alloc)
        assert bad == 0, f"restore: {bad} bytes differ, first at allocation byte {first}"
    finally:
        K.kvx_ready_destroy(ready)
        host.free()
        pool.close()


@pytest.mark.parametrize("name", ["llama8b", "trtllm_hnd"])
def test_full_size_layer_pipelined_exchange(name):
    """The benchmark's step at full size, in its launch configuration: BACKUP
    of layer 0, one kvx_exchange per layer (backup of layer l + 1, restore of
    layer l, both through the same packed buffer), RESTORE of the last
    layer, zero-copy. The whole packed buffer and the whole allocation are
    checked against the oracle's closed forms, and every layer is
    published."""
    t = torch()
    w = WORKLOADS[name]
    n = w.pages_per_request
    print(f"\n[full] {name} exchange: pool {w.pool_bytes / 2**30:.1f} GiB, n={n}", flush=True)
    L = oracle_layout(w)
    src, dst = request_pair(w)
    pool = DevicePool(w, generation=5)
    P = w.payload_bytes(n)
    host = K.HostBuffer(P)
    synth.fill_gpu(host.ptr, P, w.seed + 2, 0)
    t.cuda.synchronize()
    stream = t.cuda.Stream()
    ready = K.kvx_ready_create(w.num_layers, 5)
    try:
        Z = K.KVX_PATH_ZEROCOPY
        K.kvx_backup(pool.handle, src, host.ptr, P, 0, 1, stream, Z)
        for l in range(1, w.num_layers):
            K.kvx_exchange(pool.handle, src, host.ptr, P, (l, l + 1), host.ptr, P, dst, (l - 1, l),
                           ready, 0, stream, Z)
        K.kvx_restore(pool.handle, host.ptr, P, dst, w.num_layers - 1, w.num_layers, ready, 0,
                      stream, Z)
        K.kvx_sync(stream)
        assert K.kvx_ready_prefix(ready) == n
        t0 = time.time()
        bad, first = check_packed(w, L, w.seed, src, 0, w.num_layers, host.numpy())
        print(f"[full] packed buffer checked in {time.time() - t0:.1f} s", flush=True)
        assert bad == 0, f"backup: {bad} bytes differ, first at packed offset {first}"
        t0 = time.time()
        bad, first = check_alloc(w, L, w.seed, src, dst, 0, w.num_layers, pool.alloc)
        print(f"[full] allocation checked in {time.time() - t0:.1f} s", flush=True)
        assert bad == 0, f"restore: {bad} bytes differ, first at allocation byte {first}"
    finally:
        K.kvx_ready_destroy(ready)
        host.free()
        pool.close()


def test_full_size_host_tier_slots():
    """The llama8b request through a slot-addressed host tier of 640 slots
    (5 GiB pinned), zero-copy: BACKUP into 256 scattered slots, then RESTORE
    of those slots into the request's destination pages with per-layer
    publish. The named slots, gathered in page order, are checked against
    the oracle's closed form of BACKUP; every unnamed slot of the first and
    last layer keeps its prefill; the whole allocation is checked against
    the closed form of the same round trip."""
    t = torch()
    w = WORKLOADS["llama8b"]
    n, S = w.pages_per_request, 640
    print(f"\n[full] llama8b host tier: {S} slots, n={n}", flush=True)
    L = oracle_layout(w)
    src, dst = request_pair(w)
    slots = np.random.default_rng(w.seed + 60).permutation(S)[:n].astype(np.int32)
    pool = DevicePool(w, generation=5)
    HB = w.payload_bytes(S)
    host = K.HostBuffer(HB)
    synth.fill_gpu(host.ptr, HB, w.seed + 2, 0)
    t.cuda.synchronize()
    stream = t.cuda.Stream()
    ready = K.kvx_ready_create(w.num_layers, 5)
    Z = K.KVX_PATH_ZEROCOPY
    try:
        K.kvx_backup_slots(pool.handle, src, slots, host.ptr, HB, S, 0, w.num_layers, stream, Z)
        K.kvx_sync(stream)
        rows = w.num_layers * w.num_kv
        hv = host.numpy().reshape(rows, S, w.piece_bytes)
        t0 = time.time()
        gathered = np.ascontiguousarray(hv[:, slots]).reshape(-1)
        bad, first = check_packed_named(L, w.seed, src, gathered)
        assert bad == 0, f"backup_slots: {bad} bytes differ, first at gathered offset {first}"
        unnamed = np.setdiff1d(np.arange(S), slots)
        jobs = [(r, s) for r in (0, 1, rows - 2, rows - 1) for s in unnamed]

        def keep(job):
            r, s = job
            a = (r * S + s) * w.piece_bytes
            return int(np.count_nonzero(hv[r, s] != synth.gen_bytes(w.seed + 2, a, w.piece_bytes)))

        with ThreadPoolExecutor(THREADS) as ex:
            assert sum(ex.map(keep, jobs)) == 0, "backup_slots wrote an unnamed slot"
        print(f"[full] host tier checked in {time.time() - t0:.1f} s", flush=True)
        del gathered
        K.kvx_restore_slots(pool.handle, host.ptr, HB, S, slots, dst, 0, w.num_layers, ready, 0,
                            stream, Z)
        K.kvx_sync(stream)
        assert K.kvx_ready_prefix(ready) == n
        t0 = time.time()
        bad, first = check_alloc(w, L, w.seed, src, dst, 0, w.num_layers, pool.alloc)
        print(f"[full] allocation checked in {time.time() - t0:.1f} s", flush=True)
        assert bad == 0, f"restore_slots: {bad} bytes differ, first at allocation byte {first}"
    finally:
        K.kvx_ready_destroy(ready)
        host.free()
        pool.close()


def test_full_size_tier_exchange():
    """The llama8b request through a host tier of 640 slots (5 GiB pinned),
    zero-copy, in the benchmark's default launch configuration:
    kvx_tier_backup stores the request's 256 source pages under 256 keys;
    then one kvx_tier_exchange restores those keys into the destination
    pages while it stores 256 other pages under new keys. The hits come back
    in their original slots and nothing is evicted; the new keys' slots,
    gathered in key order, hold the closed form of BACKUP of their pages;
    the hit slots still hold the first BACKUP (the exchange wrote none of
    them); the whole allocation is the closed form of the round trip; every
    layer publishes 256."""
    from synth import page_perm
    t = torch()
    w = WORKLOADS["llama8b"]
    n, S = w.pages_per_request, 640
    print(f"\n[full] llama8b tier exchange: {S} slots, n={n} per side", flush=True)
    L = oracle_layout(w)
    src, dst = request_pair(w)
    src2 = page_perm(w.seed, w.num_pages)[2 * n:3 * n].copy()   # disjoint from both
    keys1 = np.arange(1000, 1000 + n, dtype=np.uint64)
    keys2 = np.arange(5000, 5000 + n, dtype=np.uint64)
    pool = DevicePool(w, generation=6)
    HB = w.payload_bytes(S)
    host = K.HostBuffer(HB)
    synth.fill_gpu(host.ptr, HB, w.seed + 2, 0)
    t.cuda.synchronize()
    stream = t.cuda.Stream()
    ready = K.kvx_ready_create(w.num_layers, 6)
    tier = K.kvx_tier_create(S, 6)
    Z = K.KVX_PATH_ZEROCOPY
    try:
        s1, ev = K.kvx_tier_backup(tier, pool.handle, keys1, src, host.ptr, HB, stream, Z)
        K.kvx_sync(stream)
        K.kvx_tier_commit(tier, s1)
        assert ev.size == 0
        bs, ev, rs = K.kvx_tier_exchange(tier, pool.handle, keys2, src2, keys1, dst, host.ptr, HB,
                                         ready, 0, stream, Z)
        K.kvx_sync(stream)
        K.kvx_tier_commit(tier, bs)
        K.kvx_tier_release(tier, rs)
        assert ev.size == 0 and np.array_equal(rs, s1)
        assert np.intersect1d(bs, s1).size == 0 and np.unique(bs).size == n
        assert K.kvx_ready_prefix(ready) == n
        assert K.kvx_tier_get_info(tier)["resident"] == 2 * n
        rows = w.num_layers * w.num_kv
        hv = host.numpy().reshape(rows, S, w.piece_bytes)
        t0 = time.time()
        for what, ids, slots in (("new keys", src2, bs), ("hit slots", src, s1)):
            gathered = np.ascontiguousarray(hv[:, slots]).reshape(-1)
            bad, first = check_packed_named(L, w.seed, ids, gathered)
            del gathered
            assert bad == 0, f"{what}: {bad} bytes differ, first at gathered offset {first}"
        print(f"[full] tier slots checked in {time.time() - t0:.1f} s", flush=True)
        t0 = time.time()
        bad, first = check_alloc(w, L, w.seed, src, dst, 0, w.num_layers, pool.alloc)
        print(f"[full] allocation checked in {time.time() - t0:.1f} s", flush=True)
        assert bad == 0, f"tier exchange: {bad} bytes differ, first at allocation byte {first}"
    finally:
        K.kvx_tier_destroy(tier)
        K.kvx_ready_destroy(ready)
        host.free()
        pool.close()


def check_packed_named(L, seed, ids, packed):
    """A whole packed buffer of every layer against the closed form of BACKUP,
    in parallel 64 MiB ranges."""
    def one(r):
        a, b = r
        return oracle.check_backup_gen(L, seed, ids, 0, L.num_layers, packed[a:b], a)

    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(one, _ranges(packed.size)))
    return sum(r[0] for r in res), min((r[1] for r in res if r[0]), default=-1)


@pytest.mark.parametrize("name", ["llama8b", "trtllm_hnd"])
def test_whole_pool_in_one_call(name):
    """Maximum size: every page of a 16 GiB pool (llama8b: 2048 pages in five
    launches of at most 448; trtllm_hnd: 4096 head-major pages in ten) in one
    BACKUP into a device buffer, in a random order, then one RESTORE of that
    buffer into another random order of all pages with per-layer publish.
    512 sampled pieces of the packed buffer and 512 sampled pieces of the
    allocation, plus the padding before and after the pool, are checked
    against the oracle's closed forms."""
    t = torch()
    w = WORKLOADS[name]
    NB, NL = w.num_pages, w.num_layers
    print(f"\n[full] {name} whole pool: {NB} pages, {w.payload_bytes(NB) / 2**30:.0f} GiB per call",
          flush=True)
    L = oracle_layout(w)
    src = synth.page_perm(w.seed + 90, NB)
    dst = synth.page_perm(w.seed + 91, NB)
    pool = DevicePool(w, generation=5)
    P = w.payload_bytes(NB)
    pb = w.piece_bytes
    dev = t.empty(P, dtype=t.uint8, device="cuda")
    stream = t.cuda.Stream()
    ready = K.kvx_ready_create(NL, 5)
    rng = np.random.default_rng(w.seed + 92)
    D = K.KVX_PATH_DEVICE
    try:
        K.kvx_backup(pool.handle, src, dev.data_ptr(), P, 0, NL, stream, D)
        K.kvx_sync(stream)
        for q in rng.choice(NL * w.num_kv * NB, 512, replace=False):
            a = int(q) * pb
            bad, first = oracle.check_backup_gen(L, w.seed, src, 0, NL, dev[a:a + pb].cpu().numpy(), a)
            assert bad == 0, f"backup: piece at packed offset {a}: {bad} bytes differ, first {first}"
        K.kvx_restore(pool.handle, dev.data_ptr(), P, dst, 0, NL, ready, 0, stream, D)
        K.kvx_sync(stream)
        assert K.kvx_ready_prefix(ready) == NB
        ranges = [(0, w.byte_offset), (w.byte_offset + w.pool_bytes, w.alloc_bytes)]
        ranges += [(w.byte_offset + int(q) * pb, w.byte_offset + (int(q) + 1) * pb)
                   for q in rng.choice(NL * w.num_kv * NB, 512, replace=False)]
        for a, b in ranges:
            if a == b:
                continue
            bad, first = oracle.check_alloc_roundtrip(L, w.seed, w.seed + 1, src, dst, 0, NL,
                                                      pool.alloc[a:b].cpu().numpy(), a)
            assert bad == 0, f"restore: allocation bytes [{a}, {b}): {bad} differ, first at {first}"
    finally:
        K.kvx_ready_destroy(ready)
        del dev
        pool.close()
