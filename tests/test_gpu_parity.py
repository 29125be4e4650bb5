"""GPU parity: kvx backup/restore through the C ABI vs the CPU oracle, byte for
byte, on pools small enough for the oracle (several work units per piece,
ragged tails, more pages than one launch carries, offsets and padding), for
every path and both inner layouts; plus per-layer publish, the ready
prefix, a GPU-side consumer and the GPU-only argument checks."""
import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import WORKLOADS, Workload
from tests.gpu_util import PATHS, DevicePool, Packed, oracle_layout, torch

pytestmark = pytest.mark.gpu

KIB = 1024

SMALL = {
    "tiny": (WORKLOADS["tiny"], 8),
    "llama_small": (WORKLOADS["llama8b"].scaled(name="llama_small", num_pages=96, num_layers=3), 24),
    "mla_small": (WORKLOADS["mla_fp8"].scaled(name="mla_small", num_pages=40, num_layers=5), 10),
    "trtllm_small": (WORKLOADS["trtllm_hnd"].scaled(name="trtllm_small", num_pages=64,
                                                    num_layers=3), 16),
    # 240-byte pieces, 16-byte rows, head-major, page-major outer order, more
    # pages than one launch carries
    "ragged_hnd": (Workload(name="ragged_hnd", outer=("page", "kv", "layer"), inner="HND",
                            num_pages=1200, num_layers=3, num_kv=2, page_size=5, num_heads=3,
                            head_dim=8, dtype_bytes=2, pages_per_request=500, seed=201,
                            byte_offset=4096, alloc_tail=1008), 500),
    # 4032-byte pieces (not a multiple of a 4 KiB vector round), 192-byte rows
    "ragged_nhd": (Workload(name="ragged_nhd", outer=("kv", "layer", "page"), inner="NHD",
                            num_pages=300, num_layers=2, num_kv=2, page_size=7, num_heads=3,
                            head_dim=96, dtype_bytes=2, pages_per_request=100, seed=202,
                            byte_offset=8192, alloc_tail=4096), 100),
    "ragged_hnd2": (Workload(name="ragged_hnd2", outer=("layer", "page", "kv"), inner="HND",
                             num_pages=300, num_layers=2, num_kv=1, page_size=7, num_heads=3,
                             head_dim=96, dtype_bytes=2, pages_per_request=100, seed=203), 100),
    # degenerate head-major pools: one head, or one token per page (HND is NHD)
    "hnd_h1": (Workload(name="hnd_h1", outer=("layer", "kv", "page"), inner="HND", num_pages=100,
                        num_layers=2, num_kv=2, page_size=16, num_heads=1, head_dim=64, dtype_bytes=2,
                        pages_per_request=30, seed=205), 30),
    "hnd_t1": (Workload(name="hnd_t1", outer=("page", "layer", "kv"), inner="HND", num_pages=200,
                        num_layers=2, num_kv=2, page_size=1, num_heads=8, head_dim=64, dtype_bytes=2,
                        pages_per_request=50, seed=206), 50),
    # 4-byte elements, 16-byte rows (one vector per row), head-major
    "hnd_f32_rows16": (Workload(name="hnd_f32_rows16", outer=("kv", "page", "layer"), inner="HND",
                                num_pages=64, num_layers=3, num_kv=2, page_size=4, num_heads=3,
                                head_dim=4, dtype_bytes=4, pages_per_request=20, seed=207), 20),
}


@pytest.fixture(scope="module")
def stream():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    K.lib()
    return t.cuda.Stream()


def diff_report(got, want, limit=8):
    bad = np.flatnonzero(got != want)
    return f"{bad.size} bytes differ; first at {bad[:limit].tolist()}"


def pages(w, n):
    perm = synth.page_perm(w.seed, w.num_pages)
    return perm[:n].copy(), perm[n:2 * n].copy()


def check_backup_restore(w, n, path, stream):
    """BACKUP then RESTORE of n pages over two layer ranges on `path`, each
    compared byte for byte with the oracle (whole packed buffer, whole
    allocation)."""
    L = oracle_layout(w)
    pool = DevicePool(w)
    img = pool.host_image()
    assert np.array_equal(img, synth.pool_alloc_image(w, w.seed))
    src, dst = pages(w, n)
    nb = w.host_bytes(n)
    ranges = [(0, w.num_layers), (1, w.num_layers)] if w.num_layers > 1 else [(0, 1)]
    for l0, l1 in ranges:
        pk = Packed(w, n, path, fill_seed=w.seed + 2)
        want = oracle.backup(L, img, src, l0, l1, host=synth.gen_bytes(w.seed + 2, 0, nb))
        K.kvx_backup(pool.handle, src, pk.ptr, nb, l0, l1, stream, PATHS[path])
        K.kvx_sync(stream)
        got = pk.numpy()
        assert np.array_equal(got, want), f"backup {l0}:{l1} " + diff_report(got, want)

        pk.fill(w.seed + 3)
        hbytes = synth.gen_bytes(w.seed + 3, 0, nb)
        want_alloc = oracle.restore(L, pool.host_image(), hbytes, dst, l0, l1)
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, l0, l1, None, 0, stream, PATHS[path])
        K.kvx_sync(stream)
        after = pool.host_image()
        assert np.array_equal(after, want_alloc), f"restore {l0}:{l1} " + \
            diff_report(after, want_alloc)
        img = after
        pk.close()
    pool.close()


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("case", list(SMALL))
def test_backup_restore_parity(case, path, stream):
    w, n = SMALL[case]
    print(f"\n[parity] case={case} path={path} n={n} piece={w.piece_bytes}", flush=True)
    check_backup_restore(w, n, path, stream)


# 48 KiB head-major pieces: the only unit that tiles them without a tail is
# 12 rounds of 4 KiB
HND48K = Workload(name="hnd48k", outer=("layer", "kv", "page"), inner="HND", num_pages=40,
                  num_layers=2, num_kv=2, page_size=16, num_heads=12, head_dim=128, dtype_bytes=2,
                  pages_per_request=12, seed=204)

# (case, largest unroll, forced unit rounds, cache policy, HND through LDS);
# forced units that do not tile the piece leave a partial last unit whose
# accesses past the piece the hardware drops
VARIANTS = [
    ("llama_small", 32, 0, -1, -1), ("llama_small", 16, 0, 0, -1), ("llama_small", 8, 0, 3, -1),
    ("llama_small", 4, 0, 4, -1), ("llama_small", 32, 12, 7, -1), ("llama_small", 32, 3, 7, -1),
    ("mla_small", 32, 0, 7, -1), ("mla_small", 12, 0, 5, -1), ("mla_small", 32, 32, 7, -1),
    ("mla_small", 32, 16, 6, -1),
    ("trtllm_small", 32, 0, 7, 0), ("trtllm_small", 16, 0, 6, 1), ("trtllm_small", 8, 0, 0, 1),
    ("trtllm_small", 4, 0, 1, 1), ("trtllm_small", 32, 32, 7, 0), ("trtllm_small", 32, 12, 7, 1),
    ("hnd48k", 32, 0, -1, -1), ("hnd48k", 16, 0, 2, 1), ("hnd48k", 32, 16, 7, 1),
    ("ragged_nhd", 32, 0, 7, -1), ("ragged_hnd", 32, 0, 7, 1), ("ragged_hnd", 32, 2, 7, 0),
]


@pytest.mark.parametrize("path", ["device", "zerocopy"])
@pytest.mark.parametrize("case,unroll,rounds,policy,lds", VARIANTS)
def test_kernel_variants(case, unroll, rounds, policy, lds, path, stream):
    """Every unit size (including partial last units), cache policy and HND
    conversion form gives the oracle's bytes."""
    w, n = (HND48K, 12) if case == "hnd48k" else SMALL[case]
    opts = {K.KVX_OPT_MAX_UNROLL: unroll, K.KVX_OPT_UNIT_ROUNDS: rounds,
            K.KVX_OPT_CACHE_POLICY: policy, K.KVX_OPT_HND_LDS: lds}
    print(f"\n[variant] case={case} path={path} unroll<={unroll} rounds={rounds} policy={policy} "
          f"lds={lds} piece={w.piece_bytes}", flush=True)
    old = {o: K.kvx_get_option(o) for o in opts}
    try:
        for o, v in opts.items():
            K.kvx_set_option(o, v)
        check_backup_restore(w, n, path, stream)
    finally:
        for o, v in old.items():
            K.kvx_set_option(o, v)


# (case, backup pages, restore pages, backup layers, restore layers)
EXCHANGES = [
    ("tiny", 8, 8, None, None),
    ("llama_small", 24, 11, None, (1, 3)),
    ("mla_small", 10, 10, (0, 2), (2, 5)),
    ("trtllm_small", 16, 7, None, None),
    ("ragged_hnd", 460, 130, None, None),      # two launches per call, the second backup only
    ("ragged_nhd", 100, 50, (1, 2), (0, 2)),
]


@pytest.mark.parametrize("path", ["zerocopy", "device"])
@pytest.mark.parametrize("case,nb,nr,lb,lr", EXCHANGES)
def test_exchange_parity(case, nb, nr, lb, lr, path, stream):
    """kvx_exchange gives the bytes of kvx_backup followed by kvx_restore:
    the whole packed buffer of the backup and the whole allocation after the
    restore match the oracle, and the restore publishes its layers. Two
    exchanges run back to back without a host synchronisation (the second
    depends on the unit queue the first leaves reset)."""
    w, _ = SMALL[case]
    assert 2 * (nb + nr) <= w.num_pages
    lb = lb or (0, w.num_layers)
    lr = lr or (0, w.num_layers)
    print(f"\n[exchange] case={case} path={path} nb={nb} nr={nr} lb={lb} lr={lr}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=307, generation=8)
    img = pool.host_image()
    perm = synth.page_perm(w.seed + 11, w.num_pages)
    ready = K.kvx_ready_create(w.num_layers, 8)
    bufs = []
    try:
        want_alloc = img
        wants = []
        want_counts = [0] * w.num_layers
        for r in range(2):
            off = r * (nb + nr)
            src = perm[off:off + nb].copy()
            dst = perm[off + nb:off + nb + nr].copy()
            pk_b = Packed(w, nb, path, fill_seed=w.seed + 20 + r)
            pk_r = Packed(w, nr, path, fill_seed=w.seed + 30 + r)
            bufs += [pk_b, pk_r]
            # backup reads the pool as the previous exchange left it
            wants.append(oracle.backup(L, want_alloc, src, *lb,
                                       host=synth.gen_bytes(w.seed + 20 + r, 0, w.host_bytes(nb))))
            want_alloc = oracle.restore(L, want_alloc, synth.gen_bytes(w.seed + 30 + r, 0, w.host_bytes(nr)),
                                        dst, *lr)
            want_counts = oracle.ready_publish(want_counts, 0, *lr, nr)
            K.kvx_exchange(pool.handle, src, pk_b.ptr, w.host_bytes(nb), lb, pk_r.ptr, w.host_bytes(nr),
                           dst, lr, ready, 0, stream, PATHS[path])
        K.kvx_sync(stream)
        for r in range(2):
            got = bufs[2 * r].numpy()
            assert np.array_equal(got, wants[r]), f"exchange {r} backup: " + diff_report(got, wants[r])
        after = pool.host_image()
        assert np.array_equal(after, want_alloc), "exchange restore: " + diff_report(after, want_alloc)
        # each exchange's restore adds nr to every layer it publishes
        assert [K.kvx_layer_ready(ready, l) for l in range(w.num_layers)] == want_counts
    finally:
        K.kvx_ready_destroy(ready)
        for b in bufs:
            b.close()
        pool.close()


def test_exchange_with_overlapping_pages_in_disjoint_layers(stream):
    """A page the backup reads in layer 0 may be written by the restore in
    the other layers."""
    w, _ = SMALL["llama_small"]
    L = oracle_layout(w)
    pool = DevicePool(w, seed=309, generation=9)
    img = pool.host_image()
    ids = synth.page_perm(w.seed + 13, w.num_pages)[:12].copy()
    pk_b = Packed(w, 12, "zerocopy", fill_seed=41)
    pk_r = Packed(w, 12, "zerocopy", fill_seed=42)
    try:
        K.kvx_exchange(pool.handle, ids, pk_b.ptr, w.host_bytes(12), (0, 1), pk_r.ptr,
                       w.host_bytes(12), ids, (1, w.num_layers), None, 0, stream,
                       K.KVX_PATH_ZEROCOPY)
        K.kvx_sync(stream)
        want_b = oracle.backup(L, img, ids, 0, 1, host=synth.gen_bytes(41, 0, w.host_bytes(12)))
        want = oracle.restore(L, img, synth.gen_bytes(42, 0, w.host_bytes(12)), ids, 1, w.num_layers)
        got_b = pk_b.numpy()
        assert np.array_equal(got_b, want_b), diff_report(got_b, want_b)
        after = pool.host_image()
        assert np.array_equal(after, want), diff_report(after, want)
    finally:
        pk_b.close()
        pk_r.close()
        pool.close()


@pytest.mark.parametrize("path", ["staged", "zerocopy"])
def test_round_trip_and_duplicates(path, stream):
    w, _ = SMALL["trtllm_small"]
    L = oracle_layout(w)
    pool = DevicePool(w, seed=301)
    img = pool.host_image()
    src = np.array([5, 5, 17, 0, 63, 17], dtype=np.int32)    # duplicates allowed in a backup
    dst = np.array([40, 41, 42, 43, 44, 45], dtype=np.int32)
    nb = w.host_bytes(len(src))
    pk = Packed(w, len(src), path, fill_seed=9)
    K.kvx_backup(pool.handle, src, pk.ptr, nb, 0, w.num_layers, stream, PATHS[path])
    K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, None, 0, stream, PATHS[path])
    K.kvx_sync(stream)
    after = pool.host_image()
    host = oracle.backup(L, img, src, 0, w.num_layers)
    want = oracle.restore(L, img, host, dst, 0, w.num_layers)
    assert np.array_equal(after, want), diff_report(after, want)
    # round trip: each destination piece now equals its source piece
    for s, d in zip(src, dst):
        for l in range(w.num_layers):
            for c in range(w.num_kv):
                a, b = oracle.piece_start(L, int(s), l, c), oracle.piece_start(L, int(d), l, c)
                assert np.array_equal(after[b:b + w.piece_bytes], img[a:a + w.piece_bytes])
    pk.close()
    pool.close()


@pytest.mark.parametrize("dma_on_caller", [-1, 0, 1])
@pytest.mark.parametrize("slot_bytes", [1 << 20, 64 << 20])
@pytest.mark.parametrize("sort_pages", [0, 1])
def test_staged_chunking_by_slot_range(sort_pages, slot_bytes, dma_on_caller, stream):
    """A 1 MiB ring slot forces layers to be split into slot ranges, several
    DMA strips per chunk and ring reuse; a 64 MiB slot holds the whole
    request in one chunk. The staged DMA runs on the library's side stream,
    on the caller's stream, or on whichever the library picks (the caller's
    for one chunk); bytes must not change."""
    w, n = SMALL["llama_small"]
    L = oracle_layout(w)
    old = {o: K.kvx_get_option(o) for o in (K.KVX_OPT_STAGE_SLOT_BYTES, K.KVX_OPT_SORT_PAGES,
                                            K.KVX_OPT_STAGED_DMA_ON_CALLER)}
    try:
        K.kvx_set_option(K.KVX_OPT_STAGE_SLOT_BYTES, slot_bytes)
        K.kvx_set_option(K.KVX_OPT_SORT_PAGES, sort_pages)
        K.kvx_set_option(K.KVX_OPT_STAGED_DMA_ON_CALLER, dma_on_caller)
        pool = DevicePool(w, seed=302)
        img = pool.host_image()
        src, dst = pages(w, n)
        nb = w.host_bytes(n)
        pk = Packed(w, n, "staged", fill_seed=3)
        K.kvx_backup(pool.handle, src, pk.ptr, nb, 0, w.num_layers, stream, K.KVX_PATH_STAGED)
        K.kvx_sync(stream)
        want = oracle.backup(L, img, src, 0, w.num_layers)
        got = pk.numpy()
        assert np.array_equal(got, want), diff_report(got, want)
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, None, 0, stream,
                      K.KVX_PATH_STAGED)
        K.kvx_sync(stream)
        after = pool.host_image()
        want_alloc = oracle.restore(L, img, want, dst, 0, w.num_layers)
        assert np.array_equal(after, want_alloc), diff_report(after, want_alloc)
        pk.close()
        pool.close()
    finally:
        for o, v in old.items():
            K.kvx_set_option(o, v)


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("case", ["ragged_hnd", "llama_small", "mla_small", "trtllm_small"])
def test_publishing_restore_parity(case, path, stream):
    """Restores that publish take their work units from a queue that each
    launch leaves reset for the next: two restores in a row on one stream
    (ragged_hnd's 500 pages take two launches per layer range) must write
    exactly the oracle's bytes and publish every layer."""
    w, n = SMALL[case]
    print(f"\n[publish-parity] case={case} path={path} n={n}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=305, generation=6)
    img = pool.host_image()
    perm = synth.page_perm(w.seed + 7, w.num_pages)
    nb = w.host_bytes(n)
    ready = K.kvx_ready_create(w.num_layers, 6)
    pks = []
    try:
        want = img
        for r in range(2):
            dst = perm[r * n:(r + 1) * n].copy()
            pk = Packed(w, n, path, fill_seed=w.seed + 10 + r)
            pks.append(pk)
            hbytes = synth.gen_bytes(w.seed + 10 + r, 0, nb)
            want = oracle.restore(L, want, hbytes, dst, 0, w.num_layers)
            # no host synchronisation between the two: the second launch
            # depends on the queue the first one left reset
            K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, ready, 0, stream,
                          PATHS[path])
        K.kvx_sync(stream)
        # each restore adds its n to every layer's count (no reset between)
        counts = [0] * w.num_layers
        for _ in range(2):
            counts = oracle.ready_publish(counts, 0, 0, w.num_layers, n)
        assert [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)] == counts
        after = pool.host_image()
        assert np.array_equal(after, want), diff_report(after, want)
    finally:
        K.kvx_ready_destroy(ready)
        for pk in pks:
            pk.close()
        pool.close()


@pytest.mark.parametrize("path", list(PATHS))
def test_restore_publishes_every_layer(path, stream):
    w, n = SMALL["mla_small"]
    pool = DevicePool(w, seed=303, generation=4)
    src, dst = pages(w, n)
    nb = w.host_bytes(n)
    pk = Packed(w, n, path, fill_seed=5)
    ready = K.kvx_ready_create(w.num_layers + 3, 4)
    try:
        assert K.kvx_ready_prefix(ready) == 0
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, ready, 2, stream, PATHS[path])
        K.kvx_sync(stream)
        counts = [K.kvx_layer_ready(ready, s) for s in range(w.num_layers + 3)]
        assert counts == [0, 0] + [n] * w.num_layers + [0]
        assert K.kvx_ready_prefix(ready) == 0 == oracle.ready_prefix(counts)
        K.kvx_ready_reset(ready)
        assert K.kvx_ready_prefix(ready) == 0
        # a partial layer range publishes only its slots
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, 1, 3, ready, 0, stream, PATHS[path])
        K.kvx_sync(stream)
        counts = [K.kvx_layer_ready(ready, s) for s in range(w.num_layers + 3)]
        assert counts == [0, n, n] + [0] * (w.num_layers)
        # repeated calls on the same stream reuse the self-clearing counters
        for _ in range(3):
            K.kvx_ready_reset(ready)
            K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, ready, 3, stream,
                          PATHS[path])
            K.kvx_sync(stream)
            counts = [K.kvx_layer_ready(ready, s) for s in range(w.num_layers + 3)]
            assert counts == [0, 0, 0] + [n] * w.num_layers
        assert K.kvx_ready_prefix(ready) == 0
        full = K.kvx_ready_create(w.num_layers, 4)
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, full, 0, stream, PATHS[path])
        K.kvx_sync(stream)
        assert K.kvx_ready_prefix(full) == n
        K.kvx_ready_destroy(full)
    finally:
        K.kvx_ready_destroy(ready)
        pk.close()
        pool.close()


def test_ready_generation_range_and_lifetime(stream):
    w, n = SMALL["tiny"]
    pool = DevicePool(w, seed=304, generation=9)
    nb = w.host_bytes(n)
    pk = Packed(w, n, "zerocopy", fill_seed=1)
    _, dst = pages(w, n)
    other = K.kvx_ready_create(w.num_layers, 8)
    mine = K.kvx_ready_create(w.num_layers, 9)
    before = pool.host_image()

    def code(fn):
        with pytest.raises(K.KvxError) as e:
            fn()
        return e.value.code

    assert code(lambda: K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, 2, other, 0, stream,
                                      K.KVX_PATH_ZEROCOPY)) == K.KVX_E_STALE
    assert code(lambda: K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, 2, mine, 1, stream,
                                      K.KVX_PATH_ZEROCOPY)) == K.KVX_E_RANGE
    K.kvx_ready_destroy(mine)
    K.kvx_ready_destroy(mine)   # second teardown is logged, not an error
    assert code(lambda: K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, 2, mine, 0, stream,
                                      K.KVX_PATH_ZEROCOPY)) == K.KVX_E_STALE
    assert code(lambda: K.kvx_ready_prefix(mine)) == K.KVX_E_STALE
    K.kvx_sync(stream)
    assert np.array_equal(pool.host_image(), before)   # fail closed: nothing was written
    K.kvx_ready_destroy(other)
    pk.close()
    pool.close()


@pytest.mark.parametrize("path,policy,block", [("zerocopy", -1, 0), ("device", -1, 0),
                                               ("device", 0, 0), ("device", 0, 1),
                                               ("zerocopy", 0, 0), ("device", 3, 5)])
def test_gpu_consumer_waits_for_published_layer(path, policy, block, stream):
    """A consumer stream waits (bounded) for the last layer's count, then
    reads that layer back; the bytes must be the restored ones. Also with
    plain stores that stay in L2 until written back (cache policy 0 or 3)
    and with other publish blocks."""
    t = torch()
    w, n = SMALL["llama_small"]
    L = oracle_layout(w)
    old = {o: K.kvx_get_option(o) for o in (K.KVX_OPT_CACHE_POLICY, K.KVX_OPT_PUBLISH_BLOCK)}
    K.kvx_set_option(K.KVX_OPT_CACHE_POLICY, policy)
    K.kvx_set_option(K.KVX_OPT_PUBLISH_BLOCK, block)
    pool = DevicePool(w, seed=305, generation=2)
    img = pool.host_image()
    _, dst = pages(w, n)
    nb = w.host_bytes(n)
    pk = Packed(w, n, path, fill_seed=11)
    hbytes = synth.gen_bytes(11, 0, nb)
    ready = K.kvx_ready_create(w.num_layers, 2)
    consumer = t.cuda.Stream()
    status = t.zeros(1, dtype=t.int32, device="cuda")
    out = Packed(w, n, "device")
    t.cuda.synchronize()
    last = w.num_layers - 1
    try:
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, ready, 0, stream, PATHS[path])
        # everything the producer needs is enqueued before the consumer waits
        K.kvx_ready_wait_gpu(ready, last, n, consumer, 2_000_000, status)
        K.kvx_backup(pool.handle, dst, out.ptr, nb, last, w.num_layers, consumer,
                     K.KVX_PATH_DEVICE)
        K.kvx_sync(consumer)
        K.kvx_sync(stream)
        assert int(status.item()) == 1
        restored = oracle.restore(L, img, hbytes, dst, 0, w.num_layers)
        want = oracle.backup(L, restored, dst, last, w.num_layers)
        got = out.numpy()
        lo = last * w.num_kv * n * w.piece_bytes
        assert np.array_equal(got[lo:], want[lo:]), diff_report(got[lo:], want[lo:])
        assert K.kvx_ready_prefix(ready) == n
        # a wait that can never be satisfied gives up after its spin limit
        status.zero_()
        t.cuda.synchronize()
        K.kvx_ready_wait_gpu(ready, 0, n + 1, consumer, 1000, status)
        K.kvx_sync(consumer)
        assert int(status.item()) == 0
    finally:
        for o, v in old.items():
            K.kvx_set_option(o, v)
        K.kvx_ready_destroy(ready)
        pk.close()
        pool.close()


@pytest.mark.parametrize("path,policy", [("device", -1), ("device", 0), ("zerocopy", -1),
                                         ("zerocopy", 0)])
@pytest.mark.parametrize("case", ["mla_small", "llama_small"])
def test_consumer_reads_every_layer_as_it_is_published(case, path, policy, stream):
    """Eight rounds, each restoring fresh bytes into the same pages: a
    consumer stream waits (bounded) for each layer's count in turn and
    copies that layer out at once, while the producer still writes later
    layers. Every copy holds the round's bytes, never an earlier round's:
    the producer's stores reach the consumer's reads through the count
    alone. Also with plain stores that stay in L2 until written back
    (cache policy 0)."""
    t = torch()
    w, n = SMALL[case]
    L = oracle_layout(w)
    NL = w.num_layers
    old = K.kvx_get_option(K.KVX_OPT_CACHE_POLICY)
    K.kvx_set_option(K.KVX_OPT_CACHE_POLICY, policy)
    pool = DevicePool(w, seed=306, generation=2)
    img = pool.host_image()
    _, dst = pages(w, n)
    nb = w.host_bytes(n)
    ready = K.kvx_ready_create(NL, 2)
    consumer = t.cuda.Stream()
    status = t.zeros(NL, dtype=t.int32, device="cuda")
    out = Packed(w, n, "device")
    print(f"\n[consumer] case={case} path={path} policy={policy} n={n} layers={NL}", flush=True)
    try:
        for r in range(8):
            pk = Packed(w, n, path, fill_seed=500 + r)
            status.zero_()
            K.kvx_ready_reset(ready)
            t.cuda.synchronize()
            K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, NL, ready, 0, stream, PATHS[path])
            for l in range(NL):
                K.kvx_ready_wait_gpu(ready, l, n, consumer, 2_000_000, status[l:l + 1])
                K.kvx_backup(pool.handle, dst, out.ptr, nb, l, l + 1, consumer, K.KVX_PATH_DEVICE)
            K.kvx_sync(consumer)
            K.kvx_sync(stream)
            assert status.tolist() == [1] * NL, f"round {r}: a wait gave up"
            want = oracle.backup(L, oracle.restore(L, img, synth.gen_bytes(500 + r, 0, nb), dst, 0, NL),
                                 dst, 0, NL)
            got = out.numpy()
            assert np.array_equal(got, want), f"round {r}: " + diff_report(got, want)
            pk.close()
    finally:
        K.kvx_set_option(K.KVX_OPT_CACHE_POLICY, old)
        K.kvx_ready_destroy(ready)
        pool.close()


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("case", ["trtllm_small", "ragged_nhd"])
def test_byte_offset_moves_the_pool_and_nothing_else(case, path, stream):
    """The same pool bytes placed at byte offset 0 and at offsets of 16 B,
    4 KiB and 12 KiB + 16 B of their allocations: every BACKUP gives the
    same packed bytes (the oracle's), every RESTORE of the same host bytes
    leaves the same pool bytes, and the padding before and after the pool
    keeps its bytes."""
    t = torch()
    w0, n = SMALL[case]
    src, dst = pages(w0, n)
    nb = w0.host_bytes(n)
    packed, pools = [], []
    for off in (0, 16, 4096, 12304):
        w = w0.scaled(byte_offset=off, alloc_tail=4096 + 48)
        L = oracle_layout(w)
        pool = DevicePool(w, seed=311, generation=3)
        # the pool region holds stream 311 from its own first byte, whatever the offset
        synth.fill_gpu(pool.alloc.data_ptr() + off, w.pool_bytes, 311, 0)
        t.cuda.synchronize()
        img = pool.host_image()
        pk = Packed(w, n, path, fill_seed=21)
        K.kvx_backup(pool.handle, src, pk.ptr, nb, 0, w.num_layers, stream, PATHS[path])
        K.kvx_sync(stream)
        got = pk.numpy()
        want = oracle.backup(L, img, src, 0, w.num_layers, host=synth.gen_bytes(21, 0, nb))
        assert np.array_equal(got, want), f"offset {off}: backup " + diff_report(got, want)
        packed.append(got)
        pk.fill(22)
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, None, 0, stream, PATHS[path])
        K.kvx_sync(stream)
        after = pool.host_image()
        want_alloc = oracle.restore(L, img, synth.gen_bytes(22, 0, nb), dst, 0, w.num_layers)
        assert np.array_equal(after, want_alloc), f"offset {off}: restore " + diff_report(after, want_alloc)
        pad = np.concatenate([after[:off], after[off + w.pool_bytes:]])
        pad_want = np.concatenate([synth.gen_bytes(312, 0, off),
                                   synth.gen_bytes(312, off + w.pool_bytes, w.alloc_bytes - off - w.pool_bytes)])
        assert np.array_equal(pad, pad_want), f"offset {off}: padding changed"
        pools.append(after[off:off + w.pool_bytes].copy())
        pk.close()
        pool.close()
    for k in range(1, len(packed)):
        assert np.array_equal(packed[k], packed[0])
        assert np.array_equal(pools[k], pools[0])


@pytest.mark.parametrize("path", ["zerocopy", "staged"])
def test_gpu_consumer_reads_layer0_while_later_layers_are_held_back(path, stream):
    """The producer restores layer 0; the later layers are held back on the
    host until a consumer stream, waiting for layer 0's count, has copied
    layer 0 out. The copy equals the oracle's restored bytes, no later layer
    is published while it runs, and the later layers then complete. (The
    hold-back is on the host: streams may share a hardware queue, so a
    kernel-side delay on the producer could also delay the consumer.)"""
    t = torch()
    w, n = SMALL["llama_small"]
    print(f"\n[layer0-consumer] path={path} n={n}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=306, generation=2)
    img = pool.host_image()
    _, dst = pages(w, n)
    nb = w.host_bytes(n)
    pk = Packed(w, n, path, fill_seed=12)
    hbytes = synth.gen_bytes(12, 0, nb)
    ready = K.kvx_ready_create(w.num_layers, 2)
    consumer = t.cuda.Stream()
    status = t.zeros(1, dtype=t.int32, device="cuda")
    out = Packed(w, n, "device")
    t.cuda.synchronize()
    P = PATHS[path]
    try:
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, 1, ready, 0, stream, P)
        K.kvx_ready_wait_gpu(ready, 0, n, consumer, 5_000_000, status.data_ptr())
        K.kvx_backup(pool.handle, dst, out.ptr, nb, 0, 1, consumer, K.KVX_PATH_DEVICE)
        K.kvx_sync(consumer)
        assert int(status.item()) == 1
        assert [K.kvx_layer_ready(ready, s) for s in range(1, w.num_layers)] == \
            [0] * (w.num_layers - 1)
        restored = oracle.restore(L, img, hbytes, dst, 0, w.num_layers)
        want = oracle.backup(L, restored, dst, 0, 1)
        hi = w.num_kv * n * w.piece_bytes
        got = out.numpy()
        assert np.array_equal(got[:hi], want[:hi]), diff_report(got[:hi], want[:hi])
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, 1, w.num_layers, ready, 0, stream, P)
        K.kvx_sync(stream)
        assert [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)] == [n] * w.num_layers
        assert np.array_equal(pool.host_image(), restored)
    finally:
        K.kvx_ready_destroy(ready)
        out.close()
        pk.close()
        pool.close()


# bf16 words a float path would change: quiet and signalling NaNs with
# payloads and either sign, infinities, denormals, negative zero
BF16_SPECIALS = [0x7FC0, 0xFFC0, 0x7F81, 0xFF81, 0x7FBF, 0x7FC1, 0x7F80, 0xFF80, 0x0001, 0x8001,
                 0x007F, 0x807F, 0x8000, 0x0000, 0xFFFF, 0x7FFF]


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("case", ["llama_small", "mla_small"])
def test_bits_survive_whatever_they_would_mean(case, path, stream):
    """Dtype neutrality: a bf16 pool holding every NaN, infinity, denormal and
    signed-zero class in every position of a row, and an fp8 pool holding
    all 256 byte values, round-trip through BACKUP and RESTORE bit for bit
    (the oracle's bytes, and the restored pages equal the sources)."""
    t = torch()
    w, n = SMALL[case]
    print(f"\n[dtype] case={case} eb={w.dtype_bytes} path={path}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=308, generation=4)
    rng = np.random.default_rng(308)
    if w.dtype_bytes == 2:
        words = rng.integers(0, 1 << 16, w.alloc_bytes // 2, dtype=np.uint16)
        specials = np.array(BF16_SPECIALS, dtype=np.uint16)
        # runs of the special words, shifted by one word each row of 64 so
        # every class meets every position of a row
        idx = np.arange(words.size)
        pick = (idx // 64 + idx) % (2 * specials.size)
        words = np.where(pick < specials.size, specials[pick % specials.size], words)
        img = words.view(np.uint8)
    else:
        img = (np.arange(w.alloc_bytes, dtype=np.int64) * 73 % 256).astype(np.uint8)
        assert np.unique(img).size == 256
    pool.alloc.copy_(t.from_numpy(img.copy()))
    t.cuda.synchronize()
    src, dst = pages(w, n)
    nb = w.host_bytes(n)
    pk = Packed(w, n, path, fill_seed=22)
    try:
        K.kvx_backup(pool.handle, src, pk.ptr, nb, 0, w.num_layers, stream, PATHS[path])
        K.kvx_sync(stream)
        want = oracle.backup(L, img, src, 0, w.num_layers)
        got = pk.numpy()
        assert np.array_equal(got, want), "backup " + diff_report(got, want)
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, None, 0, stream, PATHS[path])
        K.kvx_sync(stream)
        want_alloc = oracle.restore(L, img, want, dst, 0, w.num_layers)
        after = pool.host_image()
        assert np.array_equal(after, want_alloc), "restore " + diff_report(after, want_alloc)
        for i in (0, n - 1):
            for l in range(w.num_layers):
                for c in range(w.num_kv):
                    a, b = oracle.piece_start(L, src[i], l, c), oracle.piece_start(L, dst[i], l, c)
                    assert np.array_equal(after[b:b + w.piece_bytes], img[a:a + w.piece_bytes])
    finally:
        pk.close()
        pool.close()


# 300 layers: more than the per-layer counters a lane starts with (256)
MANY_LAYERS = Workload(name="many_layers", outer=("layer", "kv", "page"), inner="NHD", num_pages=16,
                       num_layers=300, num_kv=2, page_size=2, num_heads=1, head_dim=64,
                       dtype_bytes=2, pages_per_request=4, seed=211)


def test_injected_allocation_failures_fail_closed_and_recover():
    """With the allocation test hook armed, a staged BACKUP whose staging ring
    must be (re)allocated (a slot size no other test uses) and a publishing
    RESTORE of a 300-layer pool whose per-layer counters must grow both
    return KVX_E_NOMEM with nothing written (pool, packed buffer and ready
    counts unchanged); the hook is spent, the ready object resets, and the
    same calls then succeed with the oracle's bytes."""
    t = torch()
    w, n = SMALL["llama_small"]
    L = oracle_layout(w)
    pool = DevicePool(w, seed=307, generation=3)
    img = pool.host_image()
    src, _ = pages(w, n)
    nb = w.host_bytes(n)
    s_staged, s_zc = t.cuda.Stream(), t.cuda.Stream()
    pk = Packed(w, n, "staged", fill_seed=21)
    w2, n2 = MANY_LAYERS, MANY_LAYERS.pages_per_request
    L2 = oracle_layout(w2)
    pool2 = DevicePool(w2, generation=3)
    img2 = pool2.host_image()
    src2, dst2 = pages(w2, n2)
    nb2 = w2.host_bytes(n2)
    pk2 = Packed(w2, n2, "zerocopy", fill_seed=23)
    ready = K.kvx_ready_create(w2.num_layers, 3)
    old_slot = K.kvx_get_option(K.KVX_OPT_STAGE_SLOT_BYTES)
    try:
        K.kvx_set_option(K.KVX_OPT_STAGE_SLOT_BYTES, (96 << 20) + 4096)
        K.kvx_set_option(K.KVX_OPT_FAIL_ALLOCS, 1)
        with pytest.raises(K.KvxError) as e:
            K.kvx_backup(pool.handle, src, pk.ptr, nb, 0, w.num_layers, s_staged, K.KVX_PATH_STAGED)
        assert e.value.code == K.KVX_E_NOMEM, e.value.message
        assert K.kvx_get_option(K.KVX_OPT_FAIL_ALLOCS) == 0
        K.kvx_sync(s_staged)
        assert np.array_equal(pk.numpy(), synth.gen_bytes(21, 0, nb))
        K.kvx_backup(pool.handle, src, pk.ptr, nb, 0, w.num_layers, s_staged, K.KVX_PATH_STAGED)
        K.kvx_sync(s_staged)
        want = oracle.backup(L, img, src, 0, w.num_layers)
        assert np.array_equal(pk.numpy(), want), diff_report(pk.numpy(), want)

        hbytes = synth.gen_bytes(23, 0, nb2)
        K.kvx_set_option(K.KVX_OPT_FAIL_ALLOCS, 1)
        with pytest.raises(K.KvxError) as e:
            K.kvx_restore(pool2.handle, pk2.ptr, nb2, dst2, 0, w2.num_layers, ready, 0, s_zc,
                          K.KVX_PATH_ZEROCOPY)
        assert e.value.code == K.KVX_E_NOMEM, e.value.message
        assert K.kvx_get_option(K.KVX_OPT_FAIL_ALLOCS) == 0
        K.kvx_sync(s_zc)
        assert np.array_equal(pool2.host_image(), img2)
        assert K.kvx_ready_prefix(ready) == 0
        K.kvx_ready_reset(ready)
        K.kvx_restore(pool2.handle, pk2.ptr, nb2, dst2, 0, w2.num_layers, ready, 0, s_zc,
                      K.KVX_PATH_ZEROCOPY)
        K.kvx_sync(s_zc)
        assert K.kvx_ready_prefix(ready) == n2
        want2 = oracle.restore(L2, img2, hbytes, dst2, 0, w2.num_layers)
        after = pool2.host_image()
        assert np.array_equal(after, want2), diff_report(after, want2)
    finally:
        K.kvx_set_option(K.KVX_OPT_FAIL_ALLOCS, 0)
        K.kvx_set_option(K.KVX_OPT_STAGE_SLOT_BYTES, old_slot)
        K.kvx_ready_destroy(ready)
        pk.close()
        pk2.close()
        pool.close()
        pool2.close()


def test_memory_kind_checks(stream):
    t = torch()
    w, n = SMALL["tiny"]
    pool = DevicePool(w, seed=308)
    nb = w.host_bytes(n)
    src, _ = pages(w, n)
    pageable = np.zeros(nb + 16, dtype=np.uint8)
    pp = (pageable.ctypes.data + 15) // 16 * 16
    dev = t.empty(nb, dtype=t.uint8, device="cuda")
    pinned = K.HostBuffer(nb)

    def code(fn):
        with pytest.raises(K.KvxError) as e:
            fn()
        return e.value.code

    assert code(lambda: K.kvx_backup(pool.handle, src, pp, nb, 0, 2, stream,
                                     K.KVX_PATH_STAGED)) == K.KVX_E_NOTPINNED
    assert code(lambda: K.kvx_backup(pool.handle, src, pp, nb, 0, 2, stream,
                                     K.KVX_PATH_ZEROCOPY)) == K.KVX_E_NOTPINNED
    assert code(lambda: K.kvx_backup(pool.handle, src, dev, nb, 0, 2, stream,
                                     K.KVX_PATH_STAGED)) == K.KVX_E_INVAL
    assert code(lambda: K.kvx_backup(pool.handle, src, pinned.ptr, nb, 0, 2, stream,
                                     K.KVX_PATH_DEVICE)) == K.KVX_E_INVAL
    # torch's own pinned memory is accepted
    tp = t.empty(nb, dtype=t.uint8, pin_memory=True)
    K.kvx_backup(pool.handle, src, tp, nb, 0, 2, stream, K.KVX_PATH_ZEROCOPY)
    K.kvx_backup(pool.handle, src, pinned.ptr, nb, 0, 2, stream, K.KVX_PATH_STAGED)
    K.kvx_sync(stream)
    assert np.array_equal(tp.numpy(), pinned.numpy())
    pinned.free()
    pool.close()


def test_unregister_with_work_in_flight(stream):
    w, n = SMALL["llama_small"]
    pool = DevicePool(w, seed=309)
    src, _ = pages(w, n)
    pk = Packed(w, n, "staged")
    K.kvx_backup(pool.handle, src, pk.ptr, pk.nbytes, 0, w.num_layers, stream, K.KVX_PATH_STAGED)
    K.kvx_unregister_pool(pool.handle)   # waits for the backup, never raises
    with pytest.raises(K.KvxError) as e:
        K.kvx_backup(pool.handle, src, pk.ptr, pk.nbytes, 0, 1, stream, K.KVX_PATH_STAGED)
    assert e.value.code == K.KVX_E_STALE
    want = oracle.backup(oracle_layout(w), synth.pool_alloc_image(w, 309), src, 0, w.num_layers)
    assert np.array_equal(pk.numpy(), want)
    pool.handle = 0
    pk.close()


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("case", ["ragged_hnd2", "trtllm_small"])
def test_every_page_and_single_page(case, path, stream):
    """Edge sizes: a request naming every page of the pool (in a random
    order), and a one-page request, through backup and restore."""
    w, _ = SMALL[case]
    L = oracle_layout(w)
    pool = DevicePool(w, seed=401)
    img = pool.host_image()
    for ids in (synth.page_perm(77, w.num_pages), np.array([w.num_pages - 1], dtype=np.int32)):
        n = len(ids)
        nb = w.host_bytes(n)
        pk = Packed(w, n, path, fill_seed=6)
        K.kvx_backup(pool.handle, ids, pk.ptr, nb, 0, w.num_layers, stream, PATHS[path])
        K.kvx_sync(stream)
        want = oracle.backup(L, img, ids, 0, w.num_layers)
        got = pk.numpy()
        assert np.array_equal(got, want), f"n={n} " + diff_report(got, want)
        # restore the same bytes to the reversed page list
        rev = ids[::-1].copy()
        K.kvx_restore(pool.handle, pk.ptr, nb, rev, 0, w.num_layers, None, 0, stream, PATHS[path])
        K.kvx_sync(stream)
        after = pool.host_image()
        want_alloc = oracle.restore(L, img, want, rev, 0, w.num_layers)
        assert np.array_equal(after, want_alloc), f"n={n} " + diff_report(after, want_alloc)
        img = after
        pk.close()
    pool.close()


HND_LDS_CASES = {
    "trtllm_small": SMALL["trtllm_small"],
    # 128 KiB head-major pieces: two 64 KiB LDS token blocks (32 tokens x 8 heads) per piece
    "hnd_two_blocks": (Workload(name="hnd_two_blocks", outer=("layer", "kv", "page"), inner="HND",
                                num_pages=64, num_layers=2, num_kv=2, page_size=64, num_heads=8,
                                head_dim=128, dtype_bytes=2, pages_per_request=16, seed=204,
                                byte_offset=4096, alloc_tail=4096), 16),
    # 32 KiB pieces of 2 heads x 128 tokens of 128 B rows: one block of all 128 tokens
    "hnd_narrow_rows": (Workload(name="hnd_narrow_rows", outer=("page", "layer", "kv"),
                                 inner="HND", num_pages=48, num_layers=3, num_kv=2, page_size=128,
                                 num_heads=2, head_dim=64, dtype_bytes=2, pages_per_request=12,
                                 seed=205), 12),
}


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("case", list(HND_LDS_CASES))
def test_hnd_through_lds(case, path, stream):
    """The LDS token-block conversion gives the oracle's bytes, for backup,
    restore and restore with publish."""
    w, n = HND_LDS_CASES[case]
    L = oracle_layout(w)
    old = K.kvx_get_option(K.KVX_OPT_HND_LDS)
    K.kvx_set_option(K.KVX_OPT_HND_LDS, 1)
    try:
        pool = DevicePool(w, seed=501)
        img = pool.host_image()
        src, dst = pages(w, n)
        nb = w.host_bytes(n)
        pk = Packed(w, n, path, fill_seed=7)
        K.kvx_backup(pool.handle, src, pk.ptr, nb, 0, w.num_layers, stream, PATHS[path])
        K.kvx_sync(stream)
        want = oracle.backup(L, img, src, 0, w.num_layers)
        got = pk.numpy()
        assert np.array_equal(got, want), diff_report(got, want)
        ready = K.kvx_ready_create(w.num_layers, 1)
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, ready, 0, stream,
                      PATHS[path])
        K.kvx_sync(stream)
        assert K.kvx_ready_prefix(ready) == n
        K.kvx_ready_destroy(ready)
        after = pool.host_image()
        want_alloc = oracle.restore(L, img, want, dst, 0, w.num_layers)
        assert np.array_equal(after, want_alloc), diff_report(after, want_alloc)
        pk.close()
        pool.close()
    finally:
        K.kvx_set_option(K.KVX_OPT_HND_LDS, old)


@pytest.mark.parametrize("path", ["staged", "zerocopy", "device"])
def test_device_ready_object(path, stream):
    """Ready counts in device memory: a restore publishes into them, the host
    queries copy them back, a GPU wait sees them, a second handle attached
    to the same counts reads the same values, and reset clears them."""
    t = torch()
    w, n = SMALL["mla_small"]
    L = oracle_layout(w)
    pool = DevicePool(w, seed=311, generation=12)
    img = pool.host_image()
    src, dst = pages(w, n)
    nb = w.host_bytes(n)
    pk = Packed(w, n, path, fill_seed=51)
    ready = K.kvx_ready_create_device(0, w.num_layers + 2, 12)
    other = K.kvx_ready_attach_device(K.kvx_ready_slot_ptr(ready, 0), w.num_layers + 2, 12)
    status = t.zeros(1, dtype=t.int32, device="cuda")
    consumer = t.cuda.Stream()
    try:
        assert K.kvx_ready_prefix(ready) == 0
        K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, ready, 1, stream, PATHS[path])
        K.kvx_ready_wait_gpu(ready, w.num_layers, n, consumer, 5_000_000, status)
        K.kvx_sync(stream)
        K.kvx_sync(consumer)
        assert int(status.item()) == 1
        counts = [K.kvx_layer_ready(ready, s) for s in range(w.num_layers + 2)]
        assert counts == [0] + [n] * w.num_layers + [0]
        assert [K.kvx_layer_ready(other, s) for s in range(w.num_layers + 2)] == counts
        assert K.kvx_ready_prefix(ready) == 0 == K.kvx_ready_prefix(other)
        want = oracle.restore(L, img, synth.gen_bytes(51, 0, nb), dst, 0, w.num_layers)
        after = pool.host_image()
        assert np.array_equal(after, want), diff_report(after, want)
        K.kvx_ready_reset(other)
        assert [K.kvx_layer_ready(ready, s) for s in range(w.num_layers + 2)] == [0] * (w.num_layers + 2)
        # a ready object of another generation is refused
        stale = K.kvx_ready_create_device(0, w.num_layers, 13)
        with pytest.raises(K.KvxError) as e:
            K.kvx_restore(pool.handle, pk.ptr, nb, dst, 0, w.num_layers, stale, 0, stream,
                          PATHS[path])
        assert e.value.code == K.KVX_E_STALE
        K.kvx_ready_destroy(stale)
    finally:
        K.kvx_ready_destroy(other)
        K.kvx_ready_destroy(ready)
        pk.close()
        pool.close()


@pytest.mark.parametrize("path", list(PATHS))
def test_empty_work_is_a_noop_on_the_gpu(path, stream):
    """n = 0 and empty layer ranges move nothing and publish nothing (a
    restore of 0 pages has nothing to publish: every count stays at its
    value, and a count of 0 already equals n)."""
    w, n = SMALL["llama_small"]
    pool = DevicePool(w, seed=313, generation=14)
    img = pool.host_image()
    pk = Packed(w, n, path, fill_seed=61)
    ready = K.kvx_ready_create(w.num_layers, 14)
    try:
        src, dst = pages(w, n)
        K.kvx_restore(pool.handle, pk.ptr, pk.nbytes, [], 0, w.num_layers, ready, 0, stream, PATHS[path])
        K.kvx_restore(pool.handle, pk.ptr, pk.nbytes, dst, 1, 1, ready, 0, stream, PATHS[path])
        K.kvx_backup(pool.handle, [], pk.ptr, pk.nbytes, 0, w.num_layers, stream, PATHS[path])
        if path != "staged":
            K.kvx_exchange(pool.handle, [], pk.ptr, pk.nbytes, (0, w.num_layers), pk.ptr, pk.nbytes,
                           [], (0, w.num_layers), ready, 0, stream, PATHS[path])
        K.kvx_sync(stream)
        assert [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)] == [0] * w.num_layers
        assert np.array_equal(pool.host_image(), img)
        assert np.array_equal(pk.numpy(), synth.gen_bytes(61, 0, pk.nbytes))
    finally:
        K.kvx_ready_destroy(ready)
        pk.close()
        pool.close()


def test_trace_ranges_leave_results_unchanged():
    """With KVX_TRACE=1 every data-moving call opens and closes a roctx
    range; the smoke round trip (staged path and kvx_exchange, checked
    against the oracle) still passes. A process of its own, since the
    setting is read once."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, KVX_TRACE="1")
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.smoke()"], cwd=root,
                       env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "smoke ok" in r.stdout
