"""GPU parity on seeded random pool geometries: every outer order of
{page, layer, kv}, both inner layouts, 1-, 2- and 4-byte elements, rows of
16-624 bytes, 1-69 tokens and 1-9 heads per page, 1-5 layers, K alone or K
and V, byte offsets and trailing padding, merged or split piece axes in the
caller's tensor view. Each geometry runs BACKUP and a publishing RESTORE on
random paths and layer ranges, one kvx_exchange, the slot-addressed calls
and one kvx_exchange_slots, each compared byte for byte with the oracle
(whole packed buffer or host pool, whole allocation) and the per-layer
counts with what the restore published.

The geometries come from numpy's seeded generator (seed 9000 + k); the
CPU test at the end checks that every one of them is a valid pool for the
library's own host-side checks, so the GPU cases only exercise valid input."""
import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import Workload
from tests.gpu_util import PATHS, DevicePool, Packed, kvx_layout, oracle_layout, torch

NUM_GEOMS = 160
POOL_CAP = 12 << 20   # pool bytes at most (about), so the oracle stays fast


def random_workload(k: int, exotic: bool = False) -> Workload:
    rng = np.random.default_rng(9000 + k)
    outer = tuple(str(a) for a in rng.permutation(["page", "layer", "kv"]))
    inner = str(rng.choice(["NHD", "HND"]))
    if not exotic:
        eb = int(rng.choice([1, 2, 4]))
        row = 16 * int(rng.integers(1, 40))
    else:
        # element sizes no torch dtype has: rows stay 16-byte multiples
        eb = int(rng.choice([3, 6, 8, 12, 16, 64]))
        unit = int(np.lcm(16, eb))
        row = unit * int(rng.integers(1, max(2, 640 // unit + 1)))
    T = int(rng.integers(1, 70))
    H = int(rng.integers(1, 10))
    KV = int(rng.integers(1, 3))
    NL = int(rng.integers(1, 6))
    piece = T * H * row
    NB = int(rng.integers(4, max(5, min(1400, POOL_CAP // (piece * NL * KV))) + 1))
    return Workload(name=f"random{k}", outer=outer, inner=inner, num_pages=NB, num_layers=NL,
                    num_kv=KV, page_size=T, num_heads=H, head_dim=row // eb, dtype_bytes=eb,
                    pages_per_request=max(1, NB // 3), seed=9100 + k,
                    byte_offset=16 * int(rng.integers(0, 300)),
                    alloc_tail=16 * int(rng.integers(0, 300)),
                    merged_inner=bool(rng.integers(0, 2)))


GEOMS = [random_workload(k) for k in range(NUM_GEOMS)]
NUM_EXOTIC = 24
EXOTIC = [random_workload(NUM_GEOMS + k, exotic=True) for k in range(NUM_EXOTIC)]


def layer_range(rng, NL):
    l0 = int(rng.integers(0, NL))
    return l0, int(rng.integers(l0 + 1, NL + 1))


def diff_report(got, want, limit=8):
    bad = np.flatnonzero(got != want)
    return f"{bad.size} bytes differ; first at {bad[:limit].tolist()}"


@pytest.fixture(scope="module")
def stream():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    K.lib()
    return t.cuda.Stream()


# every tuning knob with the values it accepts (a sample of the wide ranges)
TUNING = {
    "GRID_MAX": [0, 0, 1, 3, 8, 13, 64, 1024],
    "HOST_GRID_MAX": [0, 0, 1, 2, 7, 32, 100],
    "UNIT_ORDER": [-1, -1, 0, 1, 2, 3],
    "MAX_UNROLL": [32, 32, 1, 2, 3, 4, 8, 16],
    "UNIT_ROUNDS": [0, 0, 0, 1, 2, 3, 4, 6, 8, 12, 16, 32],
    "CACHE_POLICY": [-1, -1, 0, 1, 2, 3, 4, 5, 6, 7],
    "HND_LDS": [-1, -1, 0, 1],
    "SORT_PAGES": [0, 1],
    "STAGE_SLOT_BYTES": [128 << 20, 1 << 20, 3 << 20],
    "STAGE_SLOTS": [3, 2, 8],
    "RESTORE_CHUNK_LAYERS": [0, 0, 1, 2],
    "STAGED_DMA_ON_CALLER": [-1, 0, 1],
    "PUBLISH_BLOCK": [0, 0, 1, 3, 16, 4096],
    "COALESCE_RUNS": [1, 1, 0],
    "TAIL_UNITS": [1, 1, 0],
    "DEVICE_LISTS": [1, 1, 0],
}
NUM_TUNED = 60


@pytest.mark.gpu
@pytest.mark.parametrize("k", range(NUM_GEOMS))
def test_random_geometry_parity(k, stream):
    run_geometry(k, np.random.default_rng(9500 + k), stream)


@pytest.mark.gpu
@pytest.mark.parametrize("k", range(NUM_TUNED))
def test_random_geometry_with_random_tuning(k, stream):
    """The same sequence with every tuning knob drawn at random (grid caps,
    unit order, unit size, cache policy, HND form, page sorting, staging
    ring and chunking, staged DMA stream): knobs change speed, never bytes."""
    rng = np.random.default_rng(9700 + k)
    opts = {name: int(rng.choice(vals)) for name, vals in TUNING.items()}
    print(f"\n[random] tuning {opts}", flush=True)
    old = {name: K.kvx_get_option(getattr(K, "KVX_OPT_" + name)) for name in TUNING}
    try:
        for name, v in opts.items():
            K.kvx_set_option(getattr(K, "KVX_OPT_" + name), v)
        run_geometry(k, rng, stream)
    finally:
        for name, v in old.items():
            K.kvx_set_option(getattr(K, "KVX_OPT_" + name), v)


@pytest.mark.gpu
@pytest.mark.parametrize("k", range(NUM_EXOTIC))
def test_random_geometry_with_other_element_sizes(k, stream):
    """Element sizes of 3, 6, 8, 12, 16 and 64 bytes: the library only sizes
    rows with them, so the bytes must come out as for any other size."""
    run_geometry(k, np.random.default_rng(9900 + k), stream, EXOTIC[k])


def run_geometry(k, rng, stream, w=None):
    w = GEOMS[k] if w is None else w
    NB, NL = w.num_pages, w.num_layers
    print(f"\n[random] k={k} outer={w.outer} inner={w.inner} NB={NB} NL={NL} KV={w.num_kv} "
          f"T={w.page_size} H={w.num_heads} row={w.row_bytes} eb={w.dtype_bytes} "
          f"offset={w.byte_offset} tail={w.alloc_tail} merged={w.merged_inner} "
          f"piece={w.piece_bytes}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, generation=4)
    ready = K.kvx_ready_create(NL, 4)
    bufs = []

    def packed(n, path, seed):
        b = Packed(w, n, path, fill_seed=seed)
        bufs.append(b)
        return b

    try:
        img = pool.host_image()
        perm = synth.page_perm(w.seed, NB)

        # BACKUP (source pages may repeat) then a publishing RESTORE
        n = int(rng.integers(1, NB // 2 + 1))
        src = perm[:n].copy()
        if n > 2 and rng.integers(0, 2):
            src[-1] = src[0]
        dst = perm[n:2 * n].copy()
        p1, p2 = (str(p) for p in rng.choice(list(PATHS), 2))
        l0, l1 = layer_range(rng, NL)
        print(f"[random] backup n={n} {p1} {l0}:{l1}; restore {p2}", flush=True)
        nb = w.host_bytes(n)
        pk = packed(n, p1, w.seed + 2)
        want = oracle.backup(L, img, src, l0, l1, host=synth.gen_bytes(w.seed + 2, 0, nb))
        K.kvx_backup(pool.handle, src, pk.ptr, nb, l0, l1, stream, PATHS[p1])
        K.kvx_sync(stream)
        got = pk.numpy()
        assert np.array_equal(got, want), "backup: " + diff_report(got, want)
        pr = packed(n, p2, w.seed + 3)
        want_alloc = oracle.restore(L, img, synth.gen_bytes(w.seed + 3, 0, nb), dst, l0, l1)
        K.kvx_restore(pool.handle, pr.ptr, nb, dst, l0, l1, ready, 0, stream, PATHS[p2])
        K.kvx_sync(stream)
        img = pool.host_image()
        assert np.array_equal(img, want_alloc), "restore: " + diff_report(img, want_alloc)
        counts = [K.kvx_layer_ready(ready, l) for l in range(NL)]
        assert counts == [n if l0 <= l < l1 else 0 for l in range(NL)]

        # one exchange: disjoint page lists, independent layer ranges
        xpath = str(rng.choice(["zerocopy", "device"]))
        nb_ = int(rng.integers(0, NB // 2 + 1))
        nr_ = int(rng.integers(1, NB - nb_ + 1))
        perm = synth.page_perm(w.seed + 1, NB)
        bsrc, rdst = perm[:nb_].copy(), perm[nb_:nb_ + nr_].copy()
        lb, lr = layer_range(rng, NL), layer_range(rng, NL)
        print(f"[random] exchange {xpath} nb={nb_} {lb} nr={nr_} {lr}", flush=True)
        K.kvx_ready_reset(ready)
        xb = packed(max(nb_, 1), xpath, w.seed + 4)   # a side of 0 pages runs nothing
        xr = packed(nr_, xpath, w.seed + 5)
        want_b = oracle.backup(L, img, bsrc, *lb, host=synth.gen_bytes(w.seed + 4, 0, xb.nbytes))
        want_alloc = oracle.restore(L, img, synth.gen_bytes(w.seed + 5, 0, w.host_bytes(nr_)), rdst, *lr)
        K.kvx_exchange(pool.handle, bsrc, xb.ptr, w.host_bytes(nb_), lb, xr.ptr, w.host_bytes(nr_),
                       rdst, lr, ready, 0, stream, PATHS[xpath])
        K.kvx_sync(stream)
        got = xb.numpy()
        assert np.array_equal(got, want_b), "exchange backup: " + diff_report(got, want_b)
        img = pool.host_image()
        assert np.array_equal(img, want_alloc), "exchange restore: " + diff_report(img, want_alloc)
        counts = [K.kvx_layer_ready(ready, l) for l in range(NL)]
        assert counts == [nr_ if lr[0] <= l < lr[1] else 0 for l in range(NL)]

        # slot-addressed host pool: backup into distinct scattered slots, then
        # restore of slots drawn with repeats into other pages
        spath = str(rng.choice(["zerocopy", "device"]))
        n = int(rng.integers(1, NB // 2 + 1))
        S = n + int(rng.integers(0, n + 4))
        perm = synth.page_perm(w.seed + 2, NB)
        src, dst = perm[:n].copy(), perm[n:2 * n].copy()
        bslots = rng.permutation(S)[:n].astype(np.int32)
        rslots = rng.integers(0, S, n).astype(np.int32)
        l0, l1 = layer_range(rng, NL)
        print(f"[random] slots {spath} n={n} S={S} {l0}:{l1}", flush=True)
        HB = w.host_bytes(S)
        hp = packed(S, spath, w.seed + 6)
        host = oracle.backup_slots(L, img, src, bslots, S, l0, l1,
                                   host=synth.gen_bytes(w.seed + 6, 0, HB))
        K.kvx_backup_slots(pool.handle, src, bslots, hp.ptr, HB, S, l0, l1, stream, PATHS[spath])
        K.kvx_sync(stream)
        got = hp.numpy()
        assert np.array_equal(got, host), "backup_slots: " + diff_report(got, host)
        K.kvx_ready_reset(ready)
        want_alloc = oracle.restore_slots(L, img, host, rslots, dst, S, l0, l1)
        K.kvx_restore_slots(pool.handle, hp.ptr, HB, S, rslots, dst, l0, l1, ready, 0, stream,
                            PATHS[spath])
        K.kvx_sync(stream)
        img = pool.host_image()
        assert np.array_equal(img, want_alloc), "restore_slots: " + diff_report(img, want_alloc)
        counts = [K.kvx_layer_ready(ready, l) for l in range(NL)]
        assert counts == [n if l0 <= l < l1 else 0 for l in range(NL)]

        # one exchange_slots on that host pool: the backup writes slots the
        # restore does not read, into pages the restore does not write
        nb_ = int(rng.integers(0, min(S, NB) // 2 + 1))
        nr_ = int(rng.integers(1, min(S, NB) - nb_ + 1))
        sperm = rng.permutation(S).astype(np.int32)
        xbs, xrs = sperm[:nb_].copy(), sperm[nb_:nb_ + nr_].copy()
        perm = synth.page_perm(w.seed + 3, NB)
        bsrc, rdst = perm[:nb_].copy(), perm[nb_:nb_ + nr_].copy()
        lb, lr = layer_range(rng, NL), layer_range(rng, NL)
        print(f"[random] exchange_slots {spath} nb={nb_} {lb} nr={nr_} {lr}", flush=True)
        K.kvx_ready_reset(ready)
        want_host = oracle.backup_slots(L, img, bsrc, xbs, S, *lb, host=host.copy())
        want_alloc = oracle.restore_slots(L, img, host, xrs, rdst, S, *lr)
        K.kvx_exchange_slots(pool.handle, bsrc, xbs, hp.ptr, HB, S, lb, hp.ptr, HB, S, xrs, rdst, lr,
                             ready, 0, stream, PATHS[spath])
        K.kvx_sync(stream)
        got = hp.numpy()
        assert np.array_equal(got, want_host), "exchange_slots backup: " + diff_report(got, want_host)
        img = pool.host_image()
        assert np.array_equal(img, want_alloc), "exchange_slots restore: " + \
            diff_report(img, want_alloc)
        counts = [K.kvx_layer_ready(ready, l) for l in range(NL)]
        assert counts == [nr_ if lr[0] <= l < lr[1] else 0 for l in range(NL)]
    finally:
        K.kvx_ready_destroy(ready)
        for b in bufs:
            b.close()
        pool.close()


def test_random_geometries_are_valid_pools():
    """Every random geometry registers (host-side checks only, no GPU) with
    the piece size the oracle computes, and the set covers what it is meant
    to: all six outer orders, both inner layouts, every element size, K
    alone and K and V, merged and split views, pieces above one 128 KiB
    unit, and pieces that are not a multiple of 4 KiB."""
    fake = 0x7F0000000000   # never dereferenced: registration reads no memory
    for w in GEOMS + EXOTIC:
        assert w.row_bytes % 16 == 0 and w.byte_offset % 16 == 0
        shape = w.tensor_shape()
        stride = [int(np.prod(shape[i + 1:])) for i in range(len(shape))]
        h = K.kvx_register_pool(kvx_layout(w), fake, w.byte_offset, w.dtype_bytes, shape, stride, 1)
        try:
            info = K.kvx_pool_get_info(h)
            assert info.piece_bytes == oracle_layout(w).piece_bytes == w.piece_bytes
        finally:
            K.kvx_unregister_pool(h)
    assert len({w.outer for w in GEOMS}) == 6
    assert {w.inner for w in GEOMS} == {"NHD", "HND"}
    assert {w.dtype_bytes for w in GEOMS} == {1, 2, 4}
    assert {w.num_kv for w in GEOMS} == {1, 2}
    assert {w.merged_inner for w in GEOMS} == {False, True}
    assert any(w.piece_bytes > 128 * 1024 for w in GEOMS)
    assert any(w.piece_bytes % 4096 for w in GEOMS)
    assert any(w.inner == "HND" and w.num_heads > 1 and w.page_size > 1 for w in GEOMS)
    assert {w.dtype_bytes for w in EXOTIC} == {3, 6, 8, 12, 16, 64}


def test_random_tuning_values_are_accepted():
    """Every knob value the tuned GPU cases draw is one kvx_set_option
    accepts (host only); the defaults come back afterwards."""
    old = {name: K.kvx_get_option(getattr(K, "KVX_OPT_" + name)) for name in TUNING}
    try:
        for name, vals in TUNING.items():
            for v in vals:
                K.kvx_set_option(getattr(K, "KVX_OPT_" + name), v)
                assert K.kvx_get_option(getattr(K, "KVX_OPT_" + name)) == v
    finally:
        for name, v in old.items():
            K.kvx_set_option(getattr(K, "KVX_OPT_" + name), v)
    assert {name: K.kvx_get_option(getattr(K, "KVX_OPT_" + name)) for name in TUNING} == old
