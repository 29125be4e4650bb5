"""GPU parity of the slot-addressed host tier: kvx_backup_slots and
kvx_restore_slots through the C ABI against oracle.backup_slots /
oracle.restore_slots, byte for byte over the whole host pool and the whole
pool allocation, on both paths that take a host pool (zero-copy over the host
link, device memory), for pools of every outer order and both inner layouts,
ragged pieces and more pages than one launch carries."""
import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from tests.gpu_util import PATHS, DevicePool, Packed, oracle_layout, torch
from tests.test_gpu_parity import SMALL, diff_report

pytestmark = pytest.mark.gpu

SLOT_PATHS = ["zerocopy", "device"]
CASES = ["tiny", "llama_small", "mla_small", "trtllm_small", "ragged_hnd", "ragged_nhd",
         "hnd_t1", "hnd_f32_rows16"]


@pytest.fixture(scope="module")
def stream():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    K.lib()
    return t.cuda.Stream()


def slot_case(w, n):
    """Host pool of 2n + 3 slots; backup slots distinct and scattered over the
    pool, restore slots drawn with repeats (one host copy into two pages)."""
    S = 2 * n + 3
    rng = np.random.default_rng(w.seed + 40)
    perm = synth.page_perm(w.seed + 41, w.num_pages)
    src, dst = perm[:n].copy(), perm[n:2 * n].copy()
    bslots = rng.permutation(S)[:n].astype(np.int32)
    rslots = rng.integers(0, S, n).astype(np.int32)
    return S, src, dst, bslots, rslots


@pytest.mark.parametrize("path", SLOT_PATHS)
@pytest.mark.parametrize("case", CASES)
def test_slot_backup_restore_parity(case, path, stream):
    w, n = SMALL[case]
    S, src, dst, bslots, rslots = slot_case(w, n)
    print(f"\n[slots] case={case} path={path} n={n} slots={S} piece={w.piece_bytes}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=w.seed + 42, generation=3)
    nb = w.host_bytes(S)
    hp = Packed(w, S, path, fill_seed=w.seed + 43)
    ready = K.kvx_ready_create(w.num_layers, 3)
    try:
        img = pool.host_image()
        host = synth.gen_bytes(w.seed + 43, 0, nb)
        ranges = [(0, w.num_layers), (1, w.num_layers)] if w.num_layers > 1 else [(0, 1)]
        for l0, l1 in ranges:
            host = oracle.backup_slots(L, img, src, bslots, S, l0, l1, host=host)
            K.kvx_backup_slots(pool.handle, src, bslots, hp.ptr, nb, S, l0, l1, stream,
                               PATHS[path])
            K.kvx_sync(stream)
            got = hp.numpy()
            assert np.array_equal(got, host), f"backup_slots {l0}:{l1} " + diff_report(got, host)

            want = oracle.restore_slots(L, img, host, rslots, dst, S, l0, l1)
            K.kvx_ready_reset(ready)
            K.kvx_restore_slots(pool.handle, hp.ptr, nb, S, rslots, dst, l0, l1, ready, 0,
                                stream, PATHS[path])
            K.kvx_sync(stream)
            after = pool.host_image()
            assert np.array_equal(after, want), f"restore_slots {l0}:{l1} " + \
                diff_report(after, want)
            counts = [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)]
            assert counts == [0] * l0 + [n] * (l1 - l0)
            img = after
    finally:
        K.kvx_ready_destroy(ready)
        hp.close()
        pool.close()


@pytest.mark.parametrize("path", SLOT_PATHS)
def test_slot_round_trip_with_sorted_visits(path, stream):
    """With pages visited in sorted order, a backup into scattered slots and
    a restore of the same slots into other pages leaves the other pages equal
    to the source pages (oracle bytes) and every unnamed host slot as it was."""
    w, n = SMALL["ragged_nhd"]
    S, src, dst, bslots, _ = slot_case(w, n)
    print(f"\n[slots-sorted] path={path} n={n} slots={S}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=w.seed + 44, generation=2)
    nb = w.host_bytes(S)
    hp = Packed(w, S, path, fill_seed=w.seed + 45)
    old = K.kvx_get_option(K.KVX_OPT_SORT_PAGES)
    try:
        K.kvx_set_option(K.KVX_OPT_SORT_PAGES, 1)
        img = pool.host_image()
        host = oracle.backup_slots(L, img, src, bslots, S, 0, w.num_layers,
                                   host=synth.gen_bytes(w.seed + 45, 0, nb))
        want = oracle.restore_slots(L, img, host, bslots, dst, S, 0, w.num_layers)
        K.kvx_backup_slots(pool.handle, src, bslots, hp.ptr, nb, S, 0, w.num_layers, stream,
                           PATHS[path])
        K.kvx_restore_slots(pool.handle, hp.ptr, nb, S, bslots, dst, 0, w.num_layers, None, 0,
                            stream, PATHS[path])
        K.kvx_sync(stream)
        got = hp.numpy()
        assert np.array_equal(got, host), diff_report(got, host)
        after = pool.host_image()
        assert np.array_equal(after, want), diff_report(after, want)
    finally:
        K.kvx_set_option(K.KVX_OPT_SORT_PAGES, old)
        hp.close()
        pool.close()


def test_slot_memory_kind_checks(stream):
    """The zero-copy path refuses a device host pool and the device path a
    pinned one (GPU-side checks: they need the runtime's pointer query)."""
    w, n = SMALL["tiny"]
    pool = DevicePool(w)
    nb = w.host_bytes(4)
    dev = Packed(w, 4, "device")
    pin = Packed(w, 4, "zerocopy")
    try:
        with pytest.raises(K.KvxError) as e:
            K.kvx_backup_slots(pool.handle, [1], [2], dev.ptr, nb, 4, 0, 2, stream,
                               K.KVX_PATH_ZEROCOPY)
        assert e.value.code == K.KVX_E_INVAL
        with pytest.raises(K.KvxError) as e:
            K.kvx_restore_slots(pool.handle, pin.ptr, nb, 4, [2], [1], 0, 2, None, 0, stream,
                                K.KVX_PATH_DEVICE)
        assert e.value.code == K.KVX_E_INVAL
    finally:
        dev.close()
        pin.close()
        pool.close()


@pytest.mark.parametrize("path", SLOT_PATHS)
@pytest.mark.parametrize("case", ["llama_small", "ragged_hnd"])
def test_tier_write_through_sequence(case, path, stream):
    """A write-through host tier of 8 slots: kvx_tier_backup of six pages,
    then of six more (two already present, two evictions), then
    kvx_tier_restore of a hit, an evicted key and another hit into fresh
    pages. Slots and evictions equal the tier model's, the host pool equals
    the oracle's slot backups, the pool equals the oracle's slot restore of
    the hits (the miss's page untouched), and each layer publishes the hits."""
    from oracle.tier_model import TierModel
    w, _ = SMALL[case]
    S = 8
    print(f"\n[tier] case={case} path={path} slots={S}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=w.seed + 50, generation=9)
    nb = w.host_bytes(S)
    hp = Packed(w, S, path, fill_seed=w.seed + 51)
    tier = K.kvx_tier_create(S, 9)
    ready = K.kvx_ready_create(w.num_layers, 9)
    model = TierModel(S)
    perm = synth.page_perm(w.seed + 52, w.num_pages)
    keys = [1000 + 7 * i for i in range(10)]
    try:
        img = pool.host_image()
        host = synth.gen_bytes(w.seed + 51, 0, nb)
        for kk, pages in ((keys[0:6], perm[0:6]), (keys[4:10], perm[4:10])):
            slots, ev = K.kvx_tier_backup(tier, pool.handle, kk, pages, hp.ptr, nb, stream,
                                          PATHS[path])
            want_slots, want_ev = model.reserve(kk)
            assert (slots.tolist(), ev.tolist()) == (want_slots, want_ev)
            new = slots >= 0
            host = oracle.backup_slots(L, img, pages[new], slots[new], S, 0, w.num_layers,
                                       host=host)
            K.kvx_sync(stream)
            K.kvx_tier_commit(tier, slots)
            model.commit(want_slots)
        assert model.evictions == 2
        got = hp.numpy()
        assert np.array_equal(got, host), "host tier " + diff_report(got, host)

        rkeys = [keys[2], keys[0], keys[7]]
        dst = perm[20:23].copy()
        rslots = K.kvx_tier_restore(tier, pool.handle, rkeys, dst, hp.ptr, nb, ready, 0, stream,
                                    PATHS[path])
        assert rslots.tolist() == model.lookup(rkeys)
        assert rslots[1] == -1 and rslots[0] >= 0 and rslots[2] >= 0
        hit = rslots >= 0
        want = oracle.restore_slots(L, img, host, rslots[hit], dst[hit], S, 0, w.num_layers)
        K.kvx_sync(stream)
        after = pool.host_image()
        assert np.array_equal(after, want), "restore " + diff_report(after, want)
        assert [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)] == \
            [2] * w.num_layers
        K.kvx_tier_release(tier, rslots)
        model.release(rslots.tolist())
        assert [K.kvx_tier_slot(tier, s) for s in range(S)] == model.view()
    finally:
        K.kvx_ready_destroy(ready)
        K.kvx_tier_destroy(tier)
        hp.close()
        pool.close()


# (case, backup pages, restore pages, backup layers, restore layers, one host pool)
EXCHANGE_SLOTS = [
    ("llama_small", 24, 11, None, (1, 3), True),
    ("ragged_hnd", 460, 230, None, None, False),     # three launches of at most 224 pages
    ("trtllm_small", 16, 16, (0, 2), (2, 3), True),  # disjoint layers: slots may repeat
    ("mla_small", 10, 7, None, None, True),
]


@pytest.mark.parametrize("path", SLOT_PATHS)
@pytest.mark.parametrize("case,nb_,nr,lb,lr,shared", EXCHANGE_SLOTS)
def test_exchange_slots_parity(case, nb_, nr, lb, lr, shared, path, stream):
    """kvx_exchange_slots gives the bytes of kvx_backup_slots followed by
    kvx_restore_slots (oracle), publishes the restore's layers, and leaves
    every host slot it does not write as it was."""
    w, _ = SMALL[case]
    print(f"\n[xslots] case={case} path={path} backup={nb_} restore={nr} shared={shared}", flush=True)
    L = oracle_layout(w)
    lb = lb or (0, w.num_layers)
    lr = lr or (0, w.num_layers)
    S = nb_ + nr + 5
    pool = DevicePool(w, seed=w.seed + 90, generation=5)
    rng = np.random.default_rng(w.seed + 91)
    perm = synth.page_perm(w.seed + 92, w.num_pages)
    bids, rids = perm[:nb_].copy(), perm[nb_:nb_ + nr].copy()
    order = rng.permutation(S).astype(np.int32)
    bsl = order[:nb_]
    # restore slots: disjoint from the backup's in a shared pool when layers overlap
    overlap = max(lb[0], lr[0]) < min(lb[1], lr[1])
    rsl = order[nb_:nb_ + nr] if (shared and overlap) else rng.permutation(S)[:nr].astype(np.int32)
    hb = Packed(w, S, path, fill_seed=w.seed + 93)
    hr = hb if shared else Packed(w, S, path, fill_seed=w.seed + 94)
    ready = K.kvx_ready_create(w.num_layers, 5)
    try:
        img = pool.host_image()
        host_b = synth.gen_bytes(w.seed + 93, 0, hb.nbytes)
        host_r = host_b if shared else synth.gen_bytes(w.seed + 94, 0, hr.nbytes)
        want_b = oracle.backup_slots(L, img, bids, bsl, S, lb[0], lb[1], host=host_b.copy())
        src_r = want_b if shared else host_r
        want_alloc = oracle.restore_slots(L, img, src_r, rsl, rids, S, lr[0], lr[1])
        K.kvx_exchange_slots(pool.handle, bids, bsl, hb.ptr, hb.nbytes, S, lb, hr.ptr, hr.nbytes, S,
                             rsl, rids, lr, ready, 0, stream, PATHS[path])
        K.kvx_sync(stream)
        got = hb.numpy()
        assert np.array_equal(got, want_b), "backup side " + diff_report(got, want_b)
        after = pool.host_image()
        assert np.array_equal(after, want_alloc), "restore side " + diff_report(after, want_alloc)
        counts = [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)]
        assert counts == [nr if lr[0] <= s < lr[1] else 0 for s in range(w.num_layers)]
    finally:
        K.kvx_ready_destroy(ready)
        hb.close()
        if not shared:
            hr.close()
        pool.close()


@pytest.mark.parametrize("path", SLOT_PATHS)
def test_tier_exchange_stores_misses_while_loading_hits(path, stream):
    """A tier of 8 slots holding 6 entries: kvx_tier_exchange restores two
    hits (pinned first, so never evicted) while it backs up four new keys
    (two into free slots, two evicting the least recently used unpinned
    entries). Slots and evictions equal the model's; the tier and the pool
    hold the oracle's bytes; the restore publishes the two hits."""
    from oracle.tier_model import TierModel
    w, _ = SMALL["llama_small"]
    S = 8
    print(f"\n[tier-exchange] path={path}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=w.seed + 99, generation=9)
    nb = w.host_bytes(S)
    hp = Packed(w, S, path, fill_seed=w.seed + 100)
    tier = K.kvx_tier_create(S, 9)
    ready = K.kvx_ready_create(w.num_layers, 9)
    model = TierModel(S)
    perm = synth.page_perm(w.seed + 101, w.num_pages)
    keys = [500 + 3 * i for i in range(10)]
    try:
        img = pool.host_image()
        host = synth.gen_bytes(w.seed + 100, 0, nb)
        slots, _ = K.kvx_tier_backup(tier, pool.handle, keys[:6], perm[:6], hp.ptr, nb, stream,
                                     PATHS[path])
        assert slots.tolist() == model.reserve(keys[:6])[0]
        host = oracle.backup_slots(L, img, perm[:6], slots, S, 0, w.num_layers, host=host)
        K.kvx_sync(stream)
        K.kvx_tier_commit(tier, slots)
        model.commit(slots.tolist())

        rkeys, rpages = [keys[0], keys[5]], perm[20:22]
        bkeys, bpages = keys[6:10], perm[6:10]
        bs, ev, rs = K.kvx_tier_exchange(tier, pool.handle, bkeys, bpages, rkeys, rpages, hp.ptr, nb,
                                         ready, 0, stream, PATHS[path])
        want_rs = model.lookup(rkeys)
        want_bs, want_ev = model.reserve(bkeys)
        assert (bs.tolist(), ev.tolist(), rs.tolist()) == (want_bs, want_ev, want_rs)
        assert sorted(want_ev) == [keys[1], keys[2]]
        restored = oracle.restore_slots(L, img, host, rs, rpages, S, 0, w.num_layers)
        host = oracle.backup_slots(L, img, bpages, bs, S, 0, w.num_layers, host=host)
        K.kvx_sync(stream)
        got = hp.numpy()
        assert np.array_equal(got, host), "tier " + diff_report(got, host)
        after = pool.host_image()
        assert np.array_equal(after, restored), "pool " + diff_report(after, restored)
        assert K.kvx_ready_prefix(ready) == 2
        K.kvx_tier_commit(tier, bs)
        K.kvx_tier_release(tier, rs)
        model.commit(want_bs)
        model.release(want_rs)
        assert [K.kvx_tier_slot(tier, s) for s in range(S)] == model.view()
    finally:
        K.kvx_ready_destroy(ready)
        K.kvx_tier_destroy(tier)
        hp.close()
        pool.close()
