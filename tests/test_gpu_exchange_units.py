"""kvx_exchange and kvx_exchange_slots on the unit forms of single-direction
calls ([RFC] "Device IPC data path": BACKUP and RESTORE of any page lists;
both directions in one launch): shared tail units for pieces that 128 KiB
units do not tile, short pieces travelling whole several to a unit (over
the host link's 8 KiB units too), and page lists longer than the kernel
arguments carry read from device memory by one launch. Bytes and published
counts must be the oracle's, and the same with each form switched off."""
import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import WORKLOADS, Workload
from tests.gpu_util import PATHS, DevicePool, Packed, oracle_layout, torch

pytestmark = pytest.mark.gpu


def token_pool(heads, pages, seed):
    """One token per page: pieces of heads x 256 B."""
    return Workload(name=f"x_token{heads}", outer=("layer", "kv", "page"), inner="NHD", num_pages=pages,
                    num_layers=3, num_kv=2, page_size=1, num_heads=heads, head_dim=128, dtype_bytes=2,
                    pages_per_request=100, seed=seed, byte_offset=4096, alloc_tail=4096)


POOLS = {
    "token2k": token_pool(8, 3000, 251),     # 2 KiB pieces: whole, 32 a device unit, 4 a host unit
    "token1k": token_pool(4, 3000, 252),     # 1 KiB pieces: 8 a host unit
    "mla": WORKLOADS["mla_fp8"].scaled(name="x_mla", num_pages=600, num_layers=3),   # 16 KiB tails
    "ragged": Workload(name="x_ragged", outer=("kv", "layer", "page"), inner="NHD", num_pages=2400,
                       num_layers=2, num_kv=2, page_size=5, num_heads=3, head_dim=8, dtype_bytes=2,
                       pages_per_request=100, seed=253, byte_offset=8192, alloc_tail=1008),   # 240 B
}

# (pool, backup pages, restore pages): short lists, and lists longer than the
# kernel arguments carry on one side or both
CASES = [("token2k", 100, 60), ("token2k", 900, 700), ("token1k", 37, 500), ("mla", 40, 23),
         ("mla", 200, 150), ("ragged", 600, 500)]

FORMS = {"default": {}, "no_tails": {"TAIL_UNITS": 0}, "no_lists": {"DEVICE_LISTS": 0}}


def diff_report(got, want, limit=8):
    bad = np.flatnonzero(got != want)
    return f"{bad.size} bytes differ; first at {bad[:limit].tolist()}"


@pytest.fixture(scope="module")
def stream():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    K.lib()
    return t.cuda.Stream()


def with_options(opts, fn):
    old = {k: K.kvx_get_option(getattr(K, "KVX_OPT_" + k)) for k in opts}
    try:
        for k, v in opts.items():
            K.kvx_set_option(getattr(K, "KVX_OPT_" + k), v)
        return fn()
    finally:
        for k, v in old.items():
            K.kvx_set_option(getattr(K, "KVX_OPT_" + k), v)


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("path", ["zerocopy", "device"])
@pytest.mark.parametrize("pool,nb,nr", CASES)
def test_exchange_unit_forms(pool, nb, nr, path, form, stream):
    """Two exchanges back to back (the second backs up pages the first
    restored into): both packed buffers, the allocation and the counts equal
    the oracle's."""
    w = POOLS[pool]
    L = oracle_layout(w)
    assert nb + 2 * nr <= w.num_pages
    print(f"\n[xunits] pool={pool} nb={nb} nr={nr} path={path} form={form}", flush=True)
    perm = synth.page_perm(w.seed + 13, w.num_pages)

    def run():
        p = DevicePool(w, seed=401, generation=3)
        ready = K.kvx_ready_create(w.num_layers, 3)
        bufs = []
        try:
            want_alloc = p.host_image()
            wants, counts = [], [0] * w.num_layers
            for r in range(2):
                # the second backs up pages that include the first's destinations
                src = perm[r * nr:r * nr + nb].copy()
                dst = perm[nb + r * nr:nb + (r + 1) * nr].copy()
                pk_b = Packed(w, nb, path, fill_seed=410 + r)
                pk_r = Packed(w, nr, path, fill_seed=420 + r)
                bufs += [pk_b, pk_r]
                wants.append(oracle.backup(L, want_alloc, src, 0, w.num_layers,
                                           host=synth.gen_bytes(410 + r, 0, w.host_bytes(nb))))
                want_alloc = oracle.restore(L, want_alloc, synth.gen_bytes(420 + r, 0, w.host_bytes(nr)), dst,
                                            0, w.num_layers)
                counts = oracle.ready_publish(counts, 0, 0, w.num_layers, nr)
                K.kvx_exchange(p.handle, src, pk_b.ptr, w.host_bytes(nb), (0, w.num_layers), pk_r.ptr,
                               w.host_bytes(nr), dst, (0, w.num_layers), ready, 0, stream, PATHS[path])
            K.kvx_sync(stream)
            got = [bufs[0].numpy(), bufs[2].numpy()]
            for r in range(2):
                assert np.array_equal(got[r], wants[r]), f"exchange {r} backup: " + diff_report(got[r], wants[r])
            after = p.host_image()
            assert np.array_equal(after, want_alloc), "restore: " + diff_report(after, want_alloc)
            assert [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)] == counts
        finally:
            K.kvx_ready_destroy(ready)
            for b in bufs:
                b.close()
            p.close()

    with_options(FORMS[form], run)


@pytest.mark.parametrize("path", ["zerocopy", "device"])
@pytest.mark.parametrize("pool,nb,nr", [("token2k", 500, 300), ("mla", 30, 250), ("ragged", 260, 40)])
def test_exchange_slots_unit_forms(pool, nb, nr, path, stream):
    """kvx_exchange_slots of long and short (page, slot) lists into host
    pools of S slots, with device lists on and off: both host pools and the
    allocation equal the oracle's."""
    w = POOLS[pool]
    L = oracle_layout(w)
    S = nb + nr + 7
    rng = np.random.default_rng(w.seed + 17)
    perm = synth.page_perm(w.seed + 14, w.num_pages)
    bids, rids = perm[:nb].copy(), perm[nb:nb + nr].copy()
    bsl = rng.permutation(S)[:nb].astype(np.int32)
    rsl = rng.permutation(S)[:nr].astype(np.int32)
    print(f"\n[xslots units] pool={pool} nb={nb} nr={nr} path={path}", flush=True)
    for lists in (1, 0):
        def run():
            p = DevicePool(w, seed=402, generation=3)
            hb = Packed(w, S, path, fill_seed=430)
            hr = Packed(w, S, path, fill_seed=431)
            ready = K.kvx_ready_create(w.num_layers, 3)
            try:
                img = p.host_image()
                want_b = oracle.backup_slots(L, img, bids, bsl, S, 0, w.num_layers,
                                             host=synth.gen_bytes(430, 0, hb.nbytes))
                want = oracle.restore_slots(L, img, synth.gen_bytes(431, 0, hr.nbytes), rsl, rids, S, 0,
                                            w.num_layers)
                K.kvx_exchange_slots(p.handle, bids, bsl, hb.ptr, hb.nbytes, S, (0, w.num_layers), hr.ptr,
                                     hr.nbytes, S, rsl, rids, (0, w.num_layers), ready, 0, stream, PATHS[path])
                K.kvx_sync(stream)
                got = hb.numpy()
                assert np.array_equal(got, want_b), f"lists={lists} backup: " + diff_report(got, want_b)
                after = p.host_image()
                assert np.array_equal(after, want), f"lists={lists} restore: " + diff_report(after, want)
                assert [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)] == [nr] * w.num_layers
            finally:
                K.kvx_ready_destroy(ready)
                hb.close()
                hr.close()
                p.close()

        with_options({"DEVICE_LISTS": lists}, run)
