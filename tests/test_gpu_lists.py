"""Page lists longer than one launch's kernel arguments carry ([RFC] "Device
IPC data path": BACKUP and RESTORE name any number of source or destination
pages; a pool of one token per page names thousands per request). Such a
list goes to device memory on the caller's stream and one launch moves
every page and layer. Bytes and published counts must be the oracle's, and
the same as with launches of at most 448 pairs each, for fragmented lists,
lists of many runs of adjacent pages, pieces of every unit form, every
path; calls back to back on one stream reuse the device list in stream
order; a consumer reads each layer as soon as it is published."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import WORKLOADS, Workload
from tests.gpu_util import PATHS, DevicePool, Packed, oracle_layout, torch

pytestmark = pytest.mark.gpu

POOLS = {
    # one-token pages of 2 KiB (whole pieces, 32 to a unit)
    "token": (Workload(name="lists_token", outer=("layer", "kv", "page"), inner="NHD", num_pages=6000,
                       num_layers=3, num_kv=2, page_size=1, num_heads=8, head_dim=128, dtype_bytes=2,
                       pages_per_request=2600, seed=241, byte_offset=4096, alloc_tail=4096), 2600),
    # 128 KiB pieces, one unit each
    "llama": (WORKLOADS["llama8b"].scaled(name="lists_llama", num_pages=1400, num_layers=2), 600),
    # 144 KiB pieces: a unit and a shared tail each
    "mla": (WORKLOADS["mla_fp8"].scaled(name="lists_mla", num_pages=1200, num_layers=3), 520),
}


def diff_report(got, want, limit=8):
    bad = np.flatnonzero(got != want)
    return f"{bad.size} bytes differ; first at {bad[:limit].tolist()}"


def page_lists(w, kind, n, seed):
    """(source, destination) lists, disjoint: `fragmented` = a random
    permutation's first and next n; `stretches` = ascending stretches of 1 to
    12 pages at random places (hundreds of runs of adjacent pages)."""
    rng = np.random.default_rng(seed)
    if kind == "fragmented":
        perm = synth.page_perm(seed, w.num_pages)
        return perm[:n].copy(), perm[n:2 * n].copy()
    used = np.zeros(w.num_pages, dtype=bool)
    out, total = [], 0
    while total < 2 * n:
        ln = min(int(rng.integers(1, 13)), 2 * n - total)
        start = int(rng.integers(0, w.num_pages - ln + 1))
        if used[start:start + ln].any():
            continue
        used[start:start + ln] = True
        out.append(np.arange(start, start + ln, dtype=np.int32))
        total += ln
    ids = np.concatenate(out)
    return ids[:n].copy(), ids[n:2 * n].copy()


@pytest.fixture(scope="module")
def stream():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    K.lib()
    return t.cuda.Stream()


CASES = [("token", "fragmented"), ("token", "stretches"), ("llama", "fragmented"), ("mla", "fragmented"),
         ("mla", "stretches")]


@pytest.mark.parametrize("path", ["device", "zerocopy", "staged"])
@pytest.mark.parametrize("pool,kind", CASES)
def test_long_lists_move_the_oracle_bytes(pool, kind, path, stream):
    """BACKUP of a long source list, then publishing RESTOREs into a long
    destination list over two layer ranges, with device lists on and off:
    packed buffers, allocations and counts equal each other and the
    oracle's."""
    w, n = POOLS[pool]
    L = oracle_layout(w)
    src, dst = page_lists(w, kind, n, seed=w.seed + 3)
    nb = w.host_bytes(n)
    print(f"\n[lists] pool={pool} kind={kind} n={n} path={path}", flush=True)
    results = {}
    old = K.kvx_get_option(K.KVX_OPT_DEVICE_LISTS)
    try:
        for lists in (1, 0):
            K.kvx_set_option(K.KVX_OPT_DEVICE_LISTS, lists)
            p = DevicePool(w, seed=391, generation=2)
            img = p.host_image()
            ready = K.kvx_ready_create(w.num_layers, 2)
            pk = Packed(w, n, path, fill_seed=995)
            try:
                want_pk = oracle.backup(L, img, src, 0, w.num_layers, host=pk.numpy())
                K.kvx_backup(p.handle, src, pk.ptr, nb, 0, w.num_layers, stream, PATHS[path])
                K.kvx_sync(stream)
                got = pk.numpy()
                assert np.array_equal(got, want_pk), "backup " + diff_report(got, want_pk)
                want, counts = img, [0] * w.num_layers
                for l0 in (0, 1):
                    want = oracle.restore(L, want, got, dst, l0, w.num_layers)
                    counts = oracle.ready_publish(counts, 0, l0, w.num_layers, n)
                    K.kvx_restore(p.handle, pk.ptr, nb, dst, l0, w.num_layers, ready, 0, stream, PATHS[path])
                K.kvx_sync(stream)
                after = p.host_image()
                assert np.array_equal(after, want), "restore " + diff_report(after, want)
                assert [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)] == counts
                results[lists] = (got, after)
            finally:
                K.kvx_ready_destroy(ready)
                pk.close()
                p.close()
    finally:
        K.kvx_set_option(K.KVX_OPT_DEVICE_LISTS, old)
    assert np.array_equal(results[0][0], results[1][0])
    assert np.array_equal(results[0][1], results[1][1])


@pytest.mark.parametrize("path", ["device", "zerocopy"])
def test_long_list_calls_back_to_back(path, stream):
    """Seven BACKUPs of seven different long lists enqueued on one stream
    with no wait between them (more calls than the pinned list buffers a
    stream rotates through; each call's device list is overwritten by the
    next call's copy in stream order), then every packed buffer checked."""
    w, _ = POOLS["token"]
    n = 800
    L = oracle_layout(w)
    p = DevicePool(w, seed=392, generation=2)
    img = p.host_image()
    pks, srcs = [], []
    try:
        for i in range(7):
            src, _ = page_lists(w, "fragmented" if i % 2 else "stretches", n, seed=500 + i)
            pk = Packed(w, n, path, fill_seed=700 + i)
            pks.append(pk)
            srcs.append(src)
        for i in range(7):
            K.kvx_backup(p.handle, srcs[i], pks[i].ptr, pks[i].nbytes, 0, w.num_layers, stream, PATHS[path])
        K.kvx_sync(stream)
        for i in range(7):
            want = oracle.backup(L, img, srcs[i], 0, w.num_layers,
                                 host=synth.gen_bytes(700 + i, 0, pks[i].nbytes))
            got = pks[i].numpy()
            assert np.array_equal(got, want), f"call {i}: " + diff_report(got, want)
    finally:
        for pk in pks:
            pk.close()
        p.close()


@pytest.mark.parametrize("path", ["device", "zerocopy"])
@pytest.mark.parametrize("pool", ["token", "mla"])
def test_long_list_consumer_reads_every_layer(pool, path, stream):
    """Three rounds of fresh bytes into the same long destination list
    without a reset: a consumer stream waits (bounded) for each layer's
    cumulative count and copies the layer out at once; every copy holds that
    round's bytes."""
    t = torch()
    w, n = POOLS[pool]
    L = oracle_layout(w)
    NL = w.num_layers
    _, dst = page_lists(w, "fragmented", n, seed=w.seed + 4)
    nb = w.host_bytes(n)
    p = DevicePool(w, seed=393, generation=2)
    img = p.host_image()
    ready = K.kvx_ready_create(NL, 2)
    consumer = t.cuda.Stream()
    status = t.zeros(NL, dtype=t.int32, device="cuda")
    out = Packed(w, n, "device")
    try:
        for r in range(3):
            pk = Packed(w, n, path, fill_seed=610 + r)
            status.zero_()
            t.cuda.synchronize()
            K.kvx_restore(p.handle, pk.ptr, nb, dst, 0, NL, ready, 0, stream, PATHS[path])
            for l in range(NL):
                K.kvx_ready_wait_gpu(ready, l, (r + 1) * n, consumer, 4_000_000, status[l:l + 1])
                K.kvx_backup(p.handle, dst, out.ptr, nb, l, l + 1, consumer, K.KVX_PATH_DEVICE)
            K.kvx_sync(consumer)
            K.kvx_sync(stream)
            assert status.tolist() == [1] * NL, f"round {r}: a wait gave up"
            want = oracle.backup(L, oracle.restore(L, img, synth.gen_bytes(610 + r, 0, nb), dst, 0, NL),
                                 dst, 0, NL)
            got = out.numpy()
            assert np.array_equal(got, want), f"round {r}: " + diff_report(got, want)
            pk.close()
    finally:
        out.close()
        K.kvx_ready_destroy(ready)
        p.close()


def test_release_of_a_stream_that_used_a_device_list():
    """A stream that ran a long-list call is released and destroyed; a new
    stream then runs one as well, exact both times."""
    t = torch()
    t.cuda.init()
    hip = ctypes.CDLL(K.hip_runtimes_mapped()[0])
    hip.hipStreamCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    w, _ = POOLS["token"]
    n = 1000
    L = oracle_layout(w)
    p = DevicePool(w, seed=394, generation=2)
    img = p.host_image()
    try:
        for i in range(2):
            s = ctypes.c_void_p()
            assert hip.hipStreamCreateWithFlags(ctypes.byref(s), 1) == 0
            src, _ = page_lists(w, "fragmented", n, seed=520 + i)
            pk = Packed(w, n, "device", fill_seed=720 + i)
            K.kvx_backup(p.handle, src, pk.ptr, pk.nbytes, 0, w.num_layers, s.value, K.KVX_PATH_DEVICE)
            K.kvx_sync(s.value)
            want = oracle.backup(L, img, src, 0, w.num_layers, host=synth.gen_bytes(720 + i, 0, pk.nbytes))
            assert np.array_equal(pk.numpy(), want), f"stream {i}"
            K.kvx_release_stream(s.value)
            assert hip.hipStreamDestroy(s) == 0
            pk.close()
    finally:
        p.close()
