"""Runs of adjacent pages on the data path: pages that are adjacent in the
pool and land in consecutive slots move as one span, in fewer and fuller
work units ([RFC] "Device IPC data path": BACKUP names source pages,
RESTORE destination pages; a scheduler that allocates a request's pages
together hands over long runs). Bytes must be those of the oracle, and the
same with coalescing switched off, for page lists that are wholly
contiguous, partly contiguous or fragmented, on pools whose pieces a unit
tiles, does not tile, or is much larger than."""
import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import WORKLOADS, Workload
from tests.gpu_util import PATHS, DevicePool, Packed, oracle_layout, torch

pytestmark = pytest.mark.gpu

POOLS = {
    # 4 KiB pieces
    "tiny": WORKLOADS["tiny"].scaled(name="tiny_runs", num_pages=600),
    # 144 KiB pieces (a 128 KiB unit does not tile them)
    "mla_small": WORKLOADS["mla_fp8"].scaled(name="mla_small", num_pages=200, num_layers=3),
    # 128 KiB pieces (runs take as many units as pieces: not used)
    "llama_small": WORKLOADS["llama8b"].scaled(name="llama_small", num_pages=96, num_layers=2),
    # one token per page: 2 KiB pieces, half a 4 KiB round
    "token_pages": Workload(name="token_pages", outer=("layer", "kv", "page"), inner="NHD",
                            num_pages=4096, num_layers=2, num_kv=2, page_size=1, num_heads=8,
                            head_dim=128, dtype_bytes=2, pages_per_request=1000, seed=211,
                            byte_offset=4096, alloc_tail=4096),
    # 240-byte pieces, pages adjacent, the pool at a byte offset
    "ragged_nhd": Workload(name="ragged_runs", outer=("kv", "layer", "page"), inner="NHD",
                           num_pages=1200, num_layers=2, num_kv=2, page_size=5, num_heads=3,
                           head_dim=8, dtype_bytes=2, pages_per_request=500, seed=212,
                           byte_offset=8192, alloc_tail=1008),
}


def diff_report(got, want, limit=8):
    bad = np.flatnonzero(got != want)
    return f"{bad.size} bytes differ; first at {bad[:limit].tolist()}"


def page_lists(w, kind, n, seed):
    """(source pages, destination pages), disjoint: `contiguous` = two
    ascending ranges; `mixed` = ascending stretches of 1 to 40 pages at
    random places; `pairs` = stretches of exactly two pages (more runs than
    one launch carries for large n)."""
    rng = np.random.default_rng(seed)
    if kind == "contiguous":
        a = int(rng.integers(0, w.num_pages - 2 * n + 1))
        return np.arange(a, a + n, dtype=np.int32), np.arange(a + n, a + 2 * n, dtype=np.int32)
    used = np.zeros(w.num_pages, dtype=bool)
    out = []
    while sum(len(b) for b in out) < 2 * n:
        ln = 2 if kind == "pairs" else int(rng.integers(1, 41))
        ln = min(ln, 2 * n - sum(len(b) for b in out))
        start = int(rng.integers(0, w.num_pages - ln + 1))
        if used[start:start + ln].any():
            continue
        used[start:start + ln] = True
        out.append(np.arange(start, start + ln, dtype=np.int32))
    ids = np.concatenate(out)
    return ids[:n].copy(), ids[n:2 * n].copy()


CASES = [("tiny", "contiguous", 64), ("tiny", "mixed", 200), ("mla_small", "contiguous", 40),
         ("mla_small", "mixed", 60), ("llama_small", "contiguous", 30), ("token_pages", "contiguous", 1000),
         ("token_pages", "pairs", 1000), ("token_pages", "mixed", 900), ("ragged_nhd", "mixed", 500)]


@pytest.fixture(scope="module")
def stream():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    K.lib()
    return t.cuda.Stream()


@pytest.mark.parametrize("path", ["device", "zerocopy"])
@pytest.mark.parametrize("pool,kind,n", CASES)
def test_runs_move_the_oracle_bytes(pool, kind, n, path, stream):
    """BACKUP of the source list and a publishing RESTORE into the
    destination list over two layer ranges, with coalescing on and off: the
    packed buffers, the allocations and the published counts are equal to
    each other and to the oracle's."""
    w = POOLS[pool]
    L = oracle_layout(w)
    src, dst = page_lists(w, kind, n, seed=w.seed + n)
    nb = w.host_bytes(n)
    print(f"\n[runs] pool={pool} kind={kind} n={n} path={path}", flush=True)
    results = {}
    old = K.kvx_get_option(K.KVX_OPT_COALESCE_RUNS)
    try:
        for coalesce in (1, 0):
            K.kvx_set_option(K.KVX_OPT_COALESCE_RUNS, coalesce)
            p = DevicePool(w, seed=361, generation=4)
            img = p.host_image()
            ready = K.kvx_ready_create(w.num_layers, 4)
            pk = Packed(w, n, path, fill_seed=970)
            try:
                ranges = [(0, w.num_layers), (1, w.num_layers)] if w.num_layers > 1 else [(0, 1)]
                want_alloc, counts = img, [0] * w.num_layers
                for l0, l1 in ranges:
                    want_pk = oracle.backup(L, want_alloc, src, l0, l1, host=pk.numpy())
                    K.kvx_backup(p.handle, src, pk.ptr, nb, l0, l1, stream, PATHS[path])
                    K.kvx_sync(stream)
                    got = pk.numpy()
                    assert np.array_equal(got, want_pk), f"backup {l0}:{l1} " + diff_report(got, want_pk)
                    want_alloc = oracle.restore(L, want_alloc, got, dst, l0, l1)
                    counts = oracle.ready_publish(counts, 0, l0, l1, n)
                    K.kvx_restore(p.handle, pk.ptr, nb, dst, l0, l1, ready, 0, stream, PATHS[path])
                    K.kvx_sync(stream)
                    after = p.host_image()
                    assert np.array_equal(after, want_alloc), f"restore {l0}:{l1} " + diff_report(after, want_alloc)
                    assert [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)] == counts
                results[coalesce] = (pk.numpy(), p.host_image())
            finally:
                K.kvx_ready_destroy(ready)
                pk.close()
                p.close()
    finally:
        K.kvx_set_option(K.KVX_OPT_COALESCE_RUNS, old)
    assert np.array_equal(results[0][0], results[1][0])
    assert np.array_equal(results[0][1], results[1][1])


@pytest.mark.parametrize("path", ["device", "zerocopy"])
def test_runs_into_a_slot_addressed_host_pool(path, stream):
    """Consecutive pages into consecutive host slots of a slot-addressed pool
    (runs), then back into other pages from those slots."""
    w = POOLS["tiny"]
    L = oracle_layout(w)
    S, n = 300, 96
    src, dst = page_lists(w, "mixed", n, seed=77)
    slots = np.concatenate([np.arange(10, 10 + n // 2), np.arange(200, 200 + n - n // 2)]).astype(np.int32)
    p = DevicePool(w, seed=362, generation=4)
    img = p.host_image()
    hp = Packed(w, S, path, fill_seed=971)
    try:
        want_host = oracle.backup_slots(L, img, src, slots, S, 0, w.num_layers, host=hp.numpy())
        K.kvx_backup_slots(p.handle, src, slots, hp.ptr, hp.nbytes, S, 0, w.num_layers, stream, PATHS[path])
        K.kvx_sync(stream)
        got = hp.numpy()
        assert np.array_equal(got, want_host), diff_report(got, want_host)
        want = oracle.restore_slots(L, img, got, slots, dst, S, 0, w.num_layers)
        K.kvx_restore_slots(p.handle, hp.ptr, hp.nbytes, S, slots, dst, 0, w.num_layers, None, 0, stream,
                            PATHS[path])
        K.kvx_sync(stream)
        after = p.host_image()
        assert np.array_equal(after, want), diff_report(after, want)
    finally:
        hp.close()
        p.close()
