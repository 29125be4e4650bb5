"""Backups and restores queued on streams of their own, both directions of
the host link in flight at once, so the host-link grid takes its
direction-aware shares (a kernel that writes host memory beside one that
reads it, beside staged copies of the other direction, and beside calls of
its own direction only): every backup gives the oracle's packed bytes and
every destination set ends up with its last restore's bytes, the rest of
the allocation untouched."""
import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from tests.gpu_util import PATHS, DevicePool, Packed, oracle_layout, torch
from tests.test_gpu_parity import SMALL, diff_report

pytestmark = pytest.mark.gpu

REQUESTS = 8   # per direction


@pytest.mark.parametrize("bpath,rpath", [("zerocopy", "zerocopy"), ("zerocopy", "staged"),
                                         ("staged", "zerocopy")])
@pytest.mark.parametrize("streams_per_direction", [1, 2])
@pytest.mark.parametrize("case", ["llama_small", "mla_small", "ragged_hnd"])
def test_both_directions_on_streams_of_their_own(case, streams_per_direction, bpath, rpath):
    t = torch()
    w, _ = SMALL[case]
    n = min(w.num_pages // 6, 64)
    print(f"\n[duplex] case={case} streams/direction={streams_per_direction} backups={bpath} "
          f"restores={rpath} n={n}", flush=True)
    L = oracle_layout(w)
    pool = DevicePool(w, seed=w.seed + 70, generation=5)
    img = pool.host_image()
    perm = synth.page_perm(w.seed + 71, w.num_pages)
    srcs = [perm[(r % 2) * n:(r % 2 + 1) * n].copy() for r in range(REQUESTS)]   # never written
    dst_sets = [perm[(2 + k) * n:(3 + k) * n].copy() for k in range(streams_per_direction)]
    nb = w.host_bytes(n)
    bstreams = [t.cuda.Stream() for _ in range(streams_per_direction)]
    rstreams = [t.cuda.Stream() for _ in range(streams_per_direction)]
    ready = K.kvx_ready_create(streams_per_direction * w.num_layers, 5)
    backups = [Packed(w, n, bpath, fill_seed=3000 + r) for r in range(REQUESTS)]
    restores = [Packed(w, n, rpath, fill_seed=4000 + r) for r in range(REQUESTS)]
    try:
        # interleaved as a scheduler would issue them; a destination set and
        # its restores stay on one stream
        for r in range(REQUESTS):
            k = r % streams_per_direction
            K.kvx_backup(pool.handle, srcs[r], backups[r].ptr, nb, 0, w.num_layers, bstreams[k],
                         PATHS[bpath])
            K.kvx_restore(pool.handle, restores[r].ptr, nb, dst_sets[k], 0, w.num_layers, ready,
                          k * w.num_layers, rstreams[k], PATHS[rpath])
        for s in bstreams + rstreams:
            K.kvx_sync(s)
        per_set = REQUESTS // streams_per_direction
        assert K.kvx_ready_prefix(ready) == per_set * n
        for r in range(REQUESTS):
            got = backups[r].numpy()
            want = oracle.backup(L, img, srcs[r], 0, w.num_layers)
            assert np.array_equal(got, want), f"backup {r}: " + diff_report(got, want)
        want_alloc = img
        for k in range(streams_per_direction):
            last = max(r for r in range(REQUESTS) if r % streams_per_direction == k)
            want_alloc = oracle.restore(L, want_alloc, synth.gen_bytes(4000 + last, 0, nb), dst_sets[k], 0,
                                        w.num_layers)
        after = pool.host_image()
        assert np.array_equal(after, want_alloc), "allocation: " + diff_report(after, want_alloc)
    finally:
        K.kvx_ready_destroy(ready)
        for b in backups + restores:
            b.close()
        pool.close()
