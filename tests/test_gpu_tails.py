"""Tail units: pieces that 128 KiB work units do not tile (the MLA pool's
144 KiB pieces) end in a tail, and the tails of several pieces share a unit
(one to eight per wave) instead of each piece ending in a mostly idle
partial unit; pieces no longer than a wave's share of a unit (32 KiB in
device memory, 2 KiB over the host link's 8 KiB units) travel whole, several
to a unit. Bytes and published counts must be the oracle's, and the
same with tail units switched off, for every tail size class, tails that are
not a whole number of 1 KiB rounds, more pages than one launch carries, a
last tail unit only partly filled, and every path (the staged path's
publishing chunks keep partial units)."""
import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import Workload
from tests.gpu_util import PATHS, DevicePool, Packed, oracle_layout, torch

pytestmark = pytest.mark.gpu


def pool(tokens, row_elems, eb=1, pages=1100, seed=221):
    """A layer-major NHD pool of one head whose piece is tokens x row bytes."""
    return Workload(name=f"tails_{tokens}x{row_elems}", outer=("layer", "kv", "page"), inner="NHD",
                    num_pages=pages, num_layers=2, num_kv=2, page_size=tokens, num_heads=1,
                    head_dim=row_elems, dtype_bytes=eb, pages_per_request=500, seed=seed,
                    byte_offset=4096, alloc_tail=2048)


# piece bytes -> tail after one 128 KiB unit (tails per wave)
CASES = {
    "tail2k": pool(130, 1024),       # 2 KiB tail (8 a wave)
    "tail8k": pool(136, 1024),       # 8 KiB (4 a wave)
    "tail16k": pool(144, 1024),      # 16 KiB, the MLA pool's (2 a wave)
    "tail24k": pool(152, 1024),      # 24 KiB (1 a wave)
    "tail1_5k": pool(224, 592),      # 132,608 B: a 1.5 KiB tail, half a round in its last
    "two_units": pool(272, 1024),    # 272 KiB: two whole units and a 16 KiB tail
    # pieces no longer than a wave's share of a unit are all tail: device
    # memory packs 32 KiB or less (1 to 8 a wave), the host link 2 KiB or less
    "whole240": pool(5, 48),         # 240 B: 8 a wave; host 2 a wave, a fraction of a round each
    "whole1k": pool(1, 1024),        # 1 KiB: 8 a wave, one round of four used; host 2 a wave
    "whole2k": pool(2, 1024),        # 2 KiB, a one-token bf16 page of 8 heads: 8 a wave; host 1
    "whole4k": pool(4, 1024),        # 4 KiB: 8 a wave, every round used; host: a unit each
    "whole6k": pool(6, 1024),        # 6 KiB: 4 a wave
    "whole20k": pool(20, 1024),      # 20 KiB: 1 a wave
    "whole32k": pool(32, 1024),      # 32 KiB: 1 a wave, the largest
}


def diff_report(got, want, limit=8):
    bad = np.flatnonzero(got != want)
    return f"{bad.size} bytes differ; first at {bad[:limit].tolist()}"


@pytest.fixture(scope="module")
def stream():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    K.lib()
    return t.cuda.Stream()


@pytest.mark.parametrize("n,path", [(500, "device"), (500, "zerocopy"), (37, "device"), (37, "zerocopy"),
                                    (37, "staged")])
@pytest.mark.parametrize("case", list(CASES))
def test_tail_units_move_the_oracle_bytes(case, n, path, stream):
    w = CASES[case]
    L = oracle_layout(w)
    perm = synth.page_perm(w.seed + n, w.num_pages)
    src, dst = perm[:n].copy(), perm[n:2 * n].copy()
    nb = w.host_bytes(n)
    print(f"\n[tails] case={case} piece={w.piece_bytes} n={n} path={path}", flush=True)
    results = {}
    old = K.kvx_get_option(K.KVX_OPT_TAIL_UNITS)
    try:
        for tails in (1, 0):
            K.kvx_set_option(K.KVX_OPT_TAIL_UNITS, tails)
            p = DevicePool(w, seed=371, generation=3)
            img = p.host_image()
            ready = K.kvx_ready_create(w.num_layers, 3)
            pk = Packed(w, n, path, fill_seed=980)
            try:
                want_pk = oracle.backup(L, img, src, 0, w.num_layers, host=pk.numpy())
                K.kvx_backup(p.handle, src, pk.ptr, nb, 0, w.num_layers, stream, PATHS[path])
                K.kvx_sync(stream)
                got = pk.numpy()
                assert np.array_equal(got, want_pk), "backup " + diff_report(got, want_pk)
                want = oracle.restore(L, img, got, dst, 0, w.num_layers)
                K.kvx_restore(p.handle, pk.ptr, nb, dst, 0, w.num_layers, ready, 0, stream, PATHS[path])
                K.kvx_restore(p.handle, pk.ptr, nb, dst, 1, w.num_layers, ready, 0, stream, PATHS[path])
                K.kvx_sync(stream)
                after = p.host_image()
                assert np.array_equal(after, want), "restore " + diff_report(after, want)
                counts = oracle.ready_publish(oracle.ready_publish([0] * w.num_layers, 0, 0, w.num_layers, n),
                                              0, 1, w.num_layers, n)
                assert [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)] == counts
                # a plain restore too (short pieces travel whole by another
                # rule without publish), the slots into the pages reversed
                rdst = dst[::-1].copy()
                want2 = oracle.restore(L, want, got, rdst, 0, w.num_layers)
                K.kvx_restore(p.handle, pk.ptr, nb, rdst, 0, w.num_layers, None, 0, stream, PATHS[path])
                K.kvx_sync(stream)
                after2 = p.host_image()
                assert np.array_equal(after2, want2), "plain restore " + diff_report(after2, want2)
                results[tails] = (got, after, after2)
            finally:
                K.kvx_ready_destroy(ready)
                pk.close()
                p.close()
    finally:
        K.kvx_set_option(K.KVX_OPT_TAIL_UNITS, old)
    for k in range(3):
        assert np.array_equal(results[0][k], results[1][k])
