"""kvx_restore_noalloc, the restore entry point that allocates nothing (its
per-layer counters and unit queue live in a static device scratch), against
kvx_restore on twin pools: two calls in a row on one stream, the second
with fewer pages and fewer layers, no host synchronisation between them.
Both pools, both ready objects and the oracle agree byte for byte."""
import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import WORKLOADS, Workload
from tests.gpu_util import PATHS, DevicePool, Packed, oracle_layout, torch

pytestmark = pytest.mark.gpu

CASES = {
    # 128 KiB NHD pieces (one unit each)
    "llama_small": (WORKLOADS["llama8b"].scaled(name="llama_small", num_pages=96, num_layers=3), 24, 9),
    # head-major through LDS token blocks, pool at a byte offset
    "trtllm_small": (WORKLOADS["trtllm_hnd"].scaled(name="trtllm_small", num_pages=64, num_layers=3), 16, 5),
    # 144 KiB pieces (a 128 KiB unit and a 16 KiB partial one)
    "mla_small": (WORKLOADS["mla_fp8"].scaled(name="mla_small", num_pages=40, num_layers=5), 10, 3),
    # 240-byte head-major pieces, more pages than one launch carries
    "ragged_hnd": (Workload(name="ragged_hnd", outer=("page", "kv", "layer"), inner="HND",
                            num_pages=1200, num_layers=3, num_kv=2, page_size=5, num_heads=3,
                            head_dim=8, dtype_bytes=2, pages_per_request=500, seed=201,
                            byte_offset=4096, alloc_tail=1008), 500, 130),
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


@pytest.mark.parametrize("publish", [True, False])
@pytest.mark.parametrize("path", ["zerocopy", "device"])
@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_restore_equals_restore(case, path, publish, stream):
    w, n1, n2 = CASES[case]
    L = oracle_layout(w)
    print(f"\n[noalloc] case={case} path={path} publish={publish} n1={n1} n2={n2}", flush=True)
    a = DevicePool(w, seed=341, generation=5)
    b = DevicePool(w, seed=341, generation=5)
    img = a.host_image()
    assert np.array_equal(img, b.host_image())
    perm = synth.page_perm(w.seed + 50, w.num_pages)
    calls = [(perm[:n1].copy(), 0, w.num_layers, 800), (perm[n1:n1 + n2].copy(), 1, w.num_layers, 801)]
    ra = K.kvx_ready_create(w.num_layers + 2, 5) if publish else None
    rb = K.kvx_ready_create(w.num_layers + 2, 5) if publish else None
    bufs = []
    try:
        want = img
        counts = [0] * (w.num_layers + 2)
        for dst, l0, l1, seed in calls:
            pk = Packed(w, dst.size, path, fill_seed=seed)
            bufs.append(pk)
            want = oracle.restore(L, want, synth.gen_bytes(seed, 0, pk.nbytes), dst, l0, l1)
            counts = oracle.ready_publish(counts, 1, l0, l1, dst.size)
        torch().cuda.synchronize()
        for (dst, l0, l1, _), pk in zip(calls, bufs):
            K.kvx_restore(a.handle, pk.ptr, pk.nbytes, dst, l0, l1, ra, 1, stream, PATHS[path])
            K.kvx_restore_noalloc(b.handle, pk.ptr, pk.nbytes, dst, l0, l1, rb, 1, stream, PATHS[path])
        K.kvx_sync(stream)
        got_a, got_b = a.host_image(), b.host_image()
        assert np.array_equal(got_b, got_a), "noalloc vs restore: " + diff_report(got_b, got_a)
        assert np.array_equal(got_b, want), "noalloc vs oracle: " + diff_report(got_b, want)
        if publish:
            ca = [K.kvx_layer_ready(ra, s) for s in range(w.num_layers + 2)]
            cb = [K.kvx_layer_ready(rb, s) for s in range(w.num_layers + 2)]
            assert cb == ca == counts
    finally:
        for r in (ra, rb):
            if r:
                K.kvx_ready_destroy(r)
        for pk in bufs:
            pk.close()
        a.close()
        b.close()


def test_noalloc_restore_refuses_what_it_cannot_serve(stream):
    """The staged path (it needs the staging ring) and a pool of more layers
    than the scratch counts are refused before anything is enqueued."""
    w, n, _ = CASES["llama_small"]
    pool = DevicePool(w, seed=342, generation=5)
    img = pool.host_image()
    dst = synth.page_perm(w.seed + 51, w.num_pages)[:n].copy()
    pk = Packed(w, n, "zerocopy", fill_seed=802)
    deep = Workload(name="deep", outer=("layer", "kv", "page"), inner="NHD", num_pages=2,
                    num_layers=K.KVX_NOALLOC_MAX_LAYERS + 1, num_kv=1, page_size=1, num_heads=1,
                    head_dim=8, dtype_bytes=2, pages_per_request=1, seed=209)
    dpool = DevicePool(deep, seed=343, generation=5)
    dpk = Packed(deep, 1, "zerocopy", fill_seed=803)
    try:
        with pytest.raises(K.KvxError) as e:
            K.kvx_restore_noalloc(pool.handle, pk.ptr, pk.nbytes, dst, 0, w.num_layers, None, 0, stream,
                                  K.KVX_PATH_STAGED)
        assert e.value.code == K.KVX_E_INVAL, e.value.message
        with pytest.raises(K.KvxError) as e:
            K.kvx_restore_noalloc(dpool.handle, dpk.ptr, dpk.nbytes, [1], 0, deep.num_layers, None, 0,
                                  stream, K.KVX_PATH_ZEROCOPY)
        assert e.value.code == K.KVX_E_RANGE, e.value.message
        K.kvx_sync(stream)
        assert np.array_equal(pool.host_image(), img)
    finally:
        pk.close()
        dpk.close()
        pool.close()
        dpool.close()
