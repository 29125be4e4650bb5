"""GPU parity of per-layer publish and the ready prefix when one ready object
serves several pools and several restores ([TICKET] "PP Prefetch Ticket
Path" diagram: KV and sidecars publish progress layer by layer, and the
minimum over all of it is the globally safe prefix).

- Sidecars: a main pool and a sidecar pool of another geometry (head-major,
  at a byte offset, other layer count) are restored with the same
  destination page IDs, round after round, into one ready object with no
  reset between rounds. A host thread observes the counts and the prefix
  while the kernels publish; a GPU consumer waits on every slot of both
  pools and copies both allocations out; every copy, and both allocations
  at the end, match the oracle byte for byte.
- Back-to-back restores into the same slots: a consumer that waits for the
  second restore's count reads the second restore's bytes, never the first's.
"""
import threading

import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import WORKLOADS
from tests.gpu_util import PATHS, DevicePool, Packed, oracle_layout, torch

pytestmark = pytest.mark.gpu

MAIN = (WORKLOADS["mla_fp8"].scaled(name="mla_small", num_pages=40, num_layers=5), 10)
# head-major, page-major outer order, byte offset 12288, its own layer count
SIDE = WORKLOADS["trtllm_hnd"].scaled(name="side_hnd", num_pages=40, num_layers=2)

SPIN = 20_000_000


def diff_report(got, want, limit=8):
    bad = np.flatnonzero(got != want)
    return f"{bad.size} bytes differ; first at {bad[:limit].tolist()}"


class Observer(threading.Thread):
    """Reads the counts, then the prefix, then the counts again, until told
    to stop. Counts only grow, so at every observation the prefix lies
    between the oracle's prefix of the snapshot before it and that of the
    snapshot after it, and it never decreases."""

    def __init__(self, ready, num_slots):
        super().__init__(daemon=True)
        self.ready, self.num_slots = ready, num_slots
        self.stop = threading.Event()
        self.errors, self.seen = [], set()
        self.observations = 0

    def run(self):
        last = 0
        while not self.stop.is_set() and len(self.errors) < 5:
            before = [K.kvx_layer_ready(self.ready, s) for s in range(self.num_slots)]
            p = K.kvx_ready_prefix(self.ready)
            after = [K.kvx_layer_ready(self.ready, s) for s in range(self.num_slots)]
            lo, hi = oracle.ready_prefix(before), oracle.ready_prefix(after)
            if not lo <= p <= hi:
                self.errors.append(f"prefix {p} outside [{lo}, {hi}]: {before} / {after}")
            if p < last:
                self.errors.append(f"prefix went back from {last} to {p}")
            if any(b > a for b, a in zip(before, after)):
                self.errors.append(f"a count went back: {before} -> {after}")
            last = p
            self.seen.add(tuple(after))
            self.observations += 1


@pytest.mark.parametrize("path", ["zerocopy", "staged"])
def test_sidecar_pool_and_main_pool_publish_one_safe_prefix(path):
    """Main pool slots [0, NL), sidecar slots [NL, NL + NL_side) of one ready
    object; the two restores run on two streams (disjoint slots), round
    after round without a reset, so each round's target is the pages of
    all rounds so far."""
    t = torch()
    (w, n), ws = MAIN, SIDE
    rounds = 4
    Lm, Ls = oracle_layout(w), oracle_layout(ws)
    main = DevicePool(w, seed=331, generation=7)
    side = DevicePool(ws, seed=332, generation=7)
    want_main, want_side = main.host_image(), side.host_image()
    dst = synth.page_perm(w.seed + 40, w.num_pages)[:n].copy()
    slots = w.num_layers + ws.num_layers
    ready = K.kvx_ready_create(slots, 7)
    s_main, s_side, consumer = t.cuda.Stream(), t.cuda.Stream(), t.cuda.Stream()
    status = t.zeros(slots, dtype=t.int32, device="cuda")
    P = PATHS[path]
    pks = []
    obs = Observer(ready, slots)
    counts = [0] * slots
    print(f"\n[sidecar] path={path} rounds={rounds} n={n} slots={slots}", flush=True)
    try:
        obs.start()
        for r in range(rounds):
            pm = Packed(w, n, path, fill_seed=500 + r)
            ps = Packed(ws, n, path, fill_seed=600 + r)
            pks += [pm, ps]
            t.cuda.synchronize()
            want_main = oracle.restore(Lm, want_main, synth.gen_bytes(500 + r, 0, pm.nbytes), dst, 0,
                                       w.num_layers)
            want_side = oracle.restore(Ls, want_side, synth.gen_bytes(600 + r, 0, ps.nbytes), dst, 0,
                                       ws.num_layers)
            counts = oracle.ready_publish(counts, 0, 0, w.num_layers, n)
            counts = oracle.ready_publish(counts, w.num_layers, 0, ws.num_layers, n)
            target = oracle.ready_prefix(counts)
            assert target == (r + 1) * n
            # producers first, then the consumer's waits (streams share
            # hardware queues, which run their kernels in order)
            K.kvx_restore(main.handle, pm.ptr, pm.nbytes, dst, 0, w.num_layers, ready, 0, s_main, P)
            K.kvx_restore(side.handle, ps.ptr, ps.nbytes, dst, 0, ws.num_layers, ready, w.num_layers,
                          s_side, P)
            with t.cuda.stream(consumer):
                status.zero_()
            for s in range(slots):
                K.kvx_ready_wait_gpu(ready, s, target, consumer, SPIN, status.data_ptr() + 4 * s)
            with t.cuda.stream(consumer):
                got_main, got_side = main.alloc.clone(), side.alloc.clone()
            consumer.synchronize()
            assert status.cpu().tolist() == [1] * slots, "the consumer gave up waiting"
            gm, gs = got_main.cpu().numpy(), got_side.cpu().numpy()
            assert np.array_equal(gm, want_main), f"round {r} main: " + diff_report(gm, want_main)
            assert np.array_equal(gs, want_side), f"round {r} sidecar: " + diff_report(gs, want_side)
            K.kvx_sync(s_main)
            K.kvx_sync(s_side)
            assert [K.kvx_layer_ready(ready, s) for s in range(slots)] == counts
            assert K.kvx_ready_prefix(ready) == oracle.ready_prefix(counts)
        obs.stop.set()
        obs.join(10)
        print(f"[sidecar] {obs.observations} observations, {len(obs.seen)} distinct count vectors",
              flush=True)
        assert not obs.errors, obs.errors
        assert np.array_equal(main.host_image(), want_main)
        assert np.array_equal(side.host_image(), want_side)
    finally:
        obs.stop.set()
        obs.join(10)
        K.kvx_ready_destroy(ready)
        for pk in pks:
            pk.close()
        main.close()
        side.close()


@pytest.mark.parametrize("path", list(PATHS))
def test_consumer_of_the_second_restore_reads_its_bytes(path):
    """Two restores of different bytes into the same pages and the same
    slots, back to back on one stream with no host reset or wait: a
    consumer stream that waits for the second restore's count of each
    layer (2n) and copies that layer out gets the second restore's bytes."""
    t = torch()
    w, n = MAIN
    L = oracle_layout(w)
    pool = DevicePool(w, seed=333, generation=8)
    img = pool.host_image()
    dst = synth.page_perm(w.seed + 41, w.num_pages)[:n].copy()
    ready = K.kvx_ready_create(w.num_layers, 8)
    producer, consumer = t.cuda.Stream(), t.cuda.Stream()
    status = t.zeros(w.num_layers, dtype=t.int32, device="cuda")
    first = Packed(w, n, path, fill_seed=700)
    second = Packed(w, n, path, fill_seed=701)
    out = Packed(w, n, "device")
    P = PATHS[path]
    print(f"\n[second-restore] path={path} n={n}", flush=True)
    try:
        t.cuda.synchronize()
        K.kvx_restore(pool.handle, first.ptr, first.nbytes, dst, 0, w.num_layers, ready, 0, producer, P)
        K.kvx_restore(pool.handle, second.ptr, second.nbytes, dst, 0, w.num_layers, ready, 0, producer, P)
        counts = oracle.ready_publish(oracle.ready_publish([0] * w.num_layers, 0, 0, w.num_layers, n),
                                      0, 0, w.num_layers, n)
        for l in range(w.num_layers):
            K.kvx_ready_wait_gpu(ready, l, counts[l], consumer, SPIN, status.data_ptr() + 4 * l)
            K.kvx_backup(pool.handle, dst, out.ptr, out.nbytes, l, l + 1, consumer, K.KVX_PATH_DEVICE)
        K.kvx_sync(consumer)
        assert status.cpu().tolist() == [1] * w.num_layers
        after_first = oracle.restore(L, img, synth.gen_bytes(700, 0, first.nbytes), dst, 0, w.num_layers)
        after_second = oracle.restore(L, after_first, synth.gen_bytes(701, 0, second.nbytes), dst, 0,
                                      w.num_layers)
        want = oracle.backup(L, after_second, dst, 0, w.num_layers)
        got = out.numpy()
        assert np.array_equal(got, want), diff_report(got, want)
        K.kvx_sync(producer)
        assert [K.kvx_layer_ready(ready, s) for s in range(w.num_layers)] == counts
        assert np.array_equal(pool.host_image(), after_second)
    finally:
        K.kvx_ready_destroy(ready)
        for b in (first, second, out):
            b.close()
        pool.close()
