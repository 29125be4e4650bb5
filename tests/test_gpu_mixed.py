"""GPU parity for the mixed hit/miss stream on the 64 GiB pool: 128 requests of
256 pages alternating BACKUP (miss) and RESTORE (hit), four in flight on
four streams, for both host paths.

The timed run's final state is checked in full (the four rotating backup
slots and the whole allocation) against the oracle's closed forms; an
untimed replay of the same seeded schedule, one request at a time, checks a
random sample of pieces of every request as it completes."""
import os
import time

import numpy as np
import pytest

import oracle
import synth
from paged_kv_offload_amd import kvx as K
from synth.workloads import WORKLOADS, mixed_schedule
from tests.gpu_util import PATHS, DevicePool, oracle_layout, torch
from tests.test_gpu_full import check_alloc, check_packed

pytestmark = pytest.mark.gpu

NREQ = 128
NSTREAMS = 4
PRIMED = 4
ROTATING = 4
SAMPLE_PIECES = 48


def build_plan(w):
    """(kind, page ids, host slot, src pages of the bytes it moves) per
    request. Primed slot r holds the backup of prime request r."""
    perm = synth.page_perm(w.seed, w.num_pages)
    resident = perm[:w.num_pages // 2]
    prime = [np.ascontiguousarray(resident[256 * r:256 * (r + 1)]) for r in range(PRIMED)]
    plan = []
    nb = 0
    nr = 0
    for kind, ids in mixed_schedule(w, NREQ):
        if kind == "backup":
            plan.append(("backup", ids, PRIMED + nb % ROTATING, ids))
            nb += 1
        else:
            slot = nr % PRIMED
            plan.append(("restore", ids, slot, prime[slot]))
            nr += 1
    return prime, plan


def piece_bytes_of(pool, w, page, layer, kv):
    # the pool tensor is [NL][KV][NB][T][H][D]
    return pool.tensor[layer, kv, page].contiguous().view(-1).view(torch().uint8).cpu().numpy()


@pytest.mark.parametrize("path", ["zerocopy", "staged", "exchange"])
def test_mixed_stream(path):
    t = torch()
    w = WORKLOADS["mixed"]
    L = oracle_layout(w)
    P = w.payload_bytes()
    print(f"\n[mixed] {path}: pool {w.pool_bytes / 2**30:.0f} GiB, {NREQ} requests, "
          f"{NSTREAMS} streams", flush=True)
    pool = DevicePool(w, generation=7)
    slots = [K.HostBuffer(P) for _ in range(PRIMED + ROTATING)]
    streams = [t.cuda.Stream() for _ in range(NSTREAMS)]
    prime, plan = build_plan(w)
    try:
        # prime the host slots that restores read (untimed), and check them
        for r in range(PRIMED):
            K.kvx_backup(pool.handle, prime[r], slots[r].ptr, P, 0, w.num_layers, streams[0],
                         K.KVX_PATH_STAGED)
        K.kvx_sync(streams[0])
        for r in range(PRIMED):
            bad, first = check_packed(w, L, w.seed, prime[r], 0, w.num_layers, slots[r].numpy())
            assert bad == 0, f"primed slot {r} differs at {first}"

        # the timed run: request k on stream k mod 4 (buffer reuse stays on
        # one stream: rotating slots every 8 requests, destination sets every 32)
        t.cuda.synchronize()
        t0 = time.perf_counter()
        if path == "exchange":
            # backup k and restore k + 1 as one kvx_exchange, pairs on two streams
            for i in range(0, len(plan), 2):
                (kb, ib, sb, _), (kr, ir, sr, _) = plan[i], plan[i + 1]
                assert kb == "backup" and kr == "restore"
                K.kvx_exchange(pool.handle, ib, slots[sb].ptr, P, (0, w.num_layers), slots[sr].ptr, P,
                               ir, (0, w.num_layers), None, 0, streams[(i // 2) % 2],
                               K.KVX_PATH_ZEROCOPY)
        else:
            for k, (kind, ids, slot, _) in enumerate(plan):
                s = streams[k % NSTREAMS]
                if kind == "backup":
                    K.kvx_backup(pool.handle, ids, slots[slot].ptr, P, 0, w.num_layers, s, PATHS[path])
                else:
                    K.kvx_restore(pool.handle, slots[slot].ptr, P, ids, 0, w.num_layers, None, 0, s,
                                  PATHS[path])
        for s in streams:
            K.kvx_sync(s)
        wall = time.perf_counter() - t0
        print(f"[mixed] {path}: {NREQ * P / wall / 1e9:.1f} GB/s aggregate "
              f"({wall * 1e3:.0f} ms for {NREQ * P / 1e9:.0f} GB)", flush=True)

        # final state: the last backup into each rotating slot ...
        last = {}
        for kind, ids, slot, src in plan:
            if kind == "backup":
                last[slot] = ids
        for slot, ids in last.items():
            bad, first = check_packed(w, L, w.seed, ids, 0, w.num_layers, slots[slot].numpy())
            assert bad == 0, f"rotating slot {slot} differs at {first}"
        # ... and every destination set holds its last restore's bytes
        dst_last = {}
        for kind, ids, slot, src in plan:
            if kind == "restore":
                dst_last[tuple(ids.tolist())] = src
        srcs = np.concatenate([v for v in dst_last.values()])
        dsts = np.concatenate([np.array(k, dtype=np.int32) for k in dst_last.keys()])
        t1 = time.time()
        bad, first = check_alloc(w, L, w.seed, srcs, dsts, 0, w.num_layers, pool.alloc)
        print(f"[mixed] whole 64 GiB allocation checked in {time.time() - t1:.1f} s", flush=True)
        assert bad == 0, f"allocation: {bad} bytes differ, first at {first}"

        # untimed replay, one request at a time, sampled check of each
        if path == "exchange":
            path = "zerocopy"
        rng = np.random.default_rng(99)
        s = streams[0]
        for k, (kind, ids, slot, src) in enumerate(plan[:32]):
            if kind == "backup":
                K.kvx_backup(pool.handle, ids, slots[slot].ptr, P, 0, w.num_layers, s, PATHS[path])
                K.kvx_sync(s)
                host = slots[slot].numpy()
                for _ in range(SAMPLE_PIECES):
                    l, c, i = rng.integers(w.num_layers), rng.integers(w.num_kv), rng.integers(256)
                    off = ((l * w.num_kv + c) * 256 + i) * w.piece_bytes
                    bad, first = oracle.check_backup_gen(L, w.seed, ids, 0, w.num_layers,
                                                         host[off:off + w.piece_bytes], off)
                    assert bad == 0, f"replay request {k}: packed offset {first}"
            else:
                K.kvx_restore(pool.handle, slots[slot].ptr, P, ids, 0, w.num_layers, None, 0, s,
                              PATHS[path])
                K.kvx_sync(s)
                for _ in range(SAMPLE_PIECES):
                    l, c, i = rng.integers(w.num_layers), rng.integers(w.num_kv), rng.integers(256)
                    got = piece_bytes_of(pool, w, int(ids[i]), int(l), int(c))
                    a = oracle.piece_start(L, int(ids[i]), int(l), int(c))
                    bad, first = oracle.check_alloc_roundtrip(L, w.seed, w.seed + 1, src, ids, 0,
                                                              w.num_layers, got, a)
                    assert bad == 0, f"replay request {k}: allocation byte {first}"
    finally:
        for h in slots:
            h.free()
        pool.close()
