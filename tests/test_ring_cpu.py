"""Submission / completion rings between a scheduler process and a
data-plane process (CPU only): order, capacity and role checks, descriptors
carried intact between two processes, peer-death detection, one data-plane
side at a time, and the executor's refusals (wrong generation, unknown
pool or buffer, unknown operation), which complete at once without touching
the GPU."""
import os
import signal
import subprocess
import sys
import textwrap
import time

import pytest

import paged_kv_offload_amd as kvx
from paged_kv_offload_amd import kvx as K
from synth.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_BASE = 0x7F0000000000
_n = [0]


def ring_name():
    _n[0] += 1
    return f"/kvx-test-{os.getpid()}-{_n[0]}"


def code(fn):
    with pytest.raises(K.KvxError) as e:
        fn()
    return e.value.code


def test_fifo_capacity_roles_and_names():
    name = ring_name()
    r = K.kvx_ring_create(name, 4, 11)
    o = K.kvx_ring_open(name)
    try:
        for i in range(4):
            K.kvx_ring_submit(r, K.make_sqe(K.KVX_OP_BACKUP, 100 + i, 11, 0, 0, range(i), 0, 1))
        assert code(lambda: K.kvx_ring_submit(r, K.make_sqe(1, 9, 11, 0, 0, [], 0, 1))) == K.KVX_E_FULL
        assert K.kvx_ring_pending(o) == (4, 0)
        for i in range(4):
            q = K.kvx_ring_take(o)
            assert (q.op_id, q.n, list(q.page_ids[:q.n])) == (100 + i, i, list(range(i)))
            K.kvx_ring_complete(o, q.op_id, q.generation, -i)
        assert K.kvx_ring_take(o) is None
        assert code(lambda: K.kvx_ring_complete(o, 1, 1, 0)) == K.KVX_E_FULL
        assert K.kvx_ring_reap(r, 3) == [(100, 11, 0), (101, 11, -1), (102, 11, -2)]
        assert K.kvx_ring_reap(r, 8) == [(103, 11, -3)]
        # each side keeps to its role
        assert code(lambda: K.kvx_ring_take(r)) == K.KVX_E_INVAL
        assert code(lambda: K.kvx_ring_submit(o, K.make_sqe(1, 1, 1, 0, 0, [], 0, 1))) == K.KVX_E_INVAL
        assert code(lambda: K.kvx_ring_serve(r, [], [], [])) == K.KVX_E_INVAL
        # one data-plane side at a time
        assert code(lambda: K.kvx_ring_open(name)) == K.KVX_E_INVAL
        q = K.make_sqe(1, 1, 1, 0, 0, [], 0, 1)
        q.n = K.KVX_RING_MAX_PAGES + 1
        assert code(lambda: K.kvx_ring_submit(r, q)) == K.KVX_E_RANGE
        K.kvx_ring_submit(r, K.make_sqe(1, 5, 11, 0, 0, [1], 0, 1))
        K.kvx_ring_submit(r, K.make_sqe(1, 6, 11, 0, 0, [1], 0, 1))
        assert K.kvx_ring_discard(o) == 2 and K.kvx_ring_pending(r) == (0, 0)
    finally:
        K.kvx_ring_close(o)
        K.kvx_ring_close(r)
    assert not os.path.exists("/dev/shm" + name)
    assert code(lambda: K.kvx_ring_submit(r, K.make_sqe(1, 1, 1, 0, 0, [], 0, 1))) == K.KVX_E_STALE
    K.kvx_ring_close(r)                                   # logged, not an error
    for bad in ("noslash", "/a/b", "/", "/" + "x" * 70):
        assert code(lambda: K.kvx_ring_create(bad, 4, 1)) == K.KVX_E_INVAL
    for entries in (0, 1, 3, 6, 8192):
        assert code(lambda: K.kvx_ring_create(ring_name(), entries, 1)) == K.KVX_E_RANGE
    assert code(lambda: K.kvx_ring_open("/kvx-test-missing")) == K.KVX_E_INVAL
    name = ring_name()
    r = K.kvx_ring_create(name, 2, 1)
    assert code(lambda: K.kvx_ring_create(name, 2, 1)) == K.KVX_E_INVAL
    K.kvx_ring_close(r)


CHILD = textwrap.dedent("""
    import sys, time
    sys.path.insert(0, {root!r})
    from paged_kv_offload_amd import kvx as K
    o = K.kvx_ring_open({name!r})
    print("open", flush=True)
    done = 0
    while done < {count}:
        q = K.kvx_ring_take(o)
        if q is None:
            time.sleep(0.0005)
            continue
        # the status proves the descriptor arrived whole
        s = (sum(q.page_ids[:q.n]) + q.layer_begin * 7 + q.layer_end + q.pool) % 100000
        while True:
            try:
                K.kvx_ring_complete(o, q.op_id, q.generation, s)
                break
            except K.KvxError:
                time.sleep(0.0005)
        done += 1
    print("done", flush=True)
    if {linger}:
        time.sleep(60)
    K.kvx_ring_close(o)
""")


def spawn(name, count, linger=False):
    p = subprocess.Popen([sys.executable, "-c", CHILD.format(root=ROOT, name=name, count=count,
                                                             linger=linger)],
                         stdout=subprocess.PIPE, text=True)
    assert p.stdout.readline().strip() == "open"
    return p


def test_descriptors_cross_processes_in_order():
    """2000 descriptors through an 8-entry ring to another process; each
    completion carries a checksum of its descriptor, in submission order."""
    name = ring_name()
    r = K.kvx_ring_create(name, 8, 5)
    p = spawn(name, 2000)
    try:
        assert K.kvx_ring_peer_alive(r)
        sent, got = 0, []
        want = []
        deadline = time.time() + 60
        while len(got) < 2000 and time.time() < deadline:
            while sent < 2000:
                ids = [(sent * 31 + k) % 997 for k in range(sent % 50)]
                q = K.make_sqe(K.KVX_OP_RESTORE, 1000 + sent, 5, sent % 3, 0, ids, sent % 4,
                               sent % 4 + 2)
                try:
                    K.kvx_ring_submit(r, q)
                except K.KvxError as e:
                    assert e.code == K.KVX_E_FULL
                    break
                want.append((1000 + sent, 5, (sum(ids) + (sent % 4) * 7 + sent % 4 + 2 + sent % 3)
                             % 100000))
                sent += 1
            got += K.kvx_ring_reap(r, 16)
        assert got == want
        assert p.stdout.readline().strip() == "done"
        assert p.wait(30) == 0
    finally:
        if p.poll() is None:
            p.kill()
            p.wait()
        K.kvx_ring_close(r)


def test_peer_death_is_seen_and_frees_the_data_plane_seat():
    name = ring_name()
    r = K.kvx_ring_create(name, 4, 1)
    p = spawn(name, 0, linger=True)
    try:
        assert p.stdout.readline().strip() == "done"
        assert K.kvx_ring_peer_alive(r)
        assert code(lambda: K.kvx_ring_open(name)) == K.KVX_E_INVAL   # the child holds it
        p.send_signal(signal.SIGKILL)
        deadline = time.time() + 10
        while K.kvx_ring_peer_alive(r) and time.time() < deadline:   # dead even before reaped
            time.sleep(0.01)
        assert not K.kvx_ring_peer_alive(r)
        p.wait(10)
        o = K.kvx_ring_open(name)                                     # the seat is free again
        assert K.kvx_ring_peer_alive(o) and K.kvx_ring_peer_alive(r)
        K.kvx_ring_close(o)
        assert not K.kvx_ring_peer_alive(r)
    finally:
        if p.poll() is None:
            p.kill()
            p.wait()
        K.kvx_ring_close(r)


def test_executor_refusals_complete_at_once():
    """Descriptors the executor refuses complete in submission order with
    their error, before any GPU call: another generation, a pool or buffer
    outside the tables, an offset past the buffer, an unknown operation, a
    publish with no ready object, and the call's own checks (an ID outside
    the pool)."""
    w = WORKLOADS["tiny"]
    shape = w.tensor_shape()
    st, acc = [], 1
    for d in reversed(shape):
        st.append(acc)
        acc *= d
    lay = kvx.make_layout(w.outer, w.inner, w.num_pages, w.num_layers, w.num_kv, w.page_size,
                          w.num_heads, w.head_dim)
    pool = K.kvx_register_pool(lay, FAKE_BASE, 0, w.dtype_bytes, shape, list(reversed(st)), 7)
    name = ring_name()
    r = K.kvx_ring_create(name, 16, 7)
    o = K.kvx_ring_open(name)
    nb = w.host_bytes(4)
    try:
        cases = [
            (dict(generation=6), K.KVX_E_STALE),
            (dict(pool=1), K.KVX_E_RANGE),
            (dict(buffer=2), K.KVX_E_RANGE),
            (dict(buffer_offset=nb + 16), K.KVX_E_RANGE),
            (dict(op=9), K.KVX_E_INVAL),
            (dict(op=K.KVX_OP_RESTORE, ready_slot_base=0), K.KVX_E_INVAL),
            (dict(page_ids=[1, 64]), K.KVX_E_RANGE),
            (dict(op=K.KVX_OP_RESTORE, page_ids=[2, 2]), K.KVX_E_DUP),
        ]
        for i, (change, _) in enumerate(cases):
            a = dict(op=K.KVX_OP_BACKUP, op_id=i, generation=7, pool=0, buffer=0,
                     page_ids=[1, 2], layer_begin=0, layer_end=2)
            a.update(change)
            K.kvx_ring_submit(r, K.make_sqe(**a))
        taken, done = K.kvx_ring_serve(o, [pool], [0x1000000], [nb])
        assert (taken, done) == (len(cases), len(cases))
        got = K.kvx_ring_reap(r, 32)
        assert [(g[0], g[2]) for g in got] == [(i, c) for i, (_, c) in enumerate(cases)]
        assert K.kvx_ring_drain(o) == 0
    finally:
        K.kvx_ring_close(o)
        K.kvx_ring_close(r)
        K.kvx_unregister_pool(pool)


WAITER = textwrap.dedent("""
    import sys, time
    sys.path.insert(0, {root!r})
    from paged_kv_offload_amd import kvx as K
    o = K.kvx_ring_open({name!r})
    print("open", flush=True)
    t0 = time.monotonic()
    got = K.kvx_ring_wait(o, 5_000_000)
    waited = time.monotonic() - t0
    q = K.kvx_ring_take(o)
    K.kvx_ring_complete(o, q.op_id, q.generation, 0)
    print(f"{{int(got)}} {{waited:.4f}}", flush=True)
    K.kvx_ring_close(o)
""")


def test_wait_sleeps_until_a_push_and_honours_timeouts_and_death():
    """A data-plane process sleeps in kvx_ring_wait until the scheduler
    submits (woken within milliseconds, not at its 5 s limit); the
    scheduler's own wait returns the completion; a wait with nothing to take
    returns False at its timeout, and at once when the other side is gone."""
    name = ring_name()
    r = K.kvx_ring_create(name, 4, 2)
    p = subprocess.Popen([sys.executable, "-c", WAITER.format(root=ROOT, name=name)],
                         stdout=subprocess.PIPE, text=True)
    try:
        assert p.stdout.readline().strip() == "open"
        t0 = time.monotonic()
        assert not K.kvx_ring_wait(r, 200_000)                 # nothing posted yet
        assert 0.15 < time.monotonic() - t0 < 2.0
        K.kvx_ring_submit(r, K.make_sqe(K.KVX_OP_BACKUP, 77, 2, 0, 0, [1], 0, 1))
        assert K.kvx_ring_wait(r, 5_000_000)
        assert K.kvx_ring_reap(r) == [(77, 2, 0)]
        got, waited = p.stdout.readline().split()
        assert got == "1" and 0.15 < float(waited) < 2.0, (got, waited)
        assert p.wait(30) == 0
        t0 = time.monotonic()
        assert not K.kvx_ring_wait(r, 5_000_000)               # the data plane is gone
        assert time.monotonic() - t0 < 1.0
        assert not K.kvx_ring_wait(r, 0)
    finally:
        if p.poll() is None:
            p.kill()
            p.wait()
        K.kvx_ring_close(r)
