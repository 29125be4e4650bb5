"""CPU tests of the C ABI: the library loads and exports every declared
symbol, and the host-side logic (layout validation, page-list checks, run
planning, handle lifecycle, fail-closed error paths) behaves as specified.
No call here reaches the GPU: every call either needs no HIP API or is
rejected by validation before the first one."""
import os
import re

import numpy as np
import pytest

import paged_kv_offload_amd as kvx
from paged_kv_offload_amd import kvx as K
from synth.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_BASE = 0x7F0000000000   # never dereferenced: registration is pure validation


def header_functions():
    with open(os.path.join(ROOT, "include", "kvx.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvx_[a-z_0-9]+)\s*\(", text)))


def dense_stride(shape):
    st, acc = [], 1
    for d in reversed(shape):
        st.append(acc)
        acc *= d
    return list(reversed(st))


def layout_of(w):
    return kvx.make_layout(w.outer, w.inner, w.num_pages, w.num_layers, w.num_kv, w.page_size,
                           w.num_heads, w.head_dim)


def register(w, base=FAKE_BASE, offset=None, shape=None, stride=None, gen=7):
    shape = shape or w.tensor_shape()
    stride = stride or dense_stride(shape)
    off = w.byte_offset if offset is None else offset
    return K.kvx_register_pool(layout_of(w), base, off, w.dtype_bytes, shape, stride, gen)


def test_library_exports_every_header_function():
    L = kvx.lib()
    names = header_functions()
    assert len(names) >= 20
    for name in names:
        assert hasattr(L, name), name
    assert {s[0] for s in K.SIGNATURES} == set(names)
    assert K.kvx_version() == 1


def test_single_hip_runtime_in_process():
    kvx.lib()
    assert len(K.hip_runtimes_mapped()) <= 1


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_register_derives_strides(name):
    w = WORKLOADS[name]
    p = register(w)
    info = K.kvx_pool_get_info(p)
    assert info.piece_bytes == w.piece_bytes
    assert info.row_bytes == w.row_bytes
    assert info.pool_bytes == w.pool_bytes
    assert info.generation == 7
    size = {"page": w.num_pages, "layer": w.num_layers, "kv": w.num_kv}
    # row-major over the outer axes in their physical order, pieces innermost
    s = w.piece_bytes
    want = {}
    for a in reversed(w.outer):
        want[a] = s
        s *= size[a]
    assert (info.page_stride, info.layer_stride, info.kv_stride) == \
        (want["page"], want["layer"], want["kv"])
    assert K.kvx_packed_bytes(p, 10) == w.num_layers * w.num_kv * 10 * w.piece_bytes
    K.kvx_unregister_pool(p)


def test_noncontiguous_is_hard_error_with_shape_and_stride():
    w = WORKLOADS["tiny"]
    shape = w.tensor_shape()
    stride = dense_stride(shape)
    stride[0], stride[1] = stride[1], stride[0]   # a transposed view of the same bytes
    with pytest.raises(kvx.KvxError) as e:
        register(w, shape=shape, stride=stride)
    assert e.value.code == K.KVX_E_NONCONTIG
    assert str(shape).replace(" ", "") in e.value.message.replace(" ", "")
    assert str(stride).replace(" ", "") in e.value.message.replace(" ", "")


def test_padded_stride_rejected_and_size1_stride_ignored():
    w = WORKLOADS["tiny"]
    shape = w.tensor_shape()
    stride = dense_stride(shape)
    padded = [s * 2 for s in stride[:-1]] + [1]
    with pytest.raises(kvx.KvxError) as e:
        register(w, shape=shape, stride=padded)
    assert e.value.code == K.KVX_E_NONCONTIG
    # a size-1 dimension may carry any stride
    sh1 = shape[:1] + [1] + shape[1:]
    st1 = dense_stride(sh1)
    st1[1] = 12345
    K.kvx_unregister_pool(register(w, shape=sh1, stride=st1))


def test_merged_and_split_views():
    w = WORKLOADS["trtllm_hnd"]
    K.kvx_unregister_pool(register(w, shape=[4096, 32, 2, 8 * 32 * 128]))
    K.kvx_unregister_pool(register(w, shape=[4096, 32, 2, 8, 32, 128]))
    K.kvx_unregister_pool(register(w, shape=[4096 * 32 * 2 * 8 * 32 * 128]))
    with pytest.raises(kvx.KvxError) as e:   # splits inside the head axis
        register(w, shape=[4096, 32, 2, 4, 64, 128])
    assert e.value.code == K.KVX_E_INVAL
    with pytest.raises(kvx.KvxError) as e:   # wrong element count
        register(w, shape=[4096, 32, 2, 8 * 32 * 64])
    assert e.value.code == K.KVX_E_INVAL


def test_alignment_errors():
    w = WORKLOADS["trtllm_hnd"]
    with pytest.raises(kvx.KvxError) as e:
        register(w, offset=12288 + 8)
    assert e.value.code == K.KVX_E_ALIGN
    odd = WORKLOADS["tiny"].scaled(head_dim=60)   # 120-byte rows
    with pytest.raises(kvx.KvxError) as e:
        register(odd)
    assert e.value.code == K.KVX_E_ALIGN


def test_bad_layouts():
    w = WORKLOADS["tiny"]
    L = layout_of(w)
    L.outer[:] = [0, 0, 2]
    shape = w.tensor_shape()
    with pytest.raises(kvx.KvxError) as e:
        K.kvx_register_pool(L, FAKE_BASE, 0, 2, shape, dense_stride(shape), 1)
    assert e.value.code == K.KVX_E_INVAL
    L = layout_of(w)
    L.num_heads = 0
    with pytest.raises(kvx.KvxError):
        K.kvx_register_pool(L, FAKE_BASE, 0, 2, shape, dense_stride(shape), 1)
    with pytest.raises(kvx.KvxError):
        K.kvx_register_pool(layout_of(w), 0, 0, 2, shape, dense_stride(shape), 1)


def test_plan_runs_sorted_and_coalesced():
    w = WORKLOADS["tiny"]   # layer-major: consecutive pages are adjacent
    p = register(w)
    ids = [9, 10, 11, 3, 40, 41, 5, 4]
    runs = K.kvx_plan_runs(p, ids)
    # (first page, first slot, pages): sorted by page, merged only where page
    # and slot both continue
    assert runs.tolist() == [[3, 3, 1], [4, 7, 1], [5, 6, 1], [9, 0, 3], [40, 4, 2]]
    cover = sorted((int(r[1]) + k, int(r[0]) + k) for r in runs for k in range(r[2]))
    assert cover == sorted(enumerate(ids))
    K.kvx_unregister_pool(p)
    q = register(WORKLOADS["trtllm_hnd"])   # page-major: pages are not adjacent
    runs = K.kvx_plan_runs(q, [7, 8, 9])
    assert runs.tolist() == [[7, 0, 1], [8, 1, 1], [9, 2, 1]]
    K.kvx_unregister_pool(q)


def test_validation_fails_closed_before_any_gpu_call():
    w = WORKLOADS["tiny"]
    p = register(w)
    host = np.zeros(w.host_bytes(8) + 64, dtype=np.uint8)
    hp = (host.ctypes.data + 15) // 16 * 16
    nb = w.host_bytes(8)

    def code(fn):
        with pytest.raises(kvx.KvxError) as e:
            fn()
        return e.value.code

    assert code(lambda: K.kvx_backup(p, [0, 64], hp, nb, 0, 2)) == K.KVX_E_RANGE
    assert code(lambda: K.kvx_backup(p, [-1], hp, nb, 0, 2)) == K.KVX_E_RANGE
    assert code(lambda: K.kvx_backup(p, [1, 2], hp, nb, 0, 3)) == K.KVX_E_RANGE
    assert code(lambda: K.kvx_backup(p, [1, 2], hp, nb, 1, 0)) == K.KVX_E_RANGE
    assert code(lambda: K.kvx_backup(p, list(range(8)), hp, nb - 16, 0, 2)) == K.KVX_E_RANGE
    assert code(lambda: K.kvx_backup(p, list(range(8)), hp + 8, nb, 0, 2)) == K.KVX_E_ALIGN
    assert code(lambda: K.kvx_backup(p, [1], hp, nb, 0, 2, path=9)) == K.KVX_E_INVAL
    assert code(lambda: K.kvx_backup(p, [1], 0, nb, 0, 2)) == K.KVX_E_INVAL
    assert code(lambda: K.kvx_restore(p, hp, nb, [3, 5, 3], 0, 2)) == K.KVX_E_DUP
    assert code(lambda: K.kvx_restore(p, hp, nb, [3, 64], 0, 2)) == K.KVX_E_RANGE
    # duplicates are fine for a backup; it fails later only because it reaches HIP
    # empty work is a no-op that succeeds without touching the GPU
    K.kvx_backup(p, [], hp, nb, 0, 2)
    K.kvx_restore(p, hp, nb, [1, 2], 1, 1)
    K.kvx_unregister_pool(p)


def test_handle_lifecycle_and_teardown_never_raises():
    w = WORKLOADS["tiny"]
    p = register(w)
    K.kvx_unregister_pool(p)
    K.kvx_unregister_pool(p)          # second teardown: logged, not an error
    K.kvx_unregister_pool(0)          # NULL: nothing to do
    for fn in (lambda: K.kvx_pool_get_info(p), lambda: K.kvx_packed_bytes(p, 1),
               lambda: K.kvx_backup(p, [1], 16, 1 << 20, 0, 1),
               lambda: K.kvx_restore(p, 16, 1 << 20, [1], 0, 1),
               lambda: K.kvx_plan_runs(p, [1])):
        with pytest.raises(kvx.KvxError) as e:
            fn()
        assert e.value.code == K.KVX_E_STALE
    with pytest.raises(kvx.KvxError) as e:
        K.kvx_pool_get_info(0x1234560)
    assert e.value.code == K.KVX_E_INVAL


def test_options_roundtrip():
    old = K.kvx_get_option(K.KVX_OPT_STAGE_SLOTS)
    K.kvx_set_option(K.KVX_OPT_STAGE_SLOTS, 4)
    assert K.kvx_get_option(K.KVX_OPT_STAGE_SLOTS) == 4
    K.kvx_set_option(K.KVX_OPT_STAGE_SLOTS, old)
    with pytest.raises(kvx.KvxError):
        K.kvx_set_option(K.KVX_OPT_STAGE_SLOTS, 1)
    with pytest.raises(kvx.KvxError):
        K.kvx_set_option(99, 1)
    assert "unknown option" in K.kvx_last_error()
    # staged DMA stream: -1 auto (the default), 0 side stream, 1 caller's stream
    dma = K.KVX_OPT_STAGED_DMA_ON_CALLER
    assert K.kvx_get_option(dma) == -1
    for v in (0, 1, -1):
        K.kvx_set_option(dma, v)
        assert K.kvx_get_option(dma) == v
    for v in (-2, 2):
        with pytest.raises(kvx.KvxError):
            K.kvx_set_option(dma, v)
    assert K.kvx_get_option(dma) == -1
    # publish block: 0 auto (the default), else 1..4096 units per draw
    pb = K.KVX_OPT_PUBLISH_BLOCK
    assert K.kvx_get_option(pb) == 0
    for v in (1, 4096, 0):
        K.kvx_set_option(pb, v)
        assert K.kvx_get_option(pb) == v
    for v in (-1, 4097):
        with pytest.raises(kvx.KvxError):
            K.kvx_set_option(pb, v)
    # duplex shares of the host link: 6 writers and 18 readers by default,
    # 0 (the direction-blind share) to 1024
    for opt, default in ((K.KVX_OPT_DUPLEX_WRITERS, 6), (K.KVX_OPT_DUPLEX_READERS, 18)):
        assert K.kvx_get_option(opt) == default
        for v in (0, 1, 1024, default):
            K.kvx_set_option(opt, v)
            assert K.kvx_get_option(opt) == v
        for v in (-1, 1025):
            with pytest.raises(kvx.KvxError):
                K.kvx_set_option(opt, v)
        assert K.kvx_get_option(opt) == default


def test_ipc_handle_layout_matches_the_header(tmp_path):
    """The binding's kvx_ipc_handle has the C struct's size and field
    offsets (compiled from include/kvx.h with gcc)."""
    import ctypes
    import subprocess
    src = tmp_path / "h.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "kvx.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(kvx_ipc_handle), '
                   'offsetof(kvx_ipc_handle, mem_handle), offsetof(kvx_ipc_handle, device_uuid), '
                   'offsetof(kvx_ipc_handle, alloc_bytes), offsetof(kvx_ipc_handle, offset), '
                   'offsetof(kvx_ipc_handle, version), offsetof(kvx_ipc_handle, reserved)); return 0; }\n')
    exe = tmp_path / "h"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    c = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                        text=True).stdout.split()]
    H = K.kvx_ipc_handle
    py = [ctypes.sizeof(H)] + [getattr(H, f).offset for f in
                               ("mem_handle", "device_uuid", "alloc_bytes", "offset", "version",
                                "reserved")]
    assert c == py == [104, 0, 64, 80, 88, 96, 100]


def test_ipc_import_and_close_validate_before_any_gpu_call():
    """Malformed or oversized handles (2 GiB, exactly, and more) and unknown
    bases are refused by validation alone (no HIP call is reached)."""
    h = K.kvx_ipc_handle()
    h.version, h.alloc_bytes, h.offset = 1, 1 << 20, 0
    good = bytes(h)
    for field, value, code in (("version", 0, K.KVX_E_INVAL), ("reserved", 1, K.KVX_E_INVAL),
                               ("alloc_bytes", 0, K.KVX_E_INVAL),
                               ("offset", 1 << 20, K.KVX_E_INVAL),
                               ("alloc_bytes", (2 << 30) + 4096, K.KVX_E_RANGE),
                               ("alloc_bytes", 2 << 30, K.KVX_E_RANGE),
                               ("alloc_bytes", 1 << 31, K.KVX_E_RANGE)):
        bad = K.kvx_ipc_handle.from_buffer_copy(good)
        setattr(bad, field, value)
        with pytest.raises(K.KvxError) as e:
            K.kvx_ipc_import(bytes(bad))
        assert e.value.code == code, (field, value)
    with pytest.raises(K.KvxError) as e:
        K.kvx_ipc_import(good[:-1])
    assert e.value.code == K.KVX_E_INVAL
    with pytest.raises(K.KvxError) as e:
        K.kvx_ipc_close(FAKE_BASE)
    assert e.value.code == K.KVX_E_INVAL
    with pytest.raises(K.KvxError) as e:
        K.kvx_ipc_export(0)
    assert e.value.code == K.KVX_E_INVAL


def test_exchange_validation_fails_closed():
    """kvx_exchange refuses the staged path, overlapping packed buffers and a
    page both sides touch in a common layer before any HIP call."""
    w = WORKLOADS["tiny"]
    pool = register(w)
    nb = w.host_bytes(2)
    base = dict(pool=pool, backup_ids=[1, 2], backup_dst=0x1000000, backup_bytes=nb,
                backup_layers=(0, 2), restore_src=0x2000000, restore_bytes=nb, restore_ids=[3, 4],
                restore_layers=(0, 2), path=K.KVX_PATH_ZEROCOPY)
    try:
        for change, code, text in (
                (dict(path=K.KVX_PATH_STAGED), K.KVX_E_INVAL, "zero-copy or device path"),
                (dict(restore_ids=[2, 5]), K.KVX_E_INVAL, "page 2 is read by the backup"),
                (dict(restore_src=0x1000000 + 16), K.KVX_E_INVAL, "overlap"),
                (dict(backup_dst=0x2000000 + nb - 16), K.KVX_E_INVAL, "overlap"),
                # one buffer for both sides: their layer slices must not overlap
                (dict(restore_src=0x1000000, backup_layers=(0, 2), restore_layers=(1, 2)),
                 K.KVX_E_INVAL, "overlap"),
                (dict(restore_ids=[3, 3]), K.KVX_E_DUP, "more than once"),
                (dict(backup_ids=[1, 64]), K.KVX_E_RANGE, "outside"),
                (dict(restore_layers=(1, 3)), K.KVX_E_RANGE, "layer range"),
                (dict(restore_bytes=nb - 1), K.KVX_E_RANGE, "needs")):
            args = dict(base)
            args.update(change)
            with pytest.raises(K.KvxError) as e:
                K.kvx_exchange(**args)
            assert e.value.code == code and text in e.value.message, (change, e.value.message)
    finally:
        K.kvx_unregister_pool(pool)


def test_slot_validation_fails_closed():
    """kvx_backup_slots / kvx_restore_slots refuse the staged path, slots
    outside the host pool, a slot a backup would write twice, a page a
    restore would write twice and a host pool too small for its slots before
    any HIP call; empty work succeeds without one."""
    w = WORKLOADS["tiny"]
    pool = register(w)
    S = 5
    nb = w.host_bytes(S)
    hp = 0x1000000
    zc = K.KVX_PATH_ZEROCOPY
    try:
        for fn, code, text in (
                (lambda: K.kvx_backup_slots(pool, [1, 2], [0, 1], hp, nb, S, 0, 2,
                                            path=K.KVX_PATH_STAGED), K.KVX_E_INVAL, "zero-copy"),
                (lambda: K.kvx_backup_slots(pool, [1, 2], [0, 5], hp, nb, S, 0, 2, path=zc),
                 K.KVX_E_RANGE, "host_slots[1] = 5"),
                (lambda: K.kvx_backup_slots(pool, [1, 2], [-1, 0], hp, nb, S, 0, 2, path=zc),
                 K.KVX_E_RANGE, "host_slots[0]"),
                (lambda: K.kvx_backup_slots(pool, [1, 2], [3, 3], hp, nb, S, 0, 2, path=zc),
                 K.KVX_E_DUP, "host slot 3"),
                (lambda: K.kvx_backup_slots(pool, [1, 64], [0, 1], hp, nb, S, 0, 2, path=zc),
                 K.KVX_E_RANGE, "page_ids[1]"),
                (lambda: K.kvx_backup_slots(pool, [1, 2], [0, 1], hp, nb - 16, S, 0, 2, path=zc),
                 K.KVX_E_RANGE, "needs"),
                (lambda: K.kvx_backup_slots(pool, [1, 2], [0, 1], hp, nb, -1, 0, 2, path=zc),
                 K.KVX_E_RANGE, "negative"),
                (lambda: K.kvx_backup_slots(pool, [1, 2], [0, 1], hp + 8, nb, S, 0, 2, path=zc),
                 K.KVX_E_ALIGN, "aligned"),
                (lambda: K.kvx_restore_slots(pool, hp, nb, S, [0, 1], [4, 4], 0, 2, path=zc),
                 K.KVX_E_DUP, "destination page 4"),
                (lambda: K.kvx_restore_slots(pool, hp, nb, S, [0, 9], [4, 5], 0, 2, path=zc),
                 K.KVX_E_RANGE, "host_slots[1] = 9"),
                (lambda: K.kvx_restore_slots(pool, hp, nb, S, [0, 1], [4, 5], 0, 3, path=zc),
                 K.KVX_E_RANGE, "layer range"),
                (lambda: K.kvx_restore_slots(pool, hp, nb, S, [0], [4, 5], 0, 2, path=zc),
                 K.KVX_E_INVAL, "host slots")):
            with pytest.raises(K.KvxError) as e:
                fn()
            assert e.value.code == code and text in e.value.message, (code, e.value.message)
        # empty work: no-ops that never reach the GPU
        K.kvx_backup_slots(pool, [], [], hp, nb, S, 0, 2, path=zc)
        K.kvx_restore_slots(pool, hp, nb, S, [2, 2], [4, 5], 1, 1, path=zc)
        K.kvx_backup_slots(pool, [], [], 0, 0, 0, 0, 2, path=zc)
    finally:
        K.kvx_unregister_pool(pool)


def test_tier_policy_calls_fail_closed():
    """kvx_tier_backup / kvx_tier_restore: a tier of another generation is
    STALE; a refusal by the transfer's own checks (here a host pool too
    small) leaves the tier exactly as it was, evictions included; all
    before any HIP call."""
    w = WORKLOADS["tiny"]
    pool = register(w, gen=7)
    S = 2
    nb = w.host_bytes(S)
    hp = 0x1000000
    t = K.kvx_tier_create(S, 7)
    old = K.kvx_tier_create(S, 6)
    try:
        slots, _ = K.kvx_tier_reserve(t, [11, 12])
        K.kvx_tier_commit(t, slots)
        view = [K.kvx_tier_slot(t, s) for s in range(S)]
        info = K.kvx_tier_get_info(t)
        for fn, code, text in (
                (lambda: K.kvx_tier_backup(old, pool, [13], [1], hp, nb), K.KVX_E_STALE,
                 "generation"),
                # 13 and 14 would evict 11 and 12, then the transfer refuses
                (lambda: K.kvx_tier_backup(t, pool, [13, 14], [1, 2], hp, nb - 16), K.KVX_E_RANGE,
                 "needs"),
                (lambda: K.kvx_tier_backup(t, pool, [13, 14], [1, 2], hp, nb,
                                           path=K.KVX_PATH_STAGED), K.KVX_E_INVAL, "zero-copy"),
                (lambda: K.kvx_tier_backup(t, pool, [13], [64], hp, nb), K.KVX_E_RANGE, "outside"),
                (lambda: K.kvx_tier_restore(t, pool, [11, 12], [3, 3], hp, nb), K.KVX_E_DUP,
                 "destination page 3"),
                (lambda: K.kvx_tier_restore(t, pool, [11, 12], [3, 4], hp, nb - 1), K.KVX_E_RANGE,
                 "needs")):
            with pytest.raises(K.KvxError) as e:
                fn()
            assert e.value.code == code and text in e.value.message, (code, e.value.message)
            assert [K.kvx_tier_slot(t, s) for s in range(S)] == view
            assert K.kvx_tier_get_info(t) == info
        # nothing new and no hit: no transfer, no HIP call
        assert K.kvx_tier_backup(t, pool, [11], [1], hp, nb)[0].tolist() == [-1]
        assert K.kvx_tier_restore(t, pool, [99], [1], hp, nb).tolist() == [-1]
    finally:
        K.kvx_tier_destroy(t)
        K.kvx_tier_destroy(old)
        K.kvx_unregister_pool(pool)


def test_exchange_slots_validation_fails_closed():
    """kvx_exchange_slots refuses the staged path, a host slot both sides use
    in a common layer of one host pool, overlapping layer slices of two host
    pools, a page both sides touch in a common layer, and each side's own
    slot and page errors, before any HIP call."""
    w = WORKLOADS["tiny"]
    pool = register(w)
    S = 6
    nb = w.host_bytes(S)
    base = dict(pool=pool, backup_ids=[1, 2], backup_slots=[0, 1], backup_pool=0x1000000,
                backup_pool_bytes=nb, backup_num_slots=S, backup_layers=(0, 2),
                restore_pool=0x1000000, restore_pool_bytes=nb, restore_num_slots=S,
                restore_slots=[2, 3], restore_ids=[3, 4], restore_layers=(0, 2),
                path=K.KVX_PATH_ZEROCOPY)
    try:
        for change, code, text in (
                (dict(path=K.KVX_PATH_STAGED), K.KVX_E_INVAL, "zero-copy or device path"),
                (dict(restore_slots=[1, 5]), K.KVX_E_INVAL, "host slot 1"),
                (dict(restore_ids=[2, 5]), K.KVX_E_INVAL, "page 2 is read by the backup"),
                (dict(restore_pool=0x1000000 + 16), K.KVX_E_INVAL, "overlap"),
                (dict(backup_slots=[4, 4]), K.KVX_E_DUP, "host slot 4"),
                (dict(restore_ids=[3, 3]), K.KVX_E_DUP, "destination page 3"),
                (dict(restore_slots=[2, 6]), K.KVX_E_RANGE, "host_slots[1] = 6"),
                (dict(backup_pool_bytes=nb - 16), K.KVX_E_RANGE, "needs")):
            args = dict(base)
            args.update(change)
            with pytest.raises(K.KvxError) as e:
                K.kvx_exchange_slots(**args)
            assert e.value.code == code and text in e.value.message, (change, e.value.message)
        # nothing to move on either side is a no-op that touches no GPU
        K.kvx_exchange_slots(**dict(base, backup_ids=[], backup_slots=[], restore_ids=[],
                                    restore_slots=[]))
    finally:
        K.kvx_unregister_pool(pool)


def test_tier_exchange_fails_closed():
    """kvx_tier_exchange: when the exchange refuses the pair (a page the
    backup reads is one the restore writes), the lookup's pins and the
    reservation's evictions are undone; all before any HIP call."""
    w = WORKLOADS["tiny"]
    pool = register(w, gen=7)
    S = 2
    nb = w.host_bytes(S)
    t = K.kvx_tier_create(S, 7)
    try:
        slots, _ = K.kvx_tier_reserve(t, [11, 12])
        K.kvx_tier_commit(t, slots)
        view = [K.kvx_tier_slot(t, s) for s in range(S)]
        info = K.kvx_tier_get_info(t)
        with pytest.raises(K.KvxError) as e:
            K.kvx_tier_exchange(t, pool, [13], [1], [11], [1], 0x1000000, nb)
        assert e.value.code == K.KVX_E_INVAL and "page 1" in e.value.message, e.value.message
        assert [K.kvx_tier_slot(t, s) for s in range(S)] == view
        assert K.kvx_tier_get_info(t) == info
        old = K.kvx_tier_create(S, 6)
        with pytest.raises(K.KvxError) as e:
            K.kvx_tier_exchange(old, pool, [13], [1], [11], [2], 0x1000000, nb)
        assert e.value.code == K.KVX_E_STALE
        K.kvx_tier_destroy(old)
    finally:
        K.kvx_tier_destroy(t)
        K.kvx_unregister_pool(pool)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library every entry point raises; there is no
    other implementation to fall back to."""
    monkeypatch.setattr(K, "_lib", None)
    monkeypatch.setattr(K, "LIB_PATH", str(tmp_path / "libkvx.so"))
    with pytest.raises(ImportError, match="not built"):
        K.lib()
    with pytest.raises(ImportError, match="not built"):
        K.kvx_version()
    with pytest.raises(ImportError, match="not built"):
        K.kvx_backup(1, [0], 16, 4096, 0, 1)
