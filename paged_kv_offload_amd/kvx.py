"""ctypes binding of libkvx.so (include/kvx.h).

Argument marshalling only: every step of backup, restore, publish and the
ready queries runs inside libkvx.so (HIP kernels and the HIP runtime). The
functions keep the C names. There is no fallback: if the library is not
built, loading fails with an error.

PyTorch is used only as a source of device memory and streams: a tensor is
passed as its data pointer, a stream as its hipStream_t handle.
"""
import ctypes
import os
from typing import Iterable, Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvx.so")

KVX_OK = 0
KVX_E_INVAL, KVX_E_NONCONTIG, KVX_E_ALIGN, KVX_E_RANGE, KVX_E_DUP = -1, -2, -3, -4, -5
KVX_E_STALE, KVX_E_NOTPINNED, KVX_E_NOMEM, KVX_E_HIP, KVX_E_FULL = -6, -7, -8, -9, -10
KVX_NOALLOC_MAX_LAYERS = 4096      # layers kvx_restore_noalloc serves (its scratch)
TIER_FREE, TIER_WRITING, TIER_RESIDENT = 0, 1, 2
KVX_RING_MAX_PAGES = 1024
KVX_OP_BACKUP, KVX_OP_RESTORE, KVX_OP_BACKUP_SLOTS, KVX_OP_RESTORE_SLOTS = 1, 2, 3, 4
KVX_AX_PAGE, KVX_AX_LAYER, KVX_AX_KV = 0, 1, 2
KVX_NHD, KVX_HND = 0, 1
KVX_PATH_STAGED, KVX_PATH_ZEROCOPY, KVX_PATH_DEVICE = 0, 1, 2
KVX_OPT_GRID_MAX, KVX_OPT_STAGE_SLOT_BYTES, KVX_OPT_STAGE_SLOTS = 0, 1, 2
KVX_OPT_SORT_PAGES, KVX_OPT_CACHE_POLICY, KVX_OPT_RESTORE_CHUNK_LAYERS = 3, 4, 5
KVX_OPT_HOST_GRID_MAX, KVX_OPT_UNIT_ORDER, KVX_OPT_MAX_UNROLL = 6, 7, 8
KVX_OPT_STAGED_DMA_ON_CALLER, KVX_OPT_HND_LDS, KVX_OPT_UNIT_ROUNDS = 9, 10, 11
KVX_OPT_FAIL_ALLOCS, KVX_OPT_RING_PAIRING, KVX_OPT_PUBLISH_BLOCK = 12, 13, 14
KVX_OPT_COALESCE_RUNS, KVX_OPT_TAIL_UNITS, KVX_OPT_DEVICE_LISTS = 15, 16, 17
KVX_OPT_DUPLEX_WRITERS, KVX_OPT_DUPLEX_READERS = 18, 19

ERROR_NAMES = {0: "KVX_OK", -1: "KVX_E_INVAL", -2: "KVX_E_NONCONTIG", -3: "KVX_E_ALIGN",
               -4: "KVX_E_RANGE", -5: "KVX_E_DUP", -6: "KVX_E_STALE", -7: "KVX_E_NOTPINNED",
               -8: "KVX_E_NOMEM", -9: "KVX_E_HIP", -10: "KVX_E_FULL"}
PATHS = {"staged": KVX_PATH_STAGED, "zerocopy": KVX_PATH_ZEROCOPY, "device": KVX_PATH_DEVICE}
_AXES = {"page": KVX_AX_PAGE, "layer": KVX_AX_LAYER, "kv": KVX_AX_KV}


class KvxError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code
        self.message = message


class kvx_layout(ctypes.Structure):
    _fields_ = [("outer", ctypes.c_int32 * 3), ("inner", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("num_kv", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class kvx_pool_info(ctypes.Structure):
    _fields_ = [(k, ctypes.c_uint64) for k in ("row_bytes", "piece_bytes", "page_stride",
                                               "layer_stride", "kv_stride", "pool_bytes",
                                               "generation")]


class kvx_xfer(ctypes.Structure):
    _fields_ = [("page_ids", ctypes.c_void_p), ("n", ctypes.c_int32), ("packed", ctypes.c_void_p),
                ("packed_bytes", ctypes.c_uint64), ("layer_begin", ctypes.c_int32),
                ("layer_end", ctypes.c_int32)]


class kvx_xfer_slots(ctypes.Structure):
    _fields_ = [("page_ids", ctypes.c_void_p), ("host_slots", ctypes.c_void_p), ("n", ctypes.c_int32),
                ("num_host_slots", ctypes.c_int32), ("host_pool", ctypes.c_void_p),
                ("host_pool_bytes", ctypes.c_uint64), ("layer_begin", ctypes.c_int32),
                ("layer_end", ctypes.c_int32)]


class kvx_ipc_handle(ctypes.Structure):
    _fields_ = [("mem_handle", ctypes.c_uint8 * 64), ("device_uuid", ctypes.c_uint8 * 16),
                ("alloc_bytes", ctypes.c_uint64), ("offset", ctypes.c_uint64),
                ("version", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class kvx_tier_info(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32) for k in ("num_slots", "free_slots", "writing", "resident",
                                              "pinned", "doomed")] + \
               [("evictions", ctypes.c_uint64), ("generation", ctypes.c_uint64)]


class kvx_sqe(ctypes.Structure):
    _fields_ = [("op_id", ctypes.c_uint64), ("generation", ctypes.c_uint64),
                ("buffer_offset", ctypes.c_uint64)] + \
               [(k, ctypes.c_int32) for k in ("op", "pool", "buffer", "n", "layer_begin",
                                              "layer_end", "path", "ready_slot_base",
                                              "num_host_slots", "reserved")] + \
               [("page_ids", ctypes.c_int32 * KVX_RING_MAX_PAGES),
                ("host_slots", ctypes.c_int32 * KVX_RING_MAX_PAGES)]


class kvx_cqe(ctypes.Structure):
    _fields_ = [("op_id", ctypes.c_uint64), ("generation", ctypes.c_uint64),
                ("status", ctypes.c_int32), ("reserved", ctypes.c_int32)]


# (name, restype, argtypes) of every exported function
_vp, _i32, _u32, _i64, _u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64, \
    ctypes.c_uint64
_P = ctypes.POINTER
SIGNATURES = [
    ("kvx_register_pool", ctypes.c_int, [_P(kvx_layout), _vp, _u64, _u32, _i32, _P(_i64), _P(_i64),
                                         _u64, _P(_vp)]),
    ("kvx_unregister_pool", ctypes.c_int, [_vp]),
    ("kvx_pool_get_info", ctypes.c_int, [_vp, _P(kvx_pool_info)]),
    ("kvx_packed_bytes", ctypes.c_int, [_vp, _i32, _P(_u64)]),
    ("kvx_backup", ctypes.c_int, [_vp, _P(_i32), _i32, _vp, _u64, _i32, _i32, _vp, _i32]),
    ("kvx_restore", ctypes.c_int, [_vp, _vp, _u64, _P(_i32), _i32, _i32, _i32, _vp, _i32, _vp,
                                   _i32]),
    ("kvx_restore_noalloc", ctypes.c_int, [_vp, _vp, _u64, _P(_i32), _i32, _i32, _i32, _vp, _i32,
                                           _vp, _i32]),
    ("kvx_plan_runs", ctypes.c_int, [_vp, _P(_i32), _i32, _P(_i32), _i32, _P(_i32)]),
    ("kvx_ready_create", ctypes.c_int, [_i32, _u64, _P(_vp)]),
    ("kvx_ready_create_device", ctypes.c_int, [_i32, _i32, _u64, _P(_vp)]),
    ("kvx_ready_attach_device", ctypes.c_int, [_vp, _i32, _u64, _P(_vp)]),
    ("kvx_ready_reset", ctypes.c_int, [_vp]),
    ("kvx_ready_destroy", ctypes.c_int, [_vp]),
    ("kvx_layer_ready", ctypes.c_int, [_vp, _i32, _P(_i32)]),
    ("kvx_ready_prefix", ctypes.c_int, [_vp, _P(_i32)]),
    ("kvx_ready_slot_ptr", ctypes.c_int, [_vp, _i32, _P(_vp)]),
    ("kvx_ready_wait_gpu", ctypes.c_int, [_vp, _i32, _i32, _vp, _u32, _vp]),
    ("kvx_host_alloc", ctypes.c_int, [_u64, _P(_vp)]),
    ("kvx_host_free", ctypes.c_int, [_vp]),
    ("kvx_alloc_range", ctypes.c_int, [_vp, _P(_vp), _P(_u64)]),
    ("kvx_sync", ctypes.c_int, [_vp]),
    ("kvx_release_stream", ctypes.c_int, [_vp]),
    ("kvx_last_error", ctypes.c_char_p, []),
    ("kvx_version", ctypes.c_int, []),
    ("kvx_set_option", ctypes.c_int, [_i32, _i64]),
    ("kvx_get_option", ctypes.c_int, [_i32, _P(_i64)]),
    ("kvx_backup_slots", ctypes.c_int, [_vp, _P(_i32), _P(_i32), _i32, _vp, _u64, _i32, _i32, _i32,
                                        _vp, _i32]),
    ("kvx_restore_slots", ctypes.c_int, [_vp, _vp, _u64, _i32, _P(_i32), _P(_i32), _i32, _i32, _i32,
                                         _vp, _i32, _vp, _i32]),
    ("kvx_exchange", ctypes.c_int, [_vp, _P(kvx_xfer), _P(kvx_xfer), _vp, _i32, _vp, _i32]),
    ("kvx_exchange_slots", ctypes.c_int, [_vp, _P(kvx_xfer_slots), _P(kvx_xfer_slots), _vp, _i32, _vp,
                                          _i32]),
    ("kvx_ipc_export", ctypes.c_int, [_vp, _P(kvx_ipc_handle)]),
    ("kvx_ipc_import", ctypes.c_int, [_P(kvx_ipc_handle), _P(_vp), _P(_i32)]),
    ("kvx_ipc_close", ctypes.c_int, [_vp]),
    ("kvx_ring_create", ctypes.c_int, [ctypes.c_char_p, _i32, _u64, _P(_vp)]),
    ("kvx_ring_open", ctypes.c_int, [ctypes.c_char_p, _P(_vp)]),
    ("kvx_ring_close", ctypes.c_int, [_vp]),
    ("kvx_ring_submit", ctypes.c_int, [_vp, _P(kvx_sqe)]),
    ("kvx_ring_reap", ctypes.c_int, [_vp, _P(kvx_cqe), _i32, _P(_i32)]),
    ("kvx_ring_take", ctypes.c_int, [_vp, _P(kvx_sqe), _P(_i32)]),
    ("kvx_ring_complete", ctypes.c_int, [_vp, _P(kvx_cqe)]),
    ("kvx_ring_peer_alive", ctypes.c_int, [_vp, _P(_i32)]),
    ("kvx_ring_pending", ctypes.c_int, [_vp, _P(_i32), _P(_i32)]),
    ("kvx_ring_wait", ctypes.c_int, [_vp, _i32, _P(_i32)]),
    ("kvx_ring_serve", ctypes.c_int, [_vp, _P(_vp), _i32, _P(_vp), _P(_u64), _i32, _vp, _vp, _i32,
                                      _P(_i32), _P(_i32)]),
    ("kvx_ring_drain", ctypes.c_int, [_vp, _P(_i32)]),
    ("kvx_ring_discard", ctypes.c_int, [_vp, _P(_i32)]),
    ("kvx_tier_create", ctypes.c_int, [_i32, _u64, _P(_vp)]),
    ("kvx_tier_destroy", ctypes.c_int, [_vp]),
    ("kvx_tier_reserve", ctypes.c_int, [_vp, _P(_u64), _i32, _P(_i32), _P(_u64), _P(_i32)]),
    ("kvx_tier_commit", ctypes.c_int, [_vp, _P(_i32), _i32]),
    ("kvx_tier_abort", ctypes.c_int, [_vp, _P(_i32), _i32]),
    ("kvx_tier_lookup", ctypes.c_int, [_vp, _P(_u64), _i32, _P(_i32), _P(_i32)]),
    ("kvx_tier_release", ctypes.c_int, [_vp, _P(_i32), _i32]),
    ("kvx_tier_invalidate", ctypes.c_int, [_vp, _P(_u64), _i32, _P(_i32)]),
    ("kvx_tier_get_info", ctypes.c_int, [_vp, _P(kvx_tier_info)]),
    ("kvx_tier_slot", ctypes.c_int, [_vp, _i32, _P(_u64), _P(_i32), _P(_i32)]),
    ("kvx_tier_backup", ctypes.c_int, [_vp, _vp, _P(_u64), _P(_i32), _i32, _vp, _u64, _vp, _i32,
                                       _P(_i32), _P(_u64), _P(_i32)]),
    ("kvx_tier_restore", ctypes.c_int, [_vp, _vp, _P(_u64), _P(_i32), _i32, _vp, _u64, _vp, _i32,
                                        _vp, _i32, _P(_i32), _P(_i32)]),
    ("kvx_tier_exchange", ctypes.c_int, [_vp, _vp, _P(_u64), _P(_i32), _i32, _P(_u64), _P(_i32), _i32,
                                         _vp, _u64, _vp, _i32, _vp, _i32, _P(_i32), _P(_u64),
                                         _P(_i32), _P(_i32), _P(_i32)]),
]

_lib: Optional[ctypes.CDLL] = None


def hip_runtimes_mapped() -> list:
    """Distinct libamdhip64 files mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return sorted(paths)


def lib() -> ctypes.CDLL:
    """Loads libkvx.so. Raises if it is not built or if the process ends up
    with two HIP runtimes (torch's and another), which would make torch's
    streams and pointers meaningless to kvx."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libkvx.so is not built ({LIB_PATH}); run "
                              "`python -c 'import __graft_entry__ as g; g.build()'` first")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.kvx_version() != 1:
            raise ImportError("libkvx.so ABI version mismatch")
        rts = hip_runtimes_mapped()
        if len(rts) > 1:
            raise ImportError(f"two HIP runtimes are loaded: {rts}")
        _lib = L
    return _lib


def kvx_last_error() -> str:
    return lib().kvx_last_error().decode(errors="replace")


def _check(rc: int) -> None:
    if rc != KVX_OK:
        raise KvxError(rc, kvx_last_error())


def _ptr(x) -> int:
    """Address of a tensor, numpy array or integer pointer."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(s) -> int:
    if s is None:
        return 0
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    raise TypeError(f"not a stream: {type(s)}")


def _ids(page_ids) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(page_ids, dtype=np.int32).reshape(-1))
    return a


def _ids_ptr(a: np.ndarray):
    return a.ctypes.data_as(_P(_i32))


# ---------------------------------------------------------------------------
# layout and registration
# ---------------------------------------------------------------------------
def make_layout(outer: Sequence[str], inner: str, num_pages: int, num_layers: int, num_kv: int,
                page_size: int, num_heads: int, head_dim: int) -> kvx_layout:
    L = kvx_layout()
    L.outer[:] = [_AXES[a] for a in outer]
    L.inner = {"NHD": KVX_NHD, "HND": KVX_HND}[inner]
    L.num_pages, L.num_layers, L.num_kv = num_pages, num_layers, num_kv
    L.page_size, L.num_heads, L.head_dim = page_size, num_heads, head_dim
    return L


def kvx_register_pool(layout: kvx_layout, base: int, byte_offset: int, dtype_bytes: int,
                      shape: Sequence[int], stride: Sequence[int], generation: int) -> int:
    nd = len(shape)
    sh = (_i64 * max(nd, 1))(*shape)
    st = (_i64 * max(nd, 1))(*stride)
    out = _vp()
    _check(lib().kvx_register_pool(ctypes.byref(layout), base, byte_offset, dtype_bytes, nd, sh, st,
                                   generation, ctypes.byref(out)))
    return out.value


def kvx_unregister_pool(pool: int) -> None:
    _check(lib().kvx_unregister_pool(pool))


def kvx_pool_get_info(pool: int) -> kvx_pool_info:
    info = kvx_pool_info()
    _check(lib().kvx_pool_get_info(pool, ctypes.byref(info)))
    return info


def kvx_packed_bytes(pool: int, n: int) -> int:
    out = _u64()
    _check(lib().kvx_packed_bytes(pool, n, ctypes.byref(out)))
    return out.value


def kvx_alloc_range(ptr: int):
    base, size = _vp(), _u64()
    _check(lib().kvx_alloc_range(ptr, ctypes.byref(base), ctypes.byref(size)))
    return base.value, size.value


# ---------------------------------------------------------------------------
# device-memory IPC
# ---------------------------------------------------------------------------
def kvx_ipc_export(device_ptr: int) -> bytes:
    """Handle of the allocation holding device_ptr, as bytes to send to
    another process."""
    h = kvx_ipc_handle()
    _check(lib().kvx_ipc_export(device_ptr, ctypes.byref(h)))
    return bytes(h)


def ipc_handle_from_bytes(data: bytes) -> kvx_ipc_handle:
    if len(data) != ctypes.sizeof(kvx_ipc_handle):
        raise KvxError(KVX_E_INVAL, f"an IPC handle is {ctypes.sizeof(kvx_ipc_handle)} bytes, "
                                    f"got {len(data)}")
    return kvx_ipc_handle.from_buffer_copy(data)


def kvx_ipc_import(data: bytes):
    """Maps an exported allocation: returns (base, device ordinal, byte
    offset of the exported pointer, allocation bytes)."""
    h = ipc_handle_from_bytes(data)
    base, dev = _vp(), _i32()
    _check(lib().kvx_ipc_import(ctypes.byref(h), ctypes.byref(base), ctypes.byref(dev)))
    return base.value, dev.value, h.offset, h.alloc_bytes


def kvx_ipc_close(base: int) -> None:
    _check(lib().kvx_ipc_close(base))


def dense_strides(shape: Sequence[int]) -> list:
    st, acc = [], 1
    for d in reversed(list(shape)):
        st.append(acc)
        acc *= d
    return st[::-1]


def register_imported(data: bytes, layout: kvx_layout, dtype_bytes: int, shape: Sequence[int],
                      generation: int):
    """Imports a pool exported by another process and registers it with the
    given layout and dense shape. Returns (pool handle, mapping base); the
    base goes to kvx_ipc_close after the pool is unregistered."""
    base, _, offset, _ = kvx_ipc_import(data)
    try:
        pool = kvx_register_pool(layout, base, offset, dtype_bytes, list(shape),
                                 dense_strides(shape), generation)
    except KvxError:
        kvx_ipc_close(base)
        raise
    return pool, base


def permute_to_dense_view(t):
    """Metadata-only permute of a non-contiguous tensor view to a contiguous
    one when its strides allow it (the RawCudaIPCWrapper article, sender
    validation: permute first, then check; never copy)."""
    if t.is_contiguous():
        return t
    order = sorted(range(t.dim()), key=lambda d: (-t.stride(d), d))
    p = t.permute(*order)
    return p if p.is_contiguous() else t


def register_tensor(t, layout: kvx_layout, generation: int) -> int:
    """Registers a torch tensor as a pool: permutes it to a dense view if its
    strides allow (metadata only), finds its allocation base, and passes
    base, byte offset, element size, shape and stride to kvx_register_pool,
    which rejects any view that is still not dense."""
    v = permute_to_dense_view(t)
    base, _ = kvx_alloc_range(v.data_ptr())
    return kvx_register_pool(layout, base, v.data_ptr() - base, v.element_size(), list(v.shape),
                             list(v.stride()), generation)


# ---------------------------------------------------------------------------
# data movement
# ---------------------------------------------------------------------------
def kvx_backup(pool: int, page_ids: Iterable[int], dst, dst_bytes: int, layer_begin: int,
               layer_end: int, stream=None, path: int = KVX_PATH_STAGED) -> None:
    ids = _ids(page_ids)
    _check(lib().kvx_backup(pool, _ids_ptr(ids), ids.size, _ptr(dst), dst_bytes, layer_begin,
                            layer_end, _stream(stream), path))


def kvx_restore(pool: int, src, src_bytes: int, page_ids: Iterable[int], layer_begin: int,
                layer_end: int, ready: int = None, slot_base: int = 0, stream=None,
                path: int = KVX_PATH_STAGED) -> None:
    ids = _ids(page_ids)
    _check(lib().kvx_restore(pool, _ptr(src), src_bytes, _ids_ptr(ids), ids.size, layer_begin,
                             layer_end, ready or 0, slot_base, _stream(stream), path))


def kvx_restore_noalloc(pool: int, src, src_bytes: int, page_ids: Iterable[int], layer_begin: int,
                        layer_end: int, ready: int = None, slot_base: int = 0, stream=None,
                        path: int = KVX_PATH_ZEROCOPY) -> None:
    ids = _ids(page_ids)
    _check(lib().kvx_restore_noalloc(pool, _ptr(src), src_bytes, _ids_ptr(ids), ids.size, layer_begin,
                                     layer_end, ready or 0, slot_base, _stream(stream), path))


def kvx_backup_slots(pool: int, page_ids: Iterable[int], host_slots: Iterable[int], host_pool,
                     host_pool_bytes: int, num_host_slots: int, layer_begin: int, layer_end: int,
                     stream=None, path: int = KVX_PATH_ZEROCOPY) -> None:
    """BACKUP of page_ids[i] into slot host_slots[i] of a host pool of
    num_host_slots slots per (layer, kv)."""
    ids, sl = _ids(page_ids), _ids(host_slots)
    if sl.size != ids.size:
        raise KvxError(KVX_E_INVAL, f"{ids.size} pages but {sl.size} host slots")
    _check(lib().kvx_backup_slots(pool, _ids_ptr(ids), _ids_ptr(sl), ids.size, _ptr(host_pool),
                                  host_pool_bytes, num_host_slots, layer_begin, layer_end,
                                  _stream(stream), path))


def kvx_restore_slots(pool: int, host_pool, host_pool_bytes: int, num_host_slots: int,
                      host_slots: Iterable[int], page_ids: Iterable[int], layer_begin: int,
                      layer_end: int, ready: int = None, slot_base: int = 0, stream=None,
                      path: int = KVX_PATH_ZEROCOPY) -> None:
    """RESTORE of slot host_slots[i] of a host pool into page page_ids[i]."""
    ids, sl = _ids(page_ids), _ids(host_slots)
    if sl.size != ids.size:
        raise KvxError(KVX_E_INVAL, f"{sl.size} host slots but {ids.size} pages")
    _check(lib().kvx_restore_slots(pool, _ptr(host_pool), host_pool_bytes, num_host_slots,
                                   _ids_ptr(sl), _ids_ptr(ids), ids.size, layer_begin, layer_end,
                                   ready or 0, slot_base, _stream(stream), path))


# ---------------------------------------------------------------------------
# host tier
# ---------------------------------------------------------------------------
def _keys(keys) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(keys, dtype=np.uint64).reshape(-1))


def _kp(a: np.ndarray):
    return a.ctypes.data_as(_P(_u64))


def _sp(a: np.ndarray):
    return a.ctypes.data_as(_P(_i32))


def kvx_tier_create(num_slots: int, generation: int) -> int:
    out = _vp()
    _check(lib().kvx_tier_create(num_slots, generation, ctypes.byref(out)))
    return out.value


def kvx_tier_destroy(tier: int) -> None:
    _check(lib().kvx_tier_destroy(tier))


def kvx_tier_reserve(tier: int, keys):
    """(slots, evicted keys) of a reservation; slot -1 for a key present."""
    k = _keys(keys)
    slots = np.empty(k.size, dtype=np.int32)
    ev = np.empty(max(k.size, 1), dtype=np.uint64)
    ne = _i32()
    _check(lib().kvx_tier_reserve(tier, _kp(k), k.size, _sp(slots), _kp(ev), ctypes.byref(ne)))
    return slots, ev[:ne.value].copy()


def kvx_tier_commit(tier: int, slots) -> None:
    s = _ids(slots)
    _check(lib().kvx_tier_commit(tier, _sp(s), s.size))


def kvx_tier_abort(tier: int, slots) -> None:
    s = _ids(slots)
    _check(lib().kvx_tier_abort(tier, _sp(s), s.size))


def kvx_tier_lookup(tier: int, keys) -> np.ndarray:
    """Slots of the keys (pinned), -1 for a miss."""
    k = _keys(keys)
    slots = np.empty(k.size, dtype=np.int32)
    hits = _i32()
    _check(lib().kvx_tier_lookup(tier, _kp(k), k.size, _sp(slots), ctypes.byref(hits)))
    return slots


def kvx_tier_release(tier: int, slots) -> None:
    s = _ids(slots)
    _check(lib().kvx_tier_release(tier, _sp(s), s.size))


def kvx_tier_invalidate(tier: int, keys) -> int:
    k = _keys(keys)
    nd = _i32()
    _check(lib().kvx_tier_invalidate(tier, _kp(k), k.size, ctypes.byref(nd)))
    return nd.value


def kvx_tier_get_info(tier: int) -> dict:
    info = kvx_tier_info()
    _check(lib().kvx_tier_get_info(tier, ctypes.byref(info)))
    return {k: getattr(info, k) for k, _ in kvx_tier_info._fields_}


def kvx_tier_slot(tier: int, slot: int):
    """(key, state, pins) of one slot."""
    key, state, pins = _u64(), _i32(), _i32()
    _check(lib().kvx_tier_slot(tier, slot, ctypes.byref(key), ctypes.byref(state),
                               ctypes.byref(pins)))
    return key.value, state.value, pins.value


def kvx_tier_backup(tier: int, pool: int, keys, page_ids, host_pool, host_pool_bytes: int,
                    stream=None, path: int = KVX_PATH_ZEROCOPY):
    """Reserve + backup of the new keys' pages; (slots, evicted keys)."""
    k, ids = _keys(keys), _ids(page_ids)
    if k.size != ids.size:
        raise KvxError(KVX_E_INVAL, f"{k.size} keys but {ids.size} pages")
    slots = np.empty(k.size, dtype=np.int32)
    ev = np.empty(max(k.size, 1), dtype=np.uint64)
    ne = _i32()
    _check(lib().kvx_tier_backup(tier, pool, _kp(k), _ids_ptr(ids), k.size, _ptr(host_pool),
                                 host_pool_bytes, _stream(stream), path, _sp(slots), _kp(ev),
                                 ctypes.byref(ne)))
    return slots, ev[:ne.value].copy()


def kvx_tier_restore(tier: int, pool: int, keys, page_ids, host_pool, host_pool_bytes: int,
                     ready: int = None, slot_base: int = 0, stream=None,
                     path: int = KVX_PATH_ZEROCOPY) -> np.ndarray:
    """Lookup + restore of the hits into their pages; the slots (-1 = miss)."""
    k, ids = _keys(keys), _ids(page_ids)
    if k.size != ids.size:
        raise KvxError(KVX_E_INVAL, f"{k.size} keys but {ids.size} pages")
    slots = np.empty(k.size, dtype=np.int32)
    hits = _i32()
    _check(lib().kvx_tier_restore(tier, pool, _kp(k), _ids_ptr(ids), k.size, _ptr(host_pool),
                                  host_pool_bytes, ready or 0, slot_base, _stream(stream), path,
                                  _sp(slots), ctypes.byref(hits)))
    return slots


def kvx_tier_exchange(tier: int, pool: int, backup_keys, backup_pages, restore_keys,
                      restore_pages, host_pool, host_pool_bytes: int, ready: int = None,
                      slot_base: int = 0, stream=None, path: int = KVX_PATH_ZEROCOPY):
    """Lookup of restore_keys + reserve of backup_keys + one exchange;
    (backup slots, evicted keys, restore slots)."""
    bk, bp, rk, rp = _keys(backup_keys), _ids(backup_pages), _keys(restore_keys), _ids(restore_pages)
    if bk.size != bp.size or rk.size != rp.size:
        raise KvxError(KVX_E_INVAL, "one page per key on each side")
    bs = np.empty(bk.size, dtype=np.int32)
    rs = np.empty(rk.size, dtype=np.int32)
    ev = np.empty(max(bk.size, 1), dtype=np.uint64)
    ne, hits = _i32(), _i32()
    _check(lib().kvx_tier_exchange(tier, pool, _kp(bk), _ids_ptr(bp), bk.size, _kp(rk), _ids_ptr(rp),
                                   rk.size, _ptr(host_pool), host_pool_bytes, ready or 0, slot_base,
                                   _stream(stream), path, _sp(bs), _kp(ev), ctypes.byref(ne),
                                   _sp(rs), ctypes.byref(hits)))
    return bs, ev[:ne.value].copy(), rs


# ---------------------------------------------------------------------------
# submission / completion rings
# ---------------------------------------------------------------------------
def make_sqe(op: int, op_id: int, generation: int, pool: int, buffer: int, page_ids,
             layer_begin: int, layer_end: int, path: int = KVX_PATH_ZEROCOPY,
             buffer_offset: int = 0, ready_slot_base: int = -1, host_slots=None,
             num_host_slots: int = 0) -> kvx_sqe:
    ids = _ids(page_ids)
    if ids.size > KVX_RING_MAX_PAGES:
        raise KvxError(KVX_E_RANGE, f"{ids.size} pages exceed {KVX_RING_MAX_PAGES} per descriptor")
    q = kvx_sqe()
    q.op_id, q.generation, q.buffer_offset = op_id, generation, buffer_offset
    q.op, q.pool, q.buffer, q.n = op, pool, buffer, ids.size
    q.layer_begin, q.layer_end, q.path = layer_begin, layer_end, path
    q.ready_slot_base, q.num_host_slots = ready_slot_base, num_host_slots
    ctypes.memmove(q.page_ids, ids.ctypes.data, ids.nbytes)
    if host_slots is not None:
        sl = _ids(host_slots)
        if sl.size != ids.size:
            raise KvxError(KVX_E_INVAL, f"{ids.size} pages but {sl.size} host slots")
        ctypes.memmove(q.host_slots, sl.ctypes.data, sl.nbytes)
    return q


def kvx_ring_create(name: str, entries: int, generation: int) -> int:
    out = _vp()
    _check(lib().kvx_ring_create(name.encode(), entries, generation, ctypes.byref(out)))
    return out.value


def kvx_ring_open(name: str) -> int:
    out = _vp()
    _check(lib().kvx_ring_open(name.encode(), ctypes.byref(out)))
    return out.value


def kvx_ring_close(ring: int) -> None:
    _check(lib().kvx_ring_close(ring))


def kvx_ring_submit(ring: int, sqe: kvx_sqe) -> None:
    _check(lib().kvx_ring_submit(ring, ctypes.byref(sqe)))


def kvx_ring_reap(ring: int, max_n: int = 64) -> list:
    """[(op_id, generation, status), ...] of up to max_n completions."""
    buf = (kvx_cqe * max(max_n, 1))()
    got = _i32()
    _check(lib().kvx_ring_reap(ring, buf, max_n, ctypes.byref(got)))
    return [(buf[i].op_id, buf[i].generation, buf[i].status) for i in range(got.value)]


def kvx_ring_take(ring: int):
    """The next descriptor, or None."""
    q = kvx_sqe()
    got = _i32()
    _check(lib().kvx_ring_take(ring, ctypes.byref(q), ctypes.byref(got)))
    return q if got.value else None


def kvx_ring_complete(ring: int, op_id: int, generation: int, status: int) -> None:
    c = kvx_cqe(op_id, generation, status, 0)
    _check(lib().kvx_ring_complete(ring, ctypes.byref(c)))


def kvx_ring_peer_alive(ring: int) -> bool:
    a = _i32()
    _check(lib().kvx_ring_peer_alive(ring, ctypes.byref(a)))
    return bool(a.value)


def kvx_ring_wait(ring: int, timeout_us: int) -> bool:
    """True once the caller's side has something to take; False on timeout
    or when the other side has died."""
    r = _i32()
    _check(lib().kvx_ring_wait(ring, timeout_us, ctypes.byref(r)))
    return bool(r.value)


def kvx_ring_pending(ring: int):
    """(submitted and not taken, completed and not reaped)."""
    a, b = _i32(), _i32()
    _check(lib().kvx_ring_pending(ring, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def kvx_ring_serve(ring: int, pools, buffers, buffer_bytes, ready: int = None, stream=None,
                   max_ops: int = 64):
    """Runs up to max_ops descriptors against the tables; (taken, completed)."""
    P = (_vp * max(len(pools), 1))(*pools)
    B = (_vp * max(len(buffers), 1))(*[_ptr(b) for b in buffers])
    N = (_u64 * max(len(buffer_bytes), 1))(*buffer_bytes)
    taken, done = _i32(), _i32()
    _check(lib().kvx_ring_serve(ring, P, len(pools), B, N, len(buffers), ready or 0,
                                _stream(stream), max_ops, ctypes.byref(taken), ctypes.byref(done)))
    return taken.value, done.value


def kvx_ring_drain(ring: int) -> int:
    d = _i32()
    _check(lib().kvx_ring_drain(ring, ctypes.byref(d)))
    return d.value


def kvx_ring_discard(ring: int) -> int:
    d = _i32()
    _check(lib().kvx_ring_discard(ring, ctypes.byref(d)))
    return d.value


def kvx_exchange(pool: int, backup_ids: Iterable[int], backup_dst, backup_bytes: int,
                 backup_layers, restore_src, restore_bytes: int, restore_ids: Iterable[int],
                 restore_layers, ready: int = None, slot_base: int = 0, stream=None,
                 path: int = KVX_PATH_ZEROCOPY) -> None:
    """BACKUP of backup_ids into backup_dst and RESTORE of restore_src into
    restore_ids in one launch sequence; *_layers are (begin, end)."""
    bi, ri = _ids(backup_ids), _ids(restore_ids)
    b = kvx_xfer(bi.ctypes.data if bi.size else None, bi.size, _ptr(backup_dst), backup_bytes,
                 *backup_layers)
    r = kvx_xfer(ri.ctypes.data if ri.size else None, ri.size, _ptr(restore_src), restore_bytes,
                 *restore_layers)
    _check(lib().kvx_exchange(pool, ctypes.byref(b), ctypes.byref(r), ready, slot_base,
                              _stream(stream), path))


def kvx_exchange_slots(pool: int, backup_ids, backup_slots, backup_pool, backup_pool_bytes: int,
                       backup_num_slots: int, backup_layers, restore_pool, restore_pool_bytes: int,
                       restore_num_slots: int, restore_slots, restore_ids, restore_layers,
                       ready: int = None, slot_base: int = 0, stream=None,
                       path: int = KVX_PATH_ZEROCOPY) -> None:
    """kvx_backup_slots of backup_ids into backup_slots and kvx_restore_slots
    of restore_slots into restore_ids in one launch sequence."""
    bi, bs, ri, rsl = _ids(backup_ids), _ids(backup_slots), _ids(restore_ids), _ids(restore_slots)
    if bi.size != bs.size or ri.size != rsl.size:
        raise KvxError(KVX_E_INVAL, "each side needs one host slot per page")
    b = kvx_xfer_slots(bi.ctypes.data if bi.size else None, bs.ctypes.data if bs.size else None,
                       bi.size, backup_num_slots, _ptr(backup_pool), backup_pool_bytes, *backup_layers)
    r = kvx_xfer_slots(ri.ctypes.data if ri.size else None, rsl.ctypes.data if rsl.size else None,
                       ri.size, restore_num_slots, _ptr(restore_pool), restore_pool_bytes,
                       *restore_layers)
    _check(lib().kvx_exchange_slots(pool, ctypes.byref(b), ctypes.byref(r), ready, slot_base,
                                    _stream(stream), path))


def kvx_plan_runs(pool: int, page_ids: Iterable[int]) -> np.ndarray:
    ids = _ids(page_ids)
    cap = max(ids.size, 1)
    runs = np.zeros(3 * cap, dtype=np.int32)
    num = _i32()
    _check(lib().kvx_plan_runs(pool, _ids_ptr(ids), ids.size, runs.ctypes.data_as(_P(_i32)), cap,
                               ctypes.byref(num)))
    return runs[:3 * num.value].reshape(-1, 3)


# ---------------------------------------------------------------------------
# readiness
# ---------------------------------------------------------------------------
def kvx_ready_create(num_slots: int, generation: int) -> int:
    out = _vp()
    _check(lib().kvx_ready_create(num_slots, generation, ctypes.byref(out)))
    return out.value


def kvx_ready_create_device(device: int, num_slots: int, generation: int) -> int:
    out = _vp()
    _check(lib().kvx_ready_create_device(device, num_slots, generation, ctypes.byref(out)))
    return out.value


def kvx_ready_attach_device(counts_dev: int, num_slots: int, generation: int) -> int:
    out = _vp()
    _check(lib().kvx_ready_attach_device(counts_dev, num_slots, generation, ctypes.byref(out)))
    return out.value


def kvx_ready_reset(ready: int) -> None:
    _check(lib().kvx_ready_reset(ready))


def kvx_ready_destroy(ready: int) -> None:
    _check(lib().kvx_ready_destroy(ready))


def kvx_layer_ready(ready: int, slot: int) -> int:
    out = _i32()
    _check(lib().kvx_layer_ready(ready, slot, ctypes.byref(out)))
    return out.value


def kvx_ready_prefix(ready: int) -> int:
    out = _i32()
    _check(lib().kvx_ready_prefix(ready, ctypes.byref(out)))
    return out.value


def kvx_ready_slot_ptr(ready: int, slot: int) -> int:
    out = _vp()
    _check(lib().kvx_ready_slot_ptr(ready, slot, ctypes.byref(out)))
    return out.value


def kvx_ready_wait_gpu(ready: int, slot: int, min_count: int, stream, spin_limit: int,
                       status_dev) -> None:
    _check(lib().kvx_ready_wait_gpu(ready, slot, min_count, _stream(stream), spin_limit,
                                    _ptr(status_dev)))


# ---------------------------------------------------------------------------
# memory, sync, options
# ---------------------------------------------------------------------------
def kvx_host_alloc(nbytes: int) -> int:
    out = _vp()
    _check(lib().kvx_host_alloc(nbytes, ctypes.byref(out)))
    return out.value


def kvx_host_free(ptr: int) -> None:
    _check(lib().kvx_host_free(ptr))


def kvx_release_stream(stream) -> None:
    """Frees the library's per-stream state (see include/kvx.h)."""
    _check(lib().kvx_release_stream(_stream(stream)))


def kvx_sync(stream=None) -> None:
    _check(lib().kvx_sync(_stream(stream)))


def kvx_set_option(option: int, value: int) -> None:
    _check(lib().kvx_set_option(option, value))


def kvx_get_option(option: int) -> int:
    out = _i64()
    _check(lib().kvx_get_option(option, ctypes.byref(out)))
    return out.value


def kvx_version() -> int:
    return lib().kvx_version()


class HostBuffer:
    """Pinned, device-mapped host memory from kvx_host_alloc, viewable as a
    numpy uint8 array."""

    def __init__(self, nbytes: int):
        self.nbytes = nbytes
        self.ptr = kvx_host_alloc(nbytes)

    def numpy(self) -> np.ndarray:
        buf = (ctypes.c_uint8 * self.nbytes).from_address(self.ptr)
        return np.frombuffer(buf, dtype=np.uint8)

    def free(self) -> None:
        if self.ptr:
            kvx_host_free(self.ptr)
            self.ptr = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
