"""ctypes access to the CPU oracle for paged-KV backup/restore.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path
(``paged_kv_offload_amd``) never does, and this package imports nothing from
it. The arithmetic lives in ``kvx_oracle.c``; this module only marshals numpy
arrays into it.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Sequence, Tuple

import numpy as np

from . import build as _build

PAGE, LAYER, KV = 0, 1, 2
NHD, HND = 0, 1


class _CLayout(ctypes.Structure):
    _fields_ = [("outer", ctypes.c_int32 * 3), ("inner", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("num_layers", ctypes.c_int64),
                ("num_kv", ctypes.c_int64), ("page_size", ctypes.c_int64),
                ("num_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("dtype_bytes", ctypes.c_int64), ("byte_offset", ctypes.c_int64)]


@dataclass(frozen=True)
class Layout:
    """Pool geometry, in the oracle's own terms (outer order of {page, layer,
    kv}, inner NHD/HND, dims, element bytes, byte offset in the allocation)."""
    outer: Tuple[int, int, int]
    inner: int
    num_pages: int
    num_layers: int
    num_kv: int
    page_size: int
    num_heads: int
    head_dim: int
    dtype_bytes: int
    byte_offset: int = 0

    def c(self) -> _CLayout:
        s = _CLayout()
        s.outer[:] = list(self.outer)
        s.inner = self.inner
        s.num_pages, s.num_layers, s.num_kv = self.num_pages, self.num_layers, self.num_kv
        s.page_size, s.num_heads, s.head_dim = self.page_size, self.num_heads, self.head_dim
        s.dtype_bytes, s.byte_offset = self.dtype_bytes, self.byte_offset
        return s

    @property
    def row_bytes(self) -> int:
        return self.head_dim * self.dtype_bytes

    @property
    def piece_bytes(self) -> int:
        return self.page_size * self.num_heads * self.row_bytes

    @property
    def pool_bytes(self) -> int:
        return self.num_pages * self.num_layers * self.num_kv * self.piece_bytes

    def host_bytes(self, n: int) -> int:
        return self.num_layers * self.num_kv * n * self.piece_bytes


_lib = None
_P = ctypes.POINTER


def lib() -> ctypes.CDLL:
    """Loads oracle/libkvx_oracle.so, compiling it first only if it is absent.
    KVX_ORACLE_LIB names another build of the same source instead: the
    mutation tests point it at copies with a planted mistake to show that the
    pins catch each one."""
    global _lib
    if _lib is None:
        path = os.environ.get("KVX_ORACLE_LIB")
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        L = ctypes.CDLL(path)
        lp = _P(_CLayout)
        i64, u64, u8p, i32p = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p
        L.kvxo_piece_start.argtypes = [lp, i64, i64, i64]
        L.kvxo_piece_start.restype = i64
        L.kvxo_backup.argtypes = [lp, u8p, i32p, i64, i64, i64, u8p]
        L.kvxo_restore.argtypes = [lp, u8p, u8p, i32p, i64, i64, i64]
        L.kvxo_backup_slots.argtypes = [lp, u8p, i32p, i32p, i64, i64, i64, i64, u8p]
        L.kvxo_restore_slots.argtypes = [lp, u8p, u8p, i32p, i32p, i64, i64, i64, i64]
        L.kvxo_nhd_to_hnd.argtypes = [u8p, u8p, i64, i64, i64]
        L.kvxo_hnd_to_nhd.argtypes = [u8p, u8p, i64, i64, i64]
        L.kvxo_ready_prefix.argtypes = [ctypes.c_void_p, i64]
        L.kvxo_ready_prefix.restype = i64
        L.kvxo_ready_publish.argtypes = [ctypes.c_void_p, i64, i64, i64, i64, ctypes.c_uint32]
        L.kvxo_gen_word.argtypes = [u64, u64]
        L.kvxo_gen_word.restype = u64
        L.kvxo_splitmix64_next.argtypes = [_P(u64)]
        L.kvxo_splitmix64_next.restype = u64
        L.kvxo_gen_fill.argtypes = [u64, u64, u64, u8p]
        L.kvxo_check_backup_gen.argtypes = [lp, u64, i32p, i64, i64, i64, u8p, i64, i64, _P(i64)]
        L.kvxo_check_backup_gen.restype = i64
        L.kvxo_check_alloc_roundtrip.argtypes = [lp, u64, u64, i32p, i32p, i64, i64, i64, u8p,
                                                 i64, i64, _P(i64)]
        L.kvxo_check_alloc_roundtrip.restype = i64
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _ids(ids: Sequence[int]) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(ids, dtype=np.int32))


def piece_start(layout: Layout, page: int, layer: int, kv: int) -> int:
    c = layout.c()
    return lib().kvxo_piece_start(ctypes.byref(c), page, layer, kv)


def backup(layout: Layout, alloc: np.ndarray, ids: Sequence[int], l0: int, l1: int,
           host: np.ndarray = None) -> np.ndarray:
    """BACKUP of `ids`, layers [l0, l1), from the allocation bytes `alloc` into
    the packed host buffer (a new zero-filled one unless `host` is given)."""
    ids = _ids(ids)
    assert alloc.dtype == np.uint8 and alloc.flags.c_contiguous
    assert alloc.size >= layout.byte_offset + layout.pool_bytes
    if host is None:
        host = np.zeros(layout.host_bytes(len(ids)), dtype=np.uint8)
    assert host.dtype == np.uint8 and host.flags.c_contiguous
    assert host.size >= layout.host_bytes(len(ids))
    c = layout.c()
    lib().kvxo_backup(ctypes.byref(c), _ptr(alloc), _ptr(ids), len(ids), l0, l1, _ptr(host))
    return host


def restore(layout: Layout, alloc: np.ndarray, host: np.ndarray, ids: Sequence[int], l0: int,
            l1: int, out: np.ndarray = None) -> np.ndarray:
    """RESTORE of the packed `host` buffer into pages `ids`, layers [l0, l1).
    Returns a new allocation and leaves `alloc` as it was, unless `out` is
    given (it may be `alloc` itself), which is then written in place."""
    ids = _ids(ids)
    if out is None:
        out = np.array(alloc, dtype=np.uint8, copy=True)
    elif out is not alloc:
        out[...] = alloc
    assert out.dtype == np.uint8 and out.flags.c_contiguous
    assert host.dtype == np.uint8 and host.flags.c_contiguous
    assert host.size >= layout.host_bytes(len(ids))
    c = layout.c()
    lib().kvxo_restore(ctypes.byref(c), _ptr(out), _ptr(host), _ptr(ids), len(ids), l0, l1)
    return out


def host_pool_bytes(layout: Layout, num_slots: int) -> int:
    """Bytes of a slot-addressed host pool of num_slots slots per (layer, kv)."""
    return layout.host_bytes(num_slots)


def backup_slots(layout: Layout, alloc: np.ndarray, ids: Sequence[int], slots: Sequence[int],
                 num_slots: int, l0: int, l1: int, host: np.ndarray = None) -> np.ndarray:
    """BACKUP of `ids` into host slots `slots` of a host pool of num_slots
    slots per (layer, kv), layers [l0, l1); other slots keep their bytes."""
    ids, slots = _ids(ids), _ids(slots)
    assert ids.size == slots.size and (slots.size == 0 or 0 <= slots.min() <= slots.max() < num_slots)
    assert alloc.dtype == np.uint8 and alloc.flags.c_contiguous
    if host is None:
        host = np.zeros(layout.host_bytes(num_slots), dtype=np.uint8)
    assert host.dtype == np.uint8 and host.flags.c_contiguous
    assert host.size >= layout.host_bytes(num_slots)
    c = layout.c()
    lib().kvxo_backup_slots(ctypes.byref(c), _ptr(alloc), _ptr(ids), _ptr(slots), len(ids), num_slots,
                            l0, l1, _ptr(host))
    return host


def restore_slots(layout: Layout, alloc: np.ndarray, host: np.ndarray, slots: Sequence[int],
                  ids: Sequence[int], num_slots: int, l0: int, l1: int,
                  out: np.ndarray = None) -> np.ndarray:
    """RESTORE of host slots `slots` into pages `ids`, layers [l0, l1). A new
    allocation unless `out` is given (it may be `alloc`)."""
    ids, slots = _ids(ids), _ids(slots)
    assert ids.size == slots.size and (slots.size == 0 or 0 <= slots.min() <= slots.max() < num_slots)
    if out is None:
        out = np.array(alloc, dtype=np.uint8, copy=True)
    elif out is not alloc:
        out[...] = alloc
    assert host.dtype == np.uint8 and host.size >= layout.host_bytes(num_slots)
    c = layout.c()
    lib().kvxo_restore_slots(ctypes.byref(c), _ptr(out), _ptr(host), _ptr(slots), _ptr(ids), len(ids),
                             num_slots, l0, l1)
    return out


def nhd_to_hnd(piece: np.ndarray, T: int, H: int, row_bytes: int) -> np.ndarray:
    piece = np.ascontiguousarray(piece, dtype=np.uint8)
    assert piece.size == T * H * row_bytes
    out = np.empty_like(piece)
    lib().kvxo_nhd_to_hnd(_ptr(piece), _ptr(out), T, H, row_bytes)
    return out


def hnd_to_nhd(piece: np.ndarray, T: int, H: int, row_bytes: int) -> np.ndarray:
    piece = np.ascontiguousarray(piece, dtype=np.uint8)
    assert piece.size == T * H * row_bytes
    out = np.empty_like(piece)
    lib().kvxo_hnd_to_nhd(_ptr(piece), _ptr(out), T, H, row_bytes)
    return out


def ready_prefix(counts: Sequence[int]) -> int:
    a = np.ascontiguousarray(np.asarray(counts, dtype=np.uint32))
    return lib().kvxo_ready_prefix(_ptr(a), a.size)


def ready_publish(counts: Sequence[int], slot_base: int, l0: int, l1: int, n: int) -> list:
    """The ready counts after a RESTORE of n pages over layers [l0, l1) that
    publishes from slot_base has completed (a new list; `counts` is left as
    it was)."""
    a = np.array(np.asarray(counts, dtype=np.uint32), dtype=np.uint32, copy=True)
    lib().kvxo_ready_publish(_ptr(a), a.size, slot_base, l0, l1, n)
    return [int(x) for x in a]


def splitmix64_stream(state: int, count: int) -> list:
    s = ctypes.c_uint64(state)
    return [lib().kvxo_splitmix64_next(ctypes.byref(s)) for _ in range(count)]


def gen_word(seed: int, j: int) -> int:
    return lib().kvxo_gen_word(seed, j)


def gen_fill(seed: int, addr: int, length: int) -> np.ndarray:
    out = np.empty(length, dtype=np.uint8)
    lib().kvxo_gen_fill(seed, addr, length, _ptr(out))
    return out


def check_backup_gen(layout: Layout, seed: int, ids: Sequence[int], l0: int, l1: int,
                     host: np.ndarray, host_begin: int = 0) -> Tuple[int, int]:
    """Returns (mismatching bytes, packed offset of the first or -1) for packed
    bytes [host_begin, host_begin + host.size) of a BACKUP of a pool filled
    from generator stream `seed`."""
    ids = _ids(ids)
    host = np.ascontiguousarray(host, dtype=np.uint8)
    first = ctypes.c_int64(-1)
    c = layout.c()
    bad = lib().kvxo_check_backup_gen(ctypes.byref(c), seed, _ptr(ids), len(ids), l0, l1,
                                      _ptr(host), host_begin, host.size, ctypes.byref(first))
    return bad, first.value


def check_alloc_roundtrip(layout: Layout, seed: int, pad_seed: int, src: Sequence[int],
                          dst: Sequence[int], l0: int, l1: int, buf: np.ndarray,
                          addr_begin: int = 0) -> Tuple[int, int]:
    """Returns (mismatching bytes, address of the first or -1) for allocation
    bytes [addr_begin, addr_begin + buf.size) after BACKUP(src) then RESTORE
    into dst, starting from a generator-filled allocation."""
    src, dst = _ids(src), _ids(dst)
    assert src.size == dst.size
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    first = ctypes.c_int64(-1)
    c = layout.c()
    bad = lib().kvxo_check_alloc_roundtrip(ctypes.byref(c), seed, pad_seed, _ptr(src), _ptr(dst),
                                           src.size, l0, l1, _ptr(buf), addr_begin, buf.size,
                                           ctypes.byref(first))
    if bad < 0:
        raise MemoryError("oracle could not allocate its page table")
    return bad, first.value
