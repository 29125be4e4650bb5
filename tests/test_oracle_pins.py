"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against something it does not compute: numpy's
own advanced indexing and transposes, plain memcpy for the contiguous case,
brute force over every short page-ID tuple of a tiny pool, hand-derived
worked examples (tests/golden), the round-trip and untouched-byte
properties that the pages' BACKUP/RESTORE semantics imply, and the
published SplitMix64 outputs. The layouts use pairwise different dimension
sizes so that a swapped index or a transposed axis changes the result.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import HND, KV, LAYER, NHD, PAGE, Layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
OUTER_ORDERS = list(itertools.permutations((PAGE, LAYER, KV)))


# ---------------------------------------------------------------------------
# independent numpy model: reshape the pool by its physical dims and index it
# ---------------------------------------------------------------------------
def numpy_pool_view(L: Layout, alloc: np.ndarray) -> np.ndarray:
    """View of the pool as [layer][kv][page][token][head][row byte]."""
    sizes = {PAGE: L.num_pages, LAYER: L.num_layers, KV: L.num_kv}
    inner = ([L.page_size, L.num_heads] if L.inner == NHD else [L.num_heads, L.page_size])
    p = alloc[L.byte_offset:L.byte_offset + L.pool_bytes].reshape(
        [sizes[a] for a in L.outer] + inner + [L.row_bytes])
    p = p.transpose([L.outer.index(LAYER), L.outer.index(KV), L.outer.index(PAGE), 3, 4, 5])
    if L.inner == HND:
        p = p.transpose(0, 1, 2, 4, 3, 5)
    return p


def numpy_backup(L, alloc, ids, l0, l1):
    n = len(ids)
    host = np.zeros(L.host_bytes(n), dtype=np.uint8)
    hv = host.reshape(L.num_layers, L.num_kv, n, L.page_size, L.num_heads, L.row_bytes)
    hv[l0:l1] = numpy_pool_view(L, alloc)[l0:l1][:, :, np.asarray(ids, dtype=np.int64)]
    return host


def numpy_restore(L, alloc, host, ids, l0, l1):
    out = alloc.copy()
    n = len(ids)
    hv = host.reshape(L.num_layers, L.num_kv, n, L.page_size, L.num_heads, L.row_bytes)
    pv = numpy_pool_view(L, out)   # a view into `out`
    idx = np.asarray(ids, dtype=np.int64)
    for l in range(l0, l1):
        pv[l, :, idx] = hv[l].transpose(1, 0, 2, 3, 4)
    return out


def rand_layout(rng, outer, inner, offset=0):
    # distinct sizes everywhere: NB 7, NL 3, KV 2, T 5, H 4 (or 1), D 3, eb 2
    return Layout(outer=outer, inner=inner, num_pages=7, num_layers=3, num_kv=2, page_size=5,
                  num_heads=4, head_dim=3, dtype_bytes=2, byte_offset=offset)


def rand_alloc(rng, L, tail=11):
    return rng.integers(0, 256, L.byte_offset + L.pool_bytes + tail, dtype=np.uint8)


# ---------------------------------------------------------------------------
# the generator: published vector, and numpy vs C
# ---------------------------------------------------------------------------
def test_splitmix64_published_outputs():
    # The worked example published with the Rosetta Code SplitMix64 task:
    # seed 1234567 gives these first five outputs.
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert oracle.splitmix64_stream(1234567, 5) == want
    assert [oracle.gen_word(1234567, j) for j in range(5)] == want
    assert [int(x) for x in synth.gen_words(1234567, 0, 5)] == want


@pytest.mark.parametrize("seed,addr,length", [(101, 0, 64), (7, 3, 1001), (2**40 + 5, 8 * 999, 77),
                                              (0, 1, 1)])
def test_generator_c_matches_numpy(seed, addr, length):
    assert np.array_equal(oracle.gen_fill(seed, addr, length), synth.gen_bytes(seed, addr, length))


def test_generator_byte_order_little_endian():
    w = oracle.gen_word(9, 4)
    got = oracle.gen_fill(9, 32, 8)
    assert [int(b) for b in got] == [(w >> (8 * k)) & 0xFF for k in range(8)]


# ---------------------------------------------------------------------------
# BACKUP / RESTORE vs numpy indexing, every outer order, both inner layouts
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("outer", OUTER_ORDERS)
@pytest.mark.parametrize("inner", [NHD, HND])
def test_backup_matches_numpy_indexing(outer, inner):
    rng = np.random.default_rng(hash((outer, inner)) % 2**32)
    L = rand_layout(rng, outer, inner, offset=48)
    alloc = rand_alloc(rng, L)
    for ids, l0, l1 in [([4, 0, 6], 0, 3), ([2, 2, 5, 1], 1, 3), ([6], 2, 3), ([3, 1], 0, 1),
                        (list(rng.permutation(7)), 0, 3)]:
        got = oracle.backup(L, alloc, ids, l0, l1)
        assert np.array_equal(got, numpy_backup(L, alloc, ids, l0, l1)), (ids, l0, l1)


@pytest.mark.parametrize("outer", OUTER_ORDERS)
@pytest.mark.parametrize("inner", [NHD, HND])
def test_restore_matches_numpy_assignment(outer, inner):
    rng = np.random.default_rng(1 + hash((outer, inner)) % 2**32)
    L = rand_layout(rng, outer, inner, offset=16)
    alloc = rand_alloc(rng, L)
    for ids, l0, l1 in [([4, 0, 6], 0, 3), ([5, 1], 1, 3), ([6], 2, 3), ([0, 3, 2], 0, 2)]:
        host = rng.integers(0, 256, L.host_bytes(len(ids)), dtype=np.uint8)
        got = oracle.restore(L, alloc, host, ids, l0, l1)
        assert np.array_equal(got, numpy_restore(L, alloc, host, ids, l0, l1)), (ids, l0, l1)


def test_backup_contiguous_ids_is_memcpy():
    # layer-major [NL][KV][NB] NHD with ids = p0 .. p0+n-1: each (layer, kv)
    # host slice is one memcpy of n pieces starting at piece (p0, l, c),
    # whose byte address is off + ((l*KV + c)*NB + p0) * piece_bytes.
    L = Layout(outer=(LAYER, KV, PAGE), inner=NHD, num_pages=9, num_layers=3, num_kv=2,
               page_size=4, num_heads=3, head_dim=8, dtype_bytes=2, byte_offset=32)
    rng = np.random.default_rng(5)
    alloc = rand_alloc(rng, L)
    p0, n = 3, 5
    host = oracle.backup(L, alloc, range(p0, p0 + n), 0, 3)
    pb = L.piece_bytes
    for l in range(3):
        for c in range(2):
            a = L.byte_offset + ((l * 2 + c) * 9 + p0) * pb
            h = ((l * 2 + c) * n) * pb
            assert np.array_equal(host[h:h + n * pb], alloc[a:a + n * pb])


@pytest.mark.parametrize("inner", [NHD, HND])
@pytest.mark.parametrize("outer", [(LAYER, KV, PAGE), (PAGE, LAYER, KV)])
def test_brute_force_tiny_pool(inner, outer):
    # every ordered page tuple of length 1..3 over a 5-page, 2-layer pool
    L = Layout(outer=outer, inner=inner, num_pages=5, num_layers=2, num_kv=2, page_size=3,
               num_heads=2, head_dim=1, dtype_bytes=2, byte_offset=8)
    rng = np.random.default_rng(11)
    alloc = rand_alloc(rng, L)
    for k in (1, 2, 3):
        for ids in itertools.product(range(5), repeat=k):
            for l0, l1 in ((0, 2), (1, 2)):
                assert np.array_equal(oracle.backup(L, alloc, ids, l0, l1),
                                      numpy_backup(L, alloc, ids, l0, l1)), (ids, l0, l1)
                if len(set(ids)) == k:
                    host = rng.integers(0, 256, L.host_bytes(k), dtype=np.uint8)
                    assert np.array_equal(oracle.restore(L, alloc, host, ids, l0, l1),
                                          numpy_restore(L, alloc, host, ids, l0, l1))


# ---------------------------------------------------------------------------
# round trip and untouched bytes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("outer", OUTER_ORDERS)
@pytest.mark.parametrize("inner", [NHD, HND])
def test_round_trip_moves_pieces_and_nothing_else(outer, inner):
    rng = np.random.default_rng(3 + hash((outer, inner)) % 2**32)
    L = rand_layout(rng, outer, inner, offset=64)
    alloc = rand_alloc(rng, L)
    src, dst = [5, 2, 0], [1, 6, 3]
    l0, l1 = 1, 3
    host = oracle.backup(L, alloc, src, l0, l1)
    out = oracle.restore(L, alloc, host, dst, l0, l1)
    pb = L.piece_bytes
    touched = np.zeros(alloc.size, dtype=bool)
    for s, d in zip(src, dst):
        for l in range(l0, l1):
            for c in range(L.num_kv):
                a_s = oracle.piece_start(L, s, l, c)
                a_d = oracle.piece_start(L, d, l, c)
                assert np.array_equal(out[a_d:a_d + pb], alloc[a_s:a_s + pb])
                touched[a_d:a_d + pb] = True
    assert touched.sum() == len(dst) * (l1 - l0) * L.num_kv * pb
    assert np.array_equal(out[~touched], alloc[~touched])


def test_piece_start_is_row_major_over_outer_axes():
    L = Layout(outer=(KV, PAGE, LAYER), inner=NHD, num_pages=7, num_layers=3, num_kv=2,
               page_size=1, num_heads=1, head_dim=8, dtype_bytes=1, byte_offset=40)
    for p, l, c in itertools.product(range(7), range(3), range(2)):
        assert oracle.piece_start(L, p, l, c) == 40 + ((c * 7 + p) * 3 + l) * 8


# ---------------------------------------------------------------------------
# layout permutation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,rb", [(5, 4, 6), (32, 8, 16), (1, 7, 4), (9, 1, 2), (3, 3, 1)])
def test_permutation_inverse_and_transpose(T, H, rb):
    rng = np.random.default_rng(T * 100 + H)
    x = rng.integers(0, 256, T * H * rb, dtype=np.uint8)
    y = oracle.nhd_to_hnd(x, T, H, rb)
    assert np.array_equal(y, x.reshape(T, H, rb).transpose(1, 0, 2).reshape(-1))
    assert np.array_equal(oracle.hnd_to_nhd(y, T, H, rb), x)
    assert np.array_equal(oracle.nhd_to_hnd(oracle.hnd_to_nhd(x, T, H, rb), T, H, rb), x)
    if T == 1 or H == 1:
        assert np.array_equal(y, x)


# ---------------------------------------------------------------------------
# hand-derived worked examples
# ---------------------------------------------------------------------------
def _read_golden(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            d[k] = v
    axis = {"page": PAGE, "layer": LAYER, "kv": KV}
    L = Layout(outer=tuple(axis[a] for a in d["outer"].split()),
               inner=NHD if d["inner"] == "NHD" else HND,
               **{k: int(d[k]) for k in ("num_pages", "num_layers", "num_kv", "page_size",
                                         "num_heads", "head_dim", "dtype_bytes", "byte_offset")})
    ints = lambda k: [int(x) for x in d[k].split()]  # noqa: E731
    changes = dict(tuple(int(x) for x in kv.split(":")) for kv in d["alloc_changes"].split())
    return L, int(d["alloc_bytes"]), ints("backup_ids"), ints("restore_ids"), ints("layers"), \
        ints("host"), changes


@pytest.mark.parametrize("name", ["trtllm_hnd_tiny.txt", "llama_nhd_tiny.txt"])
def test_golden_worked_example(name):
    L, nbytes, bids, rids, (l0, l1), host_want, changes = _read_golden(name)
    alloc = np.arange(nbytes, dtype=np.uint8)
    host = oracle.backup(L, alloc, bids, l0, l1)
    assert [int(b) for b in host] == host_want
    out = oracle.restore(L, alloc, host, rids, l0, l1)
    want = alloc.copy()
    for a, v in changes.items():
        want[a] = v
    assert np.array_equal(out, want)


# ---------------------------------------------------------------------------
# closed forms against the materialized oracle, and that they catch errors
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("inner,outer", [(NHD, (LAYER, KV, PAGE)), (HND, (PAGE, LAYER, KV))])
def test_closed_forms_match_materialized_oracle(inner, outer):
    L = Layout(outer=outer, inner=inner, num_pages=11, num_layers=3, num_kv=2, page_size=4,
               num_heads=2, head_dim=8, dtype_bytes=2, byte_offset=4096)
    seed, pad = 77, 78
    w = synth.Workload(name="t", outer=tuple({PAGE: "page", LAYER: "layer", KV: "kv"}[a]
                                             for a in outer),
                       inner="NHD" if inner == NHD else "HND", num_pages=11, num_layers=3,
                       num_kv=2, page_size=4, num_heads=2, head_dim=8, dtype_bytes=2,
                       pages_per_request=3, seed=seed, byte_offset=4096, alloc_tail=512)
    alloc = synth.pool_alloc_image(w, seed)
    src, dst = [7, 2, 9], [0, 10, 4]
    for l0, l1 in ((0, 3), (1, 2)):
        host = oracle.backup(L, alloc, src, l0, l1)
        lo, hi = l0 * 2 * 3 * L.piece_bytes, l1 * 2 * 3 * L.piece_bytes
        assert oracle.check_backup_gen(L, seed, src, l0, l1, host[lo:hi], lo) == (0, -1)
        # a sub-range starting mid-row
        assert oracle.check_backup_gen(L, seed, src, l0, l1, host[lo + 5:hi - 3], lo + 5)[0] == 0
        bad = host.copy()
        bad[lo + 100] ^= 1
        assert oracle.check_backup_gen(L, seed, src, l0, l1, bad[lo:hi], lo) == (1, lo + 100)
        out = oracle.restore(L, alloc, host, dst, l0, l1)
        assert oracle.check_alloc_roundtrip(L, seed, pad, src, dst, l0, l1, out) == (0, -1)
        assert oracle.check_alloc_roundtrip(L, seed, pad, src, dst, l0, l1, out[100:5000],
                                            100)[0] == 0
        # a changed byte in a destination piece, in an untouched piece, in padding
        for a in (oracle.piece_start(L, dst[1], l0, 1) + 7, oracle.piece_start(L, 5, l0, 0),
                  3, alloc.size - 1):
            b = out.copy()
            b[a] ^= 0x80
            assert oracle.check_alloc_roundtrip(L, seed, pad, src, dst, l0, l1, b) == (1, a)


def test_ready_prefix_is_minimum():
    assert oracle.ready_prefix([5, 3, 7]) == 3
    assert oracle.ready_prefix([256] * 61) == 256
    assert oracle.ready_prefix([64, 64, 0, 64]) == 0
    assert oracle.ready_prefix([9]) == 9


def test_ready_publish_adds_n_to_the_call_slots():
    """Hand-worked counts of a ready object serving several restores (the
    reading of the ticket page's per-layer progress: a count is the pages
    published into its slot since the object was created or reset)."""
    # six slots; a restore of 4 pages over layers [0, 3) published from slot 2
    c = oracle.ready_publish([0] * 6, 2, 0, 3, 4)
    assert c == [0, 0, 4, 4, 4, 0]
    # a second restore into layers [1, 3) of the same slots adds, never overwrites
    c = oracle.ready_publish(c, 2, 1, 3, 4)
    assert c == [0, 0, 4, 8, 8, 0]
    # an empty layer range or n = 0 changes nothing
    assert oracle.ready_publish(c, 2, 2, 2, 4) == c
    assert oracle.ready_publish(c, 0, 0, 6, 0) == c
    # main pool in slots 0-2, a sidecar in slot 3: the prefix waits for both
    c = oracle.ready_publish([0] * 4, 0, 0, 3, 16)
    assert oracle.ready_prefix(c) == 0
    c = oracle.ready_publish(c, 3, 0, 1, 16)
    assert c == [16, 16, 16, 16] and oracle.ready_prefix(c) == 16
    # the next request's main restore alone does not move the prefix
    c = oracle.ready_publish(c, 0, 0, 3, 16)
    assert c == [32, 32, 32, 16] and oracle.ready_prefix(c) == 16
    c = oracle.ready_publish(c, 3, 0, 1, 16)
    assert oracle.ready_prefix(c) == 32
    # 32-bit counts wrap
    assert oracle.ready_publish([2 ** 32 - 1, 7], 0, 0, 1, 2) == [1, 7]


# ---------------------------------------------------------------------------
# slot-addressed host pool
# ---------------------------------------------------------------------------
def numpy_backup_slots(L, alloc, ids, slots, S, l0, l1, host):
    out = host.copy()
    hv = out.reshape(L.num_layers, L.num_kv, S, L.page_size, L.num_heads, L.row_bytes)
    hv[l0:l1, :, np.asarray(slots, dtype=np.int64)] = \
        numpy_pool_view(L, alloc)[l0:l1][:, :, np.asarray(ids, dtype=np.int64)]
    return out


def numpy_restore_slots(L, alloc, host, slots, ids, S, l0, l1):
    out = alloc.copy()
    hv = host.reshape(L.num_layers, L.num_kv, S, L.page_size, L.num_heads, L.row_bytes)
    pv = numpy_pool_view(L, out)
    for l in range(l0, l1):
        pv[l, :, np.asarray(ids, dtype=np.int64)] = \
            hv[l][:, np.asarray(slots, dtype=np.int64)].transpose(1, 0, 2, 3, 4)
    return out


@pytest.mark.parametrize("outer", OUTER_ORDERS)
@pytest.mark.parametrize("inner", [NHD, HND])
def test_slot_backup_restore_match_numpy(outer, inner):
    """Host slots: the oracle equals numpy advanced-index assignment into a
    [layer][kv][slot][token][head][row] view of the host pool, slots that
    no page names keep their bytes, and a restore may read one slot twice."""
    rng = np.random.default_rng(17 + hash((outer, inner)) % 2**32)
    L = rand_layout(rng, outer, inner, offset=32)
    alloc = rand_alloc(rng, L)
    S = 9
    ids, slots = [4, 0, 6, 2], [7, 2, 0, 5]
    host0 = rng.integers(0, 256, L.host_bytes(S), dtype=np.uint8)
    for l0, l1 in ((0, 3), (1, 2)):
        got = oracle.backup_slots(L, alloc, ids, slots, S, l0, l1, host=host0.copy())
        assert np.array_equal(got, numpy_backup_slots(L, alloc, ids, slots, S, l0, l1, host0))
        rs, rd = [7, 7, 3], [1, 5, 3]          # slot 7 read twice
        got = oracle.restore_slots(L, alloc, host0, rs, rd, S, l0, l1)
        assert np.array_equal(got, numpy_restore_slots(L, alloc, host0, rs, rd, S, l0, l1))


def test_slot_brute_force_and_round_trip():
    """Every placement of up to two distinct pages of a 5-page pool into 4
    host slots, and the round trip restore_slots(backup_slots(x)) back into
    other pages: those pages receive the source pages' bytes and nothing
    else changes."""
    L = Layout(outer=(LAYER, PAGE, KV), inner=HND, num_pages=5, num_layers=2, num_kv=2,
               page_size=3, num_heads=2, head_dim=1, dtype_bytes=2, byte_offset=8)
    rng = np.random.default_rng(23)
    alloc = rand_alloc(rng, L)
    S = 4
    host0 = rng.integers(0, 256, L.host_bytes(S), dtype=np.uint8)
    pb = L.piece_bytes
    for k in (1, 2):
        for ids in itertools.permutations(range(5), k):
            for slots in itertools.permutations(range(S), k):
                got = oracle.backup_slots(L, alloc, ids, slots, S, 0, 2, host=host0.copy())
                assert np.array_equal(got, numpy_backup_slots(L, alloc, ids, slots, S, 0, 2, host0))
                dst = [(p + 2) % 5 for p in ids]
                if set(dst) & set(ids):
                    continue
                out = oracle.restore_slots(L, alloc, got, slots, dst, S, 0, 2)
                touched = np.zeros(alloc.size, dtype=bool)
                for s_, d_ in zip(ids, dst):
                    for l in range(2):
                        for c in range(2):
                            a_s, a_d = oracle.piece_start(L, s_, l, c), oracle.piece_start(L, d_, l, c)
                            assert np.array_equal(out[a_d:a_d + pb], alloc[a_s:a_s + pb])
                            touched[a_d:a_d + pb] = True
                assert np.array_equal(out[~touched], alloc[~touched])


def test_identity_slots_are_the_packed_buffer():
    """With slots 0..n-1 and n slots, the host pool is the packed buffer of
    BACKUP / RESTORE (the reading the slot form generalises)."""
    rng = np.random.default_rng(29)
    L = rand_layout(rng, (PAGE, KV, LAYER), NHD, offset=16)
    alloc = rand_alloc(rng, L)
    ids = [6, 1, 3]
    slots = list(range(len(ids)))
    assert np.array_equal(oracle.backup_slots(L, alloc, ids, slots, len(ids), 0, 3),
                          numpy_backup(L, alloc, ids, 0, 3))
    host = rng.integers(0, 256, L.host_bytes(3), dtype=np.uint8)
    assert np.array_equal(oracle.restore_slots(L, alloc, host, slots, [0, 2, 5], 3, 0, 3),
                          numpy_restore(L, alloc, host, [0, 2, 5], 0, 3))
