"""The host tier's slot allocator and residency protocol (CPU only).

Hand-worked scenarios state the expected slots, evictions and states of
each step, and run against both the runtime's tier (through the C ABI) and
the model in oracle/tier_model.py; seeded random operation sequences then
compare the two step by step: every output, every error and the key, state
and pins of every slot."""
import numpy as np
import pytest

from oracle.tier_model import FREE, RESIDENT, WRITING, TierError, TierModel
from paged_kv_offload_amd import kvx as K

_KIND = {K.KVX_E_FULL: "full", K.KVX_E_INVAL: "inval", K.KVX_E_RANGE: "range"}


class CTier:
    """The runtime's tier behind the model's interface."""

    def __init__(self, num_slots, generation=1):
        self.h = K.kvx_tier_create(num_slots, generation)
        self.num_slots = num_slots

    def _call(self, fn, *a):
        try:
            return fn(self.h, *a)
        except K.KvxError as e:
            if e.code in _KIND:
                raise TierError(_KIND[e.code]) from None
            raise

    def reserve(self, keys):
        slots, ev = self._call(K.kvx_tier_reserve, keys)
        return slots.tolist(), ev.tolist()

    def commit(self, slots):
        self._call(K.kvx_tier_commit, slots)

    def abort(self, slots):
        self._call(K.kvx_tier_abort, slots)

    def lookup(self, keys):
        return self._call(K.kvx_tier_lookup, keys).tolist()

    def release(self, slots):
        self._call(K.kvx_tier_release, slots)

    def invalidate(self, keys):
        return self._call(K.kvx_tier_invalidate, keys)

    def info(self):
        d = K.kvx_tier_get_info(self.h)
        d.pop("generation")
        return d

    def view(self):
        return [K.kvx_tier_slot(self.h, s) for s in range(self.num_slots)]

    def close(self):
        K.kvx_tier_destroy(self.h)


@pytest.fixture(params=["runtime", "model"])
def make(request):
    made = []

    def new(num_slots):
        t = CTier(num_slots) if request.param == "runtime" else TierModel(num_slots)
        made.append(t)
        return t
    yield new
    for t in made:
        if isinstance(t, CTier):
            t.close()


A, B, C, D = 0xA, 0xB, 0xC, 0xD


def test_lru_eviction_order(make):
    t = make(3)
    assert t.reserve([A, B, C]) == ([0, 1, 2], [])     # clock 1, 2, 3
    t.commit([0, 1, 2])                                 # clock 4, 5, 6
    assert t.lookup([A]) == [0]                         # A touched: 7
    t.release([0])
    assert t.reserve([D]) == ([1], [B])                 # B (5) is the oldest
    assert t.lookup([B]) == [-1]
    assert t.view()[1] == (D, WRITING, 0)
    t.commit([1])
    assert t.reserve([B]) == ([2], [C])                 # C (6) before A (7), D (9)
    assert t.info()["evictions"] == 2


def test_pins_block_eviction_and_full_changes_nothing(make):
    t = make(2)
    assert t.reserve([A, B]) == ([0, 1], [])
    t.commit([0, 1])
    assert t.lookup([A, B]) == [0, 1]
    before = (t.view(), t.info())
    with pytest.raises(TierError) as e:
        t.reserve([C])
    assert e.value.kind == "full"
    assert (t.view(), t.info()) == before
    t.release([1])
    assert t.reserve([C]) == ([1], [B])
    assert t.view() == [(A, RESIDENT, 1), (C, WRITING, 0)]


def test_keys_named_by_a_reserve_are_not_its_victims(make):
    t = make(2)
    t.reserve([A, B])
    t.commit([0, 1])                                    # A older than B
    assert t.reserve([A, C]) == ([-1, 1], [B])          # A touched and kept
    t.commit([1])
    with pytest.raises(TierError) as e:                  # A and C named: no victim for D
        t.reserve([A, C, D])
    assert e.value.kind == "full"


def test_a_named_key_later_in_the_call_is_not_a_victim(make):
    t = make(2)
    t.reserve([A, B])
    t.commit([0, 1])                                    # A older than B
    assert t.reserve([C, A]) == ([1, -1], [B])          # A is the oldest but named


def test_commit_counts_as_a_use(make):
    t = make(2)
    assert t.reserve([A, B]) == ([0, 1], [])            # A 1, B 2
    t.commit([1])                                       # B 3
    t.commit([0])                                       # A 4: now the newer one
    assert t.reserve([C]) == ([1], [B])


def test_writing_entries_miss_until_committed(make):
    t = make(4)
    assert t.reserve([A, A, B]) == ([0, -1, 1], [])     # the repeat is present by then
    assert t.lookup([A, B]) == [-1, -1]
    t.commit([-1, 0])
    assert t.lookup([A, B]) == [0, -1]
    t.abort([1])
    assert t.view()[1] == (0, FREE, 0)
    assert t.info() == {"num_slots": 4, "free_slots": 3, "writing": 0, "resident": 1,
                        "pinned": 1, "doomed": 0, "evictions": 0}


def test_invalidation_waits_for_pins_and_backups(make):
    t = make(3)
    t.reserve([A, B])
    t.commit([0])
    assert t.lookup([A, A]) == [0, 0]                   # two pins
    assert t.invalidate([A, B, C]) == 2                 # A pinned, B writing, C absent
    assert t.lookup([A]) == [-1]
    assert t.info()["doomed"] == 2
    assert t.reserve([A]) == ([2], [])                  # a fresh copy in another slot
    t.commit([1])                                       # B's backup ends: slot freed
    assert t.view()[1] == (0, FREE, 0)
    t.release([0])
    assert t.view()[0] == (A, RESIDENT, 1)
    t.release([0])                                      # last pin: freed
    assert t.view()[0] == (0, FREE, 0)
    t.commit([2])
    assert t.lookup([A]) == [2]


def test_bad_commit_release_change_nothing(make):
    t = make(3)
    t.reserve([A, B])
    t.commit([0])
    t.lookup([A])
    before = (t.view(), t.info())
    for op, arg, kind in ((t.commit, [0], "inval"),          # not writing
                          (t.commit, [1, 1], "inval"),       # named twice
                          (t.commit, [1, 3], "range"),
                          (t.abort, [2], "inval"),           # free slot
                          (t.release, [0, 0], "inval"),      # one pin only
                          (t.release, [1], "inval"),         # writing, no pin
                          (t.release, [-2], "range")):
        with pytest.raises(TierError) as e:
            op(arg)
        assert e.value.kind == kind, (op, arg)
        assert (t.view(), t.info()) == before


def test_runtime_tier_lifecycle():
    h = K.kvx_tier_create(2, 5)
    assert K.kvx_tier_get_info(h)["generation"] == 5
    K.kvx_tier_destroy(h)
    with pytest.raises(K.KvxError) as e:
        K.kvx_tier_lookup(h, [1])
    assert e.value.code == K.KVX_E_STALE
    K.kvx_tier_destroy(h)                                # logged, not an error
    K.kvx_tier_destroy(0)
    with pytest.raises(K.KvxError) as e:
        K.kvx_tier_create(-1, 0)
    assert e.value.code == K.KVX_E_RANGE
    with pytest.raises(K.KvxError) as e:
        K.kvx_tier_lookup(0x1234, [1])
    assert e.value.code == K.KVX_E_INVAL


@pytest.mark.parametrize("seed", range(40))
def test_runtime_matches_model_on_random_sequences(seed):
    rng = np.random.default_rng(1000 + seed)
    S = int(rng.integers(1, 7))
    keys = list(range(1, int(rng.integers(2, 3 * S + 3))))
    c, m = CTier(S), TierModel(S)
    held, writing = [], []         # slots returned by lookups / reserves
    try:
        for step in range(120):
            op = rng.choice(["reserve", "commit", "abort", "lookup", "release", "invalidate",
                             "bad"], p=[0.25, 0.15, 0.05, 0.2, 0.15, 0.1, 0.1])
            if op in ("reserve", "lookup", "invalidate"):
                arg = [int(k) for k in rng.choice(keys, int(rng.integers(0, S + 2)))]
            elif op in ("commit", "abort"):
                rng.shuffle(writing)
                k = int(rng.integers(0, len(writing) + 1))
                arg, writing = writing[:k], writing[k:]
            elif op == "release":
                rng.shuffle(held)
                k = int(rng.integers(0, len(held) + 1))
                arg, held = held[:k], held[k:]
            else:
                op = str(rng.choice(["commit", "abort", "release"]))
                arg = [int(s) for s in rng.integers(-2, S + 1, int(rng.integers(1, 4)))]
            results = []
            for t in (c, m):
                try:
                    results.append(("ok", getattr(t, op)(arg)))
                except TierError as e:
                    results.append(("err", e.kind))
            assert results[0] == results[1], (step, op, arg, results)
            if results[0][0] == "ok":
                if op == "reserve":
                    writing += [s for s in results[0][1][0] if s >= 0]
                elif op == "lookup":
                    held += [s for s in results[0][1] if s >= 0]
            # commits and aborts may fail when a slot left WRITING another way
            writing = [s for s in writing if m.slots[s].state == WRITING]
            assert c.view() == m.view(), (step, op, arg)
            assert c.info() == m.info(), (step, op, arg)
    finally:
        c.close()
