"""Executable model of the host tier's slot allocator and residency protocol.

TEST INFRASTRUCTURE ONLY: the tests compare the runtime's tier (C ABI) with
this model operation by operation; the product path never imports it.

What it models. The out-of-process HiCache RFC (SGLang issue #37372,
section "Ownership") gives host KV physical allocation to the data plane and
keeps cache semantics with the scheduler's index, and leaves open how the
two sides agree on eviction and invalidation so that a lookup is never
answered from an outdated view. The pages fix no algorithm for it; the
reading taken here is the plainest one that makes every answer current:

  * a slot is FREE, WRITING (a backup in flight: invisible to lookups,
    never evicted) or RESIDENT (readable; a lookup hit pins it until the
    restore releases it);
  * only RESIDENT entries without pins are evicted, least recently used
    first, and only when no slot is free; the lowest free slot is taken
    first; keys named by the reserving call are never its victims;
  * recency is a clock: every key a reserve names, every commit and every
    lookup hit takes the next clock value;
  * invalidation hides a key at once; its slot is freed when its last pin
    or its backup in flight ends.

Written as plain lists and linear scans so that it can be checked by eye.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

FREE, WRITING, RESIDENT = 0, 1, 2


class TierError(Exception):
    def __init__(self, kind: str):
        super().__init__(kind)
        self.kind = kind          # "full", "inval" or "range"


@dataclass
class Slot:
    key: int = 0
    state: int = FREE
    pins: int = 0
    doomed: bool = False
    last: int = 0


@dataclass
class TierModel:
    num_slots: int
    slots: List[Slot] = field(default_factory=list)
    clock: int = 0
    evictions: int = 0

    def __post_init__(self):
        self.slots = [Slot() for _ in range(self.num_slots)]

    # -- helpers ------------------------------------------------------------
    def find(self, key: int) -> Optional[int]:
        """Slot of a key that is present (not FREE, not invalidated)."""
        for s, x in enumerate(self.slots):
            if x.state != FREE and not x.doomed and x.key == key:
                return s
        return None

    def tick(self) -> int:
        self.clock += 1
        return self.clock

    def evictable(self, s: int) -> bool:
        x = self.slots[s]
        return x.state == RESIDENT and x.pins == 0 and not x.doomed

    # -- operations -----------------------------------------------------------
    def reserve(self, keys: Sequence[int]) -> Tuple[List[int], List[int]]:
        present = {self.find(k) for k in keys} - {None}
        new_keys = {k for k in keys if self.find(k) is None}
        free = [s for s in range(self.num_slots) if self.slots[s].state == FREE]
        victims = [s for s in range(self.num_slots) if self.evictable(s) and s not in present]
        if len(new_keys) > len(free) + len(victims):
            raise TierError("full")
        out, evicted = [], []
        for k in keys:
            s = self.find(k)
            if s is not None:
                self.slots[s].last = self.tick()
                out.append(-1)
                continue
            free = [t for t in range(self.num_slots) if self.slots[t].state == FREE]
            if free:
                s = free[0]
            else:
                cands = [t for t in range(self.num_slots) if self.evictable(t) and t not in present]
                s = min(cands, key=lambda t: self.slots[t].last)
                evicted.append(self.slots[s].key)
                self.evictions += 1
            self.slots[s] = Slot(key=k, state=WRITING, last=self.tick())
            out.append(s)
        return out, evicted

    def _check_writing(self, slots: Sequence[int]) -> None:
        seen = set()
        for s in slots:
            if s == -1:
                continue
            if not 0 <= s < self.num_slots:
                raise TierError("range")
            if self.slots[s].state != WRITING or s in seen:
                raise TierError("inval")
            seen.add(s)

    def commit(self, slots: Sequence[int]) -> None:
        self._check_writing(slots)
        for s in slots:
            if s == -1:
                continue
            if self.slots[s].doomed:
                self.slots[s] = Slot()
            else:
                self.slots[s].state = RESIDENT
                self.slots[s].last = self.tick()

    def abort(self, slots: Sequence[int]) -> None:
        self._check_writing(slots)
        for s in slots:
            if s != -1:
                self.slots[s] = Slot()

    def lookup(self, keys: Sequence[int]) -> List[int]:
        out = []
        for k in keys:
            s = self.find(k)
            if s is None or self.slots[s].state != RESIDENT:
                out.append(-1)
                continue
            self.slots[s].pins += 1
            self.slots[s].last = self.tick()
            out.append(s)
        return out

    def release(self, slots: Sequence[int]) -> None:
        named = [s for s in slots if s != -1]
        for s in named:
            if not 0 <= s < self.num_slots:
                raise TierError("range")
        for s in set(named):
            if self.slots[s].state != RESIDENT or self.slots[s].pins < named.count(s):
                raise TierError("inval")
        for s in named:
            self.slots[s].pins -= 1
            if self.slots[s].pins == 0 and self.slots[s].doomed:
                self.slots[s] = Slot()

    def invalidate(self, keys: Sequence[int]) -> int:
        dropped = 0
        for k in keys:
            s = self.find(k)
            if s is None:
                continue
            x = self.slots[s]
            if x.state == RESIDENT and x.pins == 0:
                self.slots[s] = Slot()
            else:
                x.doomed = True
            dropped += 1
        return dropped

    def info(self) -> Dict[str, int]:
        xs = self.slots
        return {"num_slots": self.num_slots,
                "free_slots": sum(x.state == FREE for x in xs),
                "writing": sum(x.state == WRITING for x in xs),
                "resident": sum(x.state == RESIDENT for x in xs),
                "pinned": sum(x.state == RESIDENT and x.pins > 0 for x in xs),
                "doomed": sum(x.doomed for x in xs),
                "evictions": self.evictions}

    def view(self) -> List[Tuple[int, int, int]]:
        """(key, state, pins) of every slot."""
        return [(x.key, x.state, x.pins) for x in self.slots]
