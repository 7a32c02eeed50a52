"""Pins of the unit cache oracle (oracle/unit_cache.py; InfLLM Guide, "Core
Innovation 3": a least-recently-used pool of hot units in GPU memory).

Each pin takes the cache class, so the mutant test at the end can run the
same pins against a copy of the oracle with one plausible mistake planted:
  - one unit per step: the textbook LRU cache (an ordered dict, move to the
    end on a hit, evict the front when full), with slots reused in place;
  - batches of units per step: every chosen unit resident afterwards, hit
    and miss counts by set arithmetic, evictions only of unchosen units and
    only of the least recently used ones, tables consistent;
  - closed cases: no eviction when the cache holds every unit; a cycle over
    C + 1 units misses every time; a full replacement; a hand-worked tie.
"""
import importlib.util
import os
import random
from collections import OrderedDict

import pytest

from oracle.unit_cache import UnitCache

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def pin_single_access_is_textbook_lru(cls):
    rng = random.Random(1)
    for C, U, n in ((1, 5, 60), (4, 12, 400), (16, 40, 2000), (8, 8, 200)):
        cache = cls(C, U)
        lru = OrderedDict()          # unit -> slot, least recent first
        for step in range(1, n + 1):
            # locality: mostly recent units, sometimes any unit
            u = rng.randrange(U) if rng.random() < 0.3 or not lru else \
                rng.choice(list(lru)[-min(len(lru), 6):])
            if u in lru:
                lru.move_to_end(u)
                want = (1, 0, [])
            else:
                if len(lru) == C:
                    _, slot = lru.popitem(last=False)
                else:
                    slot = len(lru)          # slots fill in order while empty
                lru[u] = slot
                want = (0, 1, [(slot, u)])
            assert cache.fetch(step, [u]) == want, (C, U, step, u)
            assert cache.resident() == set(lru)


def pin_batch_invariants(cls):
    rng = random.Random(2)
    for C, U, k in ((8, 30, 3), (32, 200, 12), (64, 1000, 32), (5, 6, 5)):
        cache = cls(C, U)
        for step in range(1, 300):
            before = cache.resident()
            stamp_before = {cache.unit_of[c]: cache.stamp[c] for c in range(C)
                            if cache.unit_of[c] >= 0}
            # a selection of k ids with -1 pads and repeats, overlapping the
            # residents about half the time
            pool = list(before) if before and rng.random() < 0.5 else list(range(U))
            chosen = rng.sample(pool, min(k, len(pool)))
            extra = rng.sample(range(U), max(0, k - len(chosen)))
            ids = (chosen + extra)[:k]
            ids = ids + [-1, ids[0]] if ids else [-1]
            want = {u for u in ids if u >= 0}
            if len(want) > C:
                continue
            hits, misses, filled = cache.fetch(step, ids)
            after = cache.resident()
            assert want <= after
            assert len(after) <= C
            assert hits == len(want & before) and misses == len(want - before)
            assert sorted(u for _, u in filled) == sorted(want - before)
            evicted = before - after
            assert not (evicted & want)
            kept_unchosen = (before & after) - want
            for e in evicted:   # least recently used first
                assert all(stamp_before[e] <= stamp_before[x] for x in kept_unchosen)
            for c in range(C):
                u = cache.unit_of[c]
                if u >= 0:
                    assert cache.slot_of[u] == c
                    assert cache.stamp[c] <= step
            assert sum(1 for u in range(U) if cache.slot_of[u] >= 0) == len(after)


def pin_closed_cases(cls):
    # (1) the cache holds every unit: misses = distinct units, no eviction
    rng = random.Random(3)
    cache = cls(50, 50)
    seen, total_hits, total_miss, n_acc = set(), 0, 0, 0
    for step in range(1, 200):
        ids = rng.sample(range(50), 7)
        h, m, _ = cache.fetch(step, ids)
        total_hits += h
        total_miss += m
        n_acc += 7
        seen |= set(ids)
    assert total_miss == len(seen) and total_hits == n_acc - len(seen)
    # (2) a cycle over C + 1 units, one per step: LRU misses every time
    C = 6
    cache = cls(C, C + 1)
    for step in range(1, 10 * (C + 1)):
        assert cache.fetch(step, [(step - 1) % (C + 1)])[1] == 1
    # (3) a full cache replaced by C new units in one step: every slot
    # refilled, units to slots in ascending order
    cache = cls(4, 10)
    cache.fetch(1, [0, 1, 2, 3])
    assert cache.fetch(2, [9, 8, 7, 6]) == (0, 4, [(0, 6), (1, 7), (2, 8), (3, 9)])
    # (4) a hand-worked case: stamps after steps 1-3 are slot0:u5@1, slot1:u2@2,
    # slot2:u7@2, slot3:u1@3; step 4 uses u2 and needs two slots: the least
    # recent unchosen are slot0 (stamp 1), then slot2 (stamp 2, u7) -- slot1
    # holds the chosen u2
    cache = cls(4, 10)
    cache.fetch(1, [5])
    cache.fetch(2, [2, 7])
    cache.fetch(3, [1])
    assert cache.unit_of == [5, 2, 7, 1]
    assert cache.fetch(4, [4, 2, 3]) == (1, 2, [(0, 3), (2, 4)])
    assert cache.unit_of == [3, 2, 4, 1] and cache.stamp == [4, 4, 4, 3]
    # (5) -1 entries and repeats count once
    cache = cls(3, 5)
    assert cache.fetch(1, [-1, 2, 2, -1]) == (0, 1, [(0, 2)])
    assert cache.fetch(2, [2, -1, 2]) == (1, 0, [])


PINS = [pin_single_access_is_textbook_lru, pin_batch_invariants, pin_closed_cases]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_cache_pin(pin):
    pin(UnitCache)


# (name, exact source text, replacement)
MUTANTS = [
    ("no_refresh_on_hit", "            self.stamp[self.slot_of[u]] = step\n",
     "            pass\n"),
    ("most_recent_first", "key=lambda c: (self.stamp[c], c))",
     "key=lambda c: (-self.stamp[c], c))"),
    ("ties_higher_slot", "key=lambda c: (self.stamp[c], c))",
     "key=lambda c: (self.stamp[c], -c))"),
    ("victims_before_hits",
     "        for u in hits:\n            self.stamp[self.slot_of[u]] = step\n        victims = sorted((c for c in range(self.C) if self.stamp[c] < step),\n                         key=lambda c: (self.stamp[c], c))\n",
     "        victims = sorted((c for c in range(self.C) if self.stamp[c] < step),\n                         key=lambda c: (self.stamp[c], c))\n        for u in hits:\n            self.stamp[self.slot_of[u]] = step\n"),
    ("old_unit_not_released", "                self.slot_of[old] = -1\n", "                pass\n"),
    ("misses_in_given_order",
     "misses = [u for u in chosen if self.slot_of[u] < 0]",
     "misses = [u for u in dict.fromkeys(int(x) for x in units if int(x) >= 0) if self.slot_of[u] < 0]"),
    ("fill_without_stamp", "            self.stamp[c] = step\n            filled.append",
     "            filled.append"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_cache_pins_kill_mutant(tmp_path, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "unit_cache.py")).read()
    assert src.count(old) >= 1, "mutation site vanished: " + name
    path = tmp_path / "mutant_cache.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("mutant_cache", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = 0
    for pin in PINS:
        try:
            pin(mod.UnitCache)
        except (AssertionError, IndexError, ValueError):
            failed += 1
    assert failed > 0, "mutant %s survived the cache pins" % name
