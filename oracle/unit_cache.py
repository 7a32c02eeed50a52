"""Unit cache oracle -- TEST INFRASTRUCTURE ONLY (imported by tests/ and
nothing else; it imports nothing from the HIP product package).

The GPU-resident cache of memory units in front of a host-resident unit
pool (InfLLM Guide, "Core Innovation 3": a least-recently-used pool of hot
units in GPU memory, every unit's full K/V in host memory, a miss copied in
over the host link).  The pages fix only "least recently used"; this module
states the policy in full (the reading the kernels follow), as plain Python
over one (sequence, KV head):

  state: C slots; unit_of[c] (unit or -1), stamp[c] (the last step that used
         the slot, 0 = never), slot_of[u] (slot or -1).
  fetch(step, units): units = the ids a call selects for this head (any
         number of positions; -1 entries ignored, repeats counted once),
         at most C distinct; step >= 1 and larger than every earlier step.
    1. hits: each selected unit already cached gets stamp = step;
    2. misses: the other selected units, in ascending unit order;
    3. victims: the slots whose stamp is below step (not used by this call),
       least recently used first -- ascending (stamp, slot), so empty slots
       (stamp 0) go first, lower slot first among equals;
    4. the i-th miss takes the i-th victim: the victim's old unit (if any)
       leaves the cache, the miss moves in with stamp = step.
  Returns (hits, misses, [(slot, unit) filled]).
"""
from __future__ import annotations


class UnitCache:
    def __init__(self, n_slots: int, n_units: int):
        self.C, self.U = n_slots, n_units
        self.unit_of = [-1] * n_slots
        self.stamp = [0] * n_slots
        self.slot_of = [-1] * n_units

    def fetch(self, step: int, units):
        chosen = sorted({int(u) for u in units if int(u) >= 0})
        assert step >= 1 and all(step > s for s in self.stamp)
        assert len(chosen) <= self.C and all(u < self.U for u in chosen)
        hits = [u for u in chosen if self.slot_of[u] >= 0]
        misses = [u for u in chosen if self.slot_of[u] < 0]
        for u in hits:
            self.stamp[self.slot_of[u]] = step
        victims = sorted((c for c in range(self.C) if self.stamp[c] < step),
                         key=lambda c: (self.stamp[c], c))
        filled = []
        for u, c in zip(misses, victims):
            old = self.unit_of[c]
            if old >= 0:
                self.slot_of[old] = -1
            self.unit_of[c] = u
            self.slot_of[u] = c
            self.stamp[c] = step
            filled.append((c, u))
        return len(hits), len(misses), filled

    def resident(self) -> set:
        return {u for u in self.unit_of if u >= 0}
