"""Reference policy of the HBM expert cache, in plain Python.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): used by tests/ to check
the library's cache planner, never by the product path.

The osrepos summary ("SSD Streaming for Large Models") runs models larger
than GPU memory by loading routed MoE experts from disk as they are needed,
with a cache of experts whose size the user sets.  The pages fix no
replacement policy; the reading taken is least-recently-used over decode
steps:

  * A step needs the distinct experts of its top-k choices, in order of first
    appearance (row-major over the [T, k] choices); ids outside [0, E) are
    skipped.
  * Needed experts already resident are hits.  Each miss takes a free slot if
    one exists, else evicts the resident expert used least recently among
    those the step does not need and that were not used in the last `keep`
    steps (they may still be in use by work in flight).
  * Recency: after the step every needed expert counts as used at this step,
    later-appearing ones more recently than earlier ones.
  * A step whose needs cannot be met (more distinct experts than slots that
    are free or evictable) is an error and changes nothing.

Which free slot a miss takes is not part of the policy (the library takes the
lowest free index); what is fixed is the resident set and the misses of each
step.
"""
from __future__ import annotations


class LruExpertCache:
    def __init__(self, n_experts: int, n_slots: int, keep: int = 0):
        assert n_slots >= 1 and keep >= 0
        self.E, self.n, self.keep = n_experts, n_slots, keep
        self.resident: dict[int, tuple[int, int]] = {}   # expert -> (step, order) of its last use
        self.step = 0

    def needed(self, ids) -> list[int]:
        out, seen = [], set()
        for e in ids:
            e = int(e)
            if 0 <= e < self.E and e not in seen:
                seen.add(e)
                out.append(e)
        return out

    def plan(self, ids):
        """Returns (hits, misses, evicted) in the order decided; raises
        ValueError when the step cannot be served."""
        need = self.needed(ids)
        step = self.step + 1
        hits = [e for e in need if e in self.resident]
        misses = [e for e in need if e not in self.resident]
        free = self.n - len(self.resident)
        protected = set(need) | {e for e, (s, _) in self.resident.items() if s > step - 1 - self.keep}
        victims = sorted((u, e) for e, u in self.resident.items() if e not in protected)
        n_evict = max(0, len(misses) - free)
        if n_evict > len(victims):
            raise ValueError("more distinct experts than free or evictable slots")
        evicted = [e for _, e in victims[:n_evict]]
        for e in evicted:
            del self.resident[e]
        for order, e in enumerate(need):
            self.resident[e] = (step, order)
        self.step = step
        return hits, misses, evicted
