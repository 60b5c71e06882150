"""Pins of the expert-cache policy oracle (oracle/expert_cache.py) against
hand-worked sequences and an independent recency-list simulation.

The policy is the reading the oracle states for the osrepos summary's "SSD
Streaming for Large Models" (routed experts loaded on demand into a cache of
a set size): least-recently-used over decode steps, the experts of the step
and of the last `keep` steps never evicted, free slots used first.
"""
import numpy as np
import pytest

from oracle.expert_cache import LruExpertCache


def test_hand_worked_lru_sequence():
    c = LruExpertCache(8, 3)
    assert c.plan([0, 1]) == ([], [0, 1], [])
    assert c.plan([2, 0]) == ([0], [2], [])                 # a free slot is left
    assert c.plan([3]) == ([], [3], [1])                    # 1 was used at step 1, 0 and 2 at step 2
    assert c.plan([1, 2]) == ([2], [1], [0])                # 0 (step 2, second) before 3 (step 3)
    assert c.plan([4, 5, 6]) == ([], [4, 5, 6], [3, 1, 2])  # all three; 1 before 2 (order within step 4)
    # repeated ids count once, ids outside [0, E) are skipped
    assert c.plan([4, 7, 9, -1, 4]) == ([4], [7], [5])
    assert set(c.resident) == {4, 6, 7}


def test_hand_worked_keep_previous_step():
    c = LruExpertCache(16, 4, keep=1)
    assert c.plan([0, 1]) == ([], [0, 1], [])
    assert c.plan([2, 3]) == ([], [2, 3], [])
    assert c.plan([4]) == ([], [4], [0])                    # 2, 3 (previous step) are kept
    assert c.plan([5, 6]) == ([], [5, 6], [1, 2])           # 4 (previous step) is kept
    before = (dict(c.resident), c.step)
    with pytest.raises(ValueError):
        c.plan([7, 8, 9])                                   # 3 misses, only 3 and 4 evictable
    assert (dict(c.resident), c.step) == before             # a refused step changes nothing


def _recency_list_sim(E, n, keep, steps):
    """Independent LRU: a recency list (front = least recent), per-step
    protection by an explicit window of the last `keep` steps' sets."""
    order, history, out = [], [], []
    for ids in steps:
        need = []
        for e in ids:
            if 0 <= e < E and e not in need:
                need.append(e)
        recent = set().union(*history[-keep:]) if keep else set()
        misses = [e for e in need if e not in order]
        n_evict = max(0, len(order) + len(misses) - n)
        cand = [e for e in order if e not in need and e not in recent]
        if n_evict > len(cand):
            out.append(None)
            continue
        evicted = cand[:n_evict]
        order = [e for e in order if e not in evicted and e not in need] + need
        history.append(set(need))
        out.append(([e for e in need if e not in misses], misses, evicted))
    return out


@pytest.mark.parametrize("E,n,keep,k", [(8, 3, 0, 2), (32, 8, 0, 4), (32, 16, 1, 4), (256, 64, 1, 8),
                                        (64, 8, 0, 8)])
def test_matches_recency_list_simulation(E, n, keep, k):
    rng = np.random.default_rng(E * 100 + n + keep)
    steps = []
    for _ in range(300):
        T = int(rng.integers(1, 3))
        # skewed: half the draws from a small hot set
        hot = rng.random((T, k)) < 0.5
        ids = np.where(hot, rng.integers(0, max(2, E // 8), (T, k)), rng.integers(0, E, (T, k)))
        steps.append(ids.reshape(-1).tolist())
    want = _recency_list_sim(E, n, keep, steps)
    c = LruExpertCache(E, n, keep)
    for ids, w in zip(steps, want):
        if w is None:
            with pytest.raises(ValueError):
                c.plan(ids)
        else:
            assert c.plan(ids) == w
        assert len(c.resident) <= n


# Planted mistakes in a copy of the policy: each must fail a pin above.
MUTATIONS = {
    "evicts_most_recent": ("victims = sorted((u, e)", "victims = sorted(((-u[0], -u[1]), e)"),
    "ignores_keep": ("if s > step - 1 - self.keep}", "if s > step - 1}"),
    "order_within_step_reversed": ("self.resident[e] = (step, order)", "self.resident[e] = (step, -order)"),
    "duplicates_counted": ("if 0 <= e < self.E and e not in seen:", "if 0 <= e < self.E:"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_planted_policy_mistake(name):
    import types
    import oracle.expert_cache as real
    src = open(real.__file__).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1
    mod = types.ModuleType("cache_mutant")
    exec(compile(src.replace(old, new), real.__file__ + " (mutant)", "exec"), mod.__dict__)
    g = globals()
    saved = g["LruExpertCache"]
    g["LruExpertCache"] = mod.LruExpertCache
    failed = 0
    try:
        for t in (test_hand_worked_lru_sequence, test_hand_worked_keep_previous_step,
                  lambda: test_matches_recency_list_simulation(32, 16, 1, 4),
                  lambda: test_matches_recency_list_simulation(32, 8, 0, 4)):
            try:
                t()
            except (Exception, pytest.fail.Exception):     # an assertion, or a missing expected error
                failed += 1
    finally:
        g["LruExpertCache"] = saved
    assert failed, f"no pin rejects {name}"
