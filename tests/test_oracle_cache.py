"""Pins of the expert-cache oracle (oracle/cache.py): the step-batched LRU
the GPU cache must reproduce, and Belady's optimum it is compared with.

- the textbook page-replacement example (tests/golden/lru_textbook.txt):
  LRU 12 faults, optimal 9;
- Belady's policy equals an exhaustive search over every eviction choice on
  tiny traces, including steps that need several experts at once;
- LRU's inclusion property on single-expert steps (a cache of S + 1 slots
  always holds what a cache of S holds), which FIFO-like mistakes break;
- LRU never beats the optimum; a cache that holds every expert misses only
  on first use;
- a hand-worked two-expert-per-step case fixes the tie rules (empty slots
  first by index; misses placed in ascending expert id; equal stamps go to
  the lower slot)."""
import os
import random

import pytest

from oracle import cache as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lru_textbook.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        vals[k.strip()] = v.split()
    return [int(x) for x in vals["reference"]], int(vals["frames"][0]), int(vals["lru_faults"][0]), \
        int(vals["opt_faults"][0])


def test_textbook_reference_string():
    ref, frames, lru_f, opt_f = _golden()
    steps = [[p] for p in ref]
    assert sum(s["misses"] for s in oc.lru_replay(steps, frames)) == lru_f
    hits, misses = oc.opt_replay(steps, frames)
    assert misses == opt_f and hits + misses == len(ref)
    assert oc.min_misses_bruteforce(steps, frames) == opt_f


@pytest.mark.parametrize("seed", range(6))
def test_belady_is_the_exhaustive_optimum(seed):
    rng = random.Random(seed)
    for _ in range(40):
        E, S = rng.randint(3, 7), rng.randint(2, 4)
        k = rng.randint(1, min(2, S))
        steps = [rng.sample(range(E), k) for _ in range(rng.randint(2, 9))]
        _, m = oc.opt_replay(steps, S)
        assert m == oc.min_misses_bruteforce(steps, S), (steps, S)


@pytest.mark.parametrize("seed", range(4))
def test_lru_inclusion_and_bounds(seed):
    rng = random.Random(100 + seed)
    E = 12
    steps = [[rng.randrange(E)] for _ in range(200)]
    runs = {S: oc.lru_replay(steps, S) for S in range(1, E + 1)}
    for S in range(1, E):
        for a, b in zip(runs[S], runs[S + 1]):
            assert set(a["slot_of"]) <= set(b["slot_of"])
    for S in range(1, E + 1):
        lm = sum(s["misses"] for s in runs[S])
        assert lm >= oc.opt_replay(steps, S)[1]
        if S == E:
            assert lm == len({e for st in steps for e in st})  # first uses only


def test_batched_tie_rules_hand_worked():
    # 3 slots; steps of two experts
    steps = [[5, 2], [2, 7], [9, 1], [1, 2]]
    r = oc.lru_replay(steps, 3)
    # step 1: misses 2, 5 (ascending) -> empty slots 0, 1
    assert r[0]["expert_in"] == [2, 5, -1] and (r[0]["hits"], r[0]["misses"]) == (0, 2)
    # step 2: 2 hits (slot 0); 7 takes the empty slot 2
    assert r[1]["expert_in"] == [2, 5, 7] and (r[1]["hits"], r[1]["misses"]) == (1, 1)
    # step 3: misses 1, 9; unhit slots by (time, index): slot 1 (t1), then
    # slots 0 and 2 (both t2) -> slot 0 first
    assert r[2]["expert_in"] == [9, 1, 7] and (r[2]["hits"], r[2]["misses"]) == (0, 2)
    # step 4: 1 hits (slot 1); 2 misses and takes the oldest unhit: slot 2 (t2)
    assert r[3]["expert_in"] == [9, 1, 2] and r[3]["slot_of"] == {9: 0, 1: 1, 2: 2}


def test_step_larger_than_cache_is_refused():
    with pytest.raises(ValueError):
        oc.lru_replay([[1, 2, 3]], 2)
