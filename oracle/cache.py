"""Expert-cache policies on a trace of steps -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py`` may import this
module; it shares nothing with the HIP library.

The pages' engine keeps hot experts in a bounded memory and evicts the least
recently used one, fetching a step's missing experts together before the
step's matrix work (fiv.co.kr "kimi-k3-in-c deep dive", "four reductions",
expert LRU cache paragraph; the same page compares that policy's hit rate
with Belady's offline optimum on a recorded expert trace).  The recorded
trace is not available here; these functions replay any trace of steps,
each step a collection of expert ids.

Reading (the pages give the policy, not its tie rules): a step needs the
distinct ids it selects.  Resident needed experts are hits and become most
recent.  Misses are placed in ascending expert id; each takes, among the
slots the step has not hit, the one used longest ago -- never-used (empty)
slots count as used at time 0, and equal times go to the lower slot index.
Placed experts are stamped with the step's time as well.  This is the LRU
rule with time stamps; the GPU keeps the same order as an explicit recency
list, so the two are different formulations of one policy.
"""
from __future__ import annotations


def lru_replay(steps, n_slots: int):
    """Replay step-batched LRU.  Returns a list with one dict per step:
    hits, misses, slot_of (expert -> slot, resident experts only) and
    expert_in (slot -> expert or -1), the state after the step."""
    last_use = [0] * n_slots
    expert_in = [-1] * n_slots
    slot_of = {}
    out = []
    for t, ids in enumerate(steps, start=1):
        need = sorted(set(int(e) for e in ids))
        if len(need) > n_slots:
            raise ValueError(f"step {t} needs {len(need)} experts, more than {n_slots} slots")
        hits = [e for e in need if e in slot_of]
        misses = [e for e in need if e not in slot_of]
        for e in hits:
            last_use[slot_of[e]] = t
        # slots the step has not hit, oldest first (time, then index)
        free = sorted((s for s in range(n_slots) if last_use[s] < t), key=lambda s: (last_use[s], s))
        for r, e in enumerate(misses):
            s = free[r]
            old = expert_in[s]
            if old >= 0:
                del slot_of[old]
            expert_in[s] = e
            slot_of[e] = s
            last_use[s] = t
        out.append({"hits": len(hits), "misses": len(misses), "slot_of": dict(slot_of),
                    "expert_in": list(expert_in)})
    return out


def opt_replay(steps, n_slots: int):
    """Belady's offline policy on the same step batches: on a miss, evict
    the resident expert (not needed by the current step) whose next use is
    furthest away, never-used-again first, ties to the lower expert id.
    Returns the total (hits, misses)."""
    from bisect import bisect_right
    steps = [sorted(set(int(e) for e in ids)) for ids in steps]
    uses = {}
    for t, need in enumerate(steps):
        for e in need:
            uses.setdefault(e, []).append(t)
    never = len(steps) + 1

    def next_use(x, t):  # first step after t that needs x
        u = uses[x]
        i = bisect_right(u, t)
        return u[i] if i < len(u) else never

    resident = set()
    hits = misses = 0
    for t, need in enumerate(steps):
        needset = set(need)
        for e in need:
            if e in resident:
                hits += 1
                continue
            misses += 1
            if len(resident) >= n_slots:
                cands = [x for x in resident if x not in needset]
                victim = max(cands, key=lambda x: (next_use(x, t), -x))
                resident.remove(victim)
            resident.add(e)
    return hits, misses


def min_misses_bruteforce(steps, n_slots: int) -> int:
    """The fewest misses any eviction choice achieves (demand fetching, a
    step's needed experts all resident after it): exhaustive search over
    every choice, for tiny traces only."""
    steps = [sorted(set(int(e) for e in ids)) for ids in steps]
    from itertools import combinations
    best = [None]

    def go(t, resident, misses):
        if best[0] is not None and misses >= best[0]:
            return
        if t == len(steps):
            best[0] = misses
            return
        need = steps[t]
        miss = [e for e in need if e not in resident]
        keep_pool = [x for x in resident if x not in need]
        room = n_slots - len(need)
        # after the step: the needed experts plus any `room`-sized subset of
        # the others that were resident (what eviction kept)
        if len(keep_pool) <= room:
            go(t + 1, frozenset(need) | frozenset(keep_pool), misses + len(miss))
            return
        for keep in combinations(sorted(keep_pool), room):
            go(t + 1, frozenset(need) | frozenset(keep), misses + len(miss))

    go(0, frozenset(), 0)
    return best[0]
