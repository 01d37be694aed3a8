"""Pins for the host-tier residency oracle (oracle/swap.py).

The PagedWeight page (section "Dynamic Paging") says inactive expert pages
can be swapped out to CPU memory; the replacement policy is this project's
reading, stated in oracle/swap.py. Pinned by a trace worked out by hand, by
the textbook behaviour of least-recently-used replacement (a cyclic pattern
one larger than the cache misses every time; a working set that fits hits
after its first touch) and by invariants on random traces checked against a
separately written brute-force search for the victims.
"""
import random

from oracle import swap


def test_hand_trace():
    r = swap.Residency(E=6, S=2)
    # pass 1: {1, 4}: both miss, empty slots 0, 1 in order
    assert r.forward([4, 1, 4]) == ([(1, 0), (4, 1)], [])
    # pass 2: {1, 2}: 1 hits; 2 misses, the only slot not in A is 1 (expert 4)
    assert r.forward([2, 1]) == ([(2, 1)], [])
    assert r.slot_of == [-1, 0, 1, -1, -1, -1]
    # pass 3: {0, 3, 5}: three misses, two slots: slot 0 (expert 1, used at
    # pass 2) and slot 1 (expert 2, pass 2): equal ages, lower expert first
    assert r.forward([5, 3, 0]) == ([(0, 0), (3, 1)], [5])
    # pass 4: {0, 5}: 0 hits; 5 misses and takes slot 1 (expert 3 not in A)
    assert r.forward([0, 5]) == ([(5, 1)], [])
    # pass 5: {2}: slots hold 0 (pass 4) and 5 (pass 4): lower id 0 goes
    assert r.forward([2]) == ([(2, 0)], [])
    assert r.expert_of == [2, 5]
    assert r.last_use == [4, 2, 5, 3, 1, 4]
    assert (r.hits, r.copies, r.host_reads) == (2, 7, 1)
    # requantizing expert 5 frees slot 1; expert 2 keeps slot 0
    r.invalidate([5, 3])
    assert r.expert_of == [2, -1] and r.slot_of[5] == -1
    assert r.forward([5]) == ([(5, 1)], [])


def test_cyclic_pattern_one_larger_than_the_cache_always_misses():
    r = swap.Residency(E=5, S=4)
    for t in range(50):
        copies, host = r.forward([t % 5])
        assert len(copies) == 1 and not host
    assert r.hits == 0


def test_working_set_that_fits_hits_after_first_touch():
    rng = random.Random(4)
    r = swap.Residency(E=40, S=8)
    ws = rng.sample(range(40), 8)
    r.forward(ws)
    for _ in range(30):
        copies, host = r.forward(rng.sample(ws, rng.randrange(1, 9)))
        assert copies == [] and host == []


def _victims_brute(slot_of, expert_of, last_use, A, n):
    """The n slots the policy hands out, by exhaustive comparison."""
    S = len(expert_of)
    out = []
    taken = set()
    for _ in range(n):
        best = None
        for s in range(S):
            if s in taken:
                continue
            e = expert_of[s]
            if e >= 0 and e in A:
                continue
            key = (0, s, 0) if e < 0 else (1, last_use[e], e)
            if best is None or key < best[0]:
                best = (key, s)
        if best is None:
            break
        out.append(best[1])
        taken.add(best[1])
    return out


def test_random_traces_against_brute_force_and_invariants():
    rng = random.Random(9)
    for trial in range(40):
        E = rng.randrange(1, 30)
        S = rng.randrange(0, E + 3)
        r = swap.Residency(E, S)
        for t in range(40):
            A = set(rng.sample(range(E), rng.randrange(0, E + 1)))
            before_slot, before_exp, before_use = list(r.slot_of), list(r.expert_of), list(r.last_use)
            misses = sorted(e for e in A if before_slot[e] < 0)
            want = _victims_brute(before_slot, before_exp, before_use, A, len(misses))
            copies, host = r.forward(list(A))
            assert [s for _, s in copies] == want
            assert [e for e, _ in copies] + host == misses
            # no expert of A lost its slot; slots and experts agree
            for e in A:
                if before_slot[e] >= 0:
                    assert r.slot_of[e] == before_slot[e]
            for s in range(S):
                e = r.expert_of[s]
                assert e < 0 or r.slot_of[e] == s
            assert sum(1 for e in range(E) if r.slot_of[e] >= 0) <= S
            # host reads only when every slot holds an expert of A
            if host:
                assert all(e in A for e in r.expert_of) and len(r.expert_of) == S
            if rng.random() < 0.1:
                r.invalidate(rng.sample(range(E), rng.randrange(0, E + 1)))
