"""Pins for the oracle allocator (Eq. 1 of the PagedWeight page, section
"Quality-Aware Quantization"): a hand-worked example, brute force against the
dynamic programme, and invariants of the optimisation problem."""
import json
import os
import random

import pytest

from oracle import alloc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden():
    with open(os.path.join(GOLDEN, "eq1_allocation.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("solver", [alloc.solve_bruteforce, alloc.solve_dp])
def test_hand_worked_example(solver):
    g = golden()
    for case in g["cases"]:
        if case.get("infeasible"):
            with pytest.raises(alloc.Infeasible):
                solver(g["p"], g["L"], g["W"], case["B"])
            continue
        bits, obj = solver(g["p"], g["L"], g["W"], case["B"])
        assert bits == case["bits"], case
        assert obj == pytest.approx(case["objective"], rel=1e-12)


def random_problem(rng, E, equal_W):
    W = [rng.choice([4, 6, 10])] * E if equal_W else [rng.choice([2, 3, 4, 6]) for _ in range(E)]
    p = [rng.random() for _ in range(E)]
    L = []
    for _ in range(E):
        l8 = rng.uniform(1e-4, 1e-2)
        l4 = l8 + rng.uniform(1e-3, 0.5)
        l3 = l4 + rng.uniform(1e-3, 1.0)
        L.append([l3, l4, l8])
    lo, hi = 3 * sum(W), 8 * sum(W)
    B = rng.randint(lo - 2, hi + 2)
    return p, L, W, B


def test_bruteforce_equals_dp_random():
    rng = random.Random(11)
    for trial in range(300):
        E = rng.randint(1, 6)
        p, L, W, B = random_problem(rng, E, equal_W=trial % 2 == 0)
        if 3 * sum(W) > B:
            with pytest.raises(alloc.Infeasible):
                alloc.solve_dp(p, L, W, B)
            with pytest.raises(alloc.Infeasible):
                alloc.solve_bruteforce(p, L, W, B)
            continue
        b1, o1 = alloc.solve_bruteforce(p, L, W, B)
        b2, o2 = alloc.solve_dp(p, L, W, B)
        assert alloc.used_bits(b2, W) <= B
        assert o2 == o1                       # same left-to-right sums
        assert b1 == b2, (p, L, W, B)         # generic inputs: unique optimum


def test_invariants():
    rng = random.Random(12)
    for _ in range(40):
        E = rng.randint(2, 6)
        p, L, W, _ = random_problem(rng, E, equal_W=True)
        S = sum(W)
        # B >= 8 sum W: everything at 8 bits
        assert alloc.solve_dp(p, L, W, 8 * S)[0] == [8] * E
        # 3 sum W <= B < 3 sum W + min W: everything at 3 bits
        assert alloc.solve_dp(p, L, W, 3 * S + min(W) - 1)[0] == [3] * E
        # optimum is non-increasing in B
        prev = None
        for B in range(3 * S, 8 * S + 1, max(1, S // 4)):
            bits, obj = alloc.solve_dp(p, L, W, B)
            assert alloc.used_bits(bits, W) <= B
            if prev is not None:
                assert obj <= prev
            prev = obj


def test_identical_experts_get_bits_in_importance_order():
    # same W and L for every expert: exchanging two experts' bit-widths shows
    # the more important one never gets fewer bits
    rng = random.Random(13)
    for _ in range(30):
        E = rng.randint(2, 7)
        Lrow = [1.0, rng.uniform(0.05, 0.6), rng.uniform(1e-4, 1e-2)]
        L = [Lrow] * E
        p = sorted((rng.random() for _ in range(E)), reverse=True)
        W = [5] * E
        B = rng.randint(15 * E, 40 * E)
        bits, _ = alloc.solve_bruteforce(p, L, W, B)
        assert all(bits[i] >= bits[i + 1] for i in range(E - 1)), (p, bits, B)


def test_dp_larger_instance_matches_exhaustive_bound():
    # E = 8 brute force (6561 assignments) against the DP
    rng = random.Random(14)
    for _ in range(5):
        p, L, W, B = random_problem(rng, 8, equal_W=False)
        B = max(B, 3 * sum(W))
        b1, o1 = alloc.solve_bruteforce(p, L, W, B)
        b2, o2 = alloc.solve_dp(p, L, W, B)
        assert o1 == o2 and b1 == b2
