"""Oracle for the budgeted precision allocation.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU baseline; never by the GPU library.

Follows Eq. 1 of the PagedWeight page (section "Quality-Aware
Quantization"): choose b_e in {3, 4, 8} minimising sum_e p_e * L_e(b_e)
subject to sum_e b_e * W_e <= B. B counts code bits only (scales and page
padding are not charged). The simplified proportional heuristic printed in
the page's code illustration is not a solver of this problem (its bits do not
respect the budget) and is not used.

Two independent solvers:

* ``solve_bruteforce`` enumerates all 3^E assignments (small E).
* ``solve_dp`` is an exact dynamic programme over capacity in units of
  g = gcd_e(W_e), written separately from the library's own solver.

Both sum the objective left to right over experts 0..E-1, so equal
assignments give bitwise equal objectives.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

BITS = (3, 4, 8)


class Infeasible(Exception):
    """B < 3 * sum_e W_e: even all-3-bit does not fit."""


def objective(bits, p, L) -> float:
    total = 0.0
    for e, b in enumerate(bits):
        total += float(p[e]) * float(L[e][BITS.index(int(b))])
    return total


def used_bits(bits, W) -> int:
    return sum(int(b) * int(w) for b, w in zip(bits, W))


def solve_bruteforce(p, L, W, B):
    """Minimum over all assignments; ties: fewer total bits, then the
    assignment with the larger b at the lowest differing expert index."""
    E = len(p)
    if 3 * sum(int(w) for w in W) > B:
        raise Infeasible()
    best = None
    for combo in itertools.product(BITS, repeat=E):
        if used_bits(combo, W) > B:
            continue
        key = (objective(combo, p, L), used_bits(combo, W), tuple(-b for b in combo))
        if best is None or key < best[0]:
            best = (key, combo)
    return list(best[1]), best[0][0]


def solve_dp(p, L, W, B):
    """Exact multiple-choice knapsack by dynamic programming.

    Capacity unit g = gcd(W); expert e at b bits costs b * W_e / g units;
    capacity floor(B / g). best[c] = least objective of the experts seen so
    far using exactly c units (inf if unreachable); choice[e][c] records the
    bit-width that reached it. Returns (bits, objective).
    """
    E = len(p)
    W = [int(w) for w in W]
    if 3 * sum(W) > B:
        raise Infeasible()
    g = 0
    for w in W:
        g = math.gcd(g, w)
    cap = B // g
    INF = math.inf
    best = [INF] * (cap + 1)
    best[0] = 0.0
    choice = []
    for e in range(E):
        new = [INF] * (cap + 1)
        ch = [0] * (cap + 1)
        for c in range(cap + 1):
            if best[c] == INF:
                continue
            for b in BITS:
                c2 = c + b * W[e] // g
                if c2 > cap:
                    continue
                val = best[c] + float(p[e]) * float(L[e][BITS.index(b)])
                # strict improvement, or an exact tie broken towards larger b
                if val < new[c2] or (val == new[c2] and b > ch[c2]):
                    new[c2] = val
                    ch[c2] = b
        best = new
        choice.append(ch)
    # least objective; among equal objectives the fewest units
    c_best = min(range(cap + 1), key=lambda c: (best[c], c))
    bits = [0] * E
    c = c_best
    for e in range(E - 1, -1, -1):
        b = choice[e][c]
        bits[e] = b
        c -= b * W[e] // g
    assert c == 0
    return bits, best[c_best]


def solve(p, L, W, B):
    """Brute force for E <= 8, dynamic programme otherwise."""
    if len(p) <= 8:
        return solve_bruteforce(p, L, W, B)
    return solve_dp(p, L, W, B)
