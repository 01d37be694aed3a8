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


# ---- comparison mode and a budget shared by several layers ----

def proportional(p, W, B):
    """The page's simplified illustration (PagedWeight page, the code sketch
    after "Implementation Details"): each expert's share of the budget is
    proportional to its importance, divided by its weight count, and the
    result is bucketized to {3, 4, 8} rounding up (a value equal to an option
    takes that option; above 8 it is clamped to 8).

    Reading: the budget is taken in bits, so share / W_e is bits per weight
    (the sketch divides a byte budget by a parameter count). The result need
    not respect the budget; returns (bits, used_bits).
    """
    p = [float(v) for v in p]
    W = [int(w) for w in W]
    total = sum(p)
    if not total > 0.0:
        raise ValueError("importances must not all be zero")
    bits = []
    for pe, we in zip(p, W):
        x = float(B) * pe / total / we
        if x <= 3.0:
            bits.append(3)
        elif x <= 4.0:
            bits.append(4)
        else:
            bits.append(8)
    return bits, used_bits(bits, W)


def solve_layers(ps, Ls, Ws, B, layer_weights=None):
    """Eq. 1 with one budget B over the experts of several layers: minimise
    sum_l w_l sum_e p_{l,e} L_{l,e}(b) subject to sum over all experts of
    b W <= B. The constraint and the objective are sums over the union of
    the layers' experts, so this is Eq. 1 on that union with importances
    w_l p_{l,e}. Returns (per-layer bit lists, objective)."""
    n = len(ps)
    w = [1.0] * n if layer_weights is None else [float(v) for v in layer_weights]
    p_all, L_all, W_all = [], [], []
    for l in range(n):
        p_all += [w[l] * float(v) for v in ps[l]]
        L_all += [list(map(float, row)) for row in Ls[l]]
        W_all += [int(v) for v in Ws[l]]
    bits, obj = solve(p_all, L_all, W_all, B)
    out, i = [], 0
    for l in range(n):
        out.append(bits[i:i + len(ps[l])])
        i += len(ps[l])
    return out, obj
