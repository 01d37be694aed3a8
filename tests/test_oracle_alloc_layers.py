"""Pins for the comparison allocator and the multi-layer budget
(oracle/alloc.py: proportional, solve_layers).

* proportional follows the PagedWeight page's simplified code sketch (bits
  proportional to importance, bucketized up to {3, 4, 8}); it is pinned by
  hand-worked values, including the bucket boundaries (a value equal to an
  option takes that option, as torch.bucketize does by default).
* solve_layers is Eq. 1 over the union of the layers' experts. Pinned by
  brute force over the union (the dynamic programme is used once the union
  has more than 8 experts) and by the decomposition identity: the global
  optimum equals the best split of B between the layers of the per-layer
  optima.
"""
import random

import pytest

from oracle import alloc


def test_proportional_hand_worked():
    # x_e = B p_e / sum(p) / W_e = 1800 * (0.5, 0.3, 0.2) / (100, 100, 200)
    #     = 9.0, 5.4, 1.8 -> 8, 8, 3; 2200 bits used for a budget of 1800
    bits, used = alloc.proportional([0.5, 0.3, 0.2], [100, 100, 200], 1800)
    assert bits == [8, 8, 3]
    assert used == 2200


def test_proportional_bucket_boundaries():
    # W = 1 and B = sum(p): x_e = p_e exactly (21.5 * 3 / 21.5 = 3, etc.)
    bits, used = alloc.proportional([3.0, 4.0, 4.5, 10.0, 0.0], [1] * 5, 21.5)
    assert bits == [3, 4, 8, 8, 3]
    assert used == 26
    bits, _ = alloc.proportional([3.0 + 1e-9, 4.0 - 1e-9], [1, 1], 7.0)
    assert bits == [4, 4]
    with pytest.raises(ValueError):
        alloc.proportional([0.0, 0.0], [1, 1], 10)


def test_proportional_is_smallest_option_not_below_the_share():
    rng = random.Random(5)
    for _ in range(200):
        E = rng.randrange(1, 12)
        W = [rng.randrange(1, 50) for _ in range(E)]
        p = [rng.random() for _ in range(E)]
        B = rng.randrange(1, 20 * sum(W))
        bits, used = alloc.proportional(p, W, B)
        assert used == sum(b * w for b, w in zip(bits, W))
        for e in range(E):
            x = B * p[e] / sum(p) / W[e]
            ok = [o for o in (3, 4, 8) if o >= x]
            assert bits[e] == (ok[0] if ok else 8)


def _layer(rng, E):
    W = [rng.choice([2, 3, 4, 6]) for _ in range(E)]
    p = [rng.random() for _ in range(E)]
    L = []
    for _ in range(E):
        l8 = rng.uniform(1e-4, 1e-2)
        l4 = l8 + rng.uniform(1e-3, 0.5)
        L.append([l4 + rng.uniform(1e-3, 1.0), l4, l8])
    return p, L, W


def test_layers_match_bruteforce_on_the_union():
    rng = random.Random(11)
    for trial in range(6):
        sizes = [rng.randrange(2, 6) for _ in range(2)]
        if sum(sizes) <= 8:
            sizes[0] += 9 - sum(sizes)   # make the union large enough for the DP path
        layers = [_layer(rng, E) for E in sizes]
        ps, Ls, Ws = zip(*layers)
        Wsum = sum(sum(W) for W in Ws)
        B = rng.randrange(3 * Wsum, 8 * Wsum + 1)
        wts = [rng.uniform(0.5, 2.0) for _ in layers]
        per_layer, obj = alloc.solve_layers(ps, Ls, Ws, B, wts)
        p_all = [w * v for w, p in zip(wts, ps) for v in p]
        L_all = [row for L in Ls for row in L]
        W_all = [v for W in Ws for v in W]
        bf_bits, bf_obj = alloc.solve_bruteforce(p_all, L_all, W_all, B)
        assert [b for bl in per_layer for b in bl] == bf_bits, trial
        assert obj == bf_obj
        assert alloc.used_bits(bf_bits, W_all) <= B


def test_global_optimum_is_the_best_split():
    rng = random.Random(23)
    for trial in range(10):
        (p1, L1, W1), (p2, L2, W2) = _layer(rng, 3), _layer(rng, 3)
        B = rng.randrange(3 * (sum(W1) + sum(W2)), 8 * (sum(W1) + sum(W2)) + 1)
        _, obj = alloc.solve_layers([p1, p2], [L1, L2], [W1, W2], B)
        best = None
        for B1 in range(3 * sum(W1), B - 3 * sum(W2) + 1):
            o = alloc.solve_bruteforce(p1, L1, W1, B1)[1] + alloc.solve_bruteforce(p2, L2, W2, B - B1)[1]
            best = o if best is None else min(best, o)
        assert obj == pytest.approx(best, rel=1e-12, abs=0.0), trial


def test_zero_weight_layer_gets_the_fewest_bits():
    rng = random.Random(2)
    (p1, L1, W1), (p2, L2, W2) = _layer(rng, 3), _layer(rng, 4)
    B = 6 * (sum(W1) + sum(W2))
    per_layer, _ = alloc.solve_layers([p1, p2], [L1, L2], [W1, W2], B, [0.0, 1.0])
    assert per_layer[0] == [3, 3, 3]
    # the other layer then gets what Eq. 1 gives it alone with the rest
    alone, _ = alloc.solve_bruteforce(p2, L2, W2, B - 3 * sum(W1))
    assert per_layer[1] == alone
