"""Pins for the KV-pressure budget scheduler oracle (oracle/sched.py).

The pages (PagedWeight, section "Implementation Details": the scheduler sizes
pages from the KV-cache occupancy; the news digest's paging comparison) give
no formula; the reading is stated in oracle/sched.py. These tests pin that
reading with a trace worked out by hand and with the guarantees it is meant
to give on random traces.
"""
import random

import numpy as np

from oracle import alloc, sched


def test_page_bytes_closed_form():
    assert sched.page_nbytes(1000, 3) == 512      # 375 B of codes -> 512
    assert sched.page_nbytes(1000, 8) == 1024     # 1000 B -> 1024
    assert sched.page_nbytes(1024, 4) == 512      # exactly 512
    assert sched.page_nbytes(1, 3) == 256         # 3 bits -> 1 byte -> 256
    assert sched.bits_for_bytes(1000, 2) == 8 * (1000 - 512)
    assert sched.bits_for_bytes(100, 2) == 0


def test_hand_trace():
    """Two experts of 1000 weights: budgets 6000..16000 bits; the all-3-bit
    pool is 2 x 512 B, the all-8-bit pool 2 x 1024 B. memory 4000 B, no
    reserve, headroom 0.1, at least 2 steps between a change and a grow."""
    W = [1000, 1000]
    M, R, h, n = 4000, 0, 0.1, 2

    def step(kv, pool, budget, since):
        return sched.decide(M, R, h, n, kv, W, pool, budget, since)

    # first call: avail 4000 -> 8 (3600 - 512) = 24704 -> clamped to 16000
    assert step(0, None, None, 0) == (sched.INIT, 16000, False)
    # pool 2048 fits in 3000: nothing to do (already at the maximum)
    assert step(1000, 2048, 16000, 1) == (sched.KEEP, 16000, False)
    # exactly full (avail 2048) still fits
    assert step(1952, 2048, 16000, 1) == (sched.KEEP, 16000, False)
    # avail 2000 < 2048: shrink to 8 (1800 - 512) = 10304
    assert step(2000, 2048, 16000, 2) == (sched.SHRINK, 10304, False)
    # avail 900 < a 4+4-bit pool (1024): 8 (810 - 512) = 2384 -> 6000, and
    # even the all-3-bit pool (1024) does not fit: pressure
    assert step(3100, 1024, 10304, 0) == (sched.SHRINK, 6000, True)
    # still does not fit, nothing left to shrink
    assert step(3100, 1024, 6000, 0) == (sched.KEEP, 6000, True)
    # room again, but only one step since the change: held back
    assert step(0, 1024, 6000, 1) == (sched.KEEP, 6000, False)
    # two steps: 16000 >= 1.1 x 6000, grow
    assert step(0, 1024, 6000, 2) == (sched.GROW, 16000, False)
    # a small gain (< 10%) is not worth a re-quantization: avail 1600 ->
    # 8 (1440 - 512) = 7424 < 1.1 x 7000 = 7700
    assert step(2400, 1024, 7000, 5) == (sched.KEEP, 7000, False)
    # ... a larger one is: avail 1700 -> 8 (1530 - 512) = 8144 >= 7700
    assert step(2300, 1024, 7000, 5) == (sched.GROW, 8144, False)


def _trace(rng, steps, memory):
    """KV occupancy: sequences arrive, grow by one token per step and end."""
    kv, live, out = 0, [], []
    for _ in range(steps):
        if rng.random() < 0.3:
            live.append(rng.randrange(1, 40))
        per_token = memory // 400
        kv = sum(t for t in live) * per_token
        live = [t + 1 for t in live if rng.random() > 0.05]
        out.append(min(kv, memory))
    return out


def test_random_traces_keep_the_pool_inside_the_memory():
    rng = random.Random(3)
    for trial in range(30):
        E = rng.randrange(2, 9)
        W = [8 * rng.randrange(50, 400) for _ in range(E)]
        p = np.array([rng.random() + 0.01 for _ in range(E)])
        L = [[rng.uniform(1.0, 2.0), rng.uniform(0.3, 0.9), rng.uniform(0.0, 0.2)] for _ in range(E)]
        total = sum(W)
        memory = rng.randrange(total, 3 * total)
        reserve = rng.randrange(0, total // 4)
        h = rng.choice([0.0, 0.05, 0.2])
        n = rng.randrange(0, 5)
        pool = budget = None
        since = 0
        last_change = None
        for t, kv in enumerate(_trace(rng, 60, memory)):
            action, B, pressure = sched.decide(memory, reserve, h, n, kv, W, pool, budget, since)
            avail = max(0, memory - kv - reserve)
            assert 3 * total <= B <= 8 * total
            if action == sched.GROW:
                assert since >= n and B > budget
                assert B >= budget * (1 + h) - 1e-9
            if action == sched.SHRINK:
                assert B < budget
            if action != sched.KEEP:
                bits, _ = alloc.solve(p, L, W, B)
                pool, budget, since, last_change = sched.pool_nbytes(W, bits), B, 0, t
                # the allocation the new budget buys fits in the memory
                # left, unless even the all-3-bit pool does not
                if not pressure:
                    assert pool <= avail, (trial, t, pool, avail)
            else:
                assert B == budget
                since += 1
            if not pressure and action == sched.KEEP:
                assert pool <= avail
