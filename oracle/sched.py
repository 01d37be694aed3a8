"""Oracle for the KV-pressure budget scheduler.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU baseline; never by the GPU library.

The PagedWeight page (section "Implementation Details", memory management)
says the scheduler sizes the expert pages from the current KV-cache
occupancy; the news digest's restatement compares it to operating-system
paging: as the KV cache grows some experts drop to lower precision, and
precision comes back when the pressure eases. The pages give no formula.
The reading taken here (the library implements the same one):

* Bytes the pool may use: A = memory - KV_used - reserve (at least 0).
* Bytes -> budget: a page is its codes rounded up to whole bytes and then to
  256 bytes, so a pool of X bytes always holds an allocation of
  8 (X - 256 E) code bits (never less than 0); budgets are then clamped to
  [3 W, 8 W], W = sum_e W_e.
* Shrink (at once): when the current pool no longer fits, A < pool bytes,
  move to the budget of A (1 - h) bytes (if that is lower than the current
  one; at 3 W nothing is left to shrink).
* Grow (held back): only when at least ``min_interval`` steps passed since
  the last change and the budget of A (1 - h) bytes is above the current one
  and at least (1 + h) times it; then move to it.
* The first call (no allocation yet) always sets the budget of A (1 - h).
* When even the all-3-bit pool does not fit in A, the budget is 3 W and the
  step reports pressure (the caller has to free KV cache).

Fractions are evaluated in float64 and floored to whole bytes.
"""
from __future__ import annotations

import math

KEEP, SHRINK, GROW, INIT = 0, 1, 2, 3
PAGE_ALIGN = 256


def page_nbytes(W_e: int, b: int) -> int:
    """Bytes of one page: W_e codes of b bits, rounded up to 256 bytes."""
    return ((W_e * b + 7) // 8 + PAGE_ALIGN - 1) // PAGE_ALIGN * PAGE_ALIGN


def pool_nbytes(W, bits) -> int:
    return sum(page_nbytes(int(w), int(b)) for w, b in zip(W, bits))


def bits_for_bytes(nbytes: int, E: int) -> int:
    """Code bits that certainly fit in a pool of nbytes bytes."""
    return 8 * max(0, nbytes - PAGE_ALIGN * E)


def decide(memory: int, reserve: int, headroom: float, min_interval: int,
           kv_used: int, W, pool_bytes_now: int | None, budget_now: int | None,
           steps_since_change: int):
    """One scheduling decision.

    Returns (action, budget_bits, pressure). ``pool_bytes_now`` and
    ``budget_now`` are None before the first allocation.
    """
    E = len(W)
    total = sum(int(w) for w in W)
    bmin, bmax = 3 * total, 8 * total
    avail = max(0, int(memory) - int(kv_used) - int(reserve))
    target = bits_for_bytes(math.floor(avail * (1.0 - headroom)), E)
    target = min(max(target, bmin), bmax)
    pressure = pool_nbytes(W, [3] * E) > avail
    if budget_now is None:
        return INIT, target, pressure
    if pool_bytes_now > avail:
        if target < budget_now:
            return SHRINK, target, pressure
        return KEEP, budget_now, pressure
    if (steps_since_change >= min_interval and target > budget_now
            and target >= math.ceil(budget_now * (1.0 + headroom))):
        return GROW, target, pressure
    return KEEP, budget_now, pressure
