"""Oracle for the host tier: expert pages swapped between CPU memory and a
device cache of page slots.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU baseline; never by the GPU library.

The PagedWeight page (section "Dynamic Paging") describes paging like virtual
memory: the router decides which experts a forward pass needs, their pages
are fetched, and pages of inactive experts can be swapped out to CPU
memory. It gives no replacement policy. The reading taken here (the library
implements the same one):

* Every expert's page lives in the host tier. The device holds S slots, each
  large enough for any page; a slot holds one expert's page or nothing.
* Each forward pass, with A the set of experts routed to at least once:
  - an expert of A that holds a slot is a hit;
  - the other experts of A (misses), in ascending expert id, take slots in
    this order: empty slots by ascending slot index, then the slots of
    experts not in A, least recently used first (ties: lower expert id).
    A miss takes its slot by copying its page in; the expert that held the
    slot loses it;
  - misses left without a slot (all slots hold experts of A) are read from
    the host tier directly for this pass;
  - every expert of A is then stamped as used at this pass.
* Requantizing an expert (new page bytes) frees its slot; experts whose
  pages did not change keep theirs.

Pass numbers start at 1; "last used" 0 means never.
"""
from __future__ import annotations


class Residency:
    def __init__(self, E: int, S: int):
        self.E, self.S = E, S
        self.slot_of = [-1] * E
        self.expert_of = [-1] * S
        self.last_use = [0] * E
        self.step = 0
        self.hits = self.copies = self.host_reads = 0

    def forward(self, active):
        """One pass over the set of routed experts. Returns (copies,
        host_read): copies is a list of (expert, slot) in miss order,
        host_read the misses read from the host tier."""
        A = sorted(set(int(e) for e in active))
        self.step += 1
        inA = set(A)
        misses = [e for e in A if self.slot_of[e] < 0]
        self.hits += len(A) - len(misses)
        free = [s for s in range(self.S) if self.expert_of[s] < 0]
        held = [s for s in range(self.S) if self.expert_of[s] >= 0 and self.expert_of[s] not in inA]
        held.sort(key=lambda s: (self.last_use[self.expert_of[s]], self.expert_of[s]))
        candidates = free + held
        copies, host_read = [], []
        for i, e in enumerate(misses):
            if i < len(candidates):
                s = candidates[i]
                old = self.expert_of[s]
                if old >= 0:
                    self.slot_of[old] = -1
                self.expert_of[s] = e
                self.slot_of[e] = s
                copies.append((e, s))
            else:
                host_read.append(e)
        for e in A:
            self.last_use[e] = self.step
        self.copies += len(copies)
        self.host_reads += len(host_read)
        return copies, host_read

    def invalidate(self, experts):
        """Pages rewritten: the experts lose their slots."""
        for e in experts:
            s = self.slot_of[e]
            if s >= 0:
                self.expert_of[s] = -1
                self.slot_of[e] = -1
