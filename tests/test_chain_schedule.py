"""CPU model of the chain kernel's DMA-wave schedule (the loop in csrc/kda_chain.hip):
the record of each chunk step comes in two parts, P1 and P2, each in a two-slot LDS
ring, plus (two value tiles per workgroup) L2 touches of the record TD steps ahead.
Vector-memory loads complete in issue order, and `s_waitcnt vmcnt(n)` returns once at
most the n youngest loads are outstanding. Replaying the loop's issue order and waits
for every chunk count checks that:
  - P1(j) has landed when the DMA wave reaches barrier (A) of step j, and P2(j) when it
    reaches (B) of step j (the other waves read them after those barriers);
  - a ring slot is refilled only after the step that reads it has passed its barrier;
  - every wait names at most 63 younger loads, the counter's range (a larger count is
    clamped to 63 by the kernel, which only waits for more loads: still safe).
The part sizes, touch count and distance are read from the kernel source."""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "gated_delta_rule_87_amd", "csrc", "kda_chain.hip")


def kernel_constants():
    s = open(SRC).read()
    m = re.search(r"constexpr int N1 = 32 \+ 2 \* NW \+ 1, N2 = 16 \+ 6 \+ 1;", s)
    assert m, "part sizes changed: update the model"
    t = re.search(r"constexpr int TP = NW == 2 \? (\d+) : 0, TD = (\d+);", s)
    assert t, "touch constants changed: update the model"
    return int(t.group(1)), int(t.group(2))


class Queue:
    def __init__(self):
        self.out = []          # outstanding load tags, oldest first
        self.done = set()

    def issue(self, tag, n):
        self.out += [tag] * n

    def wait(self, n):
        n = min(n, 63)         # the kernel's wait_vmcnt clamps the count
        while len(self.out) > n:
            self.done.add(self.out.pop(0))
        # a part has landed once none of its loads is outstanding
        return {t for t in self.done if t not in self.out}


def replay(nc, NW, TP, TD):
    N1, N2 = 32 + 2 * NW + 1, 16 + 6 + 1
    tp = TP if NW == 2 else 0
    q = Queue()
    counts = []
    landed = set()

    def wait(n):
        counts.append(n)
        landed.update(q.wait(n))

    reading = {}               # ring slot -> step whose part sits in it
    if nc > 0:
        q.issue(("P1", 0), N1); q.issue(("P2", 0), N2)
        reading[("P1", 0)] = 0; reading[("P2", 0)] = 0
        if nc > 1:
            q.issue(("P1", 1), N1); reading[("P1", 1)] = 1
            wait(N2 + N1)
        else:
            wait(N2)
    for j in range(nc):
        # barrier (A): P1(j) must have landed
        assert ("P1", j) in landed, (nc, NW, j, "P1 at (A)")
        touched = tp > 0 and j >= 1 and j + TD - 1 < nc
        if j + 1 < nc:
            # P2 slot (j+1)&1 held P2(j-1), read before (A) of step j
            assert reading.get(("P2", (j + 1) & 1), -1) <= j - 1
            q.issue(("P2", j + 1), N2); reading[("P2", (j + 1) & 1)] = j + 1
            wait(N1 + tp + N2 if touched else N1 + N2)
        else:
            wait(0)
        # barrier (B): P2(j) must have landed
        assert ("P2", j) in landed, (nc, NW, j, "P2 at (B)")
        if j + 2 < nc:
            # P1 slot j&1 held P1(j), read between (A) and (B) of step j
            assert reading.get(("P1", j & 1), -1) == j
            q.issue(("P1", j + 2), N1); reading[("P1", j & 1)] = j + 2
            wait(tp + N2 + N1 if touched else N2 + N1)
            if tp > 0 and j + TD < nc:
                q.issue(("T", j + TD), tp)
        elif j + 1 < nc:
            wait(N2)
    return counts


@pytest.mark.parametrize("NW", [2, 4])
@pytest.mark.parametrize("nc", list(range(0, 12)) + [64, 128])
def test_dma_schedule(nc, NW):
    TP, TD = kernel_constants()
    counts = replay(nc, NW, TP, TD)
    if NW == 2:
        assert all(c <= 63 for c in counts), counts


def test_touches_fit_the_counter():
    TP, TD = kernel_constants()
    assert 32 + 2 * 2 + 1 + 23 + TP <= 63
    assert TD >= 3      # a touch must precede the ring load of its step by at least a step
