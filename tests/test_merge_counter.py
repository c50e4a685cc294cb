"""The in-kernel merge's arrival counters, modelled on the CPU.

Each of the n splits of a unit that hold keys stores its partial, waits for
the stores to complete, then takes a ticket with an atomic add on the unit's
counter; the split whose ticket is n - 1 merges the n partials and stores 0
back into the counter.  The model below runs that protocol over every (or
many random) arrival orders and checks what the library documents: from a
zeroed counter exactly one split merges, after every partial has landed, and
the counter is zero again, ready for the next call of any shape; a stale
counter (a workspace head that was not cleared, or calls that overlap on
one workspace) breaks it -- the merge runs early or never, and the stale
value survives the call -- which is why the head must read zero when a call
starts (pkv_workspace_clear once, ordered calls)."""
import itertools
import random

import pytest


def run_unit(counter, n, order):
    """One call's arrivals in `order` (a permutation of the n splits).
    Returns (counter after the call, merger split or None, partials the
    merger saw written, number of mergers)."""
    written = set()
    merger, seen, mergers = None, None, 0
    for s in order:
        written.add(s)            # the split's partial stores, completed before its atomic
        ticket = counter          # atomicAdd returns the old value
        counter += 1
        if ticket == n - 1:
            mergers += 1
            merger, seen = s, set(written)
            counter = 0           # the merger returns the counter to zero
    return counter, merger, seen, mergers


def orders(n, rng, limit=200):
    if n <= 5:
        return list(itertools.permutations(range(n)))
    return [rng.sample(range(n), n) for _ in range(limit)]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 64, 256])
def test_clean_counter_one_merge_after_every_partial(n):
    rng = random.Random(n)
    for order in orders(n, rng):
        counter, merger, seen, mergers = run_unit(0, n, order)
        assert mergers == 1 and merger == order[-1]       # the last arrival merges
        assert seen == set(range(n))                       # every partial had landed
        assert counter == 0                                # ready for the next call


def test_consecutive_calls_of_any_shape_reuse_the_counter():
    rng = random.Random(7)
    counter = 0
    for _ in range(500):
        n = rng.randint(1, 64)
        counter, merger, seen, mergers = run_unit(counter, n, rng.sample(range(n), n))
        assert mergers == 1 and seen == set(range(n)) and counter == 0


@pytest.mark.parametrize("n,k", [(4, 1), (4, 3), (8, 5), (64, 1)])
def test_stale_counter_merges_early_and_stays_stale(n, k):
    """A counter left at 0 < k < n: the (n - k)-th arrival merges before the
    remaining k partials land, and the counter ends the call at k again."""
    rng = random.Random(n * 100 + k)
    for order in orders(n, rng, 50):
        counter, merger, seen, mergers = run_unit(k, n, order)
        assert mergers == 1 and merger == order[n - k - 1]
        assert len(seen) == n - k < n                      # merged too early: wrong output
        assert counter == k                                # and the next call is stale too


@pytest.mark.parametrize("n,k", [(4, 4), (4, 9), (16, 1 << 20)])
def test_counter_at_or_past_n_never_merges(n, k):
    counter, merger, seen, mergers = run_unit(k, n, list(range(n)))
    assert mergers == 0 and merger is None                 # the unit's output is never written
    assert counter == k + n


def test_two_unordered_calls_on_one_counter_break_it():
    """Two calls sharing a workspace on unordered streams: their arrivals
    interleave on one counter, so one call's merge may run on the other's
    partial count (the library documents that calls sharing a workspace must
    be ordered)."""
    n = 4
    # call A's splits a0..a3 and call B's b0..b3 interleaved
    events = ["a0", "b0", "a1", "b1", "a2", "b2", "a3", "b3"]
    counter, mergers = 0, []
    for e in events:
        ticket = counter
        counter += 1
        if ticket == n - 1:
            mergers.append(e)
            counter = 0
    assert mergers == ["b1", "b3"]                          # A never merges; B merges twice
