"""The work-counter protocol of the persistent paged launch, modelled on the
host: P resident workgroups, T (chunk, head) items.  Workgroup w starts with
item w; every item it processes costs one fetch-and-add on the counter, and a
fetched value v names item P + v when v < T - P and otherwise ends the
workgroup.  The launch clears the counter first: from zero, whatever the
order of the fetches, every item is processed exactly once and the launch
makes exactly T fetches.  From another starting value values that end
workgroups can come before the low ones, which is why it is cleared."""

import random

import pytest


def _run(P, T, start, rng, wrap=False):
    counter = start
    fetches = 0
    done = []
    active = {w: w for w in range(min(P, T))}  # workgroup -> its current item
    while active:
        w = rng.choice(sorted(active))
        done.append(active[w])       # the item is attended, then the next one fetched
        v = counter
        counter = (0 if v >= T - 1 else v + 1) if wrap else (v + 1) % 2**32
        fetches += 1
        if T > P and v < T - P:
            active[w] = P + v
        else:
            del active[w]
    return sorted(done), fetches


@pytest.mark.parametrize("P,T", [(1, 1), (4, 1), (4, 3), (4, 4), (4, 5), (8, 100), (512, 4208),
                                 (512, 513), (3, 1000)])
def test_every_item_once_from_a_cleared_counter(P, T):
    rng = random.Random(P * 7919 + T)
    for _ in range(5):
        done, fetches = _run(P, T, 0, rng)
        assert done == list(range(T)), (P, T)
        assert fetches == T, (P, T)


def test_a_counter_not_cleared_can_lose_items():
    """Four workgroups, five items, the counter at 1 (even with a wrapping
    increment): the four fetches return 1, 2, 3, 4, all past the single
    dynamic item, so item 4 is never attended."""
    for wrap in (False, True):
        done, _ = _run(4, 5, 1, random.Random(1), wrap=wrap)
        assert done == [0, 1, 2, 3]
