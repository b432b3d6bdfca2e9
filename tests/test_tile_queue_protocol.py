"""The tail-queue claim protocol of the tile kernels, as a model run under random
interleavings on the CPU (the GPU tests check the kernels themselves).

Each of the 8 XCD streams of a launch of n tiles ends in `queue` tiles taken at run time
through one 64-bit counter per XCD: low half = claims from the front (by the stream's own
workgroups, in L2-group order), high half = claims from the back (by workgroups that
found their own queue empty, and by spare workgroups past the tiles, which go straight
to the other queues).  A claim is one atomic add that returns the old counter; it gets a
tile iff front + back < queue before it.  A workgroup that finds no tile reads all
counters and claims from the back of the fullest queue until every queue shows none
left.  Checked here, over many random orders of the atomic operations: every queued
tile is taken exactly once, no workgroup gives up while a tile is left, and whatever the
counters hold when a launch starts, every tile id a claim can produce lies in its
stream's queue."""
import random

import pytest

MASK = (1 << 32) - 1


def claim_front(ctr, x, q):
    old = ctr[x]
    ctr[x] = (old + 1) & ((1 << 64) - 1)
    f, b = old & MASK, old >> 32
    return int(f) if f < q and b < q - f else None


def claim_back(ctr, y, q):
    old = ctr[y]
    ctr[y] = (old + (1 << 32)) & ((1 << 64) - 1)
    f, b = old & MASK, old >> 32
    return q - 1 - int(b) if b < q and f < q - b else None


def left(c, q):
    return q - (c & MASK) - (c >> 32)


def worker(ctr, x, q, spare):
    """A generator: one yield per atomic or counter read (the interleaving points);
    returns (queue, slot) or None."""
    if not spare:
        s = claim_front(ctr, x, q)
        yield
        if s is not None:
            return (x, s)
    while True:
        rest = [left(ctr[y], q) for y in range(8)]
        yield
        best = max(range(8), key=lambda y: (rest[y], -y))
        if rest[best] <= 0:
            return None
        s = claim_back(ctr, best, q)
        yield
        if s is not None:
            return (best, s)


def run(q, workers_per_xcd, spares_per_xcd, rng, init=None):
    ctr = list(init) if init is not None else [0] * 8
    gens, results = [], []
    for x in range(8):
        for _ in range(workers_per_xcd):
            gens.append(worker(ctr, x, q, False))
        for _ in range(spares_per_xcd):
            gens.append(worker(ctr, x, q, True))
    live = list(range(len(gens)))
    while live:
        i = rng.choice(live)
        try:
            next(gens[i])
        except StopIteration as e:
            results.append(e.value)
            live.remove(i)
    return results, ctr


@pytest.mark.parametrize("q,spares", [(1, 0), (3, 1), (5, 2), (32, 4), (7, 7)])
def test_every_queued_tile_taken_exactly_once(q, spares):
    rng = random.Random(1000 * q + spares)
    for _ in range(200):
        results, ctr = run(q, q, spares, rng)
        taken = [r for r in results if r is not None]
        assert len(taken) == len(set(taken))                       # at most once
        assert sorted(taken) == [(x, s) for x in range(8) for s in range(q)]  # all of them
        assert all(left(c, q) <= 0 for c in ctr)                   # every queue exhausted


def test_uneven_progress_moves_tiles_to_fast_xcds():
    """XCD 0's workgroups run first (a fast XCD): its spares take the last tile of other
    queues, and when the slow XCDs' workgroups run afterwards every tile is still taken
    exactly once."""
    q, spares = 4, 4
    ctr = [0] * 8
    fast = ([worker(ctr, 0, q, False) for _ in range(q)] +
            [worker(ctr, 0, q, True) for _ in range(spares)])
    got = []
    for g in fast:
        while True:
            try:
                next(g)
            except StopIteration as e:
                got.append(e.value)
                break
    assert sorted(s for x, s in got if x == 0) == list(range(q))
    stolen = [(x, s) for x, s in got if x != 0]
    assert len(stolen) == spares and all(s == q - 1 for _, s in stolen)   # from the backs
    rng = random.Random(7)
    slow, _ = run(q, q, 0, rng, init=ctr)
    taken = [r for r in slow if r is not None] + got
    assert sorted(taken) == [(x, s) for x in range(8) for s in range(q)]
    assert len(set(taken)) == len(taken)


@pytest.mark.parametrize("seed", range(20))
def test_any_counter_contents_give_tile_ids_in_range(seed):
    """Counters that were not cleared (any 64-bit values) may hand out wrong tiles but
    never a tile outside the stream's queue."""
    rng = random.Random(seed)
    q = rng.choice([1, 2, 32, 96, 384])
    init = [rng.choice([0, rng.getrandbits(64), (1 << 64) - 1, MASK, MASK << 32,
                        rng.randrange(0, 2 * q) | (rng.randrange(0, 2 * q) << 32)])
            for _ in range(8)]
    results, _ = run(q, 3, 2, rng, init=init)
    for r in results:
        if r is not None:
            x, s = r
            assert 0 <= x < 8 and 0 <= s < q
