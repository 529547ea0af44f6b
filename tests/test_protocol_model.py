"""A host model of the cross-workgroup protocol of the per-token fused losses.

The model replays, as a discrete-event simulation, what the kernels' workgroups
do with the workspace (one coordinator and W workers, each owning one tile):

* a worker publishes its valid count, then its partial loss, as entries tagged
  with its launch's identity; it waits for the coordinator's release of the
  global count N, or, past the release limit, gathers the counts itself; then
  it writes its gradient scaled by 1/N;
* the coordinator gathers the counts (computing itself any not published
  within the steal limit), releases N, gathers the partials the same way and
  writes the loss (the partials summed in worker order).

Stores become visible after a random delay; only `capacity` workgroups of the
launch are resident at once, dispatched in workgroup order as others retire,
as when other kernels hold the rest of the device.  The tests check, for every
capacity from 1 to W + 1, that every launch terminates, that every worker
scales by the true N, and that the loss is exactly the fixed-order sum; and
that entries left by a late workgroup of one launch never reach the next
launch on the same workspace.  The same model with waits that never fall back
(the design in which every workgroup must be resident) stalls whenever the
capacity is below W + 1: the model can tell the two apart.
"""
import heapq
import random

import pytest


class Device:
    """Event loop: workgroups are generators that yield the time to their next step."""

    def __init__(self, capacity, rng, dispatch=1.0, max_time=1e7):
        self.capacity, self.rng, self.dispatch, self.max_time = capacity, rng, dispatch, max_time
        self.mem = {}          # key -> list of (visible_time, value)
        self.now = 0.0

    def store(self, key, value):
        self.mem.setdefault(key, []).append((self.now + self.rng.uniform(5.0, 60.0), value))

    def load(self, key):
        seen = [(t, v) for t, v in self.mem.get(key, []) if t <= self.now]
        return max(seen, key=lambda e: e[0])[1] if seen else None

    def run(self, workgroups):
        """Runs a launch's workgroups (a list of generator factories) to completion;
        returns False if it stalls (no runnable workgroup ever progresses)."""
        pending = list(range(len(workgroups)))
        events, seq = [], 0
        resident = 0
        while pending and resident < self.capacity:
            heapq.heappush(events, (self.now + self.dispatch * resident, seq, workgroups[pending.pop(0)]()))
            seq += 1
            resident += 1
        while events:
            t, _, g = heapq.heappop(events)
            if t > self.max_time:
                return False
            self.now = t
            try:
                dt = next(g)
                heapq.heappush(events, (self.now + dt, seq, g))
                seq += 1
            except StopIteration:
                if pending:
                    heapq.heappush(events, (self.now + self.dispatch, seq, workgroups[pending.pop(0)]()))
                    seq += 1
        return True


def launch(dev, tag, counts, partials, steal, release, fallback=True, out=None):
    """One launch of the one-tile fused kernel: workgroup 0 coordinates, 1..W are workers."""
    W = len(counts)
    out = {} if out is None else out
    poll = 3.0

    def gather(kind, values, limit):
        # every entry polled until published or `limit` has passed, then computed here
        t0 = dev.now
        got = [None] * W
        while True:
            for w in range(W):
                if got[w] is None:
                    e = dev.load((kind, w))
                    if e is not None and e[0] == tag:
                        got[w] = e[1]
            if all(v is not None for v in got):
                break
            if fallback and dev.now - t0 > limit:
                for w in range(W):
                    if got[w] is None:
                        got[w] = values[w]        # computed from the inputs, same value
                        yield 20.0                # the cost of computing it
                break
            yield poll
        total = 0
        for v in got:                             # fixed (worker) order
            total = total + v
        return total

    def coordinator():
        n = yield from gather("cnt", counts, steal)
        dev.store(("rel",), (tag, n))
        s = yield from gather("par", partials, steal)
        out["loss"] = s / max(n, 1)
        out["N"] = n

    def worker(w):
        def run():
            yield dev.rng.uniform(30.0, 90.0)    # the mask arrives
            dev.store(("cnt", w), (tag, counts[w]))
            yield dev.rng.uniform(30.0, 90.0)    # the planes arrive, terms computed
            dev.store(("par", w), (tag, partials[w]))
            t0 = dev.now
            while True:
                e = dev.load(("rel",))
                if e is not None and e[0] == tag:
                    n = e[1]
                    break
                if fallback and dev.now - t0 > release:
                    n = yield from gather("cnt", counts, steal)
                    break
                yield poll
            out.setdefault("scales", {})[w] = n
            yield 5.0                            # gradient stores
        return run

    return [coordinator] + [worker(w) for w in range(W)], out


def check(out, counts, partials):
    n = sum(counts)
    assert out["N"] == n
    assert all(v == n for v in out["scales"].values()) and len(out["scales"]) == len(counts)
    total = 0
    for p in partials:
        total = total + p
    assert out["loss"] == total / max(n, 1)


@pytest.mark.parametrize("seed", range(6))
def test_every_capacity_terminates_with_exact_results(seed):
    rng = random.Random(seed)
    W = 12
    for capacity in range(1, W + 2):
        dev = Device(capacity, rng)
        counts = [rng.randint(0, 64) for _ in range(W)]
        partials = [rng.uniform(-3.0, 3.0) for _ in range(W)]
        wgs, out = launch(dev, tag=("q", 1), counts=counts, partials=partials, steal=400.0, release=1500.0)
        assert dev.run(wgs), f"stalled at capacity {capacity}"
        check(out, counts, partials)


@pytest.mark.parametrize("steal,release", [(0.0, 1e9), (400.0, 0.0), (0.0, 0.0), (30.0, 60.0)])
def test_forced_fallbacks_give_the_same_results(steal, release):
    rng = random.Random(7)
    W = 9
    counts = [rng.randint(0, 64) for _ in range(W)]
    partials = [rng.uniform(-3.0, 3.0) for _ in range(W)]
    for capacity in (1, 3, W + 1):
        dev = Device(capacity, rng)
        wgs, out = launch(dev, ("q", 1), counts, partials, steal, release)
        assert dev.run(wgs)
        check(out, counts, partials)


def test_late_workgroups_do_not_reach_the_next_launch():
    """Capacity 2: the coordinator finishes long before most workers start (it computes
    their values); their entries land in the workspace afterwards.  The next launch on the
    same workspace carries another tag and gets its own, different, exact results."""
    rng = random.Random(3)
    W = 8
    dev = Device(2, rng)
    for launch_id in range(1, 5):
        counts = [rng.randint(0, 64) for _ in range(W)]
        partials = [rng.uniform(-3.0, 3.0) for _ in range(W)]
        wgs, out = launch(dev, ("q", launch_id), counts, partials, steal=100.0, release=500.0)
        assert dev.run(wgs)
        check(out, counts, partials)


def test_waits_without_fallback_need_every_workgroup_resident():
    rng = random.Random(11)
    W = 8
    counts = [rng.randint(1, 64) for _ in range(W)]
    partials = [rng.uniform(-3.0, 3.0) for _ in range(W)]
    dev = Device(W + 1, rng, max_time=1e5)
    wgs, out = launch(dev, ("q", 1), counts, partials, steal=0.0, release=0.0, fallback=False)
    assert dev.run(wgs)
    check(out, counts, partials)
    dev = Device(W, rng, max_time=1e5)
    wgs, out = launch(dev, ("q", 1), counts, partials, steal=0.0, release=0.0, fallback=False)
    assert not dev.run(wgs)
