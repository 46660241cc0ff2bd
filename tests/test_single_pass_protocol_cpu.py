"""CPU model of the single-pass quantize's grid-wide amax handoff, run under
random schedules with only part of the grid resident at once.

The model follows the kernel's protocol step by step (workspace words of
launch.h; all accesses relaxed atomics on 64-bit words tag << 32 | low):

  start    read the epoch e (tag = e + 1); mark the own slot STARTED
  load     load the own tiles (takes a few steps)
  publish  own slot <- tag | max
  fast     poll (bounded): the group leader (first of each group of 64)
           waits for its members' slots and writes the group slot; every
           workgroup waits for all group slots, or for the done word.
           After a grace of some polls, a member slot without the tag (for
           the leader), or a missing group slot whose leader's slot has no
           tag (for the others), ends the fast path at once
  slow     (after the fast path) claim the slots, among SPAN from a
           spread start, that are not yet this call's (compare-and-swap to
           tag | CLAIMED), take each such workgroup's maximum from memory
           and publish it; then the first workgroup to tag the reducer word
           claims what is left over every slot, waits until every slot
           holds a maximum, reduces them and stores the done word; the
           others wait for the done word
  count    exit counter; the last workgroup advances the epoch
  encode   from its registers (a few steps); then the workgroup exits

A workgroup runs only while it holds one of R resident places; a place
frees when a workgroup exits, and the next workgroup in launch order starts.
Every run must end (no workgroup waits forever) with every workgroup
holding the true maximum, the epoch advanced once, no tagged word touched
after the epoch advanced (the last workgroup to count out may clear them
all when the epoch wraps), and no work duplicated beyond the claimed chunks
of workgroups that had not started.
"""

from __future__ import annotations

import random

import pytest

STARTED = 0xFFFFFFFE
CLAIMED = 0xFFFFFFFF
GROUP = 64
SPAN = 40  # slots each workgroup of the slow path scans for claims (the kernel: 512 of up to 2048)


class _TaggedWords(list):
    """Tagged workspace words: every access checks that the call's epoch has
    not advanced yet."""

    def __init__(self, ws, n):
        super().__init__([0] * n)
        self._ws = ws

    def __getitem__(self, i):
        self._ws.check_live()
        return super().__getitem__(i)

    def __setitem__(self, i, v):
        self._ws.check_live()
        super().__setitem__(i, v)

    def __iter__(self):
        self._ws.check_live()
        return super().__iter__()


class Workspace:
    def __init__(self, G):
        self.advanced = False  # the current call's epoch has advanced
        self.slot = _TaggedWords(self, G)
        self.group = _TaggedWords(self, (G + GROUP - 1) // GROUP)
        self._done = 0
        self._reducer = 0
        self.reducers = 0  # workgroups elected to reduce in the current call
        self.epoch = 0
        self.exits = 0
        self.memory_reads = 0  # chunks whose maximum was read from memory by a claimer

    def check_live(self):
        # once the last workgroup has counted out, the kernel may clear every
        # tagged word (the epoch's wrap-around): no workgroup of the call may
        # touch one after that
        assert not self.advanced, "a tagged word was touched after the epoch advanced"

    @property
    def done(self):
        self.check_live()
        return self._done

    @done.setter
    def done(self, v):
        self.check_live()
        self._done = v

    @property
    def reducer(self):
        self.check_live()
        return self._reducer

    @reducer.setter
    def reducer(self, v):
        self.check_live()
        self._reducer = v

    def cas_slot(self, w, expect, new):
        if self.slot[w] == expect:
            self.slot[w] = new
            return True
        return False


def workgroup(ws, wg, G, chunk_max, fast_polls, load_steps, grace):
    """A generator: each yield is one step of the workgroup (a memory access
    or a poll); the scheduler interleaves them. Returns the amax seen."""
    e = ws.epoch
    yield
    tag = (e + 1) << 32
    ws.slot[wg] = tag | STARTED
    yield
    for _ in range(load_steps):
        yield
    m = chunk_max[wg]
    ws.slot[wg] = tag | m
    yield
    amax = None
    ok = True
    # fast path: group leader, then the group slots (or the done word)
    polls = 0
    if wg % GROUP == 0:
        members = range(wg, min(wg + GROUP, G))
        while True:
            vals = [ws.slot[i] for i in members]
            yield
            polls += 1
            if all(v >> 32 == e + 1 and (v & 0xFFFFFFFF) <= 0x7FFFFFFF for v in vals):
                ws.group[wg // GROUP] = tag | max(v & 0xFFFFFFFF for v in vals)
                yield
                break
            if polls > fast_polls or (polls > grace and any(v >> 32 != e + 1 for v in vals)):
                ok = False
                break
    while ok and amax is None:
        d = ws.done
        vals = list(ws.group)
        yield
        polls += 1
        if d >> 32 == e + 1:
            amax = d & 0xFFFFFFFF
        elif all(v >> 32 == e + 1 for v in vals):
            amax = max(v & 0xFFFFFFFF for v in vals)
        elif polls > fast_polls:
            ok = False
        elif polls > grace:
            leaders = [ws.slot[GROUP * g] for g, v in enumerate(vals) if v >> 32 != e + 1]
            yield
            if any(v >> 32 != e + 1 for v in leaders):
                ok = False
    if amax is None:
        # slow path
        start = (wg * 0x9E3779B9 % (1 << 32)) * G >> 32

        def claims(limit):
            # claim untouched slots among the first `limit` of the scan order
            for k in range(limit):
                w = (start + k) % G
                old = ws.slot[w]
                yield
                if ws.done >> 32 == e + 1:
                    return
                if old >> 32 != e + 1 and ws.cas_slot(w, old, tag | CLAIMED):
                    yield
                    for _ in range(load_steps):
                        yield
                    ws.memory_reads += 1
                    # a plain store: if the owner started meanwhile, it publishes the same value
                    ws.slot[w] = tag | chunk_max[w]
                    yield

        yield from claims(min(G, SPAN))
        r = ws.reducer
        yield
        reducer = r >> 32 != e + 1 and ws.reducer == r  # compare-and-swap
        if reducer:
            ws.reducer = tag | wg
            ws.reducers += 1
            yield
            yield from claims(G)
            while True:
                vals = list(ws.slot)
                yield
                if all(v >> 32 == e + 1 and (v & 0xFFFFFFFF) <= 0x7FFFFFFF for v in vals):
                    amax = max(v & 0xFFFFFFFF for v in vals)
                    break
            ws.done = tag | amax
            yield
        else:
            while ws.done >> 32 != e + 1:
                yield
            amax = ws.done & 0xFFFFFFFF
    # count out, then encode (touches no workspace word), then exit
    ws.exits += 1
    if ws.exits == G:
        ws.epoch = e + 1
        ws.exits = 0
        ws.advanced = True
    yield
    for _ in range(load_steps):
        yield
    return amax


def run(G, R, seed, fast_polls, load_steps=3, calls=2, step_limit=2_000_000, grace=None):
    grace = fast_polls if grace is None else grace
    rng = random.Random(seed)
    ws = Workspace(G)
    for call in range(calls):
        chunk_max = [rng.randrange(0, 1 << 30) for _ in range(G)]
        epoch0 = ws.epoch
        ws.advanced = False
        pending = list(range(G))
        running = {}
        results = {}
        steps = 0
        while pending or running:
            while pending and len(running) < R:
                wg = pending.pop(0)
                running[wg] = workgroup(ws, wg, G, chunk_max, fast_polls, load_steps, grace)
            wg = rng.choice(list(running))
            try:
                next(running[wg])
            except StopIteration as stop:
                results[wg] = stop.value
                del running[wg]
            steps += 1
            assert steps < step_limit, f"no progress: G={G} R={R} seed={seed} call={call}"
        assert all(results[w] == max(chunk_max) for w in range(G)), (G, R, seed, call)
        assert ws.epoch == epoch0 + 1
        assert ws.exits == 0
        assert ws.reducers <= 1, "more than one reducer"
        ws.reducers = 0
    return ws


@pytest.mark.parametrize("G,R", [(1, 1), (5, 2), (64, 64), (70, 70), (70, 23), (130, 1), (130, 64), (200, 199),
                                 (256, 100), (300, 7)])
@pytest.mark.parametrize("seed", range(6))
def test_handoff_ends_with_the_true_maximum(G, R, seed):
    # fast_polls small enough that partly resident grids take the slow path
    run(G, R, seed, fast_polls=50)


@pytest.mark.parametrize("G,R", [(70, 23), (130, 64), (256, 128), (300, 7), (128, 64)])
@pytest.mark.parametrize("seed", range(4))
def test_non_arrival_detection_ends_with_the_true_maximum(G, R, seed):
    # a short grace: workgroups that have not started are seen early
    run(G, R, seed, fast_polls=10_000, grace=2)


def test_fully_resident_grid_claims_nothing():
    # every workgroup starts before any finishes waiting: no chunk is read twice
    ws = run(130, 130, 1, fast_polls=10_000)
    assert ws.memory_reads == 0


def test_a_half_resident_grid_reads_only_the_missing_chunks():
    G, R = 128, 64
    ws = run(G, R, 3, fast_polls=50, calls=1)
    assert 0 < ws.memory_reads <= G - R


def test_forced_slow_path_with_everything_resident():
    # a fast bound of zero polls: every workgroup takes the slow path
    run(96, 96, 4, fast_polls=0)
    run(96, 40, 5, fast_polls=0)


def test_many_calls_on_one_workspace():
    run(70, 30, 9, fast_polls=20, calls=12)
