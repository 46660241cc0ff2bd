"""CPU model of the one-launch grouped quantize's per-group amax handoff,
run under random schedules with only part of the grid resident at once and
with far fewer slots than workgroups, so that workgroups of later laps
overwrite slots that earlier ones wrote.

The model follows the kernel's protocol step by step (all accesses relaxed
atomics on 64-bit words tag << 32 | low):

  grid     per non-empty group: its head, then one workgroup per tile, in
           group order; G workgroups, S slots, laps = ceil(G / S)
  start    read the epoch e (the call's first tag b = e + 1)
  tile     load its tile (a few steps); slot[i mod S] <- (b + i // S) << 32
           | the tile's maximum; poll the group's done slot (bounded) for
           tag b; past the bound take the group's maximum from memory
  head     poll its tiles' slots (bounded): a slot with the tile's tag and a
           maximum is taken; one with a later lap's tag of this call (b + i
           // S < tag < b + laps) is read from memory at once; past the bound
           every slot still missing is read from memory; then store the
           group's maximum tagged b to the group's done slot
  count    (a tile once it holds its group's maximum, a head after its
           store) exit counter; the last workgroup advances the epoch by laps
  encode   a tile then encodes from its registers (a few steps) and exits

A workgroup runs only while it holds one of R resident places; a place frees
when a workgroup exits, and the next workgroup in launch order starts. Every
run must end (no workgroup waits forever) with every head and tile holding
its group's true maximum and the epoch advanced by laps, call after call,
and no tagged word touched after the epoch advanced (the last workgroup to
count out may clear them all when the epoch wraps).
"""

from __future__ import annotations

import random

import pytest

LOW = 0xFFFFFFFF


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


class Workspace:
    def __init__(self, S, ngroups):
        self.slot = _TaggedWords(self, S)
        self.done = _TaggedWords(self, ngroups)
        self.epoch = 0
        self.exits = 0
        self.G = 0          # workgroups of the current call
        self.laps = 0       # its laps over the slots
        self.advanced = False  # the current call's epoch has advanced
        self.tile_reads = 0   # tiles whose maximum a head read from memory
        self.group_reads = 0  # groups whose maximum a tile read from memory

    def check_live(self):
        assert not self.advanced, "a tagged word was touched after the epoch advanced"

    def count_out(self, e):
        # the last workgroup advances the epoch past the call's tags
        self.exits += 1
        if self.exits == self.G:
            self.epoch = e + self.laps
            self.exits = 0
            self.advanced = True


def plan(groups):
    """Launch order: (kind, group, index of the tile within the group)."""
    order = []
    for g, n in enumerate(groups):
        if n:
            order.append(("head", g, None))
            order += [("tile", g, u) for u in range(n)]
    return order


def tile_wg(ws, i, g, u, S, tile_max, group_max, load_steps, wait_polls):
    e = ws.epoch
    yield
    b = e + 1
    for _ in range(load_steps):
        yield
    ws.slot[i % S] = (b + i // S) << 32 | tile_max[g][u]
    yield
    amax = None
    for _ in range(wait_polls + 1):
        v = ws.done[g]
        yield
        if v >> 32 == b:
            amax = v & LOW
            break
    if amax is None:  # the group's maximum from its input
        for _ in range(load_steps):
            yield
        ws.group_reads += 1
        amax = group_max[g]
    ws.count_out(e)
    yield
    for _ in range(load_steps):  # the encode touches no workspace word
        yield
    return amax


def head_wg(ws, i, g, n, S, laps, tile_max, load_steps, lead_polls):
    e = ws.epoch
    yield
    b = e + 1
    first = i + 1  # the group's tile workgroups: first .. first + n - 1
    pending = set(range(n))
    direct = set()
    m = 0
    polls = 0
    while pending:
        vals = {u: ws.slot[(first + u) % S] for u in pending}
        yield
        polls += 1
        for u, v in vals.items():
            want = b + (first + u) // S
            tag = v >> 32
            if tag == want and (v & LOW) <= 0x7FFFFFFF:
                m = max(m, v & LOW)
                pending.discard(u)
            elif want < tag < b + laps:  # a later lap's workgroup took the slot
                pending.discard(u)
                direct.add(u)
        if pending and polls > lead_polls:
            direct |= pending
            pending = set()
    for u in sorted(direct):  # the missing tiles' maxima from the input
        for _ in range(load_steps):
            yield
        ws.tile_reads += 1
        m = max(m, tile_max[g][u])
    ws.done[g] = b << 32 | m
    yield
    ws.count_out(e)
    yield
    return m


def run(groups, S, R, seed, lead_polls=10_000, wait_polls=1_000_000, load_steps=3, calls=2,
        step_limit=3_000_000, epoch0=0):
    rng = random.Random(seed)
    order = plan(groups)
    G = len(order)
    laps = -(-G // S)
    ws = Workspace(S, len(groups))
    ws.epoch = epoch0
    ws.G, ws.laps = G, laps
    for call in range(calls):
        ws.advanced = False
        tile_max = [[rng.randrange(0, 1 << 30) for _ in range(n)] for n in groups]
        group_max = [max(t) if t else 0 for t in tile_max]
        e0 = ws.epoch
        pending = list(range(G))
        running, results = {}, {}
        steps = 0
        while pending or running:
            while pending and len(running) < R:
                i = pending.pop(0)
                kind, g, u = order[i]
                if kind == "head":
                    running[i] = head_wg(ws, i, g, groups[g], S, laps, tile_max, load_steps, lead_polls)
                else:
                    running[i] = tile_wg(ws, i, g, u, S, tile_max, group_max, load_steps, wait_polls)
            i = rng.choice(list(running))
            try:
                next(running[i])
            except StopIteration as stop:
                results[i] = stop.value
                del running[i]
            steps += 1
            assert steps < step_limit, f"no progress: groups={groups} S={S} R={R} seed={seed} call={call}"
        for i, (kind, g, u) in enumerate(order):
            assert results[i] == group_max[g], (kind, g, u, S, R, seed, call)
        assert ws.epoch == e0 + laps and ws.exits == 0
    return ws


GROUPS = {
    "moe": [3, 0, 7, 1, 0, 12, 5, 9, 2, 0, 4],
    "one": [17],
    "many_small": [1] * 30,
    "uneven": [0, 25, 0, 0, 2, 31, 0],
}


@pytest.mark.parametrize("name", sorted(GROUPS))
@pytest.mark.parametrize("S,R", [(8, 1), (8, 5), (16, 16), (16, 40), (64, 64), (64, 200), (4, 100)])
@pytest.mark.parametrize("seed", range(4))
def test_handoff_ends_with_each_groups_maximum(name, S, R, seed):
    # S below the grid size: several laps, and with R > S workgroups of a
    # later lap can overwrite slots before the head reads them
    run(GROUPS[name], S, R, seed, lead_polls=40)


@pytest.mark.parametrize("name", sorted(GROUPS))
def test_one_lap_with_the_whole_grid_resident_reads_nothing_twice(name):
    # every workgroup starts at once and no slot is reused: the heads take
    # every maximum from the slots and no tile falls back
    G = len(plan(GROUPS[name]))
    ws = run(GROUPS[name], S=G, R=G, seed=5, calls=3)
    assert ws.tile_reads == 0 and ws.group_reads == 0


def test_overwritten_slots_are_read_from_memory_not_taken():
    # a tiny slot array and the whole grid resident: later laps overwrite
    # slots, and the heads must read those tiles themselves
    ws = run(GROUPS["moe"], S=4, R=200, seed=7, calls=4)
    assert ws.tile_reads > 0


def test_one_resident_place_still_ends():
    # the head holds the only place, so its tiles cannot start: its bound
    # runs out, it reads every tile itself, and the tiles find the done slot
    ws = run(GROUPS["moe"], S=8, R=1, seed=8, lead_polls=3)
    assert ws.tile_reads > 0 and ws.group_reads == 0


def test_many_calls_keep_stale_tags_out():
    # old calls' slot and done words stay in the workspace: only this call's
    # tags may be taken
    run(GROUPS["uneven"], S=16, R=30, seed=9, lead_polls=20, calls=12)
