"""Host model of the fused backward's schedule (no GPU): per-XCD ticket
queues, key tile kt on queue kt mod nx in ascending order, each workgroup
adding its dQ slice of a step only after the previous tile of its queue
(kt - nx, same kv head) has published that step, and publishing on its own.

Random interleavings of workgroups, from one resident workgroup per XCD up,
with causal and full masks, several kv heads per launch and several query
heads per kv head, must always run every tile to the end (no state in which
no workgroup can move while work remains) and add into every row block in
ascending key-tile order, the order the results are defined by.
"""

import math
import random
from collections import defaultdict

import pytest

BKV, BQ = 128, 32  # keys per workgroup, rows per step


def _queue(x, nx, n_ktiles, nkv):
    """Tickets of queue x in hand-out order: (kt, g), kt ascending, g inner."""
    n_kt = (n_ktiles - 1 - x) // nx + 1 if x < n_ktiles else 0
    return [(x + nx * (i // nkv), i % nkv) for i in range(n_kt * nkv)]


def _steps(kt, S, heads_per_kv, causal):
    nqb = math.ceil(S / BQ)
    qb0 = kt * BKV // BQ if causal else 0
    return [(hi, qb) for hi in range(heads_per_kv) for qb in range(qb0, nqb)]


def _pred(kt, g, nx, n_ktiles):
    """The tile whose additions a tile waits for: the previous one of its queue."""
    return (kt - nx, g) if kt >= nx else None


def simulate(S, nx, slots, nkv, heads_per_kv, causal, rng, pred_of=_pred):
    """Runs the schedule with random choices; returns the additions per
    (queue, kv head, head, row block) in the order they happened. Raises on
    a deadlock."""
    n_ktiles = math.ceil(S / BKV)
    nqb = math.ceil(S / BQ)
    queues = [_queue(x, nx, n_ktiles, nkv) for x in range(nx)]
    assert sorted(t for q in queues for t in q) == sorted((kt, g) for kt in range(n_ktiles) for g in range(nkv))
    next_ticket = [0] * nx
    progress = defaultdict(int)  # (kt, g) -> published steps as code + 1
    adds = defaultdict(list)
    # a workgroup: its XCD, and (tile, steps, index of the next step, code
    # added but not yet published) or None between tiles
    wgs = [[x, None] for x in range(nx) for _ in range(slots[x])]
    finished = 0
    total = n_ktiles * nkv
    while finished < total:
        moves = []
        for w in wgs:
            x, st = w
            if st is None:
                if next_ticket[x] < len(queues[x]):
                    moves.append((w, "take"))
                continue
            (kt, g), steps, i, pending = st
            if pending is not None:
                moves.append((w, "publish"))  # depends on nothing but the workgroup's own stores
            if i < len(steps):
                hi, qb = steps[i]
                code = hi * nqb + qb
                pred = pred_of(kt, g, nx, n_ktiles)
                # a step's addition waits for the predecessor's publication of
                # that step and, in the kernel, follows its own previous
                # publication (the publish of step i - 1 comes first in step i)
                if pending is None and (pred is None or progress[pred] > code):
                    moves.append((w, "add"))
        if not moves:
            raise AssertionError("deadlock: work remains and no workgroup can move")
        w, kind = rng.choice(moves)
        x, st = w
        if kind == "take":
            kt, g = queues[x][next_ticket[x]]
            next_ticket[x] += 1
            w[1] = [(kt, g), _steps(kt, S, heads_per_kv, causal), 0, None]
        elif kind == "add":
            (kt, g), steps, i, _ = st
            hi, qb = steps[i]
            adds[(x, g, hi, qb)].append(kt)
            st[2], st[3] = i + 1, hi * nqb + qb
        else:
            (kt, g), steps, i, pending = st
            progress[(kt, g)] = pending + 1
            st[3] = None
            if i == len(steps):
                w[1] = None
                finished += 1
    return adds, n_ktiles, nqb


@pytest.mark.parametrize("S,nx,slot_counts,nkv,hpk,causal", [
    (1, 8, 1, 1, 1, True),
    (129, 8, 1, 1, 1, True),
    (2309, 8, 1, 1, 1, True),
    (2309, 8, 3, 1, 1, True),
    (5000, 8, 2, 2, 1, True),
    (5000, 8, 2, 1, 2, True),
    (3000, 8, 1, 2, 2, False),
    (4100, 4, 5, 1, 1, True),
    (4100, 1, 2, 1, 1, True),
    (4100, 8, "uneven", 1, 1, True),
])
def test_every_tile_finishes_and_adds_in_tile_order(S, nx, slot_counts, nkv, hpk, causal):
    for seed in range(6):
        rng = random.Random(1000 * seed + S)
        slots = [1 + (x % 3) for x in range(nx)] if slot_counts == "uneven" else [slot_counts] * nx
        adds, n_ktiles, nqb = simulate(S, nx, slots, nkv, hpk, causal, rng)
        for x in range(nx):
            for g in range(nkv):
                for hi in range(hpk):
                    for qb in range(nqb):
                        expected = [kt for kt in range(x, n_ktiles, nx) if not causal or kt * BKV // BQ <= qb]
                        assert adds.get((x, g, hi, qb), []) == expected, (x, g, hi, qb)


def test_waiting_for_a_later_ticket_is_caught_as_a_deadlock():
    """The model bites: pointed at the next tile of the queue (a ticket that
    is not handed out while the only resident workgroup waits), it stops."""
    later = lambda kt, g, nx, n: (kt + nx, g) if kt + nx < n else None  # noqa: E731
    with pytest.raises(AssertionError, match="deadlock"):
        simulate(2309, 8, [1] * 8, 1, 1, True, random.Random(3), pred_of=later)


def test_adding_without_waiting_breaks_the_order():
    """Without the wait, some interleaving adds a later tile first."""
    never = lambda kt, g, nx, n: None  # noqa: E731
    broken = False
    for seed in range(20):
        adds, n_ktiles, nqb = simulate(2309, 8, [3] * 8, 1, 1, True, random.Random(seed), pred_of=never)
        broken |= any(v != sorted(v) for v in adds.values())
    assert broken
