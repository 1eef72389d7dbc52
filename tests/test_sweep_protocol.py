"""A CPU model of the plain sweep kernel's hand-over between its resolver wave
and its applier waves, run under random interleavings.

The kernel (greedy_iou_nms_amd/csrc/sweep.hip) hands chunks of 64 sorted rows
between waves through LDS: a ring of staging slots with `ready` and
`app_lag` flags, a `resolved` counter, the settled words, and the removed
bitmap that the resolver reads while appliers OR far words into it.  One
wave's LDS operations take effect in the order it issues them, so the model
treats every LDS access as one atomic step and lets a random scheduler pick
which wave takes the next step.  Each wave's steps follow the kernel's
program order, including the reads it issues ahead of time (the removed
word of chunk c + 1 and the staged batch of chunk c + 2 are read before
chunk c is settled).  Global memory written by the mask kernel is input
here and needs no step.

The result of every schedule must be the greedy result of a sequential
sweep over the same mask (the definition, "LeetCUDA 14-nms" Phase 2: visit
rows in order, keep a row that is not yet removed, OR its row in).  Planted
mistakes in the protocol (an applier that reports its chunk before ORing its
words, a resolver that skips the applied check) must be caught by some
schedule, which shows the model can see the races it is meant to rule out.
"""
import random

import pytest

B = 8          # rows per chunk in the model (64 in the kernel)
NEAR = 4       # NEAR_TILES
LAG = NEAR + 1
RING = 16
APPLIERS = 7
FULL = (1 << B) - 1


def make_mask(rng, words, density):
    """Upper-triangular suppression mask: M[p] is a dict word -> bits of
    row p, bits only for columns q > p; every word of the row band."""
    n = words * B
    rows = []
    for p in range(n):
        row = {}
        for q in range(p + 1, n):
            # overlaps mostly close by, a few far away
            near = q - p <= 3 * B
            if rng.random() < (density if near else density / 8):
                row[q // B] = row.get(q // B, 0) | (1 << (q % B))
        rows.append(row)
    return rows


def greedy(rows, words):
    n = words * B
    removed = [0] * (words + NEAR + 1)
    kept = []
    for p in range(n):
        if (removed[p // B] >> (p % B)) & 1:
            continue
        kept.append(p)
        for w, v in rows[p].items():
            removed[w] |= v
    return kept


class Lds:
    def __init__(self, words):
        self.near = [[[0] * B for _ in range(NEAR + 1)] for _ in range(RING)]
        self.nzn = [0] * RING
        self.ready = [0] * RING
        self.app_lag = [t + 1 if t < LAG else 0 for t in range(RING)]
        self.settled = [(0, 0)] * RING
        self.resolved = 0
        self.removed = [0] * (words + NEAR + 1)


def resolver(lds, words, skip_applied_check=False):
    """The resolver wave: settles chunks in order (resolve_chunks /
    resolve_one).  A generator: every yield is one LDS access."""
    out = {"kept": []}

    def read_staged(x, into):
        s = x % RING
        into["ready"] = lds.ready[s]
        yield
        into["nzn"] = lds.nzn[s]
        yield
        into["nw"] = [list(lds.near[s][j]) for j in range(NEAR + 1)]
        yield

    def read_word(x, into):
        into["app_lag"] = lds.app_lag[x % RING]
        yield
        into["rem"] = lds.removed[x]
        yield

    b = [dict(), dict(), dict()]
    wb = dict()
    yield from read_staged(0, b[0])
    yield from read_staged(1, b[1])
    yield from read_word(0, wb)
    carry = 0
    total = 0
    for c in range(words):
        cur, ahead = b[c % 3], b[(c + 2) % 3]
        want = c + 1
        if cur["ready"] != want or (wb["app_lag"] != want and not skip_applied_check):
            while lds.ready[c % RING] < want:
                yield
            while lds.app_lag[c % RING] < want and not skip_applied_check:
                yield
            yield from read_staged(c, cur)
            yield from read_word(c, wb)
        rem = wb["rem"] | carry
        yield from read_word(c + 1, wb)
        yield from read_staged(c + 2, ahead)
        d = cur["nw"][0]
        for k in range(B):
            if not (rem >> k) & 1:
                rem |= d[k]
        kept = ~rem & FULL
        out["kept"].extend(c * B + k for k in range(B) if (kept >> k) & 1)
        c1 = 0
        for k in range(B):
            if (kept >> k) & 1:
                c1 |= cur["nw"][1][k]
        for j in range(2, NEAR + 1):
            v = 0
            for k in range(B):
                if (kept >> k) & 1:
                    v |= cur["nw"][j][k]
            if v:
                lds.removed[c + j] |= v
                yield
        carry = c1
        lds.settled[c % RING] = (rem, total)
        yield
        lds.resolved = want
        yield
        total += bin(kept).count("1")
    return out


def applier(lds, q, words, rows, report_early=False):
    """Applier wave q (1..APPLIERS): chunks q - 1, q - 1 + A, ... (apply_chunks
    / apply_one).  Far words (tiles beyond c + NEAR) come from the row tile's
    list, read from global memory."""

    def level1(c):
        near = [[0] * B for _ in range(NEAR + 1)]
        for k in range(B):
            for j in range(NEAR + 1):
                near[j][k] = rows[c * B + k].get(c + j, 0)
        return near

    def stage(near, c):
        s = c % RING
        for j in range(NEAR + 1):
            lds.near[s][j] = list(near[j])
        yield
        ahead = 0
        for k in range(B):
            if any(near[j][k] for j in range(1, NEAR + 1)):
                ahead |= 1 << k
        lds.nzn[s] = ahead
        yield
        lds.ready[s] = c + 1
        yield

    def far_entries(c):
        return [(k, w, v) for k in range(B) for w, v in rows[c * B + k].items()
                if w > c + NEAR]

    A = APPLIERS
    c = q - 1
    if c >= words:
        return
    l1 = level1(c)
    yield from stage(l1, c)
    if c + A < words:
        l1 = level1(c + A)
    while c < words:
        if c + A < words:
            yield from stage(l1, c + A)
            if c + 2 * A < words:
                l1 = level1(c + 2 * A)
        while lds.resolved < c + 1:
            yield
        rem, _ = lds.settled[c % RING]
        yield
        kept = ~rem & FULL
        if report_early:
            lds.app_lag[(c + LAG) % RING] = c + LAG + 1
            yield
        for k, w, v in far_entries(c):
            if (kept >> k) & 1:
                lds.removed[w] |= v
                yield
        if not report_early:
            lds.app_lag[(c + LAG) % RING] = c + LAG + 1
            yield
        c += A


def run_schedule(rows, words, seed, **mistakes):
    """One random interleaving; returns the resolver's kept rows (None if
    the schedule did not finish within its step budget)."""
    rng = random.Random(seed)
    lds = Lds(words)
    res_mistake = {k: v for k, v in mistakes.items() if k == "skip_applied_check"}
    app_mistake = {k: v for k, v in mistakes.items() if k == "report_early"}
    res = resolver(lds, words, **res_mistake)
    waves = [res] + [applier(lds, q, words, rows, **app_mistake)
                     for q in range(1, APPLIERS + 1)]
    # per-schedule speeds: some waves run much slower than others
    weight = [rng.choice([1, 1, 2, 5, 20]) for _ in waves]
    alive = list(range(len(waves)))
    result = None
    for _ in range(200000):
        if not alive:
            break
        i = rng.choices(alive, weights=[weight[a] for a in alive])[0]
        try:
            next(waves[i])
        except StopIteration as stop:
            alive.remove(i)
            if i == 0:
                result = stop.value["kept"]
    return result


def _cases(count, words):
    rng = random.Random(1234)
    return [make_mask(rng, words, rng.choice([0.05, 0.15, 0.4])) for _ in range(count)]


@pytest.mark.parametrize("words", [1, 2, 5, 9, 17, 23])
def test_protocol_matches_sequential_greedy(words):
    for ci, rows in enumerate(_cases(3, words)):
        want = greedy(rows, words)
        for seed in range(60):
            got = run_schedule(rows, words, seed)
            assert got is not None, "schedule did not finish (words=%d case=%d seed=%d)" % (
                words, ci, seed)
            assert got == want, "words=%d case=%d seed=%d" % (words, ci, seed)


@pytest.mark.parametrize("mistake", ["report_early", "skip_applied_check"])
def test_planted_protocol_mistakes_are_caught(mistake):
    words = 23
    caught = False
    for ci, rows in enumerate(_cases(4, words)):
        want = greedy(rows, words)
        for seed in range(80):
            got = run_schedule(rows, words, seed, **{mistake: True})
            if got is not None and got != want:
                caught = True
                break
        if caught:
            break
    assert caught, "no schedule exposed the planted mistake %s" % mistake
