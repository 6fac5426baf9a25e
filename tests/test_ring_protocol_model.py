"""Host model of the whole-pass kernel's in-kernel ring protocol, explored over
worker interleavings (CPU only; nothing runs on a GPU).

The whole-pass mode ran every ring round of a pass in one persistent launch
("Mixture-of-Kittens(MoK)란?" explainer, section 4 ③: a fixed ring of
mini-batch slots reused without the host). Two runs that included it hung
without a shown cause, so the library rejects the mode. This model asks
whether the protocol itself can deadlock or race. It mirrors the kernel's
claim/wait/publish steps one for one:

* items in one order: per round r (S = min(slots, G) mini-batches, ascending
  forward, descending backward), segment 3r = gather items (ceil(MB/64) per
  mini-batch), 3r+1 = producer tiles, 3r+2 = consumer tiles; tile segments are
  cut into 8 per-XCD chunks of ceil(n/8) items, numbered in the group order of
  kGroupM = 4 m-tiles;
* a worker (thread 0 of a workgroup, XCD = its index mod 8) scans segments
  from its cursor and claims with fetch-and-add, its own XCD's chunk first;
* waits: a gather of round r waits until released[slot] >= r; a worker's first
  producer tile of round r waits until every gather of round r is done;
  a consumer tile waits until its m-tile's producer tiles are done;
* publishing: gathers count full[r]; producer tiles count done[m-tile]; the
  slot's last readers (consumers forward, producers backward) count used[g]
  and release the slot when complete.

Each state is explored with every enabled step of every worker (claim, start,
finish), so all interleavings are covered, up to a state budget beyond which
random schedules take over. Checked: no state where unfinished workers are all
blocked (deadlock), every item runs exactly once, and no item starts before
what it reads is finished or while its slot's previous occupant is still read.
The schedules are the oracle's for the configurations and ring sizes of the
GPU knob tests.
"""
import random

import numpy as np
import pytest

import synth
from oracle import schedule as S

XCDS, GROUP_M, GATHER_ROWS = 8, 4, 64


def item_tile(i, nt, mtc):
    gsize = GROUP_M * nt
    grp, r = divmod(i, gsize)
    first = grp * GROUP_M
    gm = min(GROUP_M, mtc - first)
    return first + r % gm, r // gm


class Pass:
    """The item structure of one pass for a schedule (m-tiles per mini-batch)."""

    def __init__(self, mt_per_g, n_slots, MB, nt1, nt2, reverse):
        self.G = len(mt_per_g)
        self.mtfirst = np.concatenate([[0], np.cumsum(mt_per_g)]).astype(int)
        self.n_slots = n_slots
        self.S = min(n_slots, self.G)
        self.NR = (self.G + self.S - 1) // self.S
        self.cpm = (MB + GATHER_ROWS - 1) // GATHER_ROWS
        self.nt1, self.nt2, self.reverse = nt1, nt2, reverse
        self.release_cls = 2 if reverse else 3
        self.mtile_g = np.repeat(np.arange(self.G), mt_per_g)

    def span(self, r):
        if not self.reverse:
            a = r * self.S
            return a, min(self.G, a + self.S)
        b = self.G - r * self.S
        return max(0, b - self.S), b

    def seg_len(self, seg):
        r, c = divmod(seg, 3)
        a, b = self.span(r)
        if c == 0:
            return (b - a) * self.cpm
        return (self.mtfirst[b] - self.mtfirst[a]) * (self.nt1 if c == 1 else self.nt2)


def explore(p: Pass, n_workers: int, max_states: int, rng=None, walks=0):
    """Breadth-first over all interleavings (or `walks` random schedules when
    rng is given). Returns the number of states visited."""
    nseg = 3 * p.NR
    # claimed / started / finished items are keyed (seg, index in segment)

    def initial():
        heads = tuple(0 for _ in range(nseg * XCDS))
        workers = tuple((0, -1, None, "idle") for _ in range(n_workers))   # cursor, acq_round, item, phase
        counters = (tuple([0] * p.NR), tuple([0] * int(p.mtfirst[-1])), tuple([0] * p.G),
                    tuple([0] * min(p.n_slots, p.G)))
        return heads, workers, counters, frozenset(), frozenset()

    def claim(state, w):
        """The worker's claim scan; returns the new state (item claimed, or the
        worker finished when the queue is drained)."""
        heads, workers, counters, running, finished = state
        cursor, acq, _, _ = workers[w]
        heads = list(heads)
        xcd = w % XCDS
        for seg in range(cursor, nseg):
            r, c = divmod(seg, 3)
            a, b = p.span(r)
            n = p.seg_len(seg)
            if c == 0:
                h = heads[seg * XCDS]
                if h >= n:
                    continue
                heads[seg * XCDS] = h + 1
                g = a + h // p.cpm
                item = (seg, h, "gather", g, r)
                return _set(state, w, (seg, acq, item, "wait"), heads=tuple(heads))
            per = -(-n // XCDS)
            lo = int(p.mtfirst[a])
            mtc = int(p.mtfirst[b]) - lo
            for i in range(XCDS):
                x = (xcd + i) % XCDS
                start, ln = x * per, min(n - x * per, per)
                if heads[seg * XCDS + x] >= ln:
                    continue
                h = heads[seg * XCDS + x]
                heads[seg * XCDS + x] = h + 1
                j, nn = item_tile(start + h, p.nt1 if c == 1 else p.nt2, mtc)
                kind = "producer" if c == 1 else "consumer"
                item = (seg, start + h, kind, lo + j, r)
                return _set(state, w, (seg, acq, item, "wait"), heads=tuple(heads))
        return _set(state, w, (nseg, acq, None, "done"), heads=tuple(heads))

    def _set(state, w, wstate, heads=None, counters=None, running=None, finished=None):
        h0, ws, c0, r0, f0 = state
        ws = list(ws)
        ws[w] = wstate
        return (h0 if heads is None else heads, tuple(ws), c0 if counters is None else counters,
                r0 if running is None else running, f0 if finished is None else finished)

    def wait_ok(state, w):
        _, workers, (full, done, used, released), _, _ = state
        cursor, acq, item, _ = workers[w]
        seg, idx, kind, m, r = item
        if kind == "gather":
            return released[m % p.n_slots] >= r
        if kind == "producer":
            return acq >= r or full[r] >= (lambda ab: (ab[1] - ab[0]) * p.cpm)(p.span(r))
        return done[m] >= p.nt1

    def readers_of(g):
        """Tile items that read mini-batch g's ring slots: its producers (x / dy
        ring) and, forward, its consumers (a-ring)."""
        out = set()
        r = next(rr for rr in range(p.NR) if p.span(rr)[0] <= g < p.span(rr)[1])
        a, b = p.span(r)
        lo, mtc = int(p.mtfirst[a]), int(p.mtfirst[b]) - int(p.mtfirst[a])
        for c, nt in ((1, p.nt1), (2, p.nt2)):
            if c == 2 and p.reverse:
                continue
            for i in range(mtc * nt):
                j, _ = item_tile(i, nt, mtc)
                if p.mtile_g[lo + j] == g:
                    out.add((3 * r + c, i))
        return out

    prev_occupant = {}
    order = [g for r in range(p.NR) for g in (range(*p.span(r)))]
    last = {}
    for g in order:
        s = g % p.n_slots
        prev_occupant[g] = last.get(s)
        last[s] = g
    readers = {g: readers_of(g) for g in range(p.G)}

    def start(state, w):
        heads, workers, counters, running, finished = state
        cursor, acq, item, _ = workers[w]
        seg, idx, kind, m, r = item
        key = (seg, idx)
        assert key not in running and key not in finished, f"item {key} runs twice"
        if kind == "gather":
            g0 = prev_occupant[m]
            if g0 is not None:
                busy = readers[g0] - finished
                assert not busy, f"gather of mini-batch {m} overwrites slot {m % p.n_slots} while {busy} read it"
        elif kind == "producer":
            g = int(p.mtile_g[m])
            a, b = p.span(r)
            need = {(3 * r, i) for i in range((g - a) * p.cpm, (g - a + 1) * p.cpm)}
            assert need <= finished, f"producer of m-tile {m} before its gathers"
            g0 = prev_occupant[g]
            if g0 is not None and not p.reverse:     # it writes the a-ring slot the old consumers read
                busy = {k for k in readers[g0] if k[0] % 3 == 2} - finished
                assert not busy, f"producer of mini-batch {g} overwrites the a-ring slot while {busy} read it"
            acq = max(acq, r)
        else:
            a, b = p.span(r)
            lo, mtc = int(p.mtfirst[a]), int(p.mtfirst[b]) - int(p.mtfirst[a])
            need = {(seg - 1, i) for i in range(mtc * p.nt1) if lo + item_tile(i, p.nt1, mtc)[0] == m}
            assert need <= finished, f"consumer of m-tile {m} before its producers"
        return _set(state, w, (cursor, acq, item, "run"), running=running | {key})

    def finish(state, w):
        heads, workers, (full, done, used, released), running, finished = state
        cursor, acq, item, _ = workers[w]
        seg, idx, kind, m, r = item
        full, done, used, released = list(full), list(done), list(used), list(released)
        if kind == "gather":
            full[r] += 1
        else:
            cls = 2 if kind == "producer" else 3
            if kind == "producer":
                done[m] += 1
            if cls == p.release_cls:
                g = int(p.mtile_g[m])
                used[g] += 1
                expect = (p.mtfirst[g + 1] - p.mtfirst[g]) * (p.nt1 if cls == 2 else p.nt2)
                if used[g] == expect:
                    released[g % p.n_slots] += 1
        key = (seg, idx)
        return _set(state, w, (cursor, acq, None, "idle"),
                    counters=(tuple(full), tuple(done), tuple(used), tuple(released)),
                    running=running - {key}, finished=finished | {key})

    def successors(state):
        out = []
        for w, (_, _, item, phase) in enumerate(state[1]):
            if phase == "idle":
                out.append(claim(state, w))
            elif phase == "wait":
                if wait_ok(state, w):
                    out.append(start(state, w))
            elif phase == "run":
                out.append(finish(state, w))
        return out

    total_items = sum(p.seg_len(s) for s in range(nseg))

    def check_terminal(state):
        _, workers, _, running, finished = state
        live = [w for w in workers if w[3] != "done"]
        assert not live, f"deadlock: workers {live} are all blocked"
        assert not running and len(finished) == total_items

    if rng is None:
        seen = {initial()}
        frontier = [initial()]
        while frontier:
            nxt = []
            for st in frontier:
                succ = successors(st)
                if not succ:
                    check_terminal(st)
                for s2 in succ:
                    if s2 not in seen:
                        seen.add(s2)
                        nxt.append(s2)
                if len(seen) > max_states:
                    return None
            frontier = nxt
        return len(seen)
    for _ in range(walks):
        st = initial()
        while True:
            succ = successors(st)
            if not succ:
                check_terminal(st)
                break
            st = succ[rng.randrange(len(succ))]
    return walks


def pass_of(cfg, MB, ring_bytes, row_bytes, BM, nt1, nt2, reverse):
    ids, _, _ = synth.make_routing(cfg)
    s = S.build(ids, cfg.E, MB, cfg.macrobatch_tokens)
    mt = np.zeros(s.G, dtype=int)
    for (g, e, q0, n) in s.segments:
        mt[g] += -(-n // BM)
    return Pass(mt, ring_bytes // (MB * row_bytes), MB, nt1, nt2, reverse)


def tiny_pass(mt_per_g, slots, reverse, nt1=1, nt2=2):
    return Pass(np.array(mt_per_g), slots, 64, nt1, nt2, reverse)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("shape", [([1, 2, 1, 1], 2), ([2, 1, 3], 2), ([1, 1, 1, 1, 1], 3), ([3, 2], 4)])
@pytest.mark.parametrize("workers", [1, 2])
def test_every_interleaving_of_small_passes(shape, workers, reverse):
    mt, slots = shape
    n = explore(tiny_pass(mt, slots, reverse), workers, max_states=3_000_000)
    assert n is not None, "state budget exceeded"


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("workers", [3, 4])
def test_more_workers_small_pass(reverse, workers):
    n = explore(tiny_pass([1, 2, 1], 2, reverse, nt1=1, nt2=1), workers, max_states=3_000_000)
    assert n is not None, "state budget exceeded"


# the k = 1 knob-test workload on every ring size its sweep used (BF16: 768-byte
# rows, 256-row m-tiles, one gate/up n-tile of 128 i-columns, two down n-tiles)
K1 = synth.small_config("k1_macro", T=1000, H=384, I=128, E=3, k=1, minibatch_rows=64, macrobatch_tokens=300,
                        ring_bytes=4 * 64 * 768, routing="dirichlet")
K1_RINGS = [(64, 4 * 64 * 768), (64, 2 * 64 * 768), (16, 4 * 64 * 768), (64, 1 << 24), (512, 2 * 512 * 768)]
# MXFP8 variant of the same workload (396-byte rows, the removed MXFP8 pass used the same protocol)
MX1 = synth.small_config("mx_k1_macro", T=1000, H=384, I=256, E=3, k=1, minibatch_rows=64, macrobatch_tokens=300,
                         ring_bytes=4 * 64 * 396, routing="dirichlet", precision="mxfp8")
MX1_RINGS = [(64, 4 * 64 * 396), (64, 2 * 64 * 396), (16, 4 * 64 * 396), (96, 2 * 96 * 396), (64, 1 << 22)]


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("mb,ring", K1_RINGS)
def test_knob_test_schedules_bf16(mb, ring, reverse):
    p = pass_of(K1, mb, ring, 768, 256, 1, 2, reverse)
    assert explore(p, 1, max_states=50_000) is not None      # one worker: the single interleaving
    for workers in (2, 3, 4):
        explore(p, workers, 0, random.Random(7 * workers + reverse), walks=40)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("mb,ring", MX1_RINGS)
def test_knob_test_schedules_mxfp8(mb, ring, reverse):
    p = pass_of(MX1, mb, ring, 396, 256, 2, 2, reverse)
    for workers in (1, 2, 3, 4):
        explore(p, workers, 0, random.Random(11 * workers + reverse), walks=25)


def test_model_catches_a_broken_protocol():
    # control: the same model with the slot release moved to the producers in
    # the forward pass (the a-ring is then overwritten while consumers read it)
    p = tiny_pass([1, 1, 1], 2, False)
    p.release_cls = 2
    with pytest.raises(AssertionError, match="overwrites"):
        for seed in range(200):
            explore(p, 3, 0, random.Random(seed), walks=5)
