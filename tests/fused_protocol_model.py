"""CPU model of the single-launch layer's task queue and completion-flag protocol.

The single-launch form of the layer (tilelang.dataflow README, section 3.5:
GEMM-1 and GEMM-2 under one wrapper launch, their dependency resolved without a
kernel boundary) runs every step in one persistent grid.  This module models
that protocol as a discrete-event simulation, independent of the HIP code, so
that its properties can be checked on the CPU under random skews before and
besides any GPU run:

* Plan.  Every workgroup derives the same plan from the routing ids: per-expert
  counts, 16-row group blocks, padded offsets in expert order, M-tiles of MT1
  group blocks for GEMM-1 and of MT2 (a multiple of MT1) for GEMM-2, experts
  ranked by descending count (ties by id), and one task list: every GEMM-1
  task, then every GEMM-2 task, each by (rank, column block, M-tile).
* Queue.  One counter; a workgroup claims the next index with a fetch-add, the
  claim for its next task going out while its current task still runs.  An
  index past the list means no task is left.
* Flags.  A GEMM-1 task stores its rows of h, waits for the stores, then adds 1
  to the counter of the GEMM-2 M-tile its rows belong to.  A GEMM-2 task may
  load its weights first, then waits (bounded) until that counter reaches the
  number of GEMM-1 column blocks times the GEMM-1 M-tiles it holds, then reads h.
* Combine.  A GEMM-2 task stores its y rows, waits for them, then adds 1 per
  row to the arrival counter of (token, column block).  Once its queue is
  empty, workgroup b takes the (token, column block) outputs b, b + grid, ...:
  it waits (bounded) until each counter reaches the token's number of valid
  slots, sums the token's y rows in ascending slot order (zeros for a token
  without a valid slot), writes the output columns and resets the counter.
* Exit.  Each workgroup adds 1 to an exit counter after its last memory
  operation; the one that sees grid - 1 resets the queue, the exit counter and
  the M-tile counters, so the next call starts from zeros.

Deadlock freedom does not assume that all workgroups are resident: tasks are
claimed in list order by running workgroups, GEMM-1 tasks never wait, and a
GEMM-2 task waits only on GEMM-1 tasks of lower index, so the lowest unfinished
claimed task can always proceed; the combine of a workgroup whose queue is
empty waits only on GEMM-2 tasks, all claimed by then.  The simulation checks this with a resident
capacity below the grid size.
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass, field

import numpy as np

BLOCK_M = 16


@dataclass
class Plan:
    counts: np.ndarray
    tiles: np.ndarray
    poff: np.ndarray
    mt: list        # per list: M-tiles of each expert
    order: np.ndarray
    toff: list
    n1: int
    n2: int
    mtb: tuple      # group blocks per M-tile: (GEMM-1, GEMM-2)
    nb1: int
    nb2: int

    @property
    def total(self):
        return self.n1 + self.n2

    def decode(self, i):
        """Task i -> (list, expert, first padded row, row blocks, column block, M-tile)."""
        lst = 0 if i < self.n1 else 1
        j = i if lst == 0 else i - self.n1
        nb = self.nb1 if lst == 0 else self.nb2
        off = self.toff[lst]
        r = int(np.searchsorted(off, j, side="right")) - 1  # the last rank starting at or before j: never empty
        e = int(self.order[r])
        mt = int(self.mt[lst][e])
        cb, m = divmod(j - int(off[r]), mt)
        assert 0 <= cb < nb
        mtb = self.mtb[lst]
        row0 = int(self.poff[e]) + BLOCK_M * mtb * m
        nsub = min(mtb, int(self.tiles[e]) - mtb * m)
        return lst, e, row0, nsub, cb, m

    def g2_tile(self, e, row0):
        """First group block of the GEMM-2 M-tile holding padded row row0 of expert e: its counter."""
        span = BLOCK_M * self.mtb[1]
        return (int(self.poff[e]) + (row0 - int(self.poff[e])) // span * span) // BLOCK_M

    def target(self, nsub2):
        """GEMM-1 column blocks that store the h rows of a GEMM-2 M-tile of nsub2 group blocks."""
        return self.nb1 * -(-nsub2 // self.mtb[0])


def make_plan(ids, E, mtb, nb1, nb2):
    """mtb: group blocks per M-tile, an int (both GEMMs) or (GEMM-1, GEMM-2) with GEMM-2's a multiple."""
    mtb = (mtb, mtb) if isinstance(mtb, int) else tuple(mtb)
    assert mtb[1] % mtb[0] == 0
    ids = np.asarray(ids).ravel()
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E).astype(np.int64)
    tiles = (counts + BLOCK_M - 1) // BLOCK_M
    poff = np.concatenate([[0], np.cumsum(BLOCK_M * tiles)])
    mt = [(tiles + b - 1) // b for b in mtb]
    order = np.array(sorted(range(E), key=lambda e: (-counts[e], e)), dtype=np.int64)
    toff = []
    for lst, nb in enumerate((nb1, nb2)):
        per = mt[lst][order] * nb
        toff.append(np.concatenate([[0], np.cumsum(per)]))
    return Plan(counts, tiles, poff, mt, order, toff, int(toff[0][-1]), int(toff[1][-1]), mtb, nb1, nb2)


def rows_of(ids, E, plan, e, m, nsub, nsub_list=0):
    """Assignments of the M-tile's rows (ascending p within the expert), -1 on padding rows."""
    ids = np.asarray(ids).ravel()
    ps = np.nonzero(ids == e)[0]
    lo = BLOCK_M * plan.mtb[1 if nsub_list else 0] * m
    out = np.full(BLOCK_M * nsub, -1, dtype=np.int64)
    take = ps[lo:lo + BLOCK_M * nsub]
    out[:len(take)] = take
    return out


@dataclass
class Faults:
    """Planted protocol mistakes, to show that the checks below catch them."""
    g2_first: bool = False          # GEMM-2 tasks placed before GEMM-1 tasks in the list
    short_wait: bool = False        # GEMM-2 waits for one column block fewer
    flag_before_store: bool = False  # the M-tile counter is raised before h is stored
    no_reset: bool = False          # the last workgroup does not reset the counters
    arrive_off_by_one: bool = False  # the combine waits for one arrival fewer


@dataclass
class State:
    queue: int = 0
    exit: int = 0
    timeouts: int = 0
    done1: dict = field(default_factory=dict)
    arrive: dict = field(default_factory=dict)


class Sim:
    """Discrete-event run of one call.  Times are arbitrary units; every atomic
    happens at one instant, in event order."""

    def __init__(self, ids, T, k, E, nb1, nb2, mtb, grid, resident, rng, faults=None, state=None,
                 spin_limit=200000, poll=1.0):
        self.ids = np.asarray(ids).reshape(T, k)
        self.T, self.k, self.E = T, k, E
        self.plan = make_plan(self.ids, E, mtb, nb1, nb2)
        self.grid, self.resident = grid, resident
        self.rng = rng
        self.f = faults or Faults()
        self.st = state if state is not None else State()
        self.spin_limit, self.poll = spin_limit, poll
        self.valid = (self.ids >= 0) & (self.ids < E)
        self.nvalid = self.valid.sum(axis=1)
        # observations
        self.executed = {}
        self.h_ready = {}            # (rb, cb1) -> time h was stored
        self.y_ready = {}            # (p, cb2) -> time y was stored
        self.out_written = {}        # (t, cb2) -> count
        self.zero_rows = {}
        self.errors = []
        self.events = []
        self.seq = 0
        self.now = 0.0
        self.running = 0
        self.started = 0
        self.exited = 0

    # -- plan helpers -------------------------------------------------------
    def task(self, i):
        p = self.plan
        if self.f.g2_first:
            # planted: the GEMM-2 part of the list first
            i = i + p.n1 if i < p.n2 else i - p.n2
        return p.decode(i)

    def push(self, t, fn):
        self.seq += 1
        heapq.heappush(self.events, (t, self.seq, fn))

    def dur(self, scale):
        return float(self.rng.lognormal(0.0, 0.8)) * scale

    # -- workgroup ----------------------------------------------------------
    def claim(self):
        i = self.st.queue
        self.st.queue += 1
        return i if 0 <= i < self.plan.total else -1

    def start_wg(self, b):
        self.running += 1
        self.started += 1
        # prologue: the plan, then the first claim
        slot = self.claim()
        self.push(self.now + self.dur(1.0), lambda: self.run_task(b, slot))

    def run_task(self, b, slot):
        if slot < 0:
            return self.combine_share(b)
        lst, e, row0, nsub, cb, m = self.task(slot)
        if slot in self.executed:
            self.errors.append(f"task {slot} executed twice")
        self.executed[slot] = b
        rb = row0 // BLOCK_M
        g2 = self.plan.g2_tile(e, row0)  # counter of the GEMM-2 M-tile
        length = self.dur(10.0)
        nxt = {}

        def do_claim():
            nxt["slot"] = self.claim()

        # the claim for the next task goes out during the task's last K blocks
        claim_frac = float(self.rng.uniform(0.3, 0.95))
        if lst == 0:
            self.push(self.now + length * claim_frac, do_claim)
            def g1_end():
                if self.f.flag_before_store:
                    self.st.done1[g2] = self.st.done1.get(g2, 0) + 1
                    self.push(self.now + self.dur(0.5), lambda: self.h_store(rb, nsub, cb))
                else:
                    self.h_store(rb, nsub, cb)
                    self.st.done1[g2] = self.st.done1.get(g2, 0) + 1
                self.push(self.now + self.dur(0.2), lambda: self.run_task(b, nxt["slot"]))
            self.push(self.now + length, g1_end)
        else:
            target = self.plan.target(nsub) - (1 if self.f.short_wait else 0)
            polls = {"n": 0}

            def wait():
                if self.st.done1.get(g2, 0) >= target:
                    return self.g2_body(b, slot, e, row0, nsub, cb, m, rb, length, nxt, claim_frac, do_claim)
                polls["n"] += 1
                if polls["n"] > self.spin_limit:
                    self.st.timeouts += 1
                    self.errors.append(f"wait of task {slot} timed out")
                    return self.g2_body(b, slot, e, row0, nsub, cb, m, rb, length, nxt, claim_frac, do_claim)
                self.push(self.now + self.poll, wait)
            # the weight stages are requested before the wait
            self.push(self.now + self.dur(0.5), wait)

    def h_store(self, rb, nsub, cb):
        for i in range(nsub):  # every group block of the GEMM-1 M-tile
            self.h_ready[(rb + i, cb)] = self.now

    def g2_body(self, b, slot, e, row0, nsub, cb, m, rb, length, nxt, claim_frac, do_claim):
        self.push(self.now + length * claim_frac, do_claim)
        for i in range(nsub):
            for c1 in range(self.plan.nb1):
                if (rb + i, c1) not in self.h_ready:
                    self.errors.append(f"task {slot} read h of row block {rb + i}, column block {c1} before it was stored")
        rows = rows_of(self.ids, self.E, self.plan, e, m, nsub, nsub_list=1)

        def g2_end():
            for p in rows:
                if p >= 0:
                    self.y_ready[(int(p), cb)] = self.now
            # the y stores are complete: one arrival per row at (token, column block)
            for p in rows:
                if p >= 0:
                    key = (int(p) // self.k, cb)
                    self.st.arrive[key] = self.st.arrive.get(key, 0) + 1
            self.push(self.now + self.dur(0.2), lambda: self.run_task(b, nxt.get("slot", -1)))

        self.push(self.now + length, g2_end)

    def combine_share(self, b):
        nb2 = self.plan.nb2
        items = list(range(b, self.T * nb2, self.grid))
        polls = {"n": 0}

        def need(i):
            return int(self.nvalid[i // nb2]) - (1 if self.f.arrive_off_by_one else 0)

        def wait():
            if all(self.st.arrive.get((i // nb2, i % nb2), 0) >= need(i) for i in items):
                return body()
            polls["n"] += 1
            if polls["n"] > self.spin_limit:
                self.st.timeouts += 1
                self.errors.append(f"combine of workgroup {b} timed out")
                return body()
            self.push(self.now + self.poll, wait)

        def body():
            for i in items:
                t, cb = divmod(i, nb2)
                for j in range(self.k):
                    if self.valid[t, j] and (t * self.k + j, cb) not in self.y_ready:
                        self.errors.append(f"combine of token {t}, column block {cb} read slot {j} before it was stored")
                self.out_written[(t, cb)] = self.out_written.get((t, cb), 0) + 1
                self.st.arrive[(t, cb)] = 0
            self.push(self.now + self.dur(0.3), lambda: self.finish_wg(b))

        self.push(self.now + self.dur(0.2), wait)

    def finish_wg(self, b):
        old = self.st.exit
        self.st.exit += 1
        if old == self.grid - 1 and not self.f.no_reset:
            self.st.queue = 0
            self.st.exit = 0
            for key in list(self.st.done1):
                self.st.done1[key] = 0
        self.running -= 1
        self.exited += 1
        # a workgroup slot freed: the next workgroup of the grid starts there
        if self.next_wg < self.grid:
            b2 = self.next_wg
            self.next_wg += 1
            self.push(self.now + self.dur(0.3), lambda: self.start_wg(b2))

    # -- run ----------------------------------------------------------------
    def run(self, max_events=5_000_000):
        self.next_wg = min(self.grid, self.resident)
        for b in range(self.next_wg):
            self.push(self.dur(0.5), (lambda bb: (lambda: self.start_wg(bb)))(b))
        n = 0
        while self.events:
            self.now, _, fn = heapq.heappop(self.events)
            fn()
            n += 1
            if n > max_events:
                self.errors.append("no termination within the event budget")
                break
        return self

    def check(self):
        """Every property of one call; returns the list of violations."""
        err = list(self.errors)
        if self.exited != self.grid:
            err.append(f"{self.grid - self.exited} workgroups never finished")
        want = set(range(self.plan.total))
        got = set(self.executed)
        if got != want:
            err.append(f"tasks executed {len(got)} of {len(want)}")
        for t in range(self.T):
            for cb in range(self.plan.nb2):
                c = self.out_written.get((t, cb), 0)
                if c != 1:
                    err.append(f"output of token {t}, column block {cb} written {c} times")
        if self.st.queue or self.st.exit or any(self.st.done1.values()) or any(self.st.arrive.values()):
            err.append("control counters not all zero after the call")
        return err
