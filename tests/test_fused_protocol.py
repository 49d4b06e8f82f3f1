"""The single-launch protocol (task queue, M-tile completion counters,
last-arrival combine, exit reset) checked on its CPU model under random skews:
coverage, dependency order, exactly-once output, counters back at zero, and
termination with fewer resident workgroups than the grid.  Planted protocol
mistakes must be caught.  No GPU is involved."""
import numpy as np
import pytest

from tests.fused_protocol_model import Faults, Sim, State, make_plan, rows_of

pytestmark = pytest.mark.filterwarnings("ignore")


def zipf_ids(rng, T, k, E, s, empty=0, drop=0.0):
    """Distinct experts per token, Zipf(s) over a permutation; `empty` experts
    never chosen; a fraction `drop` of the ids replaced by out-of-range ones."""
    live = rng.permutation(E)[: E - empty]
    w = 1.0 / np.arange(1, len(live) + 1) ** s
    w /= w.sum()
    ids = np.empty((T, k), np.int64)
    for t in range(T):
        ids[t] = rng.choice(live, size=k, replace=False, p=w)
    if drop:
        mask = rng.random((T, k)) < drop
        ids[mask] = rng.choice([-1, E, E + 7], size=int(mask.sum()))
    return ids


CASES = [
    # T, k, E, nb1, nb2, (GEMM-1, GEMM-2 M-tile blocks), grid, resident, zipf s, empty experts, dropped fraction
    (128, 2, 32, 12, 16, (8, 8), 64, 64, 1.1, 0, 0.0),
    (256, 2, 32, 6, 16, (4, 8), 40, 40, 1.2, 4, 0.0),
    (300, 4, 16, 3, 5, (4, 8), 24, 7, 1.0, 2, 0.05),
    (64, 2, 8, 2, 2, (8, 8), 16, 1, 0.8, 0, 0.2),
    (97, 3, 20, 4, 3, (4, 4), 32, 5, 1.5, 3, 0.1),
    (40, 1, 4, 2, 3, (2, 8), 12, 12, 2.0, 1, 0.5),
    (400, 2, 6, 3, 4, (4, 8), 48, 48, 1.0, 0, 0.0),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_protocol_properties_under_random_skew(case, seed):
    T, k, E, nb1, nb2, mtb, grid, resident, s, empty, drop = case
    rng = np.random.default_rng(1000 * seed + T)
    ids = zipf_ids(rng, T, k, E, s, empty, drop)
    st = State()
    # two calls back to back on the same control block: the second starts from
    # the zeros the first left
    for call in range(2):
        sim = Sim(ids, T, k, E, nb1, nb2, mtb, grid, resident, rng, state=st).run()
        assert sim.check() == [], (call, sim.check()[:5])


def test_plan_covers_every_routed_row_once():
    rng = np.random.default_rng(5)
    T, k, E = 200, 3, 24
    ids = zipf_ids(rng, T, k, E, 1.3, 3, 0.05)
    for mtb in ((4, 8), (8, 8)):
        plan = make_plan(ids, E, mtb, 5, 7)
        seen = {}
        for i in range(plan.n1):
            lst, e, row0, nsub, cb, m = plan.decode(i)
            assert lst == 0 and 0 <= cb < 5 and nsub >= 1
            for r, p in enumerate(rows_of(ids, E, plan, e, m, nsub)):
                if p >= 0:
                    assert ids.ravel()[p] == e
                    seen[(int(p), cb)] = seen.get((int(p), cb), 0) + 1
                    # the row's padded position is its rank within the expert
                    assert row0 + r == plan.poff[e] + list(np.nonzero(ids.ravel() == e)[0]).index(p)
        valid = [p for p in range(T * k) if 0 <= ids.ravel()[p] < E]
        assert set(seen) == {(p, cb) for p in valid for cb in range(5)}
        assert all(v == 1 for v in seen.values())
        # both lists go by descending expert row count (ties by id)
        for lo, n in ((0, plan.n1), (plan.n1, plan.n2)):
            keys = [(-plan.counts[plan.decode(lo + i)[1]], plan.decode(lo + i)[1]) for i in range(n)]
            assert keys == sorted(keys)
        # every GEMM-1 M-tile sits in exactly one GEMM-2 M-tile, whose counter
        # target counts all of the GEMM-1 tasks that feed it
        feed = {}
        for i in range(plan.n1):
            _, e, row0, nsub, cb, _ = plan.decode(i)
            feed[plan.g2_tile(e, row0)] = feed.get(plan.g2_tile(e, row0), 0) + 1
        g2 = {}
        for i in range(plan.n2):
            _, e, row0, nsub, cb, _ = plan.decode(plan.n1 + i)
            assert plan.g2_tile(e, row0) == row0 // 16
            g2[row0 // 16] = plan.target(nsub)
        assert feed == g2


@pytest.mark.parametrize("fault", ["g2_first", "short_wait", "flag_before_store", "no_reset", "arrive_off_by_one"])
def test_planted_protocol_mistakes_are_caught(fault):
    rng = np.random.default_rng(11)
    T, k, E = 96, 2, 12
    ids = zipf_ids(rng, T, k, E, 1.1, 1, 0.0)
    caught = False
    # few resident workgroups (a wrong queue order then shows up as a wait that
    # never ends) and a full grid (races between producers and consumers)
    for resident in (3, 16):
        st = State()
        for call in range(4):
            sim = Sim(ids, T, k, E, 3, 4, (4, 8), 16, resident, rng, faults=Faults(**{fault: True}), state=st,
                      spin_limit=2000).run()
            if sim.check():
                caught = True
                break
    assert caught, fault
