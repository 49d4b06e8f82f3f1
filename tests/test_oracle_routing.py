"""Pins of the oracle's routing metadata (group sizes, offsets, padded offsets,
stable scatter, block map; tilelang.dataflow README section 3.5 step 1) against
brute force on tiny inputs and against the invariants the layout must keep."""
import numpy as np
import pytest


def brute_route(ids, E, bm):
    """Direct O(N^2) definitions, independent of the oracle's counting sort."""
    n = len(ids)
    valid = [0 <= v < E for v in ids]
    counts = [sum(1 for q in range(n) if valid[q] and ids[q] == e) for e in range(E)]
    offsets = [sum(counts[:e]) for e in range(E + 1)]
    tiles = [-(-c // bm) for c in counts]
    padded = [bm * sum(tiles[:e]) for e in range(E + 1)]
    pos, ppos = [], []
    for p in range(n):
        if not valid[p]:
            pos.append(-1)
            ppos.append(-1)
            continue
        rank = sum(1 for q in range(p) if valid[q] and ids[q] == ids[p])
        pos.append(offsets[ids[p]] + rank)
        ppos.append(padded[ids[p]] + rank)
    return counts, offsets, padded, pos, ppos, n - sum(valid), sum(tiles)


def _cases():
    rng = np.random.default_rng(2024)
    cases = []
    for _ in range(60):
        T = int(rng.integers(0, 40))
        k = int(rng.integers(1, 9))
        E = int(rng.integers(1, 41))
        bm = int(rng.choice([1, 2, 3, 16, 64]))
        ids = rng.integers(-3, E + 3, size=T * k)  # includes invalid ids on both sides
        if rng.random() < 0.3:
            ids = rng.integers(0, min(E, 3), size=T * k)  # heavy skew onto few experts
        cases.append((ids.astype(np.int32), E, bm))
    cases.append((np.zeros(0, np.int32), 4, 16))  # empty input
    cases.append((np.full(37, 2, np.int32), 5, 16))  # everything on one expert
    cases.append((np.full(10, 99, np.int32), 5, 16))  # everything dropped
    return cases


@pytest.mark.parametrize("case", range(63))
def test_route_matches_brute_force(oracle, case):
    ids, E, bm = _cases()[case]
    r = oracle.route(ids, E, bm)
    counts, offsets, padded, pos, ppos, dropped, ntiles = brute_route(ids.tolist(), E, bm)
    assert r["counts"].tolist() == counts
    assert r["offsets"].tolist() == offsets
    assert r["padded_offsets"].tolist() == padded
    assert r["pos"].tolist() == pos
    assert r["ppos"].tolist() == ppos
    assert r["dropped"] == dropped
    assert r["ntiles"] == ntiles


@pytest.mark.parametrize("case", range(63))
def test_route_invariants(oracle, case):
    ids, E, bm = _cases()[case]
    n = ids.size
    r = oracle.route(ids, E, bm)
    valid = (ids >= 0) & (ids < E)
    nv = int(valid.sum())
    # counts sum to tokens * top_k minus the dropped ids
    assert int(r["counts"].sum()) + r["dropped"] == n
    assert r["offsets"][E] == nv
    # pos is a bijection of the valid assignments onto [0, nv)
    pv = r["pos"][valid]
    assert sorted(pv.tolist()) == list(range(nv))
    assert np.all(r["pos"][~valid] == -1)
    # sorted_p inverts pos; assignments ascend inside each expert (stability)
    sp = r["sorted_p"]
    assert np.all(sp[nv:] == -1)
    for p in np.nonzero(valid)[0]:
        assert sp[r["pos"][p]] == p
    for e in range(E):
        seg = sp[r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(ids[seg] == e)
    # padded layout: multiples of bm, no block for an empty expert, row_src inverts ppos
    po = r["padded_offsets"]
    assert np.all(po % bm == 0)
    rs = r["row_src"]
    for e in range(E):
        c = r["counts"][e]
        assert po[e + 1] - po[e] == -(-c // bm) * bm
        assert np.all(rs[po[e]:po[e] + c] == sp[r["offsets"][e]:r["offsets"][e + 1]])
        assert np.all(rs[po[e] + c:po[e + 1]] == -1)
    assert np.all(rs[po[E]:] == -1)
    # block map: expert-ascending, one entry per bm-row block
    nt = r["ntiles"]
    te, t0 = r["tile_expert"], r["tile_row0"]
    assert nt == po[E] // bm
    assert np.all(te[nt:] == -1)
    assert np.all(t0[:nt] == np.arange(nt) * bm)
    for i in range(nt):
        assert po[te[i]] <= t0[i] < po[te[i] + 1]


def test_permutation_round_trip(oracle):
    """Gathering x rows through pos and scattering them back returns x bitwise."""
    rng = np.random.default_rng(1)
    T, k, E = 50, 3, 7
    x = rng.standard_normal((T, 16)).astype(np.float32)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    r = oracle.route(ids.ravel(), E, 16)
    n = T * k
    x_perm = np.empty((n, 16), np.float32)
    x_perm[r["pos"]] = x[np.arange(n) // k]
    # every permuted row is the token row of its assignment
    for q in range(n):
        assert np.array_equal(x_perm[q], x[r["sorted_p"][q] // k])
    back = x_perm[r["pos"]].reshape(T, k, 16)
    for j in range(k):
        assert np.array_equal(back[:, j], x)


def test_route_on_config_routings(oracle):
    """Counts on the synthetic workloads sum to tokens x top_k; the skew recipes hold."""
    from skew_aware_grouped_amd import workloads as W
    for name in ("tiny", "qwen_bf16", "qwen_fp8"):
        c = dict(W.CONFIGS[name])
        ids = W.make_routing(c["index"], c["T"], c["E"], c["k"], c["routing"])
        r = oracle.route(ids.ravel(), c["E"], 16)
        assert int(r["counts"].sum()) == c["T"] * c["k"]
    c = dict(W.CONFIGS["ds_fp8_1024"])
    ids = W.make_routing(c["index"], c["T"], c["E"], c["k"], c["routing"])
    r = oracle.route(ids.ravel(), c["E"], 16)
    cnt = np.sort(r["counts"])[::-1]
    assert cnt[0] == round(0.4 * 2048) and (cnt == 0).sum() == 3
    c = dict(W.CONFIGS["ds_fp8_8192"])
    ids = W.make_routing(c["index"], c["T"], c["E"], c["k"], c["routing"])
    r = oracle.route(ids.ravel(), c["E"], 16)
    cnt = np.sort(r["counts"])[::-1]
    assert cnt[0] == cnt[1] == 4915 and (cnt == 0).sum() == 16
    assert all(len(set(row)) == 2 for row in ids.tolist())
