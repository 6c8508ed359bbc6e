"""Owner-assignment planner (muon_owner_plan, host-only C entry point) against brute force
and closed forms, with injected cost tables (no GPU).

DMuon summary (gist.science), section 2.3: owners are chosen to minimise the predicted
makespan from measured per-shape costs of several batch sizes, exactly (a MILP) with a
greedy fallback. The exact search must reach the least makespan over every assignment of
matrices to ranks; the checks below enumerate all R^N assignments on small lists and
recompute every load from the cost model written out here on its own.
"""

import itertools

import numpy as np
import pytest

B = pytest.importorskip("matrix_orthogonalising_optimizer_muon_amd.binding")


def cost_of(points, k):
    """c(k) of the documented model: 0 at k = 0, linear from the origin to the first
    point and between points, past the last point the last segment's slope."""
    if k == 0:
        return 0.0
    bs = [b for b, _ in points]
    ts = [t for _, t in points]
    if k <= bs[0]:
        return ts[0] * k / bs[0]
    for i in range(1, len(bs)):
        if k <= bs[i]:
            return ts[i - 1] + (ts[i] - ts[i - 1]) * (k - bs[i - 1]) / (bs[i] - bs[i - 1])
    slope = (ts[-1] - ts[-2]) / (bs[-1] - bs[-2]) if len(bs) > 1 else ts[0] / bs[0]
    return ts[-1] + slope * (k - bs[-1])


def loads_of(owner, shape_of, costs, ranks):
    counts = np.zeros((len(costs), ranks), dtype=int)
    for o, s in zip(owner, shape_of):
        counts[s, o] += 1
    return [sum(cost_of(costs[s], counts[s, r]) for s in range(len(costs))) for r in range(ranks)]


def brute_force(shape_of, costs, ranks):
    best = float("inf")
    for owner in itertools.product(range(ranks), repeat=len(shape_of)):
        best = min(best, max(loads_of(owner, shape_of, costs, ranks)))
    return best


def random_costs(rng, n_shapes, batching):
    costs = []
    for _ in range(n_shapes):
        t1 = float(rng.uniform(0.5, 20.0))
        if batching:   # sub-linear: batching amortises fixed costs
            costs.append([(1, t1), (2, t1 * rng.uniform(1.2, 2.0)), (4, t1 * rng.uniform(2.4, 4.0))])
        else:
            costs.append([(1, t1)])
    return costs


@pytest.mark.parametrize("seed", range(12))
def test_exact_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    ranks = int(rng.integers(2, 4))
    n = int(rng.integers(3, 8 if ranks == 2 else 7))
    n_shapes = int(rng.integers(1, 4))
    costs = random_costs(rng, n_shapes, batching=bool(seed % 2))
    shape_of = [int(rng.integers(0, n_shapes)) for _ in range(n)]
    r = B.muon_owner_plan(shape_of, costs, ranks)
    assert r["optimal"]
    assert sorted(set(r["owner"])) <= list(range(ranks)) and len(r["owner"]) == n
    loads = loads_of(r["owner"], shape_of, costs, ranks)
    assert np.allclose(loads, r["rank_ms"], rtol=1e-12, atol=1e-12)
    assert abs(max(loads) - r["makespan_ms"]) <= 1e-12 * max(1.0, r["makespan_ms"])
    assert r["makespan_ms"] <= brute_force(shape_of, costs, ranks) * (1 + 1e-12)
    assert r["makespan_ms"] >= brute_force(shape_of, costs, ranks) * (1 - 1e-12)
    # greedy alone is a valid plan, never better than the optimum
    g = B.muon_owner_plan(shape_of, costs, ranks, greedy=True)
    assert not g["optimal"] and g["makespan_ms"] >= r["makespan_ms"] * (1 - 1e-12)
    assert np.allclose(loads_of(g["owner"], shape_of, costs, ranks), g["rank_ms"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_greedy_within_lpt_bound_for_linear_costs(seed):
    """With costs linear in the batch size the problem is makespan scheduling on identical
    machines; the greedy's first phase is longest-processing-time first, within
    (4/3 - 1/(3R)) of the optimum (Graham's bound)."""
    rng = np.random.default_rng(100 + seed)
    ranks = 3
    n_shapes = 4
    costs = random_costs(rng, n_shapes, batching=False)
    shape_of = [int(rng.integers(0, n_shapes)) for _ in range(7)]
    opt = brute_force(shape_of, costs, ranks)
    g = B.muon_owner_plan(shape_of, costs, ranks, greedy=True)
    assert g["makespan_ms"] <= (4.0 / 3.0 - 1.0 / (3 * ranks)) * opt * (1 + 1e-12)


def test_closed_forms():
    # one rank: everything of a shape in one batch
    costs = [[(1, 3.0), (4, 6.0)], [(2, 5.0)]]
    shape_of = [0, 0, 1, 0, 1, 1]
    r = B.muon_owner_plan(shape_of, costs, 1)
    assert r["optimal"] and r["owner"] == [0] * 6
    assert r["makespan_ms"] == pytest.approx(cost_of(costs[0], 3) + cost_of(costs[1], 3), rel=1e-12)
    # identical matrices, linear cost: ceil(N / R) of them on the busiest rank
    r = B.muon_owner_plan([0] * 10, [[(1, 2.5)]], 4)
    assert r["optimal"] and r["makespan_ms"] == pytest.approx(3 * 2.5, rel=1e-12)
    assert max(np.bincount(r["owner"], minlength=4)) == 3
    # more ranks than matrices, linear costs: the largest single matrix
    r = B.muon_owner_plan([0, 1, 2], [[(1, 1.0)], [(1, 7.0)], [(1, 4.0)]], 8)
    assert r["optimal"] and r["makespan_ms"] == pytest.approx(7.0, rel=1e-12)
    # strong batching (a batch of 4 costs what 1 does): keeping them together wins
    r = B.muon_owner_plan([0] * 4, [[(1, 5.0), (4, 5.0)]], 2)
    assert r["optimal"] and r["makespan_ms"] == pytest.approx(5.0, rel=1e-12)
    # no matrices
    r = B.muon_owner_plan([], [[(1, 1.0)]], 3)
    assert r["makespan_ms"] == 0.0 and r["optimal"]


def test_shapes_spread_over_the_list():
    """Matrices of one shape go to their ranks interleaved in list order (layer after layer),
    not in blocks."""
    r = B.muon_owner_plan([0] * 8, [[(1, 1.0)]], 2)
    assert r["owner"] == [0, 1, 0, 1, 0, 1, 0, 1]


def test_node_limit_falls_back():
    """A search stopped by its node limit returns a valid plan no worse than the greedy one,
    marked not proven optimal."""
    rng = np.random.default_rng(7)
    costs = random_costs(rng, 3, batching=True)
    shape_of = [int(rng.integers(0, 3)) for _ in range(60)]
    g = B.muon_owner_plan(shape_of, costs, 6, greedy=True)
    r = B.muon_owner_plan(shape_of, costs, 6, max_nodes=50)
    assert not r["optimal"]
    assert r["makespan_ms"] <= g["makespan_ms"] * (1 + 1e-12)
    assert np.allclose(loads_of(r["owner"], shape_of, costs, 6), r["rank_ms"], rtol=1e-12, atol=1e-9)


def test_beats_round_robin_on_the_7b_shape_set():
    """The 196-matrix 7B list (per layer: Q, K, V, O, gate, up, down) with costs in the ratio
    of the long-side products: round-robin by list position leaves the ranks that draw the
    18944-wide matrices as stragglers; the plan does better."""
    kinds = [0, 1, 1, 0, 2, 2, 2]       # 3584^2, 512x3584, 3584x18944
    shape_of = kinds * 28
    costs = [[(1, 2.0), (8, 14.0), (56, 95.0)], [(1, 0.15), (8, 0.5), (56, 3.0)],
             [(1, 6.0), (8, 45.0), (84, 460.0)]]
    for ranks in (2, 4, 8):
        r = B.muon_owner_plan(shape_of, costs, ranks)
        rr = [i % ranks for i in range(len(shape_of))]
        rr_mk = max(loads_of(rr, shape_of, costs, ranks))
        assert r["makespan_ms"] < rr_mk
        total_best = sum(cost_of(c, n) for c, n in zip(costs, [56, 56, 84]))
        assert r["makespan_ms"] >= total_best / ranks * (1 - 1e-12)


@pytest.mark.parametrize("bad", [
    dict(shape_of=[0, 3], costs=[[(1, 1.0)]], ranks=2),            # shape id out of range
    dict(shape_of=[0], costs=[[(1, 1.0)]], ranks=0),               # no rank
    dict(shape_of=[0], costs=[[(2, 1.0), (2, 3.0)]], ranks=2),     # batch sizes not increasing
    dict(shape_of=[0], costs=[[(0, 1.0)]], ranks=2),               # batch size 0
    dict(shape_of=[0], costs=[[(1, float("nan"))]], ranks=2),      # time not finite
    dict(shape_of=[0], costs=[[(1, -1.0)]], ranks=2),              # negative time
    dict(shape_of=[0], costs=[[]], ranks=2),                       # no point
    dict(shape_of=[0], costs=[[(1, 1.0)]], ranks=B.MUON_MAX_PLAN_RANKS + 1),
])
def test_validation(bad):
    with pytest.raises(B.MuonError):
        B.muon_owner_plan(bad["shape_of"], bad["costs"], bad["ranks"])
