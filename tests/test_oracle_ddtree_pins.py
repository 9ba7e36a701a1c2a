"""Pins of the DDTree oracle (SPOT, Sec. 4.2 Eq. 3 and App. C.2 Algorithm 2)
against hand-worked cases, closed forms and brute-force enumeration of every
state of tiny blocks."""

import math

import numpy as np
import pytest

import oracle.ddtree as dd
from oracle.rows import STATUS_EMPTY_ROW, STATUS_NONFINITE


def _log(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, np.float64))


# ---------------------------------------------------------------- hypotheses

def test_greedy_hypotheses_runner_up_below_threshold():
    """T = 0: argmax, plus the runner-up when the top-1 probability < 0.6."""
    h = dd.hypotheses(_log([0.5, 0.3, 0.2]), 0.0)["hyp"]
    assert [v for v, _ in h] == [0, 1]
    assert h[0][1] == pytest.approx(0.5, rel=1e-14) and h[1][1] == pytest.approx(0.3, rel=1e-14)
    h = dd.hypotheses(_log([0.1, 0.7, 0.2]), 0.0)["hyp"]
    assert h == [(1, pytest.approx(0.7, rel=1e-14))]
    # just above and just below 0.6
    assert len(dd.hypotheses(_log([0.6 + 1e-9, 0.25, 0.15 - 1e-9]), 0.0)["hyp"]) == 1
    assert len(dd.hypotheses(_log([0.6 - 1e-9, 0.25, 0.15 + 1e-9]), 0.0)["hyp"]) == 2


def test_greedy_hypotheses_ties_lowest_id():
    x = np.array([1.0, 3.0, 3.0, 0.0])
    h = dd.hypotheses(x, 0.0)["hyp"]
    z = math.e + 2 * math.e ** 3 + 1
    assert [v for v, _ in h] == [1, 2]
    assert h[0][1] == pytest.approx(math.e ** 3 / z, rel=1e-14)
    assert h[1][1] == pytest.approx(math.e ** 3 / z, rel=1e-14)


def test_gumbel_hypothesis():
    """T > 0: argmax of (1/T) log p^ + G (Eq. 4); the mass factor is p^ at
    temperature 1."""
    x = np.array([2.0, 1.0, 0.0, -1.0])
    p = np.exp(x) / np.exp(x).sum()
    h = dd.hypotheses(x, 1.0, np.zeros(4))["hyp"]
    assert h == [(0, pytest.approx(p[0], rel=1e-14))]
    g = np.array([0.0, 0.0, 0.0, 50.0])
    h = dd.hypotheses(x, 0.7, g)["hyp"]
    assert h == [(3, pytest.approx(p[3], rel=1e-14))]
    # a small temperature lets the logits dominate moderate noise
    g = np.array([0.0, 1.5, 0.0, 0.0])
    assert dd.hypotheses(x, 0.05, g)["hyp"][0][0] == 0
    assert dd.hypotheses(x, 1.0, g)["hyp"][0][0] == 1


# ---------------------------------------------------------- order model

def test_order_distribution_restricted_and_tempered():
    z = np.array([1.0, 5.0, 2.0, 0.0])
    q = dd.order_distribution(z, [0, 2], 2.0)
    e0, e2 = math.exp(0.5), math.exp(1.0)
    assert q[1] == 0.0 and q[3] == 0.0
    assert q[0] == pytest.approx(e0 / (e0 + e2), rel=1e-14)
    assert q[2] == pytest.approx(e2 / (e0 + e2), rel=1e-14)
    assert dd.order_distribution(np.array([np.nan, 0.0]), [0, 1], 1.0) is None
    assert dd.order_distribution(np.array([-np.inf, 0.0]), [0], 1.0) is None
    # an unused NaN entry does not matter
    assert dd.order_distribution(np.array([np.nan, 0.0]), [1], 1.0)[1] == 1.0


# ------------------------------------------------------- hand-worked tree

def _two_position_case():
    """Block of 2 masked positions; p^_0(7) = 0.9 (single hypothesis),
    p^_1(3) = 0.5 with runner-up p^_1(4) = 0.3; the root's order q = (0.7,
    0.3); a state with one masked position left has q = 1 there."""
    hyps = [[(7, 0.9)], [(3, 0.5), (4, 0.3)]]
    table = np.zeros((1, 3, 2))
    table[0, 2] = _log([0.7, 0.3])
    return hyps, dd.table_order(table)


def test_hand_worked_tree():
    hyps, order = _two_position_case()
    # candidates: (0,7): 0.63; (1,3): 0.15; (1,4): 0.09;
    # after (0,7): (0,7)(1,3): 0.315, (0,7)(1,4): 0.189;
    # after (1,3): (1,3)(0,7): 0.135; after (1,4): (1,4)(0,7): 0.081
    exp = [(((0, 7),), 0.63), (((0, 7), (1, 3)), 0.315), (((0, 7), (1, 4)), 0.189),
           (((1, 3),), 0.15), (((1, 3), (0, 7)), 0.135), (((1, 4),), 0.09),
           (((1, 4), (0, 7)), 0.081)]
    for D in range(0, 9):
        got, st = dd.best_first([1, 1], hyps, order, D)
        assert st == 0
        assert [p for p, _ in got] == [p for p, _ in exp[:D]]
        assert [m for _, m in got] == pytest.approx([m for _, m in exp[:D]], rel=1e-14)
        lb, st, _ = dd.level_batched([1, 1], hyps, order, D)
        assert lb == got
    # D = 2 takes a depth-2 state over the depth-1 state (1, 3): filling the
    # budget level by level would not
    got, _ = dd.best_first([1, 1], hyps, order, 2)
    assert got[1][0] == ((0, 7), (1, 3))


def test_hand_worked_tree_arrays():
    hyps, order = _two_position_case()
    got, _ = dd.best_first([1, 1], hyps, order, 4)
    t = dd.tree_arrays(got, [1, 1])
    assert t["parent"].tolist() == [-1, 0, 1, 1, 0]
    assert t["pos"].tolist() == [-1, 0, 1, 1, 1]
    assert t["tok"].tolist() == [-1, 7, 3, 4, 3]
    assert t["depth"].tolist() == [0, 1, 2, 2, 1]
    assert t["masked"].tolist() == [[1, 1], [0, 1], [0, 0], [0, 0], [1, 0]]


def test_floor_discards_light_states():
    hyps, order = _two_position_case()
    got, _ = dd.best_first([1, 1], hyps, order, 10, gamma=0.14)
    assert [m for _, m in got] == pytest.approx([0.63, 0.315, 0.189, 0.15], rel=1e-14)
    got, _ = dd.best_first([1, 1], hyps, order, 10, gamma=0.7)
    assert got == []


# ------------------------------------------------------------ closed forms

def test_uniform_order_one_hot_rows():
    """Uniform order logits and one-hot stale rows (p^ = 1): a depth-d state
    has mass (L - d)! / L!; ties resolve to the lexicographically first path."""
    L = 5
    hyps = [[(s + 10, 1.0)] for s in range(L)]
    order = lambda b, path: np.zeros(L)
    got, _ = dd.best_first([1] * L, hyps, order, L + 2)
    assert [p for p, _ in got[:L]] == [((s, s + 10),) for s in range(L)]
    assert [m for _, m in got[:L]] == pytest.approx([1 / L] * L, rel=1e-14)
    assert got[L][0] == ((0, 10), (1, 11)) and got[L + 1][0] == ((0, 10), (2, 12))
    assert got[L][1] == pytest.approx(1 / (L * (L - 1)), rel=1e-14)
    full, _ = dd.best_first([1] * L, hyps, order, 10 ** 6)
    by_depth = {}
    for p, m in full:
        by_depth.setdefault(len(p), set()).add(round(m * math.factorial(L) / math.factorial(L - len(p)), 12))
    assert all(v == {1.0} for v in by_depth.values())
    # number of states: sum over d of L! / (L - d)!
    assert len(full) == sum(math.factorial(L) // math.factorial(L - d) for d in range(1, L + 1))


def test_budget_zero_and_no_masked_position():
    hyps, order = _two_position_case()
    assert dd.best_first([1, 1], hyps, order, 0) == ([], 0)
    assert dd.level_batched([1, 1], hyps, order, 0)[0] == []
    assert dd.best_first([0, 0], hyps, order, 5) == ([], 0)
    assert dd.level_batched([0, 0], hyps, order, 5)[0] == []


# ------------------------------------------------------------ brute force

def _brute(masked, hyps, order_fn, D, tau, gamma):
    """Every state of the block with its mass from Eq. 3, written out from
    the definition; the D best by mass, then depth, then path."""
    L = len(masked)
    root = [s for s in range(L) if masked[s]]
    states = []

    def q_of(path, s):
        left = [t for t in root if t not in {e[0] for e in path}]
        z = np.asarray(order_fn(0, tuple(path)), np.float64) / tau
        w = {t: math.exp(z[t] - max(z[u] for u in left)) for t in left}
        return w[s] / sum(w.values())

    def walk(path, mass):
        left = [t for t in root if t not in {e[0] for e in path}]
        for s in left:
            for v, pv in hyps[s]:
                m = mass * q_of(path, s) * pv
                if m >= gamma:
                    p = path + ((s, v),)
                    states.append((p, m))
                    walk(p, m)
    walk((), 1.0)
    states.sort(key=lambda e: (-e[1], len(e[0]), e[0]))
    return states[:D]


def _random_case(rng, L, V):
    masked = (rng.random(L) < 0.8).astype(int)
    stale = rng.normal(0, 1.5, (L, V))
    hyps = []
    for s in range(L):
        hyps.append(dd.hypotheses(stale[s], 0.0)["hyp"] if masked[s] else [])
    cache = {}
    base = rng.normal(0, 1, L + 1)

    def order(b, path):
        if path not in cache:
            cache[path] = base[:L] + rng.normal(0, 1.0, L)
        return cache[path]
    return masked, hyps, order


@pytest.mark.parametrize("seed", range(12))
def test_best_first_is_the_top_d_of_all_states(seed):
    rng = np.random.default_rng(seed)
    L = 4
    masked, hyps, order = _random_case(rng, L, 6)
    for D, tau, gamma in ((1, 1.0, 0.0), (5, 1.0, 0.0), (12, 0.7, 0.0), (40, 1.3, 0.0),
                          (10, 1.0, 0.02), (1000, 1.0, 0.0)):
        want = _brute(masked, hyps, order, D, tau, gamma)
        got, st = dd.best_first(masked, hyps, order, D, tau, gamma)
        assert st == 0
        assert [p for p, _ in got] == [p for p, _ in want]
        np.testing.assert_allclose([m for _, m in got], [m for _, m in want], rtol=1e-12)


@pytest.mark.parametrize("seed", range(12))
def test_level_batched_reaches_the_best_first_set(seed):
    rng = np.random.default_rng(100 + seed)
    L = 6
    masked, hyps, order = _random_case(rng, L, 8)
    for D, gamma in ((1, 0.0), (3, 0.0), (8, 0.0), (20, 0.0), (20, 0.005), (64, 0.0)):
        want, _ = dd.best_first(masked, hyps, order, D, 1.0, gamma)
        got, _, levels = dd.level_batched(masked, hyps, order, D, 1.0, gamma)
        assert got == want
        depth = max((len(p) for p, _ in got), default=0)
        assert levels <= depth + 1


@pytest.mark.parametrize("seed", range(6))
def test_tree_invariants(seed):
    rng = np.random.default_rng(200 + seed)
    L = 7
    masked, hyps, order = _random_case(rng, L, 5)
    got, _ = dd.best_first(masked, hyps, order, 25)
    t = dd.tree_arrays(got, masked)
    n = len(got) + 1
    for z in range(1, n):
        y = t["parent"][z]
        assert 0 <= y < z
        assert t["mass"][z] <= t["mass"][y]
        assert t["depth"][z] == t["depth"][y] + 1
        assert t["masked"][y][t["pos"][z]] == 1 and t["masked"][z][t["pos"][z]] == 0
        assert t["masked"][z].sum() == t["masked"][y].sum() - 1
    assert all(t["mass"][z] >= t["mass"][z + 1] for z in range(1, n - 1))


# ------------------------------------------------------------------ status

def test_status_of_bad_rows():
    rng = np.random.default_rng(3)
    L, V = 3, 5
    stale = rng.normal(0, 1, (2, L, V))
    stale[0, 1, 2] = np.nan
    stale[1, 2, :] = 0.0  # unmasked below: never read
    masked = np.array([[1, 1, 1], [1, 1, 0]])
    stale[1, 2, 0] = np.nan
    out = dd.build_ddtree(stale, masked, lambda b, p: np.zeros(L), 4, 0.0)
    assert out["status"][0] == STATUS_NONFINITE and out["trees"][0] is None
    assert out["status"][1] == 0 and out["trees"][1] is not None
    bad = lambda b, p: np.array([-np.inf, -np.inf, 0.0])
    out = dd.build_ddtree(stale[1:], masked[1:], bad, 4, 0.0)
    assert out["status"][0] == STATUS_EMPTY_ROW


def test_build_matches_best_first_per_sequence():
    rng = np.random.default_rng(9)
    B, L, V = 3, 5, 11
    stale = rng.normal(0, 2.0, (B, L, V))
    masked = (rng.random((B, L)) < 0.8).astype(np.uint8)
    table = rng.normal(0, 1, (B, L + 1, L))
    order = dd.table_order(table)
    g = -np.log(-np.log(rng.random((B, L, V))))
    for T in (0.0, 0.8):
        out = dd.build_ddtree(stale, masked, order, 7, T, tau=1.2, gumbel=g)
        for b in range(B):
            hyps = [dd.hypotheses(stale[b, s], T, g[b, s])["hyp"] if masked[b, s] else [] for s in range(L)]
            want, _ = dd.best_first(masked[b], hyps, order, 7, 1.2, 0.0, b)
            assert out["chosen"][b] == want
            for s in range(L):
                for k, (v, pv) in enumerate(hyps[s]):
                    assert out["hyp_tok"][b, s, k] == v and out["hyp_prob"][b, s, k] == pv


def test_table_order_rows():
    table = np.arange(2 * 4 * 3, dtype=np.float64).reshape(2, 4, 3)
    f = dd.table_order(table)
    assert f(1, ()).tolist() == table[1, 3].tolist()
    assert f(0, ((2, 5), (0, 1))).tolist() == table[0, 0].tolist()
