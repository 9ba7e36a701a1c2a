"""Pins of the top-k / top-p truncation oracle (Packed-SS Sec. 3.2, the
stored nonzero entries of a truncated drafter distribution).

Checked against what the definitions fix, not against a re-sort: the full
truncation (k = V, p = 1) is the tempered softmax itself; every kept token
outranks every dropped one (ties to the lower id); the kept prefix is the
shortest whose mass reaches p; ratios between kept tokens are those of the
untruncated law; a worked example by hand.
"""

import math

import numpy as np
import pytest

import oracle


def test_no_truncation_is_the_softmax():
    rng = np.random.default_rng(81)
    for _ in range(20):
        V = int(rng.integers(1, 40))
        x = rng.normal(0, 2, V)
        T = float(rng.choice([0.5, 1.0, 1.7]))
        idx, prob = oracle.truncate_row(x, T, V, 1.0)
        q = oracle.tempered_softmax(x, T)
        assert sorted(idx.tolist()) == list(range(V))
        np.testing.assert_allclose(prob, q[idx], rtol=1e-13)
        assert (np.diff(prob) <= 0).all()


@pytest.mark.parametrize("seed", [82, 83])
def test_kept_set_order_minimality_and_ratios(seed):
    rng = np.random.default_rng(seed)
    for trial in range(200):
        V = int(rng.integers(2, 30))
        x = rng.integers(-3, 4, V).astype(float)        # ties on purpose
        T = float(rng.choice([0.6, 1.0, 2.0]))
        k = int(rng.integers(1, V + 1))
        p = float(rng.choice([1.0, 0.9, 0.5, 0.2]))
        idx, prob = oracle.truncate_row(x, T, k, p)
        kept = set(idx.tolist())
        dropped = [v for v in range(V) if v not in kept]
        # every kept token outranks every dropped one (value, then lower id)
        for v in kept:
            for w in dropped:
                assert x[v] > x[w] or (x[v] == x[w] and v < w)
        # stored order: value descending, then id ascending
        for a, b in zip(idx[:-1], idx[1:]):
            assert x[a] > x[b] or (x[a] == x[b] and a < b)
        # top-p minimality over the renormalised top-k law
        topk = sorted(range(V), key=lambda v: (-x[v], v))[:k]
        w = np.exp((x[topk] - x[topk].max()) / T)
        w /= w.sum()
        m = len(idx)
        assert m <= k and math.fsum(w[:m]) >= p - 1e-12
        if m > 1:
            assert math.fsum(w[:m - 1]) < p
        # ratios of the untruncated law, and a distribution
        assert math.fsum(prob) == pytest.approx(1.0, abs=1e-12)
        for a in range(m):
            assert prob[a] / prob[0] == pytest.approx(math.exp((x[idx[a]] - x[idx[0]]) / T), rel=1e-12)


def test_worked_example_by_hand():
    # q = (0.5, 0.2, 0.2, 0.1); top-3 keeps ids 0, 1, 2 (1 before 2 on the
    # tie) with masses (5, 2, 2)/9; p = 0.6 needs two of them: 5/9 < 0.6 <=
    # 7/9.  Renormalised: (5/7, 2/7).
    x = np.log([0.5, 0.2, 0.2, 0.1])
    idx, prob = oracle.truncate_row(x, 1.0, 3, 0.6)
    assert idx.tolist() == [0, 1]
    np.testing.assert_allclose(prob, [5 / 7, 2 / 7], rtol=1e-12)
    idx, prob = oracle.truncate_row(x, 1.0, 3, 1.0)
    assert idx.tolist() == [0, 1, 2]
    np.testing.assert_allclose(prob, [5 / 9, 2 / 9, 2 / 9], rtol=1e-12)
    idx, prob = oracle.truncate_row(x, 1.0, 1, 1.0)
    assert idx.tolist() == [0] and prob.tolist() == [1.0]


def test_rows_layout_and_bad_rows():
    rng = np.random.default_rng(84)
    rows = rng.normal(0, 1, (2, 3, 10))
    rows[1, 0, 4] = np.nan
    qi, qp, qn = oracle.truncate_rows(rows, 1.0, 4, 1.0, 6, lengths=[3, 2])
    assert qn.tolist() == [[4, 4, 4], [-1, 4, 0]]
    assert (qi[0, :, 4:] == 0).all() and (qp[0, :, 4:] == 0).all()
    with pytest.raises(ValueError):
        oracle.truncate_rows(rows, 1.0, 7, 1.0, 6)
