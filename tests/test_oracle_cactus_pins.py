"""Pins of the modified Cactus oracle ("Speculative Diffusion is a Tale of Two
Tradeoffs", App. E) against what the page and the mathematics fix.

The page defines the modified target by a constraint on whole distributions
-- the largest p~(y) with KL(p~ || p) <= delta, the other tokens rescaled --
and prints the second-order (Taylor) solution of Eq. 18.  The checks below
use those definitions directly (the KL of the two full vectors, the printed
closed form as the small-budget limit, the lossless rule at delta = 0) and
the laws any speculative sampler obeys, never the oracle's own Eq. 17 code.
"""

import math

import numpy as np
import pytest
from scipy import special, stats

import oracle


def _dist(rng, V, scale):
    x = rng.normal(0, scale, V)
    return x, oracle.tempered_softmax(x, 1.0)


def _kl(a, b):
    return float(np.sum(special.rel_entr(a, b)))


# ------------------------------------------------ the modified target (Eq. 17)

@pytest.mark.parametrize("delta", [0.01, 0.25, 1.0, 4.0])
def test_modified_target_meets_kl_budget_exactly(delta):
    # App. E: p~ maximises p~(y) subject to KL(p~ || p) <= delta, with the
    # other tokens rescaled by (1 - p~(y)) / (1 - p(y)).  The KL is computed
    # here from the two full distributions.
    rng = np.random.default_rng(31)
    hit = saturated = 0
    for trial in range(200):
        V = int(rng.integers(2, 60))
        _, p = _dist(rng, V, float(rng.choice([0.5, 2.0, 4.0])))
        y = int(rng.integers(0, V))
        g = oracle.cactus_gamma(p[y], delta)
        pt = oracle.cactus_target(p, y, g)
        assert pt.min() >= 0.0 and pt[y] == g
        assert math.fsum(pt) == pytest.approx(1.0, abs=1e-12)
        # the untouched tokens keep their ratios to one another
        others = np.arange(V) != y
        if g < 1.0 and others.any():
            np.testing.assert_allclose(pt[others] / pt[others].sum(), p[others] / p[others].sum(), rtol=1e-10)
        kl = _kl(pt, p)
        if g < 1.0:
            hit += 1
            assert kl == pytest.approx(delta, rel=1e-9, abs=1e-12), (trial, p[y], g, kl)
            # maximal: any larger mass on y breaks the budget
            g2 = g + 1e-6 * (1.0 - g)
            assert _kl(oracle.cactus_target(p, y, g2), p) > delta
            assert g >= p[y]
        else:
            saturated += 1
            assert kl <= delta + 1e-12
            assert -math.log(p[y]) <= delta + 1e-12
    assert hit > 50
    if delta >= 1.0:
        assert saturated > 0


def test_small_budget_matches_printed_taylor_solution():
    # Eq. 18's solution gamma = min{p + sqrt(2 delta p (1 - p)), 1} is the
    # second-order expansion of the exact root: the relative difference of
    # gamma - p from sqrt(2 delta p (1-p)) shrinks like sqrt(delta).
    for p in (1e-3, 0.05, 0.3, 0.6, 0.95):
        prev = None
        for delta in (1e-4, 1e-6, 1e-8):
            g = oracle.cactus_gamma(p, delta)
            taylor = math.sqrt(2 * delta * p * (1 - p))
            rel = abs((g - p) / taylor - 1.0)
            assert rel < 5.0 * math.sqrt(delta / p), (p, delta, rel)
            if prev is not None:
                assert rel < prev
            prev = rel
    # ... and the page's point: for a small p(y) and a large budget the exact
    # root is far above the Taylor value.
    assert oracle.cactus_gamma(1e-6, 5.0) > 100 * (1e-6 + math.sqrt(2 * 5.0 * 1e-6))


def test_budget_edge_cases():
    assert oracle.cactus_gamma(0.3, 0.0) == 0.3
    assert oracle.cactus_gamma(0.0, 3.0) == 0.0
    assert oracle.cactus_gamma(1.0, 0.5) == 1.0
    assert oracle.cactus_gamma(0.5, math.log(2.0)) == 1.0
    assert oracle.cactus_gamma(0.5, math.log(2.0) * (1 - 1e-9)) < 1.0
    with pytest.raises(ValueError):
        oracle.cactus_gamma(0.5, -1.0)


def test_gamma_monotone_in_budget_and_probability():
    ps = [1e-7, 1e-3, 0.1, 0.4, 0.8, 0.999]
    ds = [0.0, 1e-3, 0.1, 0.5, 2.0, 8.0]
    G = np.array([[oracle.cactus_gamma(p, d) for d in ds] for p in ps])
    assert (np.diff(G, axis=1) >= 0).all()
    assert (np.diff(G, axis=0) >= 0).all()
    assert (G >= np.array(ps)[:, None]).all()


# ---------------------------------------------------- the sampler it drives

def _chain_case(rng, B=6, K=5, V=40, sigma=1.0):
    x = rng.normal(0, 3, (B, K + 1, V))
    y = x[:, :K] + rng.normal(0, sigma, (B, K, V))
    d = np.zeros((B, K), np.int64)
    for b in range(B):
        for i in range(K):
            q = oracle.tempered_softmax(y[b, i], 1.0)
            d[b, i] = rng.choice(V, p=q)
    n = rng.integers(0, K + 1, B)
    return x, y, d, n


def test_zero_budget_is_lossless_bit_for_bit():
    rng = np.random.default_rng(32)
    x, y, d, n = _chain_case(rng)
    ua, ur = rng.random((6, 5)), rng.random((6, 6))
    a = oracle.verify_rejection(x, y, d, n, 0.8, 1.1, ua, ur)
    b = oracle.verify_cactus(x, y, d, n, 0.8, 1.1, 0.0, ua, ur)
    for k in ("accept_len", "num_out", "out_tokens", "status", "alpha", "residual_mass"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_larger_budget_never_shortens_the_accepted_prefix():
    # alpha = min{1, gamma/q} grows with delta, so under common random numbers
    # the number of leading accepts cannot fall.
    rng = np.random.default_rng(33)
    x, y, d, n = _chain_case(rng, B=40, K=8, sigma=2.0)
    ua, ur = rng.random((40, 8)), rng.random((40, 9))
    prev = None
    for delta in (0.0, 0.1, 0.5, 2.0, 8.0):
        h = oracle.verify_cactus(x, y, d, n, 1.0, 1.0, delta, ua, ur)["accept_len"]
        if prev is not None:
            assert (h >= prev).all()
        prev = h


def test_huge_budget_accepts_every_draft():
    rng = np.random.default_rng(34)
    x, y, d, n = _chain_case(rng, B=10, K=6, sigma=3.0)
    res = oracle.verify_cactus(x, y, d, n, 1.0, 1.0, 200.0, rng.random((10, 6)), rng.random((10, 7)))
    np.testing.assert_array_equal(res["accept_len"], n)
    assert (res["alpha"][np.arange(6)[None, :] < n[:, None]] == 1.0).all()


def _chi2_ok(counts, probs, pmin=1e-4):
    exp = probs * counts.sum()
    keep = exp >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] == 0:
        if obs[-1] > 0:        # draws where the law has no mass
            return False
        obs, ex = obs[:-1], ex[:-1]
    return stats.chisquare(obs, ex).pvalue > pmin


@pytest.mark.parametrize("delta", [0.05, 0.3])
def test_emitted_law_and_acceptance_rate(delta):
    # For a drafted token y ~ q the first emitted token has law
    #   sum_y q(y) [alpha(y) 1{x = y} + (1 - alpha(y)) r_y(x) / |r_y|],
    # alpha(y) = min{1, p~_y(y) / q(y)}, r_y = [p~_y - q]_+ -- the law of any
    # speculative sampler whose target for draft y is p~_y.  The whole
    # verifier, run over many seeds, must produce it, and accept draft 1 at
    # the rate sum_y q(y) alpha(y).
    rng = np.random.default_rng(35 + int(10 * delta))
    V, N = 7, 30000
    x = rng.normal(0, 1.5, (2, V))
    yl = rng.normal(0, 1.5, (1, V))
    p = oracle.tempered_softmax(x[0], 1.0)
    q = oracle.tempered_softmax(yl[0], 1.0)
    law = np.zeros(V)
    rej_law = np.zeros(V)      # the law of the corrected token, given a rejection
    rate = 0.0
    for y in range(V):
        pt = oracle.cactus_target(p, y, oracle.cactus_gamma(p[y], delta))
        alpha = min(1.0, pt[y] / q[y])
        r = np.maximum(pt - q, 0.0)
        law[y] += q[y] * alpha
        if alpha < 1.0:
            law += q[y] * (1.0 - alpha) * r / r.sum()
            rej_law += q[y] * (1.0 - alpha) * r / r.sum()
        rate += q[y] * alpha
    assert math.fsum(law) == pytest.approx(1.0, abs=1e-12)
    assert rate < 0.97      # a case where rejections (and the residual) matter
    d = rng.choice(V, size=N, p=q)[:, None]
    res = oracle.verify_cactus(np.broadcast_to(x, (N, 2, V)), np.broadcast_to(yl, (N, 1, V)), d, None,
                               1.0, 1.0, delta, rng.random((N, 1)), rng.random((N, 2)))
    counts = np.bincount(res["out_tokens"][:, 0], minlength=V)
    rejected = res["accept_len"] == 0
    rcounts = np.bincount(res["out_tokens"][rejected, 0], minlength=V)
    # tokens outside the support of the law are never emitted
    assert counts[law == 0].sum() == 0 and rcounts[rej_law == 0].sum() == 0
    assert _chi2_ok(counts, law)
    assert _chi2_ok(rcounts, rej_law / rej_law.sum())
    se = math.sqrt(rate * (1 - rate) / N)
    assert abs((res["accept_len"] == 1).mean() - rate) < 4 * se
    # the budget makes the rule lenient: more acceptance than lossless
    assert rate > 1.0 - 0.5 * float(np.abs(p - q).sum())
