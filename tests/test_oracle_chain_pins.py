"""Pins of the chain oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formula: each checks a closed form,
an identity proved on the pages, a printed value, brute force, or a Monte
Carlo law, chosen so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_dist(rng, V, scale=2.0):
    x = rng.normal(0, scale, V)
    return x, oracle.tempered_softmax(x, 1.0)


def _tv(p, q):
    return 0.5 * float(np.sum(np.abs(np.asarray(p) - np.asarray(q))))


# ---------------------------------------------------------------- softmax ---

@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 2.5])
def test_softmax_two_token_is_logistic(T):
    # V = 2: softmax(x / T)_0 = 1 / (1 + exp((x1 - x0) / T)).
    for x0, x1 in [(0.0, 0.0), (1.5, -2.0), (-3.0, 4.25), (10.0, 9.0)]:
        p = oracle.tempered_softmax(np.array([x0, x1]), T)
        assert p[0] == pytest.approx(1.0 / (1.0 + math.exp((x1 - x0) / T)), rel=1e-14)
        assert p[0] + p[1] == pytest.approx(1.0, abs=1e-15)


def test_softmax_power_form_of_tempered_law():
    # SPOT Eq. 2: pi_T(v) = p(v)^(1/T) / sum p^(1/T).  Feed logits log p + c.
    rng = np.random.default_rng(1)
    p = rng.dirichlet(np.ones(12))
    for T in (0.5, 1.0, 1.7):
        got = oracle.tempered_softmax(np.log(p) + 3.25, T)
        want = p ** (1.0 / T)
        want = want / math.fsum(want)
        np.testing.assert_allclose(got, want, rtol=1e-12)


def test_softmax_neg_inf_is_exact_zero_and_shift_invariant():
    x = np.array([1.0, -np.inf, 0.5, -np.inf, 2.0])
    p = oracle.tempered_softmax(x, 1.0)
    assert p[1] == 0.0 and p[3] == 0.0
    np.testing.assert_allclose(p, oracle.tempered_softmax(x + 100.0, 1.0), rtol=1e-13)


def test_row_status_codes():
    assert oracle.row_status([0.0, 1.0, -np.inf]) == 0
    assert oracle.row_status([0.0, np.nan]) == oracle.STATUS_NONFINITE
    assert oracle.row_status([0.0, np.inf]) == oracle.STATUS_NONFINITE
    assert oracle.row_status([-np.inf, -np.inf]) == oracle.STATUS_EMPTY_ROW


# ----------------------------------------------------------------- argmax ---

def test_argmax_lowest_index_brute_force():
    rng = np.random.default_rng(2)
    for _ in range(200):
        V = int(rng.integers(1, 40))
        x = rng.integers(-3, 4, V).astype(np.float64)  # many exact ties
        order = sorted(range(V), key=lambda i: (-x[i], i))
        assert oracle.argmax_lowest(x) == order[0]


# ------------------------------------------------------------- acceptance ---

@pytest.mark.parametrize("lam", [0.0, 0.25, 0.5, 1.0])
def test_exact_acceptance_rate_is_one_minus_tv(lam):
    # Packed-SS Lemma B.3: beta = sum_x min(P, Q); Two Tradeoffs Eq. 1-2 and
    # Theorem 1: with p~ = (1-lam)p + lam q the rate is 1 - TV(p~, q)
    # = 1 - (1 - lam) TV(p, q).  P(u < alpha) = alpha for u ~ U[0,1).
    rng = np.random.default_rng(3)
    for _ in range(50):
        _, p = _rand_dist(rng, 16)
        _, q = _rand_dist(rng, 16, 1.0)
        beta = math.fsum(q[d] * oracle.acceptance_test(0.5, p[d], q[d], lam)[1]
                         for d in range(16))
        assert beta == pytest.approx(1.0 - (1.0 - lam) * _tv(p, q), abs=1e-12)


def test_total_variation_is_the_largest_event_gap():
    # TV(p, q) = max over events A of |p(A) - q(A)|: brute force over every
    # subset of a 9-token vocabulary, plus the rejection probability of the
    # lossless test, sum_d q(d) (1 - alpha(d)) (Two Tradeoffs Sec. 2).
    import itertools
    rng = np.random.default_rng(12)
    for trial in range(6):
        V = 9
        p = oracle.tempered_softmax(rng.normal(0, 2, V), 1.0)
        q = oracle.tempered_softmax(rng.normal(0, 2, V), 1.0)
        if trial == 0:
            q = p.copy()
        best = max(abs(sum(p[list(A)]) - sum(q[list(A)]))
                   for r in range(V + 1) for A in itertools.combinations(range(V), r))
        tv = oracle.total_variation(p, q)
        assert abs(tv - best) < 1e-14
        rej = sum(q[d] * (1.0 - oracle.acceptance_test(0.5, p[d], q[d])[1]) for d in range(V))
        assert abs(tv - rej) < 1e-14
    # disjoint supports
    assert oracle.total_variation([0.5, 0.5, 0, 0], [0, 0, 0.25, 0.75]) == 1.0


def test_printed_lossless_acceptance_from_dK():
    # Two Tradeoffs App. F.4: lossless acceptance 1 - d_K.  A pair (p, q) with
    # TV = d_K gives exactly the printed acceptance through the oracle's test.
    g = json.load(open(os.path.join(GOLDEN, "two_tradeoffs_dK.json")))
    for dK, printed in zip(g["d_K"], g["lossless_acceptance"]):
        p = np.array([1.0 - dK, dK, 0.0])
        q = np.array([1.0 - dK, 0.0, dK])          # TV(p, q) = dK
        assert _tv(p, q) == pytest.approx(dK, abs=1e-15)
        beta = math.fsum(q[d] * oracle.acceptance_test(0.1, p[d], q[d])[1]
                         for d in range(3) if q[d] > 0)
        assert round(beta, 3) == pytest.approx(printed, abs=1e-12)
        # Eq. 6: alpha_K(lam) = 1 - (1 - lam) d_K
        for lam in (0.2, 0.6):
            beta_l = math.fsum(q[d] * oracle.acceptance_test(0.1, p[d], q[d], lam)[1]
                               for d in range(3) if q[d] > 0)
            assert beta_l == pytest.approx(1.0 - (1.0 - lam) * dK, abs=1e-12)


def test_acceptance_strict_inequality_and_zero_q():
    acc, alpha, _, qz = oracle.acceptance_test(0.5, 0.25, 0.5)
    assert alpha == 0.5 and acc is False          # u == alpha rejects
    acc, alpha, _, qz = oracle.acceptance_test(0.4999, 0.25, 0.5)
    assert acc is True
    acc, alpha, _, qz = oracle.acceptance_test(0.99, 0.1, 0.0)
    assert acc is True and qz is True and alpha == 1.0
    acc, alpha, _, qz = oracle.acceptance_test(0.0, 0.0, 0.0)
    assert acc is False and qz is False


# ----------------------------------------------------------- inverse CDF ---

def test_inverse_cdf_interval_measure():
    # The set of u mapped to c has measure w_c / Z; checked on a fine grid.
    rng = np.random.default_rng(4)
    w = rng.random(9)
    w[[2, 6]] = 0.0
    N = 200000
    counts = np.zeros(9)
    for k in range(N):
        c, _, _ = oracle.inverse_cdf(w, (k + 0.5) / N)
        counts[c] += 1
    np.testing.assert_allclose(counts / N, w / w.sum(), atol=2.0 / N)
    assert counts[2] == 0 and counts[6] == 0


def test_inverse_cdf_edges():
    w = np.array([0.0, 1.0, 0.0, 3.0])
    assert oracle.inverse_cdf(w, 0.0)[0] == 1
    assert oracle.inverse_cdf(w, 0.2499)[0] == 1
    assert oracle.inverse_cdf(w, 0.25)[0] == 3     # F(1) = 1 is not > 1
    assert oracle.inverse_cdf(w, 0.9999999)[0] == 3


# ------------------------------------------------- emitted law (Lemma B.3) ---

@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_emitted_law_exact_enumeration(lam):
    # Packed-SS Lemma B.3 (Two Tradeoffs App. D Prop. 2 for p~): for d ~ q,
    # sum_d q(d)[1{x = d} alpha(d) + (1 - alpha(d)) r(x) / Z] = p~(x).
    rng = np.random.default_rng(5)
    for V in (5, 64, 1024):
        _, p = _rand_dist(rng, V, 3.0)
        _, q = _rand_dist(rng, V, 2.0)
        r = oracle.residual_weights(p, q, lam)
        Z = r.sum()
        law = np.zeros(V)
        for d in range(V):
            alpha = oracle.acceptance_test(0.5, p[d], q[d], lam)[1]
            law[d] += q[d] * alpha
            law += q[d] * (1.0 - alpha) * r / Z
        np.testing.assert_allclose(law, (1 - lam) * p + lam * q, atol=1e-12)
        # rejection probability equals the residual mass (Lemma B.3)
        rej = math.fsum(q[d] * (1 - oracle.acceptance_test(0.5, p[d], q[d], lam)[1])
                        for d in range(V))
        assert rej == pytest.approx(Z, abs=1e-12)


def _sample(rng, dist, n):
    return rng.choice(len(dist), size=n, p=dist)


def _chi2_ok(counts, probs, pmin=1e-4):
    exp = probs * counts.sum()
    keep = exp >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    return stats.chisquare(obs, ex).pvalue > pmin


@pytest.mark.parametrize("miscal", [1.0, 2.0])
def test_full_oracle_emitted_law_chi2(miscal):
    # The whole verifier, run on many seeds batched on the B axis with drafts
    # drawn from q: position 1 is distributed as p_1, and position 2 given
    # that draft 1 was accepted as p_2 (SPOT App. B.4 check, incl. a
    # deliberately miscalibrated q).
    rng = np.random.default_rng(6)
    V, K, N = 8, 2, 20000
    x = rng.normal(0, 1.5, (K + 1, V))
    y = x[:K] * miscal + rng.normal(0, 1.0, (K, V))
    p = [oracle.tempered_softmax(x[i], 1.0) for i in range(K + 1)]
    q = [oracle.tempered_softmax(y[i], 1.0) for i in range(K)]
    d = np.stack([_sample(rng, q[i], N) for i in range(K)], 1)
    tgt = np.broadcast_to(x, (N, K + 1, V))
    drf = np.broadcast_to(y, (N, K, V))
    res = oracle.verify_rejection(tgt, drf, d, None, 1.0, 1.0,
                                  rng.random((N, K)), rng.random((N, K + 1)))
    first = res["out_tokens"][:, 0]
    assert _chi2_ok(np.bincount(first, minlength=V), p[0])
    sel = res["accept_len"] >= 1
    second = res["out_tokens"][sel, 1]
    assert _chi2_ok(np.bincount(second, minlength=V), p[1])
    # acceptance rate of draft 1 within 4 sigma (and 0.002 as in SPOT B.4)
    beta = 1.0 - _tv(p[0], q[0])
    se = math.sqrt(beta * (1 - beta) / N)
    assert abs(sel.mean() - beta) < max(4 * se, 0.002)


def test_lenient_emitted_law_and_rate():
    # Two Tradeoffs Theorem 1 / App. D: rejection sampling against p~ emits p~
    # at drafted positions with acceptance 1 - (1 - lam) TV(p, q).
    rng = np.random.default_rng(7)
    V, N, lam = 8, 20000, 0.5
    x = rng.normal(0, 1.5, (2, V))
    y = rng.normal(0, 1.5, (1, V))
    p = oracle.tempered_softmax(x[0], 1.0)
    q = oracle.tempered_softmax(y[0], 1.0)
    d = _sample(rng, q, N)[:, None]
    res = oracle.verify_lenient(np.broadcast_to(x, (N, 2, V)), np.broadcast_to(y, (N, 1, V)),
                                d, None, 1.0, 1.0, lam, rng.random((N, 1)), rng.random((N, 2)))
    pt = (1 - lam) * p + lam * q
    assert _chi2_ok(np.bincount(res["out_tokens"][:, 0], minlength=V), pt)
    beta = 1 - (1 - lam) * _tv(p, q)
    se = math.sqrt(beta * (1 - beta) / N)
    assert abs((res["accept_len"] == 1).mean() - beta) < 4 * se


def _chain_case(rng, B=6, K=5, V=40, sigma=1.0, n_random=True):
    x = rng.normal(0, 3, (B, K + 1, V))
    y = x[:, :K] + rng.normal(0, sigma, (B, K, V))
    d = np.zeros((B, K), np.int64)
    for b in range(B):
        for i in range(K):
            d[b, i] = _sample(rng, oracle.tempered_softmax(y[b, i], 1.0), 1)[0]
    n = rng.integers(0, K + 1, B) if n_random else np.full(B, K)
    return x, y, d, n


def test_lenient_lambda_zero_is_lossless_bit_for_bit():
    rng = np.random.default_rng(8)
    x, y, d, n = _chain_case(rng)
    ua, ur = rng.random((6, 5)), rng.random((6, 6))
    a = oracle.verify_rejection(x, y, d, n, 0.8, 1.1, ua, ur)
    b = oracle.verify_lenient(x, y, d, n, 0.8, 1.1, 0.0, ua, ur)
    for k in ("accept_len", "num_out", "out_tokens", "status", "alpha"):
        np.testing.assert_array_equal(a[k], b[k])


def test_lenient_lambda_one_accepts_everything_and_h_monotone():
    rng = np.random.default_rng(9)
    x, y, d, n = _chain_case(rng, B=20)
    ua, ur = rng.random((20, 5)), rng.random((20, 6))
    prev = None
    for lam in (0.0, 0.25, 0.5, 0.75, 1.0):
        r = oracle.verify_lenient(x, y, d, n, 1.0, 1.0, lam, ua, ur)
        if prev is not None:
            assert (r["accept_len"] >= prev).all()
        prev = r["accept_len"]
    np.testing.assert_array_equal(prev, n)


def test_expected_accept_length_fixed_drafts():
    # With fixed drafts and independent uniforms the accept indicators are
    # independent with P = alpha_i, so E[h] = sum_n prod_{i<=n} alpha_i
    # (Two Tradeoffs App. C, Eq. 10-13).
    rng = np.random.default_rng(10)
    V, K, R = 30, 6, 20000
    x = rng.normal(0, 2, (K + 1, V))
    y = x[:K] + rng.normal(0, 0.7, (K, V))
    d = np.array([oracle.argmax_lowest(y[i]) for i in range(K)])
    alphas = [oracle.acceptance_test(0.5, oracle.tempered_softmax(x[i], 1.0)[d[i]],
                                     oracle.tempered_softmax(y[i], 1.0)[d[i]])[1]
              for i in range(K)]
    expect = sum(np.prod(alphas[:m]) for m in range(1, K + 1))
    res = oracle.verify_rejection(np.broadcast_to(x, (R, K + 1, V)), np.broadcast_to(y, (R, K, V)),
                                  np.broadcast_to(d, (R, K)), None, 1.0, 1.0,
                                  rng.random((R, K)), rng.random((R, K + 1)))
    h = res["accept_len"].astype(np.float64)
    assert abs(h.mean() - expect) < 4 * h.std() / math.sqrt(R)


def test_expected_tokens_iid_closed_form():
    # Two Tradeoffs App. C Prop. 1: iid acceptance with mean mu gives
    # E[tokens per round] = sum_{n=0}^{B} mu^n = (1 - mu^(B+1)) / (1 - mu).
    rng = np.random.default_rng(11)
    V, K, R = 6, 4, 20000
    x1 = rng.normal(0, 1.5, V)
    y1 = rng.normal(0, 1.5, V)
    p = oracle.tempered_softmax(x1, 1.0)
    q = oracle.tempered_softmax(y1, 1.0)
    mu = 1 - _tv(p, q)
    d = _sample(rng, q, R * K).reshape(R, K)
    res = oracle.verify_rejection(np.broadcast_to(x1, (R, K + 1, V)), np.broadcast_to(y1, (R, K, V)),
                                  d, None, 1.0, 1.0, rng.random((R, K)), rng.random((R, K + 1)))
    toks = res["num_out"].astype(np.float64)
    assert abs(toks.mean() - (1 - mu ** (K + 1)) / (1 - mu)) < 4 * toks.std() / math.sqrt(R)


# ------------------------------------------------------------------ greedy ---

def _logits_with_argmax(rng, tokens, V):
    rows = rng.normal(0, 1, (len(tokens), V))
    for i, t in enumerate(tokens):
        rows[i, t] = rows[i].max() + 1.0
    return rows


def test_greedy_fig2_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "fig2_worked_example.json")))
    rng = np.random.default_rng(12)
    V, W, n = 50, g["W"], g["draft_len"]
    d = [11, 22, 33]
    v = [11, 7, 33, 44]                       # d1 = v1, d2 != v2, per the figure
    assert [a == b for a, b in zip(d, v)] == g["match_pattern"]
    z = [1, 2, 3, 4]
    tgt = np.zeros((1, W, V))                 # K + 1 = W rows (K = W - 1 drafts)
    tgt[0, :n + 1] = _logits_with_argmax(rng, v, V)
    tgt[0, n + 1:] = rng.normal(0, 1, (W - n - 1, V))
    dt = np.full((1, W - 1), 0)
    dt[0, :n] = d
    res = oracle.verify_greedy(tgt, dt, [n], _logits_with_argmax(rng, z, V)[None])
    e = g["expected"]
    names = dict(d1=d[0], v2=v[1], z3=z[2], z4=z[3])
    assert res["accept_len"][0] == e["accept_len"]
    assert res["num_out"][0] == e["num_out"]
    assert list(res["out_tokens"][0, :2]) == [names[t] for t in e["emitted"]]
    assert res["next_len"][0] == e["next_len"]
    assert list(res["next_draft"][0, :2]) == [names[t] for t in e["next_draft"]]


def test_greedy_brute_force_prefix_and_argmax_emission():
    rng = np.random.default_rng(13)
    for _ in range(40):
        B, K, V, W = 3, 6, 9, 7
        x = rng.integers(-2, 3, (B, K + 1, V)).astype(np.float64)  # ties
        dr = rng.normal(0, 1, (B, W, V))
        d = rng.integers(0, V, (B, K))
        for b in range(B):   # make long matches likely
            for i in range(K):
                if rng.random() < 0.7:
                    d[b, i] = int(np.argmax(x[b, i]))
        n = rng.integers(0, K + 1, B)
        res = oracle.verify_greedy(x, d, n, dr)
        for b in range(B):
            vv = [min(range(V), key=lambda j: (-x[b, i, j], j)) for i in range(K + 1)]
            h = 0
            for i in range(n[b]):
                if d[b, i] != vv[i]:
                    break
                h += 1
            assert res["accept_len"][b] == h
            toks = res["out_tokens"][b, :res["num_out"][b]]
            assert list(toks) == [vv[i] for i in range(h + 1)]   # every emitted = row argmax
            zz = [int(np.argmax(dr[b, j])) for j in range(W)]
            assert list(res["next_draft"][b, :res["next_len"][b]]) == zz[h + 1:]
            assert res["next_len"][b] == max(0, W - (h + 1))


def test_greedy_is_the_zero_temperature_limit_of_rejection():
    # Packed-SS App. B.2 ('Greedy decoding'): point masses on the argmax turn
    # Algorithm 2 into Algorithm 1.  At a small temperature with separated
    # logits, rejection sampling reproduces greedy verification.
    rng = np.random.default_rng(14)
    B, K, V = 8, 5, 30
    x = rng.normal(0, 3, (B, K + 1, V))
    y = x[:, :K] + rng.normal(0, 2, (B, K, V))
    d = np.argmax(y, axis=2)
    n = rng.integers(0, K + 1, B)
    g = oracle.verify_greedy(x, d, n)
    r = oracle.verify_rejection(x, y, d, n, 1e-3, 1e-3, rng.random((B, K)), rng.random((B, K + 1)))
    np.testing.assert_array_equal(g["accept_len"], r["accept_len"])
    np.testing.assert_array_equal(g["out_tokens"], r["out_tokens"])


def test_stopping_rule_eos_and_budget():
    # Packed-SS Algorithm 1 ending condition: a = min({A, budget} U {i: C_i = EOS}).
    assert oracle.stopping_index([5, 9, 7], 3) == 3
    assert oracle.stopping_index([5, 9, 7], 3, eos_id=9) == 2
    assert oracle.stopping_index([5, 9, 9], 3, eos_id=9) == 2
    assert oracle.stopping_index([5, 9, 7], 3, eos_id=9, budget=1) == 1
    assert oracle.stopping_index([5, 9, 7], 3, eos_id=4, budget=0) == 0
    rng = np.random.default_rng(15)
    V, K, W = 12, 4, 5
    x = _logits_with_argmax(rng, [3, 4, 6, 2, 8], V)[None]
    dr = _logits_with_argmax(rng, [0, 1, 2, 3, 4], V)[None]
    res = oracle.verify_greedy(x, [[3, 4, 6, 2]], [4], dr, eos_id=6, len_budget=[10])
    assert res["accept_len"][0] == 4 and res["num_out"][0] == 3
    assert list(res["out_tokens"][0]) == [3, 4, 6, -1, -1]
    assert res["next_len"][0] == 2 and list(res["next_draft"][0, :2]) == [3, 4]


def test_error_status_and_sentinels():
    rng = np.random.default_rng(16)
    B, K, V = 4, 3, 10
    x = rng.normal(0, 1, (B, K + 1, V))
    y = rng.normal(0, 1, (B, K, V))
    d = rng.integers(0, V, (B, K))
    d[0, 1] = V                       # out of range draft token
    x[1, 2, 4] = np.nan               # NaN in a row that is read
    x[2, :, :] = -np.inf              # every row empty
    x[3, 3, :] = np.nan               # NaN only in a row that is not read
    n = [3, 3, 3, 2]
    r = oracle.verify_rejection(x, y, d, n, 1.0, 1.0, rng.random((B, K)), rng.random((B, K + 1)))
    assert r["status"][0] == oracle.STATUS_BAD_INPUT
    assert r["status"][1] == oracle.STATUS_NONFINITE
    assert r["status"][2] == oracle.STATUS_EMPTY_ROW
    assert r["status"][3] & oracle.STATUS_ERROR_MASK == 0
    for b in range(3):
        assert r["accept_len"][b] == -1 and (r["out_tokens"][b] == -1).all()


def test_q_zero_flag_accepts():
    V = 6
    x = np.zeros((1, 2, V))
    y = np.zeros((1, 1, V))
    y[0, 0, 2] = -np.inf               # q(2) = 0, p(2) > 0
    r = oracle.verify_rejection(x, y, [[2]], None, 1.0, 1.0, [[0.999]], [[0.3, 0.3]])
    assert r["accept_len"][0] == 1
    assert r["status"][0] & oracle.STATUS_Q_ZERO


def test_lenient_bonus_is_drawn_from_p_not_p_tilde():
    # Two Tradeoffs Algorithm 1: after full acceptance the extra token comes
    # from p_{B+1}, not from the relaxed target.
    rng = np.random.default_rng(17)
    V, N, lam = 6, 20000, 0.9
    x = rng.normal(0, 1.5, (2, V))
    y = x[:1].copy()                      # q = p: every draft accepted
    d = _sample(rng, oracle.tempered_softmax(y[0], 1.0), N)[:, None]
    res = oracle.verify_lenient(np.broadcast_to(x, (N, 2, V)), np.broadcast_to(y, (N, 1, V)),
                                d, None, 1.0, 1.0, lam, rng.random((N, 1)), rng.random((N, 2)))
    assert (res["accept_len"] == 1).all()
    p2 = oracle.tempered_softmax(x[1], 1.0)
    assert _chi2_ok(np.bincount(res["out_tokens"][:, 1], minlength=V), p2)
