"""Pins of the joint-space chain oracle (SPOT App. B, Eq. 10-14 and
Proposition 3; the confidence-gated hybrid of the Table 22 discussion).

* With the drafter always proposing the target's position with q_pos = 1 the
  joint space collapses to the token chain: the result equals the lossless
  token verifier (itself pinned on its own).
* Proposition 3 on an explicit joint space: proposals drawn from
  q(s, v) = q_pos(s) qhat_s(v) over every (position, token) pair, the
  committed pair has law pi_k and the acceptance rate is 1 - TV(pi_k, q_k)
  computed over the whole joint space.
* A worked example traced by hand from Eq. 13-14.
* The hybrid: links whose drafter confidence is known by construction take
  the verifier the gate names; under match with coupled noise the commit
  law is pi and the acceptance rate lies between the coupling bound
  (1 - d)/(1 + d) quoted by the page and the maximal-coupling value 1 - d.
"""

import math

import numpy as np
import pytest
from scipy import stats

import oracle
from tests.test_oracle_cactus_pins import _chi2_ok


def _gumbel(rng, shape):
    u = rng.random(shape)
    return -np.log(-np.log(u))


# ------------------------------------------------- reduction to token chain

def test_position_certain_proposals_are_the_token_chain():
    rng = np.random.default_rng(51)
    B, K, V = 30, 6, 40
    x = rng.normal(0, 3, (B, K + 1, V))
    y = x[:, :K] + rng.normal(0, 1.5, (B, K, V))
    d = np.array([[rng.choice(V, p=oracle.tempered_softmax(y[b, i], 0.9)) for i in range(K)] for b in range(B)])
    n = rng.integers(0, K + 1, B)
    ua, ur = rng.random((B, K)), rng.random((B, K + 1))
    pos = rng.integers(0, 32, (B, K + 1))
    ref = oracle.verify_rejection(x, y, d, n, 1.1, 0.9, ua, ur, eos_id=int(d[0, 0]), len_budget=n + 1)
    got = oracle.verify_spot_chain(x, y, pos, pos[:, :K], d, np.ones((B, K)), n, 1.1, 0.9, ua, ur,
                                   eos_id=int(d[0, 0]), len_budget=n + 1)
    for k in ("accept_len", "num_out", "out_tokens", "status", "alpha", "residual_mass"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)


# ---------------------------------------------------------- Proposition 3 ---

@pytest.mark.parametrize("seed", [52, 53])
def test_joint_space_commit_law_and_acceptance(seed):
    # One verified state with L = 3 positions and V = 5 tokens; the target
    # commits at s* = 1.  The drafter's joint proposal law covers every pair.
    rng = np.random.default_rng(seed)
    L, V, N, s_star = 3, 5, 40000, 1
    xt = rng.normal(0, 1.2, V)
    p = oracle.tempered_softmax(xt, 1.0)
    q_pos = rng.dirichlet(np.full(L, 2.0))
    ylog = rng.normal(0, 1.2, (L, V))
    qhat = np.array([oracle.tempered_softmax(ylog[s], 1.0) for s in range(L)])
    pi = np.zeros((L, V))
    pi[s_star] = p
    q = q_pos[:, None] * qhat
    tv = 0.5 * np.abs(pi - q).sum()
    assert 0.2 < tv < 0.95
    flat = rng.choice(L * V, size=N, p=q.reshape(-1))
    s_prop, v_prop = flat // V, flat % V
    res = oracle.verify_spot_chain(
        np.broadcast_to(np.stack([xt, xt]), (N, 2, V)), np.broadcast_to(ylog[s_star], (N, 1, V)),
        np.tile([s_star, 0], (N, 1)), s_prop[:, None], v_prop[:, None], np.full((N, 1), q_pos[s_star]),
        None, 1.0, 1.0, rng.random((N, 1)), rng.random((N, 2)))
    counts = np.bincount(res["out_tokens"][:, 0], minlength=V)
    assert counts[p == 0].sum() == 0
    assert _chi2_ok(counts, p)
    rate = float((res["accept_len"] == 1).mean())
    se = math.sqrt((1 - tv) * tv / N)
    assert abs(rate - (1.0 - tv)) < 4 * se, (rate, 1 - tv)
    # proposals off s* are never accepted
    assert not (res["accept_len"][s_prop != s_star] == 1).any()


# --------------------------------------------------------- worked example ---

def test_worked_example_by_hand():
    # p = (0.5, 0.3, 0.2) at s* = 4; qhat = (0.2, 0.2, 0.6); q_pos(s*) = 0.5,
    # so q at (4, v) = (0.1, 0.1, 0.3).  Proposal (4, 2): alpha = 0.2 / 0.3.
    x = np.log([[0.5, 0.3, 0.2], [0.25, 0.25, 0.5]])[None]
    y = np.log([[0.2, 0.2, 0.6]])[None]
    base = dict(pos_star=[[4, 7]], prop_pos=[[4]], prop_tok=[[2]], q_pos_star=[[0.5]], draft_len=None,
                t_target=1.0, t_draft=1.0)

    def run(ua, ur, **kw):
        a = dict(base, **kw)
        return oracle.verify_spot_chain(x, y, a["pos_star"], a["prop_pos"], a["prop_tok"], a["q_pos_star"],
                                        a["draft_len"], 1.0, 1.0, [[ua]], [ur])

    # u = 0.7 >= 2/3: rejected.  Residual [p - q]_+ = (0.4, 0.2, 0), mass
    # 0.6; u' = 0.5 puts u' Z = 0.3 inside token 0's interval [0, 0.4).
    g = run(0.7, [0.5, 0.0])
    assert g["alpha"][0, 0] == pytest.approx(2.0 / 3.0, rel=1e-12)
    assert g["accept_len"][0] == 0 and g["out_tokens"][0, 0] == 0
    assert g["residual_mass"][0] == pytest.approx(0.6, rel=1e-12)
    # u' = 0.8: 0.48 falls in token 1's interval [0.4, 0.6).
    assert run(0.7, [0.8, 0.0])["out_tokens"][0, 0] == 1
    # u = 0.6 < 2/3: accepted; the bonus from row 1 = (0.25, 0.25, 0.5) with
    # u' = 0.55 lands in token 2's interval [0.5, 1).
    g = run(0.6, [0.0, 0.55])
    assert g["accept_len"][0] == 1 and g["out_tokens"][0, :2].tolist() == [2, 2]
    # The proposal sits at position 5 != s*: rejected whatever u is, and the
    # commit is drawn at s* from the same residual.
    g = run(0.0, [0.8, 0.0], prop_pos=[[5]])
    assert g["accept_len"][0] == 0 and g["alpha"][0, 0] == 0.0 and g["out_tokens"][0, 0] == 1
    # q_pos(s*) = 1 and the draft proposes token 0: p/q = 0.5/0.2 >= 1.
    g = run(0.999, [0.0, 0.0], prop_tok=[[0]], q_pos_star=[[1.0]])
    assert g["alpha"][0, 0] == 1.0 and g["accept_len"][0] == 1


# ------------------------------------------------------------------ hybrid --

def _rows_with_max(pmax, V):
    """Logits of a drafter row whose largest probability is pmax (token 0)."""
    rest = (1.0 - pmax) / (V - 1)
    return np.log(np.array([pmax] + [rest] * (V - 1)))


def test_gate_picks_the_verifier():
    # Link 0: drafter confidence 0.8 (match); link 1: 0.4 (RS); tau = 0.6.
    V = 4
    x = np.log([[0.4, 0.3, 0.2, 0.1], [0.1, 0.2, 0.3, 0.4], [0.25, 0.25, 0.25, 0.25]])[None]
    y = np.stack([_rows_with_max(0.8, V), _rows_with_max(0.4, V)])[None]
    G = np.zeros((1, 3, V))
    G[0, 0, 2] = 50.0          # the target's coupled commit at link 0 is token 2
    G[0, 2, 1] = 50.0          # and at the bonus row token 1
    args = dict(pos_star=[[3, 4, 5]], prop_pos=[[3, 4]], q_pos_star=[[1.0, 1.0]])

    def run(tok, ua, tau=0.6, gumbel=G):
        return oracle.verify_spot_chain(x, y, args["pos_star"], args["prop_pos"], [tok], args["q_pos_star"],
                                        None, 1.0, 1.0, [ua], [[0.5, 0.5, 0.5]], gumbel=gumbel, tau=tau)

    g = run([2, 3], [0.99, 0.99])
    assert g["mode"][0].tolist() == [oracle.MODE_MATCH, oracle.MODE_RS]
    assert g["conf"][0, 0] == pytest.approx(0.8) and g["conf"][0, 1] == pytest.approx(0.4)
    # match accepts token 2 whatever u is; RS at link 1: p(3) = 0.4, q(3) = 0.2
    # so alpha = 1 and token 3 is accepted too; the bonus is row 2's coupled
    # commit, token 1.
    assert g["accept_len"][0] == 2 and g["out_tokens"][0].tolist() == [2, 3, 1]
    # a draft other than the coupled commit is rejected at a match link and
    # the commit is the coupled token
    g = run([1, 3], [0.0, 0.0])
    assert g["accept_len"][0] == 0 and g["out_tokens"][0, 0] == 2
    # tau above 1: no link matches; link 0 by RS: p(2) / q(2) = 0.2 / (0.2/3)
    # >= 1 accepts; link 1 accepts too; the bonus still uses the Gumbel row
    g = run([2, 3], [0.99, 0.99], tau=1.5)
    assert g["mode"][0].tolist() == [oracle.MODE_RS, oracle.MODE_RS]
    assert g["accept_len"][0] == 2 and g["out_tokens"][0, 2] == 1
    # without Gumbel rows every link is RS and the bonus is an inverse-CDF
    # draw from p at row 2 (uniform 0.5 -> token 2 of four equal masses)
    g = run([2, 3], [0.99, 0.99], gumbel=None)
    assert g["out_tokens"][0].tolist() == [2, 3, 2]


def test_gate_off_matches_pure_rejection_sampling():
    rng = np.random.default_rng(54)
    B, K, V = 40, 5, 30
    x = rng.normal(0, 2, (B, K + 1, V))
    y = x[:, :K] + rng.normal(0, 1.0, (B, K, V))
    d = np.array([[rng.choice(V, p=oracle.tempered_softmax(y[b, i], 1.0)) for i in range(K)] for b in range(B)])
    pos = rng.integers(0, 8, (B, K + 1))
    prop = np.where(rng.random((B, K)) < 0.8, pos[:, :K], pos[:, :K] + 1)
    c = rng.uniform(0.3, 1.0, (B, K))
    ua, ur = rng.random((B, K)), rng.random((B, K + 1))
    G = _gumbel(rng, (B, K + 1, V))
    a = oracle.verify_spot_chain(x, y, pos, prop, d, c, None, 1.0, 1.0, ua, ur)
    b = oracle.verify_spot_chain(x, y, pos, prop, d, c, None, 1.0, 1.0, ua, ur, gumbel=G, tau=1.01)
    np.testing.assert_array_equal(a["accept_len"], b["accept_len"])
    np.testing.assert_array_equal(a["alpha"], b["alpha"])
    rejected = a["accept_len"] < K
    np.testing.assert_array_equal(a["out_tokens"][rejected], b["out_tokens"][rejected])
    assert rejected.sum() > 10


def test_match_links_commit_law_and_coupling_bounds():
    # Every link matches (tau = 0).  The drafter proposes its own Gumbel
    # argmax under the same noise row, at s*; the commit must have law p and
    # the agreement rate must lie between (1 - d)/(1 + d) and 1 - d, d the
    # total variation between p and qhat.
    rng = np.random.default_rng(55)
    V, N = 6, 40000
    xt = rng.normal(0, 1.0, V)
    yl = xt + rng.normal(0, 0.8, V)
    p = oracle.tempered_softmax(xt, 1.0)
    qh = oracle.tempered_softmax(yl, 1.0)
    dtv = 0.5 * np.abs(p - qh).sum()
    G = _gumbel(rng, (N, 2, V))
    prop = np.argmax(np.log(qh)[None, :] + G[:, 0], axis=1)
    res = oracle.verify_spot_chain(np.broadcast_to(np.stack([xt, xt]), (N, 2, V)), np.broadcast_to(yl, (N, 1, V)),
                                   np.zeros((N, 2), int), np.zeros((N, 1), int), prop[:, None], np.ones((N, 1)),
                                   None, 1.0, 1.0, rng.random((N, 1)), rng.random((N, 2)), gumbel=G, tau=0.0)
    assert (res["mode"][:, 0] == oracle.MODE_MATCH).all()
    counts = np.bincount(res["out_tokens"][:, 0], minlength=V)
    assert _chi2_ok(counts, p)
    rate = float((res["accept_len"] == 1).mean())
    se = math.sqrt(rate * (1 - rate) / N)
    assert (1 - dtv) / (1 + dtv) - 4 * se < rate < 1 - dtv + 4 * se, (rate, dtv)
    # an accepted link's token is the proposal; the bonus then commits
    # row 1's coupled token, again with law p
    acc = res["accept_len"] == 1
    assert (res["out_tokens"][acc, 0] == prop[acc]).all()
    assert _chi2_ok(np.bincount(res["out_tokens"][acc, 1], minlength=V), p)


def test_hybrid_chain_first_commit_law():
    # A two-link chain with random gates: the first committed token has law
    # p_0 whichever verifier the gate picked.
    rng = np.random.default_rng(56)
    V, N = 5, 30000
    x0 = rng.normal(0, 1.0, V)
    p0 = oracle.tempered_softmax(x0, 1.0)
    x = np.broadcast_to(np.stack([x0, x0 + 0.3, x0 - 0.2]), (N, 3, V))
    sharp = rng.random(N) < 0.5
    y0 = np.where(sharp[:, None], x0 * 3.0, x0 * 0.3)        # sharp or flat drafter rows
    y = np.stack([y0, y0], axis=1)
    qh = np.array([oracle.tempered_softmax(r, 1.0) for r in y0[:200]])
    assert (qh.max(axis=1)[sharp[:200]] >= 0.6).all() and (qh.max(axis=1)[~sharp[:200]] < 0.6).all()
    G = _gumbel(rng, (N, 3, V))
    q_all = np.exp(y0 - y0.max(axis=1, keepdims=True))
    q_all /= q_all.sum(axis=1, keepdims=True)
    prop = np.where(sharp, np.argmax(np.log(q_all) + G[:, 0], axis=1),
                    np.array([rng.choice(V, p=q_all[i]) for i in range(N)]))
    res = oracle.verify_spot_chain(x, y, np.zeros((N, 3), int), np.zeros((N, 2), int),
                                   np.stack([prop, prop], axis=1), np.ones((N, 2)), None, 1.0, 1.0,
                                   rng.random((N, 2)), rng.random((N, 3)), gumbel=G, tau=0.6)
    np.testing.assert_array_equal(res["mode"][:, 0] == oracle.MODE_MATCH, sharp)
    assert _chi2_ok(np.bincount(res["out_tokens"][:, 0], minlength=V), p0)


def test_bad_inputs():
    x = np.zeros((3, 3, 4))
    y = np.zeros((3, 2, 4))
    pos = np.array([[0, 1, 2], [0, -1, 2], [0, 1, 2]])
    c = np.array([[0.5, 0.5], [0.5, 0.5], [0.5, 1.5]])
    g = oracle.verify_spot_chain(x, y, pos, pos[:, :2], [[0, 1], [0, 1], [0, 1]], c, None, 1.0, 1.0,
                                 np.zeros((3, 2)), np.zeros((3, 3)))
    assert g["status"].tolist() == [0, oracle.STATUS_BAD_INPUT, oracle.STATUS_BAD_INPUT]
    g = oracle.verify_spot_chain(x, y, pos[[0, 0, 0]], pos[[0, 0, 0], :2], [[0, 4], [0, 1], [0, 1]],
                                 c[[0, 0, 0]], [2, 3, 1], 1.0, 1.0, np.zeros((3, 2)), np.zeros((3, 3)))
    assert g["status"].tolist() == [oracle.STATUS_BAD_INPUT] * 2 + [0]
    # a draft token beyond the valid length is never read
    G = np.zeros((3, 3, 4))
    G[2, 1, 0] = np.nan       # row 1 of sequence 2 is read (n = 1): nonfinite
    g = oracle.verify_spot_chain(x, y, pos[[0, 0, 0]], pos[[0, 0, 0], :2], [[0, 1]] * 3, c[[0, 0, 0]],
                                 [2, 0, 1], 1.0, 1.0, np.zeros((3, 2)), np.zeros((3, 3)), gumbel=G)
    assert g["status"].tolist() == [0, 0, oracle.STATUS_NONFINITE]
