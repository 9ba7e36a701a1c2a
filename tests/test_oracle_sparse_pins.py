"""Pins of the sparse stored-Q verifier (Packed-SS Sec. 3.2; the lossless
rule of App. B.2 with the stored drafter distribution).

* A stored list that covers the whole vocabulary is the dense drafter
  distribution: the result equals the lossless token verifier (pinned on its
  own) bit for bit, in any entry order.
* Theorem 3.3's law on a top-k truncated drafter: drafts drawn from the
  truncated Q, the first emitted token has law p and the acceptance rate is
  sum_v min(p, Q) = 1 - TV(p, Q).
* A worked example by hand, including a token outside the stored support.
"""

import math

import numpy as np
import pytest

import oracle
from tests.test_oracle_cactus_pins import _chi2_ok


def test_full_support_is_the_dense_verifier():
    rng = np.random.default_rng(71)
    B, K, V = 12, 5, 37
    x = rng.normal(0, 2.5, (B, K + 1, V))
    y = x[:, :K] + rng.normal(0, 1.0, (B, K, V))
    q = np.array([[oracle.tempered_softmax(y[b, i], 0.8) for i in range(K)] for b in range(B)])
    d = np.array([[rng.choice(V, p=q[b, i]) for i in range(K)] for b in range(B)])
    n = rng.integers(0, K + 1, B)
    ua, ur = rng.random((B, K)), rng.random((B, K + 1))
    ref = oracle.verify_rejection(x, y, d, n, 1.2, 0.8, ua, ur)
    for perm in (np.arange(V), rng.permutation(V)):
        idx = np.broadcast_to(perm, (B, K, V))
        got = oracle.verify_sparse(x, idx, np.take_along_axis(q, idx, axis=2), np.full((B, K), V), d, n, 1.2,
                                   ua, ur)
        for k in ("accept_len", "num_out", "out_tokens", "status", "alpha", "residual_mass", "q_draft"):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)


@pytest.mark.parametrize("topk", [1, 3, 6])
def test_truncated_drafter_law_and_acceptance(topk):
    rng = np.random.default_rng(72 + topk)
    V, N, kmax = 9, 30000, 8
    x = rng.normal(0, 1.2, (2, V))
    p = oracle.tempered_softmax(x[0], 1.0)
    ql = rng.normal(0, 1.5, V)
    order = np.argsort(-ql, kind="stable")[:topk]
    q = np.zeros(V)
    q[order] = np.exp(ql[order] - ql[order].max())
    q /= q.sum()
    idx = np.zeros(kmax, np.int64)
    prob = np.zeros(kmax)
    idx[:topk], prob[:topk] = order, q[order]
    d = rng.choice(V, size=N, p=q)[:, None]
    res = oracle.verify_sparse(np.broadcast_to(x, (N, 2, V)), np.broadcast_to(idx, (N, 1, kmax)),
                               np.broadcast_to(prob, (N, 1, kmax)), np.full((N, 1), topk), d, None, 1.0,
                               rng.random((N, 1)), rng.random((N, 2)))
    counts = np.bincount(res["out_tokens"][:, 0], minlength=V)
    assert _chi2_ok(counts, p)
    rate = float((res["accept_len"] == 1).mean())
    want = float(np.minimum(p, q).sum())
    assert abs(rate - want) < 4 * math.sqrt(want * (1 - want) / N) + 1e-9, (rate, want)


def test_worked_example_by_hand():
    # p = (0.4, 0.3, 0.2, 0.1); stored top-2 Q = {0: 0.6, 2: 0.4}.
    x = np.log([[0.4, 0.3, 0.2, 0.1], [0.1, 0.2, 0.3, 0.4]])[None]
    idx, prob, nnz = [[[2, 0, 3]]], [[[0.4, 0.6, 0.0]]], [[2]]      # the third entry is unused

    def run(tok, ua, ur):
        return oracle.verify_sparse(x, idx, prob, nnz, [[tok]], None, 1.0, [[ua]], [ur])

    # d = 2: alpha = 0.2 / 0.4 = 0.5.  u = 0.7 rejects; [p - Q]_+ = (0, 0.3, 0,
    # 0.1), mass 0.4.  u' = 0.5 -> 0.2 lies in token 1's interval [0, 0.3);
    # u' = 0.9 -> 0.36 lies in token 3's interval [0.3, 0.4).
    g = run(2, 0.7, [0.5, 0.0])
    assert g["alpha"][0, 0] == pytest.approx(0.5) and g["accept_len"][0] == 0
    assert g["out_tokens"][0, 0] == 1 and g["residual_mass"][0] == pytest.approx(0.4)
    assert run(2, 0.7, [0.9, 0.0])["out_tokens"][0, 0] == 3
    # u = 0.3 accepts; the bonus from row 1 with u' = 0.35 -> token 2 ([0.3, 0.6)).
    g = run(2, 0.3, [0.0, 0.35])
    assert g["accept_len"][0] == 1 and g["out_tokens"][0, :2].tolist() == [2, 2]
    # d = 1 lies outside the stored support: Q(d) = 0 < p(d) reads as an
    # infinite ratio (accepted, flagged).
    g = run(1, 0.99, [0.0, 0.0])
    assert g["accept_len"][0] == 1 and g["status"][0] == oracle.STATUS_Q_ZERO


def test_bad_inputs():
    x = np.zeros((5, 2, 4))
    idx = np.tile([[[0, 1]]], (5, 1, 1))
    prob = np.tile([[[0.5, 0.5]]], (5, 1, 1)).astype(float)
    nnz = np.full((5, 1), 2)
    idx[1, 0, 1] = 4             # index outside [0, V)
    prob[2, 0, 0] = -0.1         # negative probability
    prob[3, 0, 1] = np.nan
    nnz[4, 0] = 3                # more entries than kmax
    g = oracle.verify_sparse(x, idx, prob, nnz, np.zeros((5, 1), int), None, 1.0, np.zeros((5, 1)),
                             np.zeros((5, 2)))
    assert g["status"].tolist() == [0] + [oracle.STATUS_BAD_INPUT] * 4
    # rows beyond the draft length are not read
    g = oracle.verify_sparse(x, idx, prob, nnz, np.zeros((5, 1), int), np.zeros(5, int), 1.0,
                             np.zeros((5, 1)), np.zeros((5, 2)))
    assert (g["status"] == 0).all()
