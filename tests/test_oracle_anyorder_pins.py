"""Pins of the any-order greedy oracle (Packed-SS App. C, Algorithm 3).

* The left-to-right order with one trailing undrafted position is the
  chain verifier of Sec. 3.1 (Eq. 1-4), pinned on its own.
* Proposition C.1: on a synthetic verifier whose logits are a fixed hash of
  the conditioning context (so that a verifier row depends on the draft
  tokens before it, as in Eq. 8), the accepted pairs equal those of the
  serial reference that generates A tokens greedily in the chosen order,
  and the accepted count is the one the serial reference implies.
* A worked example, traced by hand from Algorithm 3, fixes the order, the
  missing-draft rule, the window-full rule (A = u, no extra token), the
  ending position E' and retention by position.
"""

import hashlib

import numpy as np
import pytest

import oracle


def _np(x):
    return np.asarray(x)


# --------------------------------------------------- left-to-right reduction

def test_left_to_right_is_the_chain_verifier():
    rng = np.random.default_rng(41)
    for trial in range(40):
        B, K, V = 5, 6, 9
        tgt = rng.integers(-3, 4, (B, K + 1, V)).astype(np.float64)   # ties included
        dr = rng.normal(0, 2, (B, K + 1, V))
        n = rng.integers(0, K + 1, B)
        d_chain = np.array([[int(np.argmax(tgt[b, i])) if rng.random() < 0.7 else int(rng.integers(0, V))
                             for i in range(K)] for b in range(B)])
        ref = oracle.verify_greedy(tgt, d_chain, n, dr)
        # any-order form: u = n + 1 slots at positions 1..u, identity order,
        # slot n has no draft; verifier rows by rank = chain rows 0..n
        U = K + 1
        order = np.tile(np.arange(U), (B, 1))
        drafts = np.full((B, U), -1)
        for b in range(B):
            drafts[b, :n[b]] = d_chain[b, :n[b]]
        pos = np.tile(np.arange(1, U + 1), (B, 1))
        got = oracle.verify_greedy_any_order(tgt, order, n + 1, pos, drafts, dr)
        np.testing.assert_array_equal(got["accept_len"], ref["accept_len"])
        np.testing.assert_array_equal(got["num_accepted"], ref["num_out"])
        for b in range(B):
            A = int(ref["num_out"][b])
            np.testing.assert_array_equal(got["acc_tok"][b, :A], ref["out_tokens"][b, :A])
            np.testing.assert_array_equal(got["acc_pos"][b, :A], np.arange(1, A + 1))
            # retained drafts: the chain keeps z_{A+1..W}; here slots A..u-1
            keep = int(ref["next_len"][b]) - (K + 1 - (n[b] + 1))
            np.testing.assert_array_equal(got["next_draft"][b, A:n[b] + 1], ref["next_draft"][b, :keep])
            assert (got["next_draft"][b, :A] == -1).all()


# ------------------------------------------------------ Proposition C.1 ---

class _HashModel:
    """A deterministic 'verifier': logits at a queried position given the
    ordered context of (position, token) pairs, from a hash of both."""

    def __init__(self, V, salt):
        self.V, self.salt = V, salt

    def logits(self, context, query):
        key = repr((self.salt, tuple(context), query)).encode()
        seed = int.from_bytes(hashlib.sha256(key).digest()[:8], "little")
        return np.random.default_rng(seed).integers(-2, 3, self.V).astype(np.float64)

    def greedy(self, context, query):
        x = self.logits(context, query)
        return int(np.flatnonzero(x == x.max())[0])


def test_serial_reference_of_proposition_c1():
    rng = np.random.default_rng(42)
    V, U = 4, 8
    checked = 0
    for trial in range(300):
        m = _HashModel(V, trial)
        u = int(rng.integers(1, U + 1))
        prompt = [(-1, int(rng.integers(0, V)))]
        pos = sorted(rng.choice(np.arange(1, 40), size=u, replace=False).tolist())
        pi = rng.permutation(u).tolist()
        # the serial reference's tokens in this order
        y, ctx = [], list(prompt)
        for r in range(u):
            y.append(m.greedy(ctx, pos[pi[r]]))
            ctx.append((pos[pi[r]], y[-1]))
        # drafts: mostly the serial token, sometimes wrong, sometimes missing
        d = [-1] * u
        for r in range(u):
            c = rng.random()
            d[pi[r]] = y[r] if c < 0.7 else (-1 if c < 0.85 else (y[r] + 1) % V)
        # the call's verifier rows, conditioned on the drafts at earlier ranks
        rows = np.zeros((1, U, V))
        ctx = list(prompt)
        for r in range(u):
            rows[0, r] = m.logits(ctx, pos[pi[r]])
            ctx.append((pos[pi[r]], d[pi[r]]))
        order = np.zeros((1, U), int)
        order[0, :u] = pi
        drafts = np.full((1, U), -1)
        drafts[0, :u] = d
        posa = np.zeros((1, U), int)
        posa[0, :u] = pos
        posa[0, u:] = 1000 + np.arange(U - u)
        got = oracle.verify_greedy_any_order(rows, order, [u], posa, drafts)
        # serial characterisation of A: leading ranks whose draft exists and
        # equals the serial token, plus one (capped by u)
        hs = 0
        while hs < u and d[pi[hs]] == y[hs]:
            hs += 1
        A = min(hs + 1, u)
        assert got["accept_len"][0] == hs and got["num_accepted"][0] == A
        assert got["acc_pos"][0, :A].tolist() == [pos[pi[r]] for r in range(A)]
        assert got["acc_tok"][0, :A].tolist() == y[:A]     # Prop. C.1
        checked += A
    assert checked > 500


# --------------------------------------------------------- worked example ---

def _onehot_rows(winners, V=16, U=4):
    rows = np.zeros((1, U, V))
    for r, w in enumerate(winners):
        rows[0, r, w] = 5.0
    return rows


def test_worked_example_order_end_and_retention():
    # Four unresolved positions 10..13 (slots 0..3), order pi = (slot 2,
    # slot 0, slot 3, slot 1), drafts by slot (5, 6, 9, 7); the verifier's
    # argmax by rank is (9, 5, 3, 6).  Rank 0: slot 2 drafted 9 = 9; rank 1:
    # slot 0 drafted 5 = 5; rank 2: slot 3 drafted 7 != 3.  So h = 2, A = 3
    # and C = ((12, 9), (10, 5), (13, 3)).
    V = 16
    rows = _onehot_rows([9, 5, 3, 6], V)
    dr = _onehot_rows([11, 12, 13, 14], V)          # drafter argmax by slot
    order = [[2, 0, 3, 1]]
    pos = [[10, 11, 12, 13]]
    drafts = [[5, 6, 9, 7]]
    g = oracle.verify_greedy_any_order(rows, order, None, pos, drafts, dr)
    assert g["accept_len"][0] == 2 and g["num_accepted"][0] == 3
    assert g["acc_pos"][0].tolist() == [12, 10, 13, -1]
    assert g["acc_tok"][0].tolist() == [9, 5, 3, -1]
    assert g["next_draft"][0].tolist() == [-1, 12, -1, -1]      # only slot 1 stays unresolved
    assert g["new_end"][0] == oracle.NO_END
    # EOS = 5 accepted at position 10: E' = 10 drops the pairs at 12 and 13,
    # and no unresolved position at or before 10 remains to keep a draft for.
    g = oracle.verify_greedy_any_order(rows, order, None, pos, drafts, dr, eos_id=5)
    assert g["new_end"][0] == 10 and g["num_accepted"][0] == 1
    assert g["acc_pos"][0].tolist() == [10, -1, -1, -1] and g["acc_tok"][0].tolist() == [5, -1, -1, -1]
    assert (g["next_draft"][0] == -1).all()
    # An end at 12 drops (13, 3) and keeps slot 1's draft (position 11).
    g = oracle.verify_greedy_any_order(rows, order, None, pos, drafts, dr, end_pos=[12])
    assert g["new_end"][0] == 12 and g["num_accepted"][0] == 2
    assert g["acc_pos"][0, :2].tolist() == [12, 10] and g["next_draft"][0].tolist() == [-1, 12, -1, -1]
    # Every draft matches: A = u and no token is taken outside the window.
    g = oracle.verify_greedy_any_order(rows, order, None, pos, [[5, 6, 9, 3]], dr)
    assert g["accept_len"][0] == 4 and g["num_accepted"][0] == 4
    assert g["acc_tok"][0].tolist() == [9, 5, 3, 6]
    # A missing draft at rank 2 (slot 3): kappa = 2, the verifier's token is
    # accepted there after two matches, and rank 3 is never read.
    rows_nan = rows.copy()
    rows_nan[0, 3, :] = np.nan
    g = oracle.verify_greedy_any_order(rows_nan, order, None, pos, [[5, 6, 9, -1]], dr)
    assert g["status"][0] == 0 and g["kappa"][0] == 2 and g["accept_len"][0] == 2
    assert g["acc_pos"][0, :3].tolist() == [12, 10, 13] and g["acc_tok"][0, :3].tolist() == [9, 5, 3]


def test_bad_inputs():
    rows = _onehot_rows([1, 2, 3, 4])
    for order, pos, drafts in (([[0, 0, 1, 2]], [[1, 2, 3, 4]], [[1, 2, 3, 4]]),      # not a permutation
                               ([[0, 1, 2, 3]], [[1, 3, 3, 4]], [[1, 2, 3, 4]]),      # positions not increasing
                               ([[0, 1, 2, 3]], [[1, 2, 3, 4]], [[1, -2, 3, 4]]),     # bad draft token
                               ([[0, 1, 2, 3]], [[1, 2, 3, 4]], [[1, 2, 16, 4]])):
        g = oracle.verify_greedy_any_order(rows, order, None, pos, drafts)
        assert g["status"][0] == oracle.STATUS_BAD_INPUT and g["accept_len"][0] == -1
    g = oracle.verify_greedy_any_order(rows, [[0, 1, 2, 3]], [5], None, [[1, 2, 3, 4]])
    assert g["status"][0] == oracle.STATUS_BAD_INPUT
    g = oracle.verify_greedy_any_order(rows, [[0, 1, 2, 3]], [0], None, [[1, 2, 3, 4]])
    assert g["status"][0] == 0 and g["num_accepted"][0] == 0
