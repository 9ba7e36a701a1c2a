"""Plant typical mistakes in the oracle (on the CPU) and check that some pin
catches each one.  This is evidence that the pins constrain the oracle, not a
test of the product."""

import numpy as np
import pytest

import math

import oracle
import oracle.cactus as cactus
import oracle.chain as chain
import oracle.rows as rows
import oracle.tree as tree
import tests.test_oracle_cactus_pins as kp
import tests.test_oracle_chain_pins as cp
import tests.test_oracle_tree_pins as tp


def _patch(monkeypatch, name, fn):
    for mod in (oracle, rows, chain, tree, cactus):
        if hasattr(mod, name):
            monkeypatch.setattr(mod, name, fn)


def _acc_no_min(u, p_d, q_d, lam=0.0):
    pt = (1 - lam) * p_d + lam * q_d
    alpha = pt / q_d if q_d > 0 else 1.0
    return bool(u < alpha), alpha, abs(u - alpha), False


def _acc_inverted(u, p_d, q_d, lam=0.0):
    pt = (1 - lam) * p_d + lam * q_d
    alpha = min(1.0, q_d / pt) if pt > 0 else 1.0
    return bool(u < alpha), alpha, abs(u - alpha), False


def _acc_le(u, p_d, q_d, lam=0.0):
    pt = (1 - lam) * p_d + lam * q_d
    alpha = min(1.0, pt / q_d) if q_d > 0 else (1.0 if pt > 0 else 0.0)
    return bool(u <= alpha), alpha, abs(u - alpha), bool(q_d == 0 and pt > 0)


def _acc_lam_swapped(u, p_d, q_d, lam=0.0):
    pt = lam * p_d + (1 - lam) * q_d
    alpha = min(1.0, pt / q_d) if q_d > 0 else (1.0 if pt > 0 else 0.0)
    return bool(u < alpha), alpha, abs(u - alpha), False


def _res_sign(p, q, lam=0.0):
    pt = (1 - lam) * np.asarray(p) + lam * np.asarray(q)
    return np.maximum(np.asarray(q) - pt, 0.0)


def _res_plain_p(p, q, lam=0.0):
    return np.asarray(p, np.float64).copy()


def _softmax_times_T(x, T):
    a = np.asarray(x, np.float64) * T
    w = np.exp(a - a.max())
    return w / w.sum()


def _argmax_highest(x):
    x = np.asarray(x, np.float64)
    return int(np.flatnonzero(x == x.max())[-1])


def _icdf_ge(w, u):
    w = np.asarray(w, np.float64)
    F = np.cumsum(w)
    Z = F[-1]
    c = int(np.flatnonzero(F >= u * Z)[0])
    return c, 1.0, Z


def _stop_ignores_eos(C, A, eos_id=-1, budget=None):
    return A if budget is None else min(A, budget)


def _gamma_taylor(p, delta, iters=0):
    return min(p + math.sqrt(2.0 * delta * p * (1.0 - p)), 1.0)


def _target_not_rescaled(p, y, gamma):
    pt = np.asarray(p, np.float64).copy()
    pt[y] = gamma
    return pt


def _residual_lossless(p, q, y, gamma):
    return np.maximum(np.asarray(p, np.float64) - np.asarray(q, np.float64), 0.0)


def _acceptance_ignores_budget(u, p_y, q_y, delta):
    alpha = min(1.0, p_y / q_y) if q_y > 0 else 1.0
    return bool(u < alpha), alpha, abs(u - alpha), False, p_y


MUTATIONS = [
    ("acceptance_test", _acc_no_min, cp.test_exact_acceptance_rate_is_one_minus_tv, dict(lam=0.0)),
    ("acceptance_test", _acc_inverted, cp.test_exact_acceptance_rate_is_one_minus_tv, dict(lam=0.0)),
    ("acceptance_test", _acc_le, cp.test_acceptance_strict_inequality_and_zero_q, {}),
    ("acceptance_test", _acc_lam_swapped, cp.test_exact_acceptance_rate_is_one_minus_tv, dict(lam=0.25)),
    ("residual_weights", _res_sign, cp.test_emitted_law_exact_enumeration, dict(lam=0.0)),
    ("residual_weights", _res_plain_p, cp.test_emitted_law_exact_enumeration, dict(lam=0.0)),
    ("tempered_softmax", _softmax_times_T, cp.test_softmax_two_token_is_logistic, dict(T=0.3)),
    ("argmax_lowest", _argmax_highest, cp.test_argmax_lowest_index_brute_force, {}),
    ("inverse_cdf", _icdf_ge, cp.test_inverse_cdf_edges, {}),
    ("stopping_index", _stop_ignores_eos, cp.test_stopping_rule_eos_and_budget, {}),
    ("cactus_gamma", _gamma_taylor, kp.test_modified_target_meets_kl_budget_exactly, dict(delta=0.25)),
    ("cactus_target", _target_not_rescaled, kp.test_modified_target_meets_kl_budget_exactly, dict(delta=0.25)),
    ("cactus_residual", _residual_lossless, kp.test_emitted_law_and_acceptance_rate, dict(delta=0.3)),
    ("cactus_acceptance", _acceptance_ignores_budget, kp.test_emitted_law_and_acceptance_rate, dict(delta=0.3)),
]


@pytest.mark.parametrize("name,fn,pin,kw", MUTATIONS,
                         ids=[f"{m[0]}-{m[1].__name__}" for m in MUTATIONS])
def test_pin_catches_planted_mistake(monkeypatch, name, fn, pin, kw):
    _patch(monkeypatch, name, fn)
    with pytest.raises(AssertionError):
        pin(**kw)


def test_pin_catches_retention_off_by_one(monkeypatch):
    orig = chain.verify_greedy

    def shifted(*a, **k):
        out = orig(*a, **k)
        nd = out["next_draft"]
        out["next_draft"] = np.concatenate([nd[:, 1:], np.full((nd.shape[0], 1), -1, nd.dtype)], 1)
        return out
    monkeypatch.setattr(oracle, "verify_greedy", shifted)
    with pytest.raises(AssertionError):
        cp.test_greedy_fig2_worked_example()


def test_pin_catches_gumbel_temperature_mistake(monkeypatch):
    def wrong(x, T):
        a = np.asarray(x, np.float64) * T
        m = a.max()
        return a - m - np.log(np.exp(a - m).sum())
    monkeypatch.setattr(tree, "_log_tempered_softmax", wrong)
    with pytest.raises(AssertionError):
        tp.test_gumbel_draw_has_tempered_law(T=0.5)


def test_pin_catches_walk_not_following_child(monkeypatch):
    orig = tree.verify_gumbel_tree

    def stops_at_root(*a, **k):
        out = orig(*a, **k)
        out["path_len"][:] = np.minimum(out["path_len"], 0)
        return out
    monkeypatch.setattr(oracle, "verify_gumbel_tree", stops_at_root)
    with pytest.raises(AssertionError):
        tp.test_orbit_tree_is_accepted_to_full_depth(T=1.0)


# ------------------------------------------------- any-order verification ---

import tests.test_oracle_anyorder_pins as ap  # noqa: E402
import oracle.anyorder as anyorder  # noqa: E402


def _ao_ignores_order(tgt, order, num_active, positions, draft_tokens, draft_rows=None, eos_id=-1,
                      end_pos=None):
    ident = np.tile(np.arange(np.asarray(order).shape[1]), (np.asarray(order).shape[0], 1))
    return anyorder.verify_greedy_any_order(tgt, ident, num_active, positions, draft_tokens, draft_rows,
                                            eos_id, end_pos)


def _ao_eos_truncates_by_rank(tgt, order, num_active, positions, draft_tokens, draft_rows=None, eos_id=-1,
                              end_pos=None):
    out = anyorder.verify_greedy_any_order(tgt, order, num_active, positions, draft_tokens, draft_rows,
                                           -1, end_pos)
    if eos_id >= 0:
        for b in range(out["acc_tok"].shape[0]):
            toks = out["acc_tok"][b].tolist()
            if eos_id in toks:
                k = toks.index(eos_id) + 1
                out["acc_tok"][b, k:] = -1
                out["acc_pos"][b, k:] = -1
                out["num_accepted"][b] = min(out["num_accepted"][b], k)
    return out


def _ao_keeps_beyond_end(tgt, order, num_active, positions, draft_tokens, draft_rows=None, eos_id=-1,
                         end_pos=None):
    out = anyorder.verify_greedy_any_order(tgt, order, num_active, positions, draft_tokens, draft_rows,
                                           eos_id, end_pos)
    free = anyorder.verify_greedy_any_order(tgt, order, num_active, positions, draft_tokens, draft_rows)
    out["next_draft"] = free["next_draft"]
    return out


@pytest.mark.parametrize("fn,pin", [
    (_ao_ignores_order, ap.test_serial_reference_of_proposition_c1),
    (_ao_eos_truncates_by_rank, ap.test_worked_example_order_end_and_retention),
    (_ao_keeps_beyond_end, ap.test_worked_example_order_end_and_retention),
], ids=["ignores-order", "eos-by-rank", "keeps-beyond-end"])
def test_any_order_pin_catches_planted_mistake(monkeypatch, fn, pin):
    monkeypatch.setattr(oracle, "verify_greedy_any_order", fn)
    with pytest.raises(AssertionError):
        pin()


# ------------------------------------------------ joint-space chain (SPOT) ---

import tests.test_oracle_spot_pins as sp  # noqa: E402
import oracle.spot as spot  # noqa: E402

_rs_link = spot.rs_link
_rs_residual = spot.rs_residual
_verify_spot = spot.verify_spot_chain


def _sp_residual_unscaled(p, qhat, c):
    return _rs_residual(p, qhat, 1.0)


def _sp_link_ignores_position(u, p, qhat, c, on_star, tok):
    return _rs_link(u, p, qhat, c, True, tok)


def _sp_link_unscaled(u, p, qhat, c, on_star, tok):
    return _rs_link(u, p, qhat, 1.0, on_star, tok)


@pytest.mark.parametrize("name,fn,pin", [
    ("rs_residual", _sp_residual_unscaled, sp.test_worked_example_by_hand),
    ("rs_residual", _sp_residual_unscaled, lambda: sp.test_joint_space_commit_law_and_acceptance(52)),
    ("rs_link", _sp_link_ignores_position, sp.test_worked_example_by_hand),
    ("rs_link", _sp_link_ignores_position, lambda: sp.test_joint_space_commit_law_and_acceptance(52)),
    ("rs_link", _sp_link_unscaled, lambda: sp.test_joint_space_commit_law_and_acceptance(53)),
], ids=["residual-unscaled-hand", "residual-unscaled-law", "ignores-position-hand", "ignores-position-law",
        "ratio-unscaled-law"])
def test_spot_pin_catches_planted_mistake(monkeypatch, name, fn, pin):
    monkeypatch.setattr(spot, name, fn)
    with pytest.raises(AssertionError):
        pin()


def test_spot_pin_catches_wrong_gate(monkeypatch):
    def gate_mirrored(*a, tau=0.6, **k):
        return _verify_spot(*a, tau=1.0 - tau, **k)
    monkeypatch.setattr(oracle, "verify_spot_chain", gate_mirrored)
    with pytest.raises(AssertionError):
        sp.test_gate_picks_the_verifier()


# ------------------------------------------------------- sparse stored Q ---

import tests.test_oracle_sparse_pins as zp  # noqa: E402
import oracle.sparse as sparse  # noqa: E402

_dense_q = sparse.dense_q
_residual = sparse.residual_weights


def _sq_drops_last(idx, prob, nnz, V):
    return _dense_q(idx, prob, max(int(nnz) - 1, 0), V)


def _sq_residual_on_support_only(p, q, lam=0.0):
    r = _residual(p, q, lam)
    return np.where(np.asarray(q) > 0, r, 0.0)


@pytest.mark.parametrize("name,fn,pin", [
    ("dense_q", _sq_drops_last, zp.test_worked_example_by_hand),
    ("residual_weights", _sq_residual_on_support_only, lambda: zp.test_truncated_drafter_law_and_acceptance(3)),
], ids=["drops-last-entry", "residual-on-support"])
def test_sparse_pin_catches_planted_mistake(monkeypatch, name, fn, pin):
    monkeypatch.setattr(sparse, name, fn)
    with pytest.raises(AssertionError):
        pin()


# ------------------------------------------------- top-k / top-p storage ---

import tests.test_oracle_truncate_pins as tq  # noqa: E402
import oracle.truncate as truncate  # noqa: E402

_truncate_row = truncate.truncate_row


def _tq_ties_high(x, temperature, top_k, top_p):
    x = np.asarray(x, np.float64)
    rev = x[::-1]
    idx, prob = _truncate_row(rev, temperature, top_k, top_p)
    return (x.size - 1 - idx), prob


def _tq_p_exclusive(x, temperature, top_k, top_p):
    idx, prob = _truncate_row(x, temperature, top_k, top_p)
    if top_p < 1.0 and idx.size > 1:
        idx, prob = idx[:-1], prob[:-1] / prob[:-1].sum()
    return idx, prob


def _tq_p_on_full_law(x, temperature, top_k, top_p):
    x = np.asarray(x, np.float64)
    idx, _ = _truncate_row(x, temperature, top_k, 1.0)
    q = oracle.tempered_softmax(x, temperature)
    run, keep = 0.0, idx.size
    for i, v in enumerate(idx):
        run += q[v]
        if run >= top_p:
            keep = i + 1
            break
    kept = idx[:keep]
    return kept, q[kept] / q[kept].sum()


@pytest.mark.parametrize("fn,pin", [
    (_tq_ties_high, lambda: tq.test_kept_set_order_minimality_and_ratios(82)),
    (_tq_p_exclusive, tq.test_worked_example_by_hand),
    (_tq_p_on_full_law, lambda: tq.test_kept_set_order_minimality_and_ratios(83)),
], ids=["ties-to-higher-id", "top-p-one-short", "top-p-on-full-law"])
def test_truncate_pin_catches_planted_mistake(monkeypatch, fn, pin):
    monkeypatch.setattr(oracle, "truncate_row", fn)
    with pytest.raises(AssertionError):
        pin()


# ------------------------------------------------------------------ DDTree

import oracle.ddtree as ddtree  # noqa: E402
import tests.test_oracle_ddtree_pins as dp  # noqa: E402

_DD_HYPOTHESES = ddtree.hypotheses


def _dd_fill_by_level(masked, hyps, order_fn, D, tau=1.0, gamma=0.0, b=0):
    """Fills the remaining budget from each new level, never displacing."""
    srch = ddtree._Search(masked, hyps, order_fn, b, tau, gamma)
    tree, frontier, levels = [], [((), 1.0)], 0
    while frontier and len(tree) < D:
        cand = []
        for p, m in frontier:
            cand.extend(srch.children(p, m))
        levels += 1
        cand.sort(key=lambda e: ddtree.rank_key(e[1], e[0]))
        frontier = cand[:D - len(tree)]
        tree = sorted(tree + frontier, key=lambda e: ddtree.rank_key(e[1], e[0]))
    return tree, srch.status, levels


def _dd_order_unrestricted(logits, masked_positions, tau):
    z = np.asarray(logits, np.float64) / tau
    w = np.exp(z - z.max())
    q = w / w.sum()
    out = np.zeros(z.size)
    ms = list(masked_positions)
    out[ms] = q[ms]
    return out


def _dd_runner_up_inverted(row, temperature, gumbel_row=None, runner_up_below=0.6):
    x = np.asarray(row, np.float64)
    p = ddtree.stale_softmax(x)
    if temperature == 0.0:
        v0 = rows.argmax_lowest(x)
        hyp = [(v0, float(p[v0]))]
        if p[v0] > runner_up_below and x.size > 1:
            rest = x.copy()
            rest[v0] = -np.inf
            v1 = rows.argmax_lowest(rest)
            hyp.append((v1, float(p[v1])))
        return dict(hyp=hyp, top1_margin=0.0, pick_margin=np.inf)
    return _DD_HYPOTHESES(row, temperature, gumbel_row, runner_up_below)


def _dd_gumbel_tempered_mass(row, temperature, gumbel_row=None, runner_up_below=0.6):
    x = np.asarray(row, np.float64)
    if temperature == 0.0:
        return _DD_HYPOTHESES(row, temperature, gumbel_row, runner_up_below)
    a = x / temperature
    p = np.exp(a - a.max())
    p /= p.sum()
    v = rows.argmax_lowest(np.log(p) + np.asarray(gumbel_row, np.float64))
    return dict(hyp=[(v, float(p[v]))], top1_margin=np.inf, pick_margin=np.inf)


@pytest.mark.parametrize("name,fn,pin", [
    ("level_batched", _dd_fill_by_level, dp.test_hand_worked_tree),
    ("order_distribution", _dd_order_unrestricted, lambda: dp.test_best_first_is_the_top_d_of_all_states(0)),
    ("hypotheses", _dd_runner_up_inverted, dp.test_greedy_hypotheses_runner_up_below_threshold),
    ("hypotheses", _dd_gumbel_tempered_mass, dp.test_gumbel_hypothesis),
])
def test_ddtree_pin_catches_planted_mistake(monkeypatch, name, fn, pin):
    monkeypatch.setattr(ddtree, name, fn)
    with pytest.raises(AssertionError):
        pin()


# ------------------------------------------------------------- Packed-SS loop

import oracle.loop as loopmod  # noqa: E402
import tests.test_oracle_loop_pins as lpins  # noqa: E402

_VERIFY_GREEDY = loopmod.verify_greedy


def _retain_from_a(tgt, d, n, rows, eos_id=-1, budget=None):
    """Keeps (z_A, ..., z_W) as the next draft: one position too early."""
    o = _VERIFY_GREEDY(tgt, d, n, rows, eos_id, budget)
    zs = np.asarray(rows).argmax(-1)
    for b in range(len(o["num_out"])):
        a = int(o["num_out"][b])
        if a >= 1:
            keep = zs[b, a - 1:]
            o["next_draft"][b] = -1
            o["next_draft"][b, :len(keep) - 1] = keep[:-1]
    return o


def _bonus_dropped(tgt, d, n, rows, eos_id=-1, budget=None):
    o = _VERIFY_GREEDY(tgt, d, n, rows, eos_id, budget)
    for b in range(len(o["num_out"])):
        if o["accept_len"][b] >= 1 and o["num_out"][b] == o["accept_len"][b] + 1:
            o["num_out"][b] -= 1
            o["out_tokens"][b, o["num_out"][b]] = -1
    return o


@pytest.mark.parametrize("fn,pin", [
    (_retain_from_a, lpins.test_perfect_drafter_alternates),
    (_bonus_dropped, lpins.test_perfect_drafter_alternates),
])
def test_loop_pin_catches_planted_mistake(monkeypatch, fn, pin):
    monkeypatch.setattr(loopmod, "verify_greedy", fn)
    with pytest.raises(AssertionError):
        pin()
