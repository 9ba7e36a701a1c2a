"""Parity checks of GPU outputs against the float64 oracle.

Integer outputs must agree exactly, except at a decision whose margin in the
oracle is below NEAR_MARGIN: there the GPU's choice must pass the bracket
check (it is a choice the oracle would make if the threshold moved by at most
NEAR_MARGIN), and everything downstream is recomputed from the GPU's choice
and compared exactly.  Near-margin decisions are counted and returned.
Probabilities agree within a relative tolerance fixed by the input precision.
"""

from collections import Counter

import numpy as np

import oracle
from oracle import NEAR_MARGIN

# Relative tolerance of probabilities (p(d), q(d), alpha, conf, Z): float32
# arithmetic on exact float32 inputs stays within ~2e-6; bf16 inputs are
# exact in float32 as well, the looser bound covers the exp2 / summation
# error of long rows.
PROB_RTOL = {"float32": 1e-5, "bfloat16": 2e-3}


# Near-margin counts per workload and decision kind, gathered over a test
# session (written out by tests/conftest.py when DBV_PARITY_REPORT names a
# file).
REPORT = {}


def record(config, counts):
    """Add one checker's counts (a Counter: "sequences" compared, decisions
    per kind, those whose oracle margin is below NEAR_MARGIN ("_near") and
    those the GPU took the other way ("_flip")) to the session report; keys
    starting with "max_" keep the largest value seen."""
    e = REPORT.setdefault(config, {})
    for k, v in counts.items():
        if k.startswith("max_"):
            e[k] = max(e.get(k, 0.0), float(v))
        else:
            e[k] = e.get(k, 0) + v
    return counts


def _relerr(a, b):
    m = max(abs(a), abs(b))
    return abs(a - b) / m if m > 0 else 0.0


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if hasattr(t, "detach") else np.asarray(t, np.float64)


def npi(t):
    return t.detach().cpu().numpy().astype(np.int64) if hasattr(t, "detach") else np.asarray(t, np.int64)


def _rel_ok(a, b, rtol, atol=1e-30):
    return abs(a - b) <= rtol * max(abs(a), abs(b)) + atol


# Residual mass Z = sum_v [p~_v - q_v]_+ = 1 - sum_v min(p~_v, q_v): the GPU
# forms each term as p (1 - q/p) with log2(q/p) taken from the logits and
# float64 row normalisers, so every term keeps float32 relative precision
# even where p and q nearly cancel.  What remains is the float32 evaluation
# of the two rows' exp2 terms (about one ulp each, independent between the
# rows), which leaves Z off by a fraction of an ulp of the row mass 1: Z is
# held to the probability tolerance relative to itself plus half an ulp of
# 1, the float32 resolution of a probability of order one.
Z_ATOL = 2.0 ** -24


def check_greedy(g, o):
    """Greedy outputs are integer decisions on exact values: all exact."""
    for k in ("status", "accept_len", "num_out", "out_tokens"):
        np.testing.assert_array_equal(npi(g[k]), o[k], err_msg=k)
    if o["next_draft"].shape[1] > 0:
        np.testing.assert_array_equal(npi(g["next_draft"]), o["next_draft"], err_msg="next_draft")
    np.testing.assert_array_equal(npi(g["next_len"]), o["next_len"], err_msg="next_len")


def check_any_order(g, o):
    """Any-order greedy outputs are integer decisions on exact values: all
    exact."""
    for k in ("status", "accept_len", "num_accepted", "acc_pos", "acc_tok", "new_end", "next_draft"):
        np.testing.assert_array_equal(npi(g[k]), np.asarray(o[k], np.int64), err_msg=k)


def check_sampling(g, x, o, lam, t_target, t_draft, dtype_name, eos_id=-1, len_budget=None,
                   seqs=None, delta=None, qfun=None):
    """Rejection / lenient / Cactus (``delta`` set) outputs against the oracle
    with margin accounting.  ``qfun(b, i)`` gives the drafter distribution
    of row i of sequence b where it is not the softmax of x["drf"] (stored
    sparse Q).

    g: GPU outputs (torch or numpy); x: the inputs as float64 numpy
    (tgt, drf, draft_tokens, draft_len, u_accept, u_resample); o: oracle
    result for the same inputs (possibly for the subset ``seqs``).
    """
    rtol = PROB_RTOL[dtype_name]
    near = Counter()
    st_g = npi(g["status"])
    acc_g = npi(g["accept_len"])
    out_g = npi(g["out_tokens"])
    num_g = npi(g["num_out"])
    pd_g, qd_g, al_g = (np64(g[k]) for k in ("p_draft", "q_draft", "alpha"))
    rm_g = np64(g["residual_mass"])
    B = len(st_g) if seqs is None else len(seqs)
    K = x["tgt"].shape[1] - 1
    for j in range(B):
        b = j if seqs is None else seqs[j]
        so = int(o["status"][j])
        sg = int(st_g[b])
        assert (sg & oracle.STATUS_ERROR_MASK) == (so & oracle.STATUS_ERROR_MASK), (b, sg, so)
        assert (sg & oracle.STATUS_Q_ZERO) == (so & oracle.STATUS_Q_ZERO), (b, sg, so)
        if (sg ^ so) & oracle.STATUS_Z_ZERO:
            near["z_zero_flip"] += 1
        near["sequences"] += 1
        if so & oracle.STATUS_ERROR_MASK:
            assert acc_g[b] == -1 and num_g[b] == 0 and (out_g[b] == -1).all(), b
            continue
        n = int(x["draft_len"][b])
        d = [int(v) for v in x["draft_tokens"][b, :n]]
        for i in range(n):
            assert _rel_ok(pd_g[b, i], o["p_draft"][j, i], rtol), ("p", b, i, pd_g[b, i], o["p_draft"][j, i])
            assert _rel_ok(qd_g[b, i], o["q_draft"][j, i], rtol), ("q", b, i, qd_g[b, i], o["q_draft"][j, i])
            assert _rel_ok(al_g[b, i], o["alpha"][j, i], rtol), ("alpha", b, i)
            near["max_prob_relerr"] = max(near["max_prob_relerr"], _relerr(pd_g[b, i], o["p_draft"][j, i]),
                                          _relerr(qd_g[b, i], o["q_draft"][j, i]),
                                          _relerr(al_g[b, i], o["alpha"][j, i]))
        for i in range(n, K):
            assert pd_g[b, i] == 0 and qd_g[b, i] == 0 and al_g[b, i] == 0
        h = int(acc_g[b])
        assert 0 <= h <= n, (b, h, n)
        for i in range(min(h + 1, n)):   # the tests the GPU decided: accepts i < h, the reject at h
            near["accept_tests"] += 1
            if o["accept_margin"][j, i] < NEAR_MARGIN:
                near["accept_near"] += 1
        for i in range(h):           # GPU accepted draft i
            if not o["accept_bits"][j, i]:
                assert o["accept_margin"][j, i] < NEAR_MARGIN, ("accept", b, i, o["accept_margin"][j, i])
                near["accept_flip"] += 1
        if h < n and o["accept_bits"][j, h]:   # GPU rejected draft h
            assert o["accept_margin"][j, h] < NEAR_MARGIN, ("reject", b, h, o["accept_margin"][j, h])
            near["accept_flip"] += 1
        # The draw at the GPU's row h.
        p = oracle.tempered_softmax(x["tgt"][b, h], t_target)
        if h < n:
            q = qfun(b, h) if qfun is not None else oracle.tempered_softmax(x["drf"][b, h], t_draft)
            if delta is None:
                w = oracle.residual_weights(p, q, lam)
            else:
                w = oracle.cactus_residual(p, q, d[h], oracle.cactus_gamma(p[d[h]], delta))
            Zr = float(np.sum(w))
            if Zr <= 0.0:
                w = p
        else:
            w, Zr = p, 0.0
        u = float(x["u_resample"][b, h])
        c_o, margin, Z = oracle.inverse_cdf(w, u)
        near["draws"] += 1
        near["draw_near"] += int(margin < NEAR_MARGIN)
        near["draw_below_4e-4"] += int(margin < 4e-4)
        if num_g[b] > h:
            c_g = int(out_g[b, h])
            if c_g != c_o:
                F = np.cumsum(w)
                lo = F[c_g - 1] if c_g > 0 else 0.0
                ok = (0 <= c_g < len(w) and w[c_g] > 0 and lo - NEAR_MARGIN * Z <= u * Z < F[c_g] + NEAR_MARGIN * Z)
                assert ok and margin < NEAR_MARGIN, ("draw", b, h, c_g, c_o, margin)
                near["draw_flip"] += 1
        else:
            c_g = c_o
        C = d[:h] + [c_g]
        bud = None if len_budget is None else int(len_budget[b])
        a = oracle.stopping_index(C, h + 1, eos_id, bud)
        assert num_g[b] == a, (b, num_g[b], a)
        exp = np.full(K + 1, -1)
        exp[:a] = C[:a]
        np.testing.assert_array_equal(out_g[b], exp, err_msg=f"out_tokens seq {b}")
        if h < n:
            assert _rel_ok(rm_g[b], Zr, rtol, Z_ATOL), ("Z", b, rm_g[b], Zr)
            near["max_z_relerr"] = max(near["max_z_relerr"], _relerr(rm_g[b], Zr))
        else:
            assert rm_g[b] == 0.0
        if h == o["accept_len"][j] and c_g == c_o:
            near["exact"] += 1
    return near


def check_tree(g, x, o, dtype_name, temperature, seqs=None):
    """Tree outputs against the oracle; near ties in s* or in the Gumbel
    argmax are bracket-checked and the walk is redone with the GPU's
    choices."""
    rtol = PROB_RTOL[dtype_name]
    near = Counter()
    sp_g, stk_g, sc_g = npi(g["sel_pos"]), npi(g["sel_tok"]), np64(g["sel_conf"])
    st_g = npi(g["status"])
    pl_g, pn_g = npi(g["path_len"]), npi(g["path_nodes"])
    cp_g, ct_g, nc_g = npi(g["commit_pos"]), npi(g["commit_tok"]), npi(g["num_commits"])
    B = len(st_g) if seqs is None else len(seqs)
    S = sp_g.shape[1]
    for j in range(B):
        b = j if seqs is None else seqs[j]
        so, sg = int(o["status"][j]), int(st_g[b])
        assert sg == so, (b, sg, so)
        near["sequences"] += 1
        if so & oracle.STATUS_ERROR_MASK:
            assert pl_g[b] == -1 and nc_g[b] == 0
            continue
        ns = S if x.get("num_states") is None else int(x["num_states"][b])
        pos, tok = [], []
        for y in range(ns):
            po, to = int(o["sel_pos"][j, y]), int(o["sel_tok"][j, y])
            pg, tg = int(sp_g[b, y]), int(stk_g[b, y])
            if po >= 0:
                near["states"] += 1
                near["pos_near"] += int(o["pos_margin"][j, y] < NEAR_MARGIN)
            if pg != po:
                assert o["pos_margin"][j, y] < NEAR_MARGIN, ("s*", b, y, pg, po)
                rows = x["logits"][b, y]
                cg = oracle.rows.max_probability(rows[pg])
                assert cg >= o["sel_conf"][j, y] * (1 - NEAR_MARGIN), ("s* bracket", b, y)
                near["pos_flip"] += 1
                t2 = oracle.state_transition(rows, None, None if x.get("gumbel") is None else x["gumbel"][b],
                                             temperature, fixed_pos=pg)
                to = t2["tok"]
                tmargin = t2["tok_margin"]
            else:
                tmargin = o["tok_margin"][j, y]
            if pg >= 0:
                near["tok_near"] += int(tmargin < NEAR_MARGIN)
            if tg != to:
                assert tmargin < NEAR_MARGIN, ("tok", b, y, tg, to, tmargin)
                near["tok_flip"] += 1
            if pg >= 0:
                c_o = oracle.rows.max_probability(x["logits"][b, y, pg])
                assert _rel_ok(sc_g[b, y], c_o, rtol), ("conf", b, y)
                near["max_conf_relerr"] = max(near["max_conf_relerr"], _relerr(sc_g[b, y], c_o))
            pos.append(pg)
            tok.append(tg)
        for y in range(ns, S):
            assert sp_g[b, y] == -1 and stk_g[b, y] == -1
        path, commits = oracle.walk(x["parent"][b], x["edge_pos"][b], x["edge_tok"][b], ns, pos, tok)
        assert pl_g[b] == len(path) - 1, (b, pl_g[b], path)
        exp = np.full(S, -1)
        exp[:len(path)] = path
        np.testing.assert_array_equal(pn_g[b], exp, err_msg=f"path seq {b}")
        assert nc_g[b] == len(commits)
        ep = np.full(S, -1)
        et = np.full(S, -1)
        for k, (s, v) in enumerate(commits):
            ep[k], et[k] = s, v
        np.testing.assert_array_equal(cp_g[b], ep)
        np.testing.assert_array_equal(ct_g[b], et)
        if pl_g[b] == o["path_len"][j]:
            near["exact_path"] += 1
    return near


def check_spot(g, x, o, t_target, t_draft, tau, dtype_name, eos_id=-1, len_budget=None, seqs=None):
    """Joint-space chain outputs (rejection sampling and the gated hybrid)
    against the oracle, with margin accounting as check_sampling.  A link
    whose drafter confidence lies within NEAR_MARGIN of tau may take the
    other verifier on the GPU: such a sequence is counted as near-margin
    ("gate") and its downstream outputs are not compared.

    x: inputs as float64 / int64 numpy (tgt, drf, pos_star, prop_pos,
    prop_tok, q_pos_star, draft_len, u_accept, u_resample, gumbel or None).
    """
    rtol = PROB_RTOL[dtype_name]
    near = Counter()
    st_g, acc_g, out_g, num_g = (npi(g[k]) for k in ("status", "accept_len", "out_tokens", "num_out"))
    pd_g, qd_g, al_g = (np64(g[k]) for k in ("p_draft", "q_draft", "alpha"))
    rm_g = np64(g["residual_mass"])
    B = len(st_g) if seqs is None else len(seqs)
    K = x["tgt"].shape[1] - 1
    G = x.get("gumbel")
    for j in range(B):
        b = j if seqs is None else seqs[j]
        so, sg = int(o["status"][j]), int(st_g[b])
        assert (sg & oracle.STATUS_ERROR_MASK) == (so & oracle.STATUS_ERROR_MASK), (b, sg, so)
        assert (sg & oracle.STATUS_Q_ZERO) == (so & oracle.STATUS_Q_ZERO), (b, sg, so)
        if (sg ^ so) & oracle.STATUS_Z_ZERO:
            near["z_zero_flip"] += 1
        near["sequences"] += 1
        if so & oracle.STATUS_ERROR_MASK:
            assert acc_g[b] == -1 and num_g[b] == 0 and (out_g[b] == -1).all(), b
            continue
        n = int(x["draft_len"][b])
        d = [int(v) for v in x["prop_tok"][b, :n]]
        for i in range(n):
            assert _rel_ok(pd_g[b, i], o["p_draft"][j, i], rtol), ("p", b, i, pd_g[b, i], o["p_draft"][j, i])
            assert _rel_ok(qd_g[b, i], o["q_draft"][j, i], rtol), ("q", b, i, qd_g[b, i], o["q_draft"][j, i])
        for i in range(n, K):
            assert pd_g[b, i] == 0 and qd_g[b, i] == 0 and al_g[b, i] == 0
        h = int(acc_g[b])
        assert 0 <= h <= n, (b, h, n)
        # The gate compares the drafter's float32 confidence 1/S with tau; its
        # error is ~1e-6, so only a gate within NEAR_MARGIN of tau may take
        # the other verifier.  Such a sequence is counted and not compared
        # further (its downstream law differs by construction).
        near["gates"] += min(h + 1, n)
        if (o["gate_margin"][j, :min(h + 1, n)] < NEAR_MARGIN).any():
            near["gate_near"] += 1
            continue
        for i in range(n):
            if o["mode"][j, i] == oracle.MODE_RS:
                assert _rel_ok(al_g[b, i], o["alpha"][j, i], rtol), ("alpha", b, i)
            elif al_g[b, i] != o["alpha"][j, i]:
                assert o["accept_margin"][j, i] < NEAR_MARGIN, ("match alpha", b, i)
        for i in range(min(h + 1, n)):
            near["accept_tests"] += 1
            near["accept_near"] += int(o["accept_margin"][j, i] < NEAR_MARGIN)
        for i in range(h):
            if not o["accept_bits"][j, i]:
                assert o["accept_margin"][j, i] < NEAR_MARGIN, ("accept", b, i, o["accept_margin"][j, i])
                near["accept_flip"] += 1
        if h < n and o["accept_bits"][j, h]:
            assert o["accept_margin"][j, h] < NEAR_MARGIN, ("reject", b, h, o["accept_margin"][j, h])
            near["accept_flip"] += 1
        # The commit at the GPU's row h.
        p = oracle.tempered_softmax(x["tgt"][b, h], t_target)
        Zr = 0.0
        if h < n and o["mode"][j, h] == oracle.MODE_RS or (h == n and G is None):
            if h < n:
                qh = oracle.tempered_softmax(x["drf"][b, h], t_draft)
                w = oracle.rs_residual(p, qh, x["q_pos_star"][b, h])
                Zr = float(np.sum(w))
                if Zr <= 0.0:
                    w = p
            else:
                w = p
            u = float(x["u_resample"][b, h])
            c_o, margin, Z = oracle.inverse_cdf(w, u)
            bracket = lambda c_g: (0 <= c_g < len(w) and w[c_g] > 0 and  # noqa: E731
                                   (np.cumsum(w)[c_g - 1] if c_g > 0 else 0.0) - NEAR_MARGIN * Z <= u * Z
                                   < np.cumsum(w)[c_g] + NEAR_MARGIN * Z)
        else:
            with np.errstate(invalid="ignore"):
                sc = np.asarray(x["tgt"][b, h], np.float64) / t_target + np.asarray(G[b, h], np.float64)
            c_o = oracle.argmax_lowest(sc)
            top = np.sort(sc)
            margin = float(top[-1] - top[-2]) if len(top) > 1 else np.inf
            bracket = lambda c_g: sc[c_g] >= top[-1] - NEAR_MARGIN  # noqa: E731
        near["draws"] += 1
        near["draw_near"] += int(margin < NEAR_MARGIN)
        if num_g[b] > h:
            c_g = int(out_g[b, h])
            if c_g != c_o:
                assert bracket(c_g) and margin < NEAR_MARGIN, ("commit", b, h, c_g, c_o, margin)
                near["draw_flip"] += 1
        else:
            c_g = c_o
        C = d[:h] + [c_g]
        bud = None if len_budget is None else int(len_budget[b])
        a = oracle.stopping_index(C, h + 1, eos_id, bud)
        assert num_g[b] == a, (b, num_g[b], a)
        exp = np.full(K + 1, -1)
        exp[:a] = C[:a]
        np.testing.assert_array_equal(out_g[b], exp, err_msg=f"out_tokens seq {b}")
        assert _rel_ok(rm_g[b], Zr, rtol, Z_ATOL), ("Z", b, rm_g[b], Zr)
        if Zr > 0:
            near["max_z_relerr"] = max(near["max_z_relerr"], _relerr(rm_g[b], Zr))
    return near


# ------------------------------------------------------------------ DDTree --

def check_ddtree_hypotheses(g, o, masked, dtype_name):
    """Hypothesis tokens exactly, their probabilities within PROB_RTOL.  A
    position whose top-1 probability (a float32 1/S, error ~1e-6) lies within
    NEAR_MARGIN of the runner-up threshold (T = 0) may differ in its
    runner-up slot, and one whose two best Gumbel scores lie within
    NEAR_MARGIN may differ in its token; the sequences holding such
    positions are returned (their trees are then built from different
    hypotheses and are not compared)."""
    rtol = PROB_RTOL[dtype_name]
    ht, hp = npi(g["hyp_tok"]), np64(g["hyp_prob"])
    np.testing.assert_array_equal(npi(g["status"]), o["hyp_status"], err_msg="status")
    amb = set()
    B, L = masked.shape
    for b in range(B):
        if o["hyp_status"][b] & oracle.STATUS_ERROR_MASK:
            continue
        for s in range(L):
            if not masked[b, s]:
                assert ht[b, s].tolist() == [-1, -1] and hp[b, s].tolist() == [0.0, 0.0], (b, s)
                continue
            near1 = o["top1_margin"][b, s] < NEAR_MARGIN
            nearg = o["pick_margin"][b, s] < NEAR_MARGIN
            if nearg:
                amb.add(b)
                continue
            assert ht[b, s, 0] == o["hyp_tok"][b, s, 0], (b, s)
            assert _rel_ok(hp[b, s, 0], o["hyp_prob"][b, s, 0], rtol), (b, s, hp[b, s, 0], o["hyp_prob"][b, s, 0])
            if near1 and ht[b, s, 1] != o["hyp_tok"][b, s, 1]:
                # only presence may differ; the runner-up itself is exact
                assert min(ht[b, s, 1], o["hyp_tok"][b, s, 1]) == -1, (b, s)
                amb.add(b)
                continue
            assert ht[b, s, 1] == o["hyp_tok"][b, s, 1], (b, s)
            assert _rel_ok(hp[b, s, 1], o["hyp_prob"][b, s, 1], rtol), (b, s)
    return amb


def ddtree_path_mass(path, masked_row, hyp, order_fn, b, tau):
    """Prefix mass (SPOT Eq. 3) of a path of (position, token) edges, from
    the oracle's order distribution and hypotheses (hyp[s] = [(v, p)])."""
    m = 1.0
    prefix = ()
    for s, v in path:
        done = {e[0] for e in prefix}
        ms = [t for t in range(len(masked_row)) if masked_row[t] and t not in done]
        q = oracle.order_distribution(order_fn(b, prefix), ms, tau)
        pv = dict(hyp[s])[v]
        m *= q[s] * pv
        prefix += ((s, v),)
    return m


def check_ddtree_tree(g, b, o, masked_row, hyp, order_fn, D, tau, gamma, dtype_name):
    """The GPU tree of sequence b: a valid tree (parents first, node masks,
    edges on masked positions with hypothesis tokens), masses equal to the
    oracle's prefix mass of each path and non-increasing in node order, and
    the oracle's top-D set except for states whose mass lies within the
    tolerance of the cut (the D-th mass) or of the floor gamma.  Returns the
    number of such near-cut states."""
    rtol = PROB_RTOL[dtype_name]
    n = int(npi(g["num_nodes"])[b])
    par = npi(g["parent"])[b]
    pos = npi(g["edge_pos"])[b]
    tok = npi(g["edge_tok"])[b]
    mass = np64(g["mass"])[b]
    nm = npi(g["node_masked"])[b]
    L = len(masked_row)
    assert 1 <= n <= D + 1
    assert par[0] == -1 and mass[0] == 1.0
    assert nm[0].tolist() == [int(bool(v)) for v in masked_row]
    paths = [()]
    for z in range(1, n):
        y = par[z]
        assert 0 <= y < z, (b, z, y)
        s, v = int(pos[z]), int(tok[z])
        assert nm[y][s] == 1, (b, z)
        exp_mask = nm[y].copy()
        exp_mask[s] = 0
        assert nm[z].tolist() == exp_mask.tolist(), (b, z)
        assert v in dict(hyp[s]), (b, z, s, v)
        paths.append(paths[y] + ((s, v),))
        assert mass[z] <= mass[z - 1] or z == 1, (b, z)
    assert (par[n:] == -1).all() and (nm[n:] == 0).all()
    band = lambda p: rtol * (len(p) + 1)
    for z in range(1, n):
        m = ddtree_path_mass(paths[z], masked_row, hyp, order_fn, b, tau)
        assert _rel_ok(mass[z], m, band(paths[z]), 1e-30), (b, z, mass[z], m)
    chosen = o["chosen"][b]
    omass = dict(chosen)
    theta = chosen[-1][1] if len(chosen) == D and D > 0 else None
    kset, oset = set(paths[1:]), set(omass)
    near = 0
    for p in kset - oset:
        m = ddtree_path_mass(p, masked_row, hyp, order_fn, b, tau)
        ok = (theta is not None and m >= theta * (1 - 2 * band(p))) or abs(m - gamma) <= 2 * band(p) * gamma
        assert ok, (b, "extra state", p, m, theta)
        near += 1
    for p in oset - kset:
        m = omass[p]
        ok = (theta is not None and m <= theta * (1 + 2 * band(p))) or abs(m - gamma) <= 2 * band(p) * gamma
        assert ok, (b, "missing state", p, m, theta)
        near += 1
    if not near:
        assert n - 1 == len(chosen)
    return near
