"""The per-call options of the C ABI on the GPU: per-decision margins
against the oracle's margins, the timing events, launch geometry
(max_groups) that leaves every integer output unchanged, the per-row total
variation TV(p_i, q_i) (dense, stored sparse Q and the joint-space chain,
including rows where one token holds nearly all of both rows' mass) against
the oracle's float64 TV, and the tree verifier's position and token margins
against the oracle's."""

import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as dbv
import oracle
import workloads
from tests.parity import PROB_RTOL, check_sampling, np64, npi

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _chain(seed, B, K, V, dtype, sigma):
    g = torch.Generator().manual_seed(seed)
    tgt = (torch.randn(B, K + 1, V, generator=g) * 3).to(dtype)
    drf = (tgt[:, :K].float() + sigma * torch.randn(B, K, V, generator=g)).to(dtype)
    q = torch.softmax(drf.float(), -1)
    d = torch.multinomial(q.reshape(-1, V), 1, generator=g).reshape(B, K).to(torch.int32)
    n = torch.randint(0, K + 1, (B,), generator=g).to(torch.int32)
    ua = torch.rand(B, K, generator=g)
    ur = torch.rand(B, K + 1, generator=g)
    return dict(tgt=tgt, drf=drf, draft_tokens=d, draft_len=n, u_accept=ua, u_resample=ur)


def _np(x):
    return {k: np64(v) if v.dtype.is_floating_point else npi(v) for k, v in x.items()}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_chain_margins(dev, dtype, lam):
    """accept_margin = |u - alpha| and draw_margin = the distance of u*Z from
    the drawn token's interval ends over Z, against the oracle's float64
    margins of the same decisions."""
    say("chain margins", dtype, lam)
    x = _chain(11 + int(lam * 10), 12, 9, 5003, dtype, 0.7)
    xd = {k: v.to(dev) for k, v in x.items()}
    r = dbv.verify_lenient(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"], lam,
                           draft_len=xd["draft_len"], margins=True)
    xn = _np(x)
    o = oracle.verify_lenient(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 1.0, lam,
                              xn["u_accept"], xn["u_resample"])
    rtol = PROB_RTOL[str(dtype).split(".")[-1]]
    check_sampling(r, xn, o, lam, 1.0, 1.0, str(dtype).split(".")[-1])
    am, dm = npi(r["accept_len"]), np64(r["draw_margin"])
    acm = np64(r["accept_margin"])
    B, K = x["draft_tokens"].shape
    for b in range(B):
        n = int(x["draft_len"][b])
        for i in range(K):
            if i < n:
                # |u - alpha| with alpha within rtol (relative) of the oracle's
                assert abs(acm[b, i] - o["accept_margin"][b, i]) <= rtol * max(o["alpha"][b, i], 1e-30) + 1e-7, \
                    (b, i, acm[b, i], o["accept_margin"][b, i])
            else:
                assert acm[b, i] == 0.0
        h = int(am[b])
        if int(npi(r["out_tokens"])[b, h]) != int(o["out_tokens"][b, h]):
            continue   # a near-margin draw (bracket-checked above)
        # The oracle's margin of the token drawn at row h.
        p = oracle.tempered_softmax(xn["tgt"][b, h], 1.0)
        w = oracle.residual_weights(p, oracle.tempered_softmax(xn["drf"][b, h], 1.0), lam) if h < n else p
        if np.sum(w) <= 0:
            w = p
        _, m_o, _ = oracle.inverse_cdf(w, float(xn["u_resample"][b, h]))
        assert 0.0 <= dm[b] <= 0.5 + 1e-6
        assert abs(dm[b] - m_o) <= max(rtol, 1e-5), (b, dm[b], m_o)


def test_chain_margins_errors_and_match_links(dev):
    """A sequence in error reports draw_margin 1 and accept margins 0; a
    coupled-noise match link reports accept margin 1."""
    say("margins: errors and match links")
    x = _chain(5, 4, 6, 777, torch.float32, 0.5)
    x["draft_tokens"][1, 0] = 777          # out of range: bad input
    x["draft_len"][1] = 6
    xd = {k: v.to(dev) for k, v in x.items()}
    r = dbv.verify_rejection(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"],
                             draft_len=xd["draft_len"], margins=True)
    assert int(r["status"][1]) & dbv.SEQ_BAD_INPUT
    assert float(r["draw_margin"][1]) == 1.0
    assert (r["accept_margin"][1] == 0).all()
    # joint-space chain with every link gated to match (tau = 0)
    s = workloads.spot_chain_inputs(41, 4, 5, 997, torch.float32)
    sd = {k: v.to(dev) if torch.is_tensor(v) else v for k, v in s.items()}
    g = dbv.verify_spot_chain(sd["tgt"], sd["drf"], sd["pos_star"], sd["prop_pos"], sd["prop_tok"],
                              sd["q_pos_star"], sd["u_accept"], sd["u_resample"], gumbel=sd["gumbel"], tau=0.0,
                              draft_len=sd["draft_len"], margins=True)
    n = npi(s["draft_len"])
    acm = np64(g["accept_margin"])
    for b in range(4):
        assert (acm[b, :n[b]] == 1.0).all() and (acm[b, n[b]:] == 0.0).all()
    # every commit is a Gumbel argmax: nothing was drawn
    assert (np64(g["draw_margin"]) == 1.0).all()


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_launch_geometry_leaves_outputs_unchanged(dev, name):
    """The same call with the row kernel on 1024, 256, 97 and 13 groups:
    every integer output is identical, and the probabilities agree to float32
    rounding.  (Different splits group the float32 reductions differently;
    only a decision within 1e-5 of its threshold could move, and the oracle
    shows none here.)"""
    say("launch geometry", name)
    x = workloads.config2() if name == "c2" else workloads.config3(1.0, 1.0)
    xd = {k: v.to(dev) if torch.is_tensor(v) else v for k, v in x.items()}
    call = dbv.verify_lenient(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"], 0.5,
                              draft_len=xd["draft_len"], prepare=True)
    base = {k: v.clone() for k, v in call().items()}
    for groups in (256, 97, 13):
        r = call.with_options(max_groups=groups)()
        for k in ("accept_len", "out_tokens", "num_out", "status"):
            assert torch.equal(r[k], base[k]), (groups, k)
        for k in ("p_draft", "q_draft", "alpha", "residual_mass"):
            torch.testing.assert_close(r[k], base[k], rtol=2e-5, atol=1e-9)
    # the decisions really are away from their thresholds
    xn = _np({k: v for k, v in x.items() if torch.is_tensor(v)})
    sl = slice(0, 8)
    o = oracle.verify_lenient(xn["tgt"][sl], xn["drf"][sl], xn["draft_tokens"][sl], xn["draft_len"][sl], 1.0, 1.0,
                              0.5, xn["u_accept"][sl], xn["u_resample"][sl])
    near = check_sampling({k: v[sl] for k, v in base.items()}, {k: v[sl] for k, v in xn.items()}, o, 0.5, 1.0, 1.0,
                          "bfloat16")
    assert near["accept_flip"] == 0 and near["draw_flip"] == 0


def test_launch_geometry_tree_and_greedy(dev):
    """The greedy and tree row kernels on fewer groups give the same
    outputs (integer reductions of exact values, and tree confidences whose
    decisions are away from ties)."""
    say("launch geometry: greedy and tree")
    x = workloads.config5()
    K = x["K"]
    p = x["packed"][:16].to(dev)
    call = dbv.verify_greedy(p[:, :K + 1], x["draft_tokens"][:16].to(dev), x["draft_len"][:16].to(dev),
                             p[:, K + 1:], prepare=True)
    base = {k: v.clone() for k, v in call().items()}
    for groups in (300, 31):
        r = call.with_options(max_groups=groups)()
        for k in base:
            assert torch.equal(r[k], base[k]), (groups, k)
    t = workloads.tree_inputs(61, 3, 16, 12, 20011, torch.bfloat16, sigma_node=0.05)
    td = {k: v.to(dev) if torch.is_tensor(v) else v for k, v in t.items()}
    call = dbv.verify_gumbel_tree(td["logits"], td["parent"], td["edge_pos"], td["edge_tok"], masked=td["masked"],
                                  gumbel=td["gumbel"], temperature=1.0, num_states=td["num_states"], prepare=True)
    base = {k: v.clone() for k, v in call().items()}
    for groups in (200, 17):
        r = call.with_options(max_groups=groups)()
        for k in base:
            if k == "sel_conf":
                torch.testing.assert_close(r[k], base[k], rtol=2e-5, atol=0)
            else:
                assert torch.equal(r[k], base[k]), (groups, k)


def test_timing_events_are_per_call(dev):
    """timed() stamps only its own call: a later call without options
    leaves the events as they were."""
    say("timing events")
    x = workloads.config2()
    xd = {k: v.to(dev) if torch.is_tensor(v) else v for k, v in x.items()}
    call = dbv.verify_rejection(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"],
                                draft_len=xd["draft_len"], prepare=True)
    b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.record()
    e.record()
    torch.cuda.synchronize()
    call.timed(b, e)
    torch.cuda.synchronize()
    t1 = b.elapsed_time(e)
    assert 0.0 < t1 < 50.0
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    assert b.elapsed_time(e) == t1


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("sigma,Tt,Td", [(0.7, 1.0, 1.0), (0.01, 1.0, 1.0), (1.5, 0.8, 1.3)])
def test_row_tv(dev, dtype, sigma, Tt, Td):
    """row_tv = TV(p_i, q_i) of every draft row against the oracle's float64
    TV (rows in the cancelling regime included), 0 past n_b; the outputs of
    the call are unchanged by the diagnostic."""
    say("row tv", dtype, sigma, Tt, Td)
    x = _chain(31 + int(sigma * 10), 10, 7, 4099, dtype, sigma)
    xd = {k: v.to(dev) for k, v in x.items()}
    args = (xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"], 0.5)
    kw = dict(draft_len=xd["draft_len"], temperature_target=Tt, temperature_draft=Td)
    r = dbv.verify_lenient(*args, row_tv=True, **kw)
    r0 = dbv.verify_lenient(*args, **kw)
    for k in r0:
        assert torch.equal(r[k], r0[k]), k
    xn = _np(x)
    tv = np64(r["row_tv"])
    rtol = PROB_RTOL[str(dtype).split(".")[-1]]
    B, K = x["draft_tokens"].shape
    for b in range(B):
        n = int(x["draft_len"][b])
        for i in range(K):
            if i >= n:
                assert tv[b, i] == 0.0
                continue
            p = oracle.tempered_softmax(xn["tgt"][b, i], Tt)
            q = oracle.tempered_softmax(xn["drf"][b, i], Td)
            t = oracle.total_variation(p, q)
            assert abs(tv[b, i] - t) <= rtol * t + 2.0 ** -24, (b, i, tv[b, i], t)


def test_row_tv_sparse_and_joint_space(dev):
    """Stored sparse Q: TV(p, Q) from the stored entries; joint-space chain:
    TV of the token rows p and qhat."""
    say("row tv sparse / joint space")
    x = workloads.sparse_inputs(91, 6, 5, 3001, torch.float32)
    xd = {k: v.to(dev) if torch.is_tensor(v) else v for k, v in x.items()}
    r = dbv.verify_sparse(xd["tgt"], xd["q_idx"], xd["q_prob"], xd["q_nnz"], xd["draft_tokens"], xd["u_accept"],
                          xd["u_resample"], draft_len=xd["draft_len"], row_tv=True)
    tv = np64(r["row_tv"])
    qi, qp, qn = npi(x["q_idx"]), np64(x["q_prob"]), npi(x["q_nnz"])
    for b in range(6):
        for i in range(5):
            if i >= int(x["draft_len"][b]):
                assert tv[b, i] == 0.0
                continue
            p = oracle.tempered_softmax(np64(x["tgt"][b, i]), 1.0)
            t = oracle.total_variation(p, oracle.dense_q(qi[b, i], qp[b, i], qn[b, i], 3001))
            assert abs(tv[b, i] - t) <= 1e-5 * t + 2.0 ** -24, (b, i, tv[b, i], t)
    s = workloads.spot_chain_inputs(92, 5, 4, 2003, torch.float32, random_lengths=True)
    sd = {k: v.to(dev) if torch.is_tensor(v) else v for k, v in s.items()}
    g = dbv.verify_spot_chain(sd["tgt"], sd["drf"], sd["pos_star"], sd["prop_pos"], sd["prop_tok"],
                              sd["q_pos_star"], sd["u_accept"], sd["u_resample"], gumbel=sd["gumbel"], tau=0.6,
                              draft_len=sd["draft_len"], row_tv=True)
    tv = np64(g["row_tv"])
    for b in range(5):
        for i in range(4):
            if i >= int(s["draft_len"][b]):
                assert tv[b, i] == 0.0
                continue
            p = oracle.tempered_softmax(np64(s["tgt"][b, i]), 1.0)
            q = oracle.tempered_softmax(np64(s["drf"][b, i]), 1.0)
            t = oracle.total_variation(p, q)
            assert abs(tv[b, i] - t) <= 1e-5 * t + 2.0 ** -24, (b, i, tv[b, i], t)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_tree_margins(dev, T):
    """pos_margin (relative gap of the two best confidences) and tok_margin
    (gap of the two best scores at s*) against the oracle's margins; the
    outputs of the call are unchanged by them."""
    say("tree margins", T)
    t = workloads.tree_inputs(71, 4, 24, 12, 30011, torch.float32, sigma_node=0.05, temperature=max(T, 1.0))
    td = {k: v.to(dev) if torch.is_tensor(v) else v for k, v in t.items()}
    kw = dict(masked=td["masked"], gumbel=td["gumbel"] if T > 0 else None, temperature=T,
              num_states=td["num_states"])
    r = dbv.verify_gumbel_tree(td["logits"], td["parent"], td["edge_pos"], td["edge_tok"], margins=True, **kw)
    r0 = dbv.verify_gumbel_tree(td["logits"], td["parent"], td["edge_pos"], td["edge_tok"], **kw)
    for k in r0:
        assert torch.equal(r[k], r0[k]), k
    tn = {k: (np64(v) if v.dtype.is_floating_point else npi(v)) if torch.is_tensor(v) else v for k, v in t.items()}
    o = oracle.verify_gumbel_tree(tn["logits"], t["masked"].numpy(), tn["parent"], tn["edge_pos"], tn["edge_tok"],
                                  tn["num_states"], tn["gumbel"] if T > 0 else None, T)
    pm, tm = np64(r["pos_margin"]), np64(r["tok_margin"])
    B, S = pm.shape
    for b in range(B):
        ns = int(t["num_states"][b])
        for y in range(S):
            if y >= ns or o["sel_pos"][b, y] < 0:
                assert pm[b, y] == 0.0 and tm[b, y] == 0.0
                continue
            om = o["pos_margin"][b, y]
            assert (pm[b, y] == 1.0) if not np.isfinite(om) else abs(pm[b, y] - om) <= 1e-5, (b, y, pm[b, y], om)
            if T > 0:
                assert abs(tm[b, y] - o["tok_margin"][b, y]) <= 1e-4 * max(1.0, o["tok_margin"][b, y]), (b, y)
            else:
                xs = tn["logits"][b, y, int(o["sel_pos"][b, y])]
                top = np.sort(xs)
                assert tm[b, y] == pytest.approx(top[-1] - top[-2], abs=1e-6)
