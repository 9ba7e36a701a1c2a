"""Parity of the DDTree construction path (ddtree_hypotheses, ddtree_build,
ddtree_level through the C ABI) with the float64 oracle: hypotheses at T = 0
and T > 0, the top-D tree under the first-order table and a set-dependent
order model, budgets from 0 to the maximum, the mass floor, error rows, and
the tree handed to the tree verifier."""

import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as dbv
import oracle
import workloads
from tests.parity import (check_ddtree_hypotheses, check_ddtree_tree, check_tree, np64, npi, record)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _hyp_lists(o, b, L):
    return [[(int(o["hyp_tok"][b, s, k]), float(o["hyp_prob"][b, s, k])) for k in range(2)
             if o["hyp_tok"][b, s, k] >= 0] for s in range(L)]


def _set_order(A, Bm):
    A, Bm = np.asarray(A, np.float64), np.asarray(Bm, np.float64)

    def fn(b, path):
        z = A[b].copy()
        for s, _ in path:
            z = z + Bm[b, s]
        return z
    return fn


def _run_build(x, dev, D, tau, gamma, runner_up_below=0.6):
    T = x["temperature"]
    h = dbv.ddtree_hypotheses(x["stale"].to(dev), x["masked"].to(dev), temperature=T,
                              gumbel=None if x["gumbel"] is None else x["gumbel"].to(dev),
                              runner_up_below=runner_up_below)
    st = dbv.ddtree_build(x["masked"].to(dev), h["hyp_tok"], h["hyp_prob"], x["order_table"].to(dev), D,
                          tau=tau, gamma=gamma, status=h["status"].clone())
    torch.cuda.synchronize()
    return h, st


def _oracle(x, order_fn, D, tau, gamma, runner_up_below=0.6):
    G = None if x["gumbel"] is None else np64(x["gumbel"])
    return oracle.build_ddtree(np64(x["stale"]), npi(x["masked"]), order_fn, D, x["temperature"], tau=tau,
                               gamma=gamma, gumbel=G, runner_up_below=runner_up_below)


def _check_all(h, st, o, x, order_fn, D, tau, gamma, dtype_name):
    masked = npi(x["masked"])
    amb = check_ddtree_hypotheses(h, o, masked, dtype_name)
    assert len(amb) <= 1, amb
    near = 0
    B, L = masked.shape
    np.testing.assert_array_equal(npi(st["status"]), o["status"])
    for b in range(B):
        if o["status"][b] & oracle.STATUS_ERROR_MASK:
            assert int(npi(st["num_nodes"])[b]) == 1
            continue
        assert int(npi(st["num_frontier"])[b]) == 0
        if b in amb:
            continue
        near += check_ddtree_tree(st, b, o, masked[b], _hyp_lists(o, b, L), order_fn, D, tau, gamma, dtype_name)
    return near


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T", [0.0, 1.0, 0.6])
def test_hypotheses_parity(dev, dtype, T):
    say("ddtree hypotheses", dtype, T)
    # V = 3001: several stream units per row and a ragged tail
    x = workloads.ddtree_inputs(60 + int(T * 10), 6, 24, 3001, dtype, temperature=T, peak_lo=6.0, peak_hi=20.0)
    h = dbv.ddtree_hypotheses(x["stale"].to(dev), x["masked"].to(dev), temperature=T,
                              gumbel=None if x["gumbel"] is None else x["gumbel"].to(dev))
    torch.cuda.synchronize()
    o = _oracle(x, lambda b, p: np.zeros(24), 0, 1.0, 0.0)
    amb = check_ddtree_hypotheses(h, o, npi(x["masked"]), str(dtype).split(".")[-1])
    assert len(amb) <= 1
    if T == 0.0:
        # both sides of the 0.6 test occur
        two = (npi(h["hyp_tok"])[:, :, 1] >= 0).sum()
        assert 0 < two < npi(x["masked"]).sum()


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_hypotheses_many_rows(dev, T):
    """B*L above the size at which the row stream lists its rows itself:
    the separate plan kernel lists them."""
    say("ddtree hypotheses B=200 L=48", T)
    x = workloads.ddtree_inputs(66, 200, 48, 97, torch.float32, temperature=T, peak_lo=2.0, peak_hi=8.0)
    h = dbv.ddtree_hypotheses(x["stale"].to(dev), x["masked"].to(dev), temperature=T,
                              gumbel=None if x["gumbel"] is None else x["gumbel"].to(dev))
    torch.cuda.synchronize()
    o = _oracle(x, lambda b, p: np.zeros(48), 0, 1.0, 0.0)
    amb = check_ddtree_hypotheses(h, o, npi(x["masked"]), "float32")
    assert len(amb) <= 2


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,D,tau,gamma", [
    (0.0, 8, 1.0, 0.0), (0.0, 20, 0.7, 0.0), (1.0, 12, 1.0, 0.0), (1.0, 64, 1.0, 0.0),
    (0.0, 64, 1.3, 0.01), (1.0, 64, 1.0, 0.02), (1.0, 5, 1.0, 0.05),
])
def test_build_parity(dev, dtype, T, D, tau, gamma):
    say("ddtree build", dtype, T, D, tau, gamma)
    x = workloads.ddtree_inputs(70 + D, 8, 16, 2053, dtype, temperature=T)
    h, st = _run_build(x, dev, D, tau, gamma)
    o = _oracle(x, oracle.table_order(np64(x["order_table"])), D, tau, gamma)
    near = _check_all(h, st, o, x, oracle.table_order(np64(x["order_table"])), D, tau, gamma,
                      str(dtype).split(".")[-1])
    say("near-cut states", near)


def test_build_block_of_64(dev):
    """L = 64 (every bit of the position masks), the largest budget."""
    say("ddtree build L=64 D=64")
    x = workloads.ddtree_inputs(81, 4, 64, 1024, torch.float32, temperature=0.0, masked_min=0.9)
    h, st = _run_build(x, dev, 64, 1.0, 0.0)
    fn = oracle.table_order(np64(x["order_table"]))
    o = _oracle(x, fn, 64, 1.0, 0.0)
    _check_all(h, st, o, x, fn, 64, 1.0, 0.0, "float32")


def _level_loop(x, dev, D, tau, gamma, h):
    """The search level by level with the set-dependent order model run by
    the caller between levels (torch on the device)."""
    A, Bm = x["order_A"].to(dev), x["order_B"].to(dev)
    m = x["masked"].to(dev)
    root = A[:, None, :].contiguous()
    st = dbv.ddtree_level(m, h["hyp_tok"], h["hyp_prob"], root, D, tau=tau, gamma=gamma,
                          status=h["status"].clone())
    levels = 1
    while True:
        torch.cuda.synchronize()
        nf = npi(st["num_frontier"])
        if nf.max() <= 0:
            break
        fr = st["frontier"].long().clamp(min=0)                                   # [B, D]
        nmask = torch.gather(st["node_masked"], 1, fr[:, :, None].expand(-1, -1, m.shape[1]))
        committed = (m[:, None, :].bool() & ~nmask.bool()).float()               # [B, D, L]
        rows = (A[:, None, :] + torch.bmm(committed, Bm)).contiguous()
        st = dbv.ddtree_level(m, h["hyp_tok"], h["hyp_prob"], rows, D, tau=tau, gamma=gamma, state=st)
        levels += 1
        assert levels <= D + 2
    return st, levels


@pytest.mark.parametrize("T,D", [(0.0, 16), (1.0, 24)])
def test_level_parity_set_order_model(dev, T, D):
    say("ddtree level loop", T, D)
    x = workloads.ddtree_inputs(90 + D, 6, 20, 1999, torch.bfloat16, temperature=T)
    h = dbv.ddtree_hypotheses(x["stale"].to(dev), x["masked"].to(dev), temperature=T,
                              gumbel=None if x["gumbel"] is None else x["gumbel"].to(dev))
    st, levels = _level_loop(x, dev, D, 0.9, 0.0, h)
    fn = _set_order(np64(x["order_A"]), np64(x["order_B"]))
    o = _oracle(x, fn, D, 0.9, 0.0)
    _check_all(h, st, o, x, fn, D, 0.9, 0.0, "bfloat16")
    say("levels", levels)


def test_level_equals_build_on_table(dev):
    """Level-by-level calls fed the table's rows give the one-launch tree
    bit for bit."""
    say("ddtree level == build")
    D, L = 20, 32
    x = workloads.ddtree_inputs(99, 5, L, 4096, torch.bfloat16, temperature=1.0)
    h, bst = _run_build(x, dev, D, 1.0, 0.0)
    tab = x["order_table"].to(dev)
    m = x["masked"].to(dev)
    st = dbv.ddtree_level(m, h["hyp_tok"], h["hyp_prob"], tab[:, L:L + 1, :].contiguous(), D,
                          status=h["status"].clone())
    for _ in range(D + 1):
        torch.cuda.synchronize()
        if npi(st["num_frontier"]).max() <= 0:
            break
        fr = st["frontier"].long().clamp(min=0)
        last = torch.gather(st["edge_pos"], 1, fr).long().clamp(min=0)           # [B, D]
        rows = torch.gather(tab, 1, last[:, :, None].expand(-1, -1, L)).contiguous()
        st = dbv.ddtree_level(m, h["hyp_tok"], h["hyp_prob"], rows, D, state=st)
    torch.cuda.synchronize()
    for k in ("parent", "edge_pos", "edge_tok", "mass", "node_masked", "num_nodes", "num_frontier", "status"):
        assert torch.equal(st[k].cpu(), bst[k].cpu()), k


def test_tree_goes_to_the_verifier(dev):
    """The built tree, with per-state logits from the verifier's forward,
    is what verify_gumbel_tree reads (S = D + 1 states)."""
    say("ddtree -> verify_gumbel_tree")
    D, L, V = 12, 16, 1500
    x = workloads.ddtree_inputs(101, 4, L, V, torch.float32, temperature=1.0)
    h, st = _run_build(x, dev, D, 1.0, 0.0)
    S = D + 1
    g = torch.Generator().manual_seed(7)
    logits = (x["stale"][:, None].float() + 0.3 * torch.randn(4, S, L, V, generator=g)).contiguous()
    out = dbv.verify_gumbel_tree(logits.to(dev), st["parent"], st["edge_pos"], st["edge_tok"],
                                 masked=st["node_masked"], gumbel=x["gumbel"].to(dev), temperature=1.0,
                                 num_states=st["num_nodes"])
    torch.cuda.synchronize()
    xn = dict(logits=np64(logits), masked=npi(st["node_masked"]), parent=npi(st["parent"]),
              edge_pos=npi(st["edge_pos"]), edge_tok=npi(st["edge_tok"]), num_states=npi(st["num_nodes"]),
              gumbel=np64(x["gumbel"]))
    o = oracle.verify_gumbel_tree(xn["logits"], xn["masked"], xn["parent"], xn["edge_pos"], xn["edge_tok"],
                                  xn["num_states"], xn["gumbel"], 1.0)
    check_tree(out, xn, o, "float32", 1.0)
    assert (npi(out["path_len"]) >= 0).all()


def test_edge_cases(dev):
    L, V = 8, 300
    x = workloads.ddtree_inputs(111, 6, L, V, torch.float32, temperature=0.0)
    stale = x["stale"].clone()
    masked = x["masked"].clone()
    masked[0] = 0                     # nothing masked: root alone
    masked[1] = 1
    stale[1, 3, 17] = float("nan")    # a NaN row: error
    masked[2] = 1
    stale[2, 5] = float("-inf")       # an empty row: error
    masked[3] = 1
    stale[3] = float("-inf")          # one-hot rows: p^ = 1, no runner-up
    stale[3, :, 5] = 0.0
    masked[4] = 1
    table = x["order_table"].clone()
    table[4, :, 2] = float("nan")     # an order row with NaN on a masked position: error
    masked[5, :] = 0
    masked[5, 6] = 1                  # one masked position, one-hot row
    stale[5, 6] = float("-inf")
    stale[5, 6, 9] = 1.0
    say("ddtree edge cases")
    x2 = dict(x, stale=stale, masked=masked, order_table=table)
    for D in (0, 1, 7, 64):
        h, st = _run_build(x2, dev, D, 1.0, 0.0)
        fn = oracle.table_order(np64(table))
        o = _oracle(x2, fn, D, 1.0, 0.0)
        _check_all(h, st, o, x2, fn, D, 1.0, 0.0, "float32")
        nn = npi(st["num_nodes"])
        assert nn[0] == 1 and nn[1] == 1 and nn[2] == 1
        assert nn[5] == (2 if D >= 1 else 1)
        if D >= 1:
            assert npi(st["status"])[4] & dbv.SEQ_NONFINITE


def test_floor_above_one_and_zero_budget(dev):
    x = workloads.ddtree_inputs(121, 3, 10, 700, torch.bfloat16, temperature=1.0)
    for D, gamma in ((0, 0.0), (10, 1.5)):
        say("ddtree root only", D, gamma)
        h, st = _run_build(x, dev, D, 1.0, gamma)
        assert (npi(st["num_nodes"]) == 1).all()
        assert (npi(st["parent"])[:, 0] == -1).all()


def test_full_size(dev):
    """The benchmarked configuration: B=16, L=32, V=151936 bf16, T=1, D=20;
    every hypothesis and every one of the 16 trees checked against the
    oracle (a tree is skipped only where a hypothesis decision lies within
    NEAR_MARGIN, and none may be)."""
    say("ddtree full size")
    x = workloads.config4_ddtree()
    h, st = _run_build(x, dev, 20, 1.0, 0.0)
    fn = oracle.table_order(np64(x["order_table"]))
    o = _oracle(x, fn, 20, 1.0, 0.0)
    masked = npi(x["masked"])
    amb = check_ddtree_hypotheses(h, o, masked, "bfloat16")
    assert not amb, amb
    near = _check_all(h, st, o, x, fn, 20, 1.0, 0.0, "bfloat16")
    record("c4d DDTree B=16 L=32 V=151936 bf16 T=1 D=20",
           {"blocks": masked.shape[0], "hypothesis_rows": int(masked.sum()), "trees_skipped": len(amb),
            "near_cut_states": near})
    say("near-cut states", near)
