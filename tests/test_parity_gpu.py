"""Parity of the HIP path (through the C ABI) with the float64 oracle at
sizes the oracle finishes in seconds: several vocabulary chunks, ragged tails,
rows that are not 16-byte aligned, exact ties, every mode and the edge cases.
"""

import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as dbv
import oracle
import workloads
from tests.parity import check_any_order, check_greedy, check_sampling, check_spot, check_tree, np64, npi

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _np_inputs(x):
    return {k: (np64(v) if v.dtype.is_floating_point else npi(v)) if torch.is_tensor(v) else v
            for k, v in x.items()}


def _to(x, dev):
    return {k: v.to(dev) if torch.is_tensor(v) else v for k, v in x.items()}


# ------------------------------------------------------------------ greedy ---

def _tie_logits(g, shape, dtype):
    # small integers: many exact ties between entries of a row
    return torch.randint(-4, 5, shape, generator=g).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V", [20011, 7, 4096])
def test_greedy_parity(dev, dtype, V):
    say("greedy", dtype, V)
    g = torch.Generator().manual_seed(V)
    B, K, W = 6, 7, 9
    tgt = _tie_logits(g, (B, K + 1, V), dtype) if V == 7 else (torch.randn(B, K + 1, V, generator=g) * 3).to(dtype)
    if V == 20011:   # plant exact top-1 ties in some rows
        tgt[0, 0, 5] = tgt[0, 0, 17] = 1000.0
        tgt[1, 2, 19990] = tgt[1, 2, 20005] = 1000.0
    dr = (torch.randn(B, W, V, generator=g) * 3).to(dtype)
    dr[2, 3, 100 % V] = dr[2, 3, 3000 % V] = 99.0
    d = torch.argmax(tgt[:, :K].float() + (torch.rand(B, K, V, generator=g) < 0.0002).float() * 50, -1).to(torch.int32)
    n = torch.tensor([0, 7, 3, 5, 7, 1], dtype=torch.int32)
    res = dbv.verify_greedy(tgt.to(dev), d.to(dev), n.to(dev), dr.to(dev))
    o = oracle.verify_greedy(np64(tgt), npi(d), npi(n), np64(dr))
    check_greedy(res, o)


def test_greedy_stopping_rule(dev):
    say("greedy stopping")
    g = torch.Generator().manual_seed(3)
    B, K, W, V = 8, 6, 6, 3000
    tgt = (torch.randn(B, K + 1, V, generator=g) * 3).to(torch.bfloat16)
    d = torch.argmax(tgt[:, :K].float(), -1).to(torch.int32)   # all drafts match
    d[3, 2] = (d[3, 2] + 1) % V
    eos = int(d[0, 2])
    d[1, 4] = eos
    dr = (torch.randn(B, W, V, generator=g) * 3).to(torch.bfloat16)
    bud = torch.tensor([10, 10, 2, 0, 3, 100, 1, 7], dtype=torch.int32)
    res = dbv.verify_greedy(tgt.to(dev), d.to(dev), None, dr.to(dev), eos_id=eos, len_budget=bud.to(dev))
    o = oracle.verify_greedy(np64(tgt), npi(d), None, np64(dr), eos_id=eos, len_budget=npi(bud))
    check_greedy(res, o)
    assert o["num_out"][0] == 3 and o["num_out"][2] == 2 and o["num_out"][3] == 0


def test_greedy_packed_layout(dev):
    say("greedy packed")
    x = workloads.config5(B=8, K=8, V=5003)
    p = x["packed"].to(dev)
    K, W = x["K"], x["W"]
    res = dbv.verify_greedy(p[:, :K + 1], x["draft_tokens"].to(dev), x["draft_len"].to(dev), p[:, K + 1:])
    o = oracle.verify_greedy(np64(x["packed"][:, :K + 1]), npi(x["draft_tokens"]), npi(x["draft_len"]),
                             np64(x["packed"][:, K + 1:]))
    check_greedy(res, o)
    assert W == K + 1


# ---------------------------------------------------------------- sampling ---

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("V", [20011, 9, 4104])
def test_rejection_parity(dev, dtype, T, V):
    say("rejection", dtype, T, V)
    x = workloads.chain_inputs(90 + V % 7, 6, 7, V, dtype, sigma=1.0, temperature=T, random_lengths=True)
    res = dbv.verify_rejection(x["tgt"].to(dev), x["drf"].to(dev), x["draft_tokens"].to(dev),
                               x["u_accept"].to(dev), x["u_resample"].to(dev),
                               draft_len=x["draft_len"].to(dev), temperature_target=T, temperature_draft=T)
    xn = _np_inputs(x)
    o = oracle.verify_rejection(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], T, T,
                                xn["u_accept"], xn["u_resample"])
    near = check_sampling(res, xn, o, 0.0, T, T, str(dtype).split(".")[1])
    say("near-margin", dict(near))


@pytest.mark.parametrize("lam", [0.0, 0.25, 0.5, 1.0])
@pytest.mark.parametrize("sigma", [0.25, 2.0])
def test_lenient_parity(dev, lam, sigma):
    say("lenient", lam, sigma)
    V = 12345
    x = workloads.chain_inputs(77, 8, 6, V, torch.bfloat16, sigma=sigma, temperature=1.0, random_lengths=True)
    res = dbv.verify_lenient(x["tgt"].to(dev), x["drf"].to(dev), x["draft_tokens"].to(dev),
                             x["u_accept"].to(dev), x["u_resample"].to(dev), lam,
                             draft_len=x["draft_len"].to(dev), temperature_target=1.0, temperature_draft=0.9)
    xn = _np_inputs(x)
    o = oracle.verify_lenient(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 0.9, lam,
                              xn["u_accept"], xn["u_resample"])
    near = check_sampling(res, xn, o, lam, 1.0, 0.9, "bfloat16")
    say("near-margin", dict(near))
    if lam == 1.0:
        np.testing.assert_array_equal(npi(res["accept_len"]), xn["draft_len"])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V", [3001, 32000, 600000])
def test_lenient_full_leniency_zero_residual(dev, dtype, V):
    # lambda = 1 gives p~ = q: a draft with q(d) = 0 is rejected (u q(d) < 0
    # fails) and [p~ - q]_+ is zero everywhere, so the draw falls back to p
    # and flags Z = 0 (Two Tradeoffs, Algorithm 1 with the zero-mass reading).
    # The row sizes take both draw paths: one group per sequence (V = 3001)
    # and the mass / select kernels (V = 32000; V = 600000 puts two or three
    # tiles on each select thread).
    say("lenient lambda=1 zero residual", dtype, V)
    B, K = 4, 5
    x = workloads.chain_inputs(87, B, K, V, dtype, sigma=1.0)
    for b, i in ((0, 0), (1, 2), (2, 4)):
        x["drf"][b, i, int(x["draft_tokens"][b, i])] = float("-inf")
    res = dbv.verify_lenient(x["tgt"].to(dev), x["drf"].to(dev), x["draft_tokens"].to(dev),
                             x["u_accept"].to(dev), x["u_resample"].to(dev), 1.0,
                             draft_len=x["draft_len"].to(dev))
    xn = _np_inputs(x)
    o = oracle.verify_lenient(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 1.0, 1.0,
                              xn["u_accept"], xn["u_resample"])
    assert list(o["accept_len"]) == [0, 2, 4, K]
    assert all(o["status"][:3] & oracle.STATUS_Z_ZERO) and o["status"][3] == 0
    check_sampling(res, xn, o, 1.0, 1.0, 1.0, str(dtype).split(".")[1])
    np.testing.assert_array_equal(npi(res["status"]), o["status"])
    assert (np64(res["residual_mass"]) == 0).all()


def test_max_draft_length_long_rows(dev):
    # K = 1024 with rows long enough for the mass / select draw (20 tiles of
    # 256 fp32): the select group assembles up to 1025 output positions, and
    # an EOS first drafted at position 300 or later stops sequence 0 there.
    say("max draft length, long rows")
    B, K, V = 2, 1024, 5000
    x = workloads.chain_inputs(88, B, K, V, torch.float32, sigma=1.0)
    x["drf"][0] = x["tgt"][0, :K]
    x["draft_tokens"][0] = torch.multinomial(torch.softmax(x["drf"][0], -1), 1,
                                             generator=torch.Generator().manual_seed(6))[:, 0].to(torch.int32)
    d0 = x["draft_tokens"][0].tolist()
    eos = next(t for t in d0[300:] if t not in d0[:300])
    xd = _to(x, dev)
    res = dbv.verify_rejection(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"],
                               draft_len=xd["draft_len"], eos_id=eos)
    xn = _np_inputs(x)
    o = oracle.verify_rejection(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 1.0,
                                xn["u_accept"], xn["u_resample"], eos_id=eos)
    assert o["accept_len"][0] == K and 300 < o["num_out"][0] < K
    check_sampling(res, xn, o, 0.0, 1.0, 1.0, "float32", eos_id=eos)


def test_lenient_zero_is_rejection_bit_for_bit(dev):
    say("lenient 0 == rejection")
    x = _to(workloads.chain_inputs(78, 8, 9, 30011, torch.bfloat16, sigma=1.0, random_lengths=True), dev)
    a = dbv.verify_rejection(x["tgt"], x["drf"], x["draft_tokens"], x["u_accept"], x["u_resample"],
                             draft_len=x["draft_len"])
    b = dbv.verify_lenient(x["tgt"], x["drf"], x["draft_tokens"], x["u_accept"], x["u_resample"], 0.0,
                           draft_len=x["draft_len"])
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_sampling_stopping_rule(dev):
    say("sampling stopping")
    x = workloads.chain_inputs(79, 8, 6, 2000, torch.float32, sigma=0.3)
    eos = int(x["draft_tokens"][0, 1])
    bud = torch.tensor([7, 1, 0, 3, 2, 7, 7, 4], dtype=torch.int32)
    xd = _to(x, dev)
    res = dbv.verify_rejection(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"],
                               eos_id=eos, len_budget=bud.to(dev))
    xn = _np_inputs(x)
    o = oracle.verify_rejection(xn["tgt"], xn["drf"], xn["draft_tokens"], None, 1.0, 1.0,
                                xn["u_accept"], xn["u_resample"], eos_id=eos, len_budget=npi(bud))
    check_sampling(res, xn, o, 0.0, 1.0, 1.0, "float32", eos_id=eos, len_budget=npi(bud))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("delta", [0.0, 0.25, 2.0, 12.0])
def test_cactus_parity(dev, dtype, delta):
    say("cactus", dtype, delta)
    x = workloads.chain_inputs(87, 8, 6, 12345, dtype, sigma=1.5, temperature=1.0, random_lengths=True)
    res = dbv.verify_cactus(x["tgt"].to(dev), x["drf"].to(dev), x["draft_tokens"].to(dev),
                            x["u_accept"].to(dev), x["u_resample"].to(dev), delta,
                            draft_len=x["draft_len"].to(dev), temperature_target=1.0, temperature_draft=0.9)
    xn = _np_inputs(x)
    o = oracle.verify_cactus(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 0.9, delta,
                             xn["u_accept"], xn["u_resample"])
    near = check_sampling(res, xn, o, 0.0, 1.0, 0.9, str(dtype).split(".")[1], delta=delta)
    say("near-margin", dict(near), "h", list(o["accept_len"]))


def test_cactus_zero_budget_is_rejection(dev):
    say("cactus 0 == rejection")
    x = _to(workloads.chain_inputs(88, 8, 9, 30011, torch.bfloat16, sigma=1.0, random_lengths=True), dev)
    a = dbv.verify_rejection(x["tgt"], x["drf"], x["draft_tokens"], x["u_accept"], x["u_resample"],
                             draft_len=x["draft_len"])
    b = dbv.verify_cactus(x["tgt"], x["drf"], x["draft_tokens"], x["u_accept"], x["u_resample"], 0.0,
                          draft_len=x["draft_len"])
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_cactus_edge_cases(dev):
    # p(d) = 0 (its logit is -inf): gamma = 0, always rejected; the stopping
    # rule; a bad draft token; an empty draft.
    say("cactus edge cases")
    B, K, V = 6, 4, 3001
    x = workloads.chain_inputs(89, B, K, V, torch.float32, sigma=1.0)
    tgt, d = x["tgt"].clone(), x["draft_tokens"].clone()
    n = torch.full((B,), K, dtype=torch.int32)
    tgt[0, 0, int(d[0, 0])] = float("-inf")
    d[1, 1] = -3
    n[2] = 0
    eos = int(d[3, 0])
    bud = torch.tensor([9, 9, 9, 9, 2, 0], dtype=torch.int32)
    xd = dict(x, tgt=tgt, draft_tokens=d, draft_len=n)
    res = dbv.verify_cactus(tgt.to(dev), x["drf"].to(dev), d.to(dev), x["u_accept"].to(dev),
                            x["u_resample"].to(dev), 3.0, draft_len=n.to(dev), eos_id=eos, len_budget=bud.to(dev))
    xn = _np_inputs(xd)
    o = oracle.verify_cactus(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 1.0, 3.0,
                             xn["u_accept"], xn["u_resample"], eos_id=eos, len_budget=npi(bud))
    assert o["accept_len"][0] == 0 and o["status"][1] == oracle.STATUS_BAD_INPUT
    check_sampling(res, xn, o, 0.0, 1.0, 1.0, "float32", eos_id=eos, len_budget=npi(bud), delta=3.0)


# --------------------------------------------------------------- sparse Q ---

def _sparse_run(dev, x, eos_id=-1, len_budget=None):
    g = dbv.verify_sparse(x["tgt"].to(dev), x["q_idx"].to(dev), x["q_prob"].to(dev), x["q_nnz"].to(dev),
                          x["draft_tokens"].to(dev), x["u_accept"].to(dev), x["u_resample"].to(dev),
                          draft_len=x["draft_len"].to(dev), temperature_target=x["temperature"], eos_id=eos_id,
                          len_budget=None if len_budget is None else len_budget.to(dev))
    xn = dict(tgt=np64(x["tgt"]), draft_tokens=npi(x["draft_tokens"]), draft_len=npi(x["draft_len"]),
              u_accept=np64(x["u_accept"]), u_resample=np64(x["u_resample"]))
    qi, qp, qn = npi(x["q_idx"]), np64(x["q_prob"]), npi(x["q_nnz"])
    o = oracle.verify_sparse(xn["tgt"], qi, qp, qn, xn["draft_tokens"], xn["draft_len"], x["temperature"],
                             xn["u_accept"], xn["u_resample"], eos_id=eos_id,
                             len_budget=None if len_budget is None else npi(len_budget))
    V = x["tgt"].shape[-1]
    qfun = lambda b, i: oracle.dense_q(qi[b, i], qp[b, i], qn[b, i], V)  # noqa: E731
    return g, xn, o, qfun


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V,topk,peak", [(5003, 20, 12.0), (40000, 7, 20.0), (151936, 256, 20.0)])
def test_sparse_parity(dev, dtype, V, topk, peak):
    say("sparse", dtype, V, topk)
    x = workloads.sparse_inputs(66, 12, 8, V, dtype, topk=topk, peak=peak, random_lengths=True)
    g, xn, o, qfun = _sparse_run(dev, x)
    near = check_sampling(g, xn, o, 0.0, x["temperature"], x["temperature"], str(dtype).split(".")[-1], qfun=qfun)
    say("h", list(o["accept_len"]), "near", dict(near))


def test_sparse_full_support_equals_rejection(dev):
    # every token stored: the dense drafter distribution
    say("sparse = rejection")
    B, K, V = 6, 4, 256
    x = workloads.chain_inputs(67, B, K, V, torch.float32, sigma=1.0, random_lengths=True)
    q = torch.softmax(x["drf"].float(), dim=-1)
    perm = torch.randperm(V, generator=torch.Generator().manual_seed(5))
    sx = dict(tgt=x["tgt"], q_idx=perm.expand(B, K, V).to(torch.int32).clone(),
              q_prob=q[:, :, perm].contiguous(), q_nnz=torch.full((B, K), V, dtype=torch.int32),
              draft_tokens=x["draft_tokens"], u_accept=x["u_accept"], u_resample=x["u_resample"],
              draft_len=x["draft_len"], temperature=1.0)
    g, xn, o, qfun = _sparse_run(dev, sx)
    check_sampling(g, xn, o, 0.0, 1.0, 1.0, "float32", qfun=qfun)
    r = oracle.verify_rejection(np64(x["tgt"]), np64(x["drf"]), npi(x["draft_tokens"]), npi(x["draft_len"]),
                                1.0, 1.0, np64(x["u_accept"]), np64(x["u_resample"]))
    np.testing.assert_array_equal(o["accept_len"], r["accept_len"])


def test_sparse_edge_cases(dev):
    say("sparse edge cases")
    B, K, V = 9, 4, 3001
    x = workloads.sparse_inputs(68, B, K, V, torch.float32, topk=5, kmax=8, peak=12.0)
    x["q_nnz"][0, 1] = 9                     # more entries than kmax
    x["q_idx"][1, 0, 2] = V                  # token out of range
    x["q_prob"][2, 2, 0] = -0.5              # negative probability
    x["q_prob"][3, 0, 4] = float("inf")
    x["q_idx"][4, 3, 6] = -7                 # beyond q_nnz: never read
    x["q_nnz"][5, 0] = 0                     # empty stored Q: d has Q = 0
    x["draft_len"][6] = 0                    # bonus only
    x["draft_len"][7] = 2
    x["q_prob"][7, 3, 0] = float("nan")      # row beyond n: never read
    # the draft token of sequence 8, row 1, is outside its stored support
    x["q_idx"][8, 1, :5] = torch.arange(5, dtype=torch.int32) + int(x["draft_tokens"][8, 1]) + 1
    x["q_idx"][8, 1, :5] %= V
    g, xn, o, qfun = _sparse_run(dev, x)
    assert list(o["status"][:4]) == [1, 1, 1, 1] and o["status"][4] == 0, o["status"]
    check_sampling(g, xn, o, 0.0, 1.0, 1.0, "float32", qfun=qfun)
    eos = int(x["draft_tokens"][4, 0])
    bud = torch.tensor([3, 3, 3, 3, 3, 3, 3, 1, 0], dtype=torch.int32)
    g, xn, o, qfun = _sparse_run(dev, x, eos_id=eos, len_budget=bud)
    check_sampling(g, xn, o, 0.0, 1.0, 1.0, "float32", eos_id=eos, len_budget=npi(bud), qfun=qfun)


# ------------------------------------------------------ top-k / top-p store ---

def _trunc_check(g, rows, T, k, p, kmax, lengths=None, dtype_name="float32"):
    """GPU truncation against the oracle: the same entry count (a top-p cut
    whose running mass lies within the tolerance of p may move by one), the
    same tokens in the same order, probabilities within the tolerance."""
    rtol = PROB_RTOL_T[dtype_name]
    qi, qp, qn = oracle.truncate_rows(rows, T, k, p, kmax, lengths)
    gi, gp, gn = npi(g["q_idx"]), np64(g["q_prob"]), npi(g["q_nnz"])
    B, K, V = rows.shape
    near = 0
    for b in range(B):
        for i in range(K):
            no, ng = int(qn[b, i]), int(gn[b, i])
            if no <= 0:
                assert ng == no, (b, i, ng, no)
                continue
            if ng != no:
                # the top-p cut: the running mass at the shorter count is within tolerance of p
                idx, _ = oracle.truncate_row(rows[b, i], T, k, 1.0)
                a = rows[b, i][idx] / T
                w = np.exp(a - a.max())
                w /= w.sum()
                c = np.cumsum(w)
                assert abs(ng - no) == 1 and abs(c[min(ng, no) - 1] - p) < 10 * rtol, (b, i, ng, no)
                near += 1
            m = min(ng, no)
            np.testing.assert_array_equal(gi[b, i, :m], qi[b, i, :m], err_msg=f"row {b},{i}")
            if ng == no:
                np.testing.assert_allclose(gp[b, i, :m], qp[b, i, :m], rtol=rtol, atol=1e-30)
    return near


PROB_RTOL_T = {"float32": 1e-5, "bfloat16": 1e-5}   # inputs exact in float32 either way


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V,k,p", [(1000, 20, 1.0), (1000, 20, 0.9), (151936, 20, 0.9), (151936, 256, 0.95),
                                   (50257, 1, 1.0), (37, 64, 0.5)])
def test_truncate_parity(dev, dtype, V, k, p):
    say("truncate", dtype, V, k, p)
    g0 = torch.Generator().manual_seed(91)
    rows = (torch.randn(6, 4, V, generator=g0) * 3.0).to(dtype)
    lengths = torch.tensor([4, 0, 2, 4, 1, 3], dtype=torch.int32)
    kmax = max(k, 1) if k <= 256 else 256
    kk = min(k, kmax)
    g = dbv.truncate_top_k_top_p(rows.to(dev), kk, p, kmax=kmax, lengths=lengths.to(dev), temperature=0.8)
    near = _trunc_check(g, np64(rows), 0.8, kk, p, kmax, npi(lengths), str(dtype).split(".")[-1])
    say("near top-p cuts", near)


def test_truncate_ties_and_bad_rows(dev):
    say("truncate ties / bad rows")
    g0 = torch.Generator().manual_seed(92)
    rows = torch.randint(-4, 5, (5, 3, 3001), generator=g0).float()   # many equal logits: id cut-offs
    rows[0, 1, 7] = float("nan")
    rows[1, 0] = float("-inf")                                        # no finite logit
    rows[1, 1, :] = float("-inf")
    rows[1, 1, :5] = 1.0                                               # fewer finite entries than k
    rows[2, 2, 100] = float("inf")
    rows[3, 0, :] = -0.0
    rows[3, 0, 50:60] = 0.0                                            # -0 and +0 tie
    for dtype in (torch.float32, torch.bfloat16):
        for k, p in ((12, 1.0), (12, 0.3), (200, 0.97)):
            x = rows.to(dtype)
            g = dbv.truncate_top_k_top_p(x.to(dev), k, p, kmax=200, temperature=1.3)
            _trunc_check(g, np64(x), 1.3, k, p, 200, None, str(dtype).split(".")[-1])
            assert npi(g["q_nnz"])[0, 1] == -1 and npi(g["q_nnz"])[1, 0] == -1 and npi(g["q_nnz"])[2, 2] == -1


def test_truncate_equal_logits_in_groups(dev):
    # The kernel keeps, per thread, its top logits with the start of the
    # 16-byte group each came from, and counts an entry's occurrence among
    # equal logits of its group after the stream (the entries above it with
    # the same logit and group).  Rows built from a few values repeated inside
    # every group, with the row start both aligned and off by one to six
    # elements (one-element head and tail groups), and k up to 256: token ids
    # must be the oracle's (lowest id first among equal logits).
    say("truncate equal logits inside groups")
    g0 = torch.Generator().manual_seed(95)
    pattern = torch.tensor([5.0, 5.0, 5.0, 3.0, 5.0, 5.0, 1.0, 5.0])
    for dtype in (torch.float32, torch.bfloat16):
        for V in (4099, 20000):
            base = pattern.repeat(V // 8 + 1)[:V]
            rows = torch.stack([base, base.roll(3), torch.where(torch.rand(V, generator=g0) < 0.05, 7.0, 2.0),
                                torch.randint(0, 2, (V,), generator=g0).float() * 4.0])
            for off in (0, 1, 6):
                # a column offset moves the row start off the 16-byte boundary
                big = torch.full((2, 2, V + off), -1.0e4, dtype=dtype)
                big[:, :, off:] = rows.reshape(2, 2, V).to(dtype)
                x = big[:, :, off:]
                xd = big.to(dev)[:, :, off:]      # sliced on the device: rows start off alignment
                for k, p in ((3, 1.0), (20, 0.9), (256, 0.99)):
                    g = dbv.truncate_top_k_top_p(xd, k, p, kmax=256, temperature=1.0)
                    _trunc_check(g, np64(x), 1.0, k, p, 256, None, str(dtype).split(".")[-1])


def test_truncate_flat_rows(dev):
    # More logits at or above the threshold than the LDS candidates hold:
    # a flat row, a row with a few distinct values, and a row with fewer
    # finite logits than k over a large vocabulary.
    say("truncate flat rows")
    g0 = torch.Generator().manual_seed(94)
    V = 20000
    rows = torch.zeros(3, 2, V)
    rows[0, 1] = torch.randint(0, 3, (V,), generator=g0).float()
    rows[1, 0, :] = float("-inf")
    rows[1, 0, torch.randperm(V, generator=g0)[:7]] = torch.randn(7, generator=g0)
    rows[1, 1] = torch.randn(V, generator=g0) * 1e-3
    rows[2, 0] = torch.round(torch.randn(V, generator=g0) * 2) / 2
    for dtype in (torch.float32, torch.bfloat16):
        for k, p in ((16, 1.0), (100, 0.5), (256, 0.99)):
            x = rows.to(dtype)
            g = dbv.truncate_top_k_top_p(x.to(dev), k, p, kmax=256, temperature=0.9)
            _trunc_check(g, np64(x), 0.9, k, p, 256, None, str(dtype).split(".")[-1])


def test_truncate_then_verify_sparse(dev):
    # drafter rows -> stored top-k Q -> verification, against the oracle end to end
    say("truncate -> verify_sparse")
    x = workloads.chain_inputs(93, 8, 6, 5003, torch.bfloat16, sigma=1.0, random_lengths=True)
    st = dbv.truncate_top_k_top_p(x["drf"].to(dev), 20, 0.9, kmax=24, lengths=x["draft_len"].to(dev))
    qi, qp, qn = (npi(st["q_idx"]), np64(st["q_prob"]), npi(st["q_nnz"]))
    # draft tokens: the first stored token of each row (a valid draw from Q)
    d = torch.tensor(qi[:, :, 0], dtype=torch.int32)
    g = dbv.verify_sparse(x["tgt"].to(dev), st["q_idx"], st["q_prob"], st["q_nnz"], d.to(dev),
                          x["u_accept"].to(dev), x["u_resample"].to(dev), draft_len=x["draft_len"].to(dev))
    xn = dict(tgt=np64(x["tgt"]), draft_tokens=npi(d), draft_len=npi(x["draft_len"]),
              u_accept=np64(x["u_accept"]), u_resample=np64(x["u_resample"]))
    o = oracle.verify_sparse(xn["tgt"], qi, qp, qn, xn["draft_tokens"], xn["draft_len"], 1.0, xn["u_accept"],
                             xn["u_resample"])
    check_sampling(g, xn, o, 0.0, 1.0, 1.0, "bfloat16", qfun=lambda b, i: oracle.dense_q(qi[b, i], qp[b, i], qn[b, i], 5003))


# ------------------------------------------------------- joint-space chain ---

def _spot_np(x):
    out = {k: (np64(v) if v.is_floating_point() else npi(v)) if torch.is_tensor(v) else v for k, v in x.items()}
    return out


def _spot_run(dev, x, tau=0.6, gumbel=True, eos_id=-1, len_budget=None):
    G = x["gumbel"] if gumbel else None
    g = dbv.verify_spot_chain(
        x["tgt"].to(dev), x["drf"].to(dev), x["pos_star"].to(dev), x["prop_pos"].to(dev), x["prop_tok"].to(dev),
        x["q_pos_star"].to(dev), x["u_accept"].to(dev), x["u_resample"].to(dev),
        gumbel=None if G is None else G.to(dev), tau=tau, draft_len=x["draft_len"].to(dev),
        temperature_target=x["temperature"], temperature_draft=x["temperature"], eos_id=eos_id,
        len_budget=None if len_budget is None else len_budget.to(dev))
    xn = _spot_np(dict(x, gumbel=G))
    o = oracle.verify_spot_chain(xn["tgt"], xn["drf"], xn["pos_star"], xn["prop_pos"], xn["prop_tok"],
                                 xn["q_pos_star"], xn["draft_len"], x["temperature"], x["temperature"],
                                 xn["u_accept"], xn["u_resample"], gumbel=xn["gumbel"], tau=tau, eos_id=eos_id,
                                 len_budget=None if len_budget is None else npi(len_budget))
    return g, xn, o


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V", [5003, 40000])
@pytest.mark.parametrize("gumbel", [True, False])
def test_spot_chain_parity(dev, dtype, V, gumbel):
    say("spot chain", dtype, V, gumbel)
    x = workloads.spot_chain_inputs(61, 24, 8, V, dtype, temperature=0.9, random_lengths=True, gumbel=gumbel)
    g, xn, o = _spot_run(dev, x, gumbel=gumbel)
    near = check_spot(g, xn, o, 0.9, 0.9, 0.6, str(dtype).split(".")[-1])
    say("h", list(o["accept_len"]), "match links", int(o["mode"].sum()), "near", dict(near))
    if gumbel:
        assert 0 < o["mode"].sum() < o["mode"].size


def test_spot_certain_positions_equal_rejection(dev):
    say("spot = rejection")
    x = workloads.spot_chain_inputs(62, 16, 6, 9001, torch.float32, random_lengths=True, gumbel=False)
    x["prop_pos"] = x["pos_star"][:, :6].clone()
    x["q_pos_star"] = torch.ones(16, 6)
    g, xn, o = _spot_run(dev, x, gumbel=False)
    r = dbv.verify_rejection(x["tgt"].to(dev), x["drf"].to(dev), x["prop_tok"].to(dev), x["u_accept"].to(dev),
                             x["u_resample"].to(dev), draft_len=x["draft_len"].to(dev))
    for k in ("accept_len", "out_tokens", "num_out", "status", "p_draft", "q_draft", "alpha", "residual_mass"):
        assert torch.equal(g[k], r[k]), k
    check_spot(g, xn, o, 1.0, 1.0, 0.6, "float32")


def test_spot_edge_cases(dev):
    say("spot edge cases")
    B, K, V = 10, 5, 3001
    x = workloads.spot_chain_inputs(63, B, K, V, torch.float32)
    x["q_pos_star"][0, 1] = 1.5                 # c outside [0, 1]
    x["q_pos_star"][1, 0] = float("nan")
    x["pos_star"][2, K] = -1                    # bonus row position
    x["pos_star"][3, 2] = -4
    x["prop_tok"][4, 3] = V                     # token out of range
    x["gumbel"][5, 2, 17] = float("nan")        # a Gumbel row that is read
    x["draft_len"][6] = 0                       # bonus only
    x["draft_len"][7] = 2
    x["gumbel"][7, 4, 5] = float("nan")         # beyond n: never read
    x["q_pos_star"][8] = 0.0                    # q = 0 at the proposal
    g, xn, o = _spot_run(dev, x)
    assert list(o["status"][:6]) == [1, 1, 1, 1, 1, 2], o["status"]
    assert o["status"][7] == 0
    check_spot(g, xn, o, 1.0, 1.0, 0.6, "float32")
    for tau in (1.5, 0.0, -1.0):                # no match link / every link matches
        g, xn, o = _spot_run(dev, x, tau=tau)
        check_spot(g, xn, o, 1.0, 1.0, tau, "float32")
    eos = int(x["prop_tok"][9, 0])
    bud = torch.tensor([5, 5, 5, 5, 5, 5, 5, 5, 1, 0], dtype=torch.int32)
    g, xn, o = _spot_run(dev, x, eos_id=eos, len_budget=bud)
    check_spot(g, xn, o, 1.0, 1.0, 0.6, "float32", eos_id=eos, len_budget=npi(bud))
    x0 = workloads.spot_chain_inputs(64, 4, 0, 777, torch.float32)   # K = 0
    for gum in (True, False):
        g, xn, o = _spot_run(dev, x0, gumbel=gum)
        check_spot(g, xn, o, 1.0, 1.0, 0.6, "float32")


# --------------------------------------------------------------- any-order ---

def _ao_run(dev, x, eos_id=-1, end_pos=None, draft_rows=True, positions=True):
    g = dbv.verify_greedy_any_order(
        x["tgt"].to(dev), x["order"].to(dev), x["draft_tokens"].to(dev), num_active=x["num_active"].to(dev),
        positions=x["positions"].to(dev) if positions else None,
        draft_rows=x["draft_rows"].to(dev) if draft_rows else None, eos_id=eos_id,
        end_pos=None if end_pos is None else end_pos.to(dev))
    o = oracle.verify_greedy_any_order(
        np64(x["tgt"]), npi(x["order"]), npi(x["num_active"]), npi(x["positions"]) if positions else None,
        npi(x["draft_tokens"]), np64(x["draft_rows"]) if draft_rows else None, eos_id,
        None if end_pos is None else npi(end_pos))
    return g, o


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("agree", [0.6, 0.95])
def test_any_order_parity(dev, dtype, agree):
    say("any-order", dtype, agree)
    x = workloads.anyorder_inputs(91, 12, 16, 5003, dtype, agree=agree, missing=0.15)
    g, o = _ao_run(dev, x)
    check_any_order(g, o)
    # with an EOS (a token some drafts carry) and an end position
    eos = int(x["draft_tokens"][x["draft_tokens"] >= 0][3])
    end = x["positions"][:, 5].clone()
    g, o = _ao_run(dev, x, eos_id=eos, end_pos=end)
    check_any_order(g, o)
    say("h", list(o["accept_len"]), "kept", list(o["num_accepted"]))


def test_any_order_edge_cases(dev):
    say("any-order edge cases")
    x = workloads.anyorder_inputs(92, 8, 6, 777, torch.float32, missing=0.0, full=True)
    x["tgt"] = torch.randint(-3, 4, x["tgt"].shape, generator=torch.Generator().manual_seed(3)).float()
    # drafts = the verifier argmax (lowest index on ties) so windows fill up
    for b in range(8):
        for r in range(6):
            x["draft_tokens"][b, int(x["order"][b, r])] = int(torch.argmax(x["tgt"][b, r]))
    x["order"][1, 2] = x["order"][1, 3]           # not a permutation
    x["positions"][2, 4] = x["positions"][2, 3]   # positions do not increase
    x["draft_tokens"][3, 0] = -2                  # bad token
    x["num_active"][4] = 0                        # empty window
    x["num_active"][5] = 7                        # more than U
    x["draft_tokens"][6, int(x["order"][6, 0])] = -1   # missing at rank 0: kappa = 0
    g, o = _ao_run(dev, x)
    check_any_order(g, o)
    assert o["accept_len"][0] == 6 and o["num_accepted"][0] == 6          # A = u
    assert list(o["status"][1:4]) == [1, 1, 1] and o["status"][5] == 1
    assert o["num_accepted"][4] == 0 and o["kappa"][6] == 0 and o["num_accepted"][6] == 1
    g, o = _ao_run(dev, x, draft_rows=False, positions=False)
    check_any_order(g, o)
    assert (npi(g["next_draft"]) == -1).all()


# -------------------------------------------------------------- edge cases ---

def test_chain_edge_cases(dev):
    say("chain edge cases")
    B, K, V = 9, 4, 3001
    x = workloads.chain_inputs(80, B, K, V, torch.float32, sigma=1.0)
    tgt, drf, d = x["tgt"].clone(), x["drf"].clone(), x["draft_tokens"].clone()
    n = torch.full((B,), K, dtype=torch.int32)
    d[0, 2] = V                      # out-of-range token
    tgt[1, 3, 77] = float("nan")     # NaN in a row that is read
    tgt[2, 1, :] = float("-inf")     # empty row
    tgt[3, 4, 5] = float("inf")      # +inf in the bonus row
    n[4] = 1
    tgt[4, 3, 9] = float("nan")      # NaN in a row that is not read
    n[5] = K + 1                     # bad draft length (its rows are not read)
    tgt[5, 0, 3] = float("nan")
    drf[6, 0, int(d[6, 0])] = float("-inf")   # q(d) = 0 < p(d): accepted + flagged
    n[7] = 0                         # empty draft: bonus from row 0
    tgt[8, :, : V // 2] = float("-inf")        # half the vocabulary masked out
    drf[8, :, : V // 2] = float("-inf")
    d[8] = torch.argmax(drf[8], -1).to(torch.int32)
    xd = dict(x, tgt=tgt, drf=drf, draft_tokens=d, draft_len=n)
    res = dbv.verify_rejection(tgt.to(dev), drf.to(dev), d.to(dev), x["u_accept"].to(dev),
                               x["u_resample"].to(dev), draft_len=n.to(dev))
    xn = _np_inputs(xd)
    o = oracle.verify_rejection(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 1.0,
                                xn["u_accept"], xn["u_resample"])
    assert list(o["status"][:6]) == [1, 2, 4, 2, 0, 1] and o["status"][6] & oracle.STATUS_Q_ZERO
    check_sampling(res, xn, o, 0.0, 1.0, 1.0, "float32")
    g = dbv.verify_greedy(tgt.to(dev), d.to(dev), n.to(dev), drf.to(dev))
    og = oracle.verify_greedy(xn["tgt"], xn["draft_tokens"], xn["draft_len"], xn["drf"])
    check_greedy(g, og)


@pytest.mark.parametrize("V", [1, 2, 3])
def test_tiny_vocabulary(dev, V):
    say("tiny V", V)
    x = workloads.chain_inputs(81, 5, 3, V, torch.float32, sigma=1.0, random_lengths=True)
    xd = _to(x, dev)
    res = dbv.verify_rejection(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"],
                               draft_len=xd["draft_len"])
    xn = _np_inputs(x)
    o = oracle.verify_rejection(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 1.0,
                                xn["u_accept"], xn["u_resample"])
    check_sampling(res, xn, o, 0.0, 1.0, 1.0, "float32")
    g = dbv.verify_greedy(xd["tgt"], xd["draft_tokens"], xd["draft_len"], xd["drf"])
    check_greedy(g, oracle.verify_greedy(xn["tgt"], xn["draft_tokens"], xn["draft_len"], xn["drf"]))


def test_no_drafts(dev):
    say("K=0, W=0")
    x = workloads.chain_inputs(82, 4, 0, 5000, torch.bfloat16)
    xd = _to(x, dev)
    res = dbv.verify_rejection(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"])
    xn = _np_inputs(x)
    o = oracle.verify_rejection(xn["tgt"], xn["drf"], xn["draft_tokens"], None, 1.0, 1.0,
                                xn["u_accept"], xn["u_resample"])
    check_sampling(res, xn, o, 0.0, 1.0, 1.0, "bfloat16")
    g = dbv.verify_greedy(xd["tgt"], xd["draft_tokens"])
    check_greedy(g, oracle.verify_greedy(xn["tgt"], xn["draft_tokens"]))


def test_determinism(dev):
    say("determinism")
    x = _to(workloads.chain_inputs(83, 16, 8, 32000, torch.bfloat16, random_lengths=True), dev)
    a = dbv.verify_rejection(x["tgt"], x["drf"], x["draft_tokens"], x["u_accept"], x["u_resample"],
                             draft_len=x["draft_len"])
    b = dbv.verify_rejection(x["tgt"], x["drf"], x["draft_tokens"], x["u_accept"], x["u_resample"],
                             draft_len=x["draft_len"])
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_max_draft_length(dev):
    # K = W = 1024, the largest the library takes: 2K+1 rows per sequence are
    # combined by one group.  Sequence 0 drafts from the target itself (q = p,
    # every draft accepted, bonus from row K); sequence 1 drafts with noise.
    say("max draft length")
    B, K, V = 2, 1024, 257
    x = workloads.chain_inputs(84, B, K, V, torch.float32, sigma=1.0)
    x["drf"][0] = x["tgt"][0, :K]
    x["draft_tokens"][0] = torch.multinomial(torch.softmax(x["drf"][0], -1), 1,
                                             generator=torch.Generator().manual_seed(5))[:, 0].to(torch.int32)
    xd = _to(x, dev)
    res = dbv.verify_rejection(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"],
                               draft_len=xd["draft_len"])
    xn = _np_inputs(x)
    o = oracle.verify_rejection(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 1.0,
                                xn["u_accept"], xn["u_resample"])
    assert o["accept_len"][0] == K
    check_sampling(res, xn, o, 0.0, 1.0, 1.0, "float32")
    g = dbv.verify_greedy(xd["tgt"], xd["draft_tokens"], xd["draft_len"], xd["drf"])
    check_greedy(g, oracle.verify_greedy(xn["tgt"], xn["draft_tokens"], xn["draft_len"], xn["drf"]))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_largest_vocabulary(dev, dtype):
    # V = 2^21, the largest the sampling entry points take: the draw's
    # segments are at their longest (8 elements per thread in the rescan).
    say("largest V", dtype)
    V = 1 << 21
    x = workloads.chain_inputs(85, 2, 2, V, dtype, sigma=2.0)
    x["draft_tokens"][1, 0] = (x["draft_tokens"][1, 0] + 7) % V   # a likely reject
    xd = _to(x, dev)
    res = dbv.verify_rejection(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"])
    xn = _np_inputs(x)
    o = oracle.verify_rejection(xn["tgt"], xn["drf"], xn["draft_tokens"], None, 1.0, 1.0,
                                xn["u_accept"], xn["u_resample"])
    near = check_sampling(res, xn, o, 0.0, 1.0, 1.0, str(dtype).split(".")[1])
    say("near-margin", dict(near))


def test_many_sequences(dev):
    # More sequences than one LDS directory entry each (B > 1024): rows are
    # located through blocks of sequences; some lengths are invalid.
    say("many sequences")
    B, K, V = 1500, 2, 200
    x = workloads.chain_inputs(86, B, K, V, torch.bfloat16, sigma=1.0, random_lengths=True)
    x["draft_len"][7] = K + 1
    x["draft_len"][1100] = -1
    xd = _to(x, dev)
    res = dbv.verify_rejection(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"],
                               draft_len=xd["draft_len"])
    xn = _np_inputs(x)
    o = oracle.verify_rejection(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 1.0,
                                xn["u_accept"], xn["u_resample"])
    assert o["status"][7] == oracle.STATUS_BAD_INPUT and o["status"][1100] == oracle.STATUS_BAD_INPUT
    check_sampling(res, xn, o, 0.0, 1.0, 1.0, "bfloat16")
    g = dbv.verify_greedy(xd["tgt"], xd["draft_tokens"], xd["draft_len"], xd["drf"])
    check_greedy(g, oracle.verify_greedy(xn["tgt"], xn["draft_tokens"], xn["draft_len"], xn["drf"]))


# -------------------------------------------------------------------- tree ---

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_tree_parity(dev, dtype, T):
    say("tree", dtype, T)
    x = workloads.tree_inputs(60, 3, 12, 6, 5003, dtype, sigma_node=0.05, temperature=T if T > 0 else 1.0)
    g = dbv.verify_gumbel_tree(x["logits"].to(dev), x["parent"].to(dev), x["edge_pos"].to(dev),
                               x["edge_tok"].to(dev), masked=x["masked"].to(dev),
                               gumbel=x["gumbel"].to(dev) if T > 0 else None, temperature=T,
                               num_states=x["num_states"].to(dev))
    xn = _np_inputs(x)
    xn["masked"] = x["masked"].numpy()
    o = oracle.verify_gumbel_tree(xn["logits"], xn["masked"], xn["parent"], xn["edge_pos"], xn["edge_tok"],
                                  xn["num_states"], xn["gumbel"], T)
    near = check_tree(g, xn, o, str(dtype).split(".")[1], T)
    say("near", dict(near), "path_len", list(o["path_len"]))


@pytest.mark.parametrize("B,S,L", [(33, 64, 64), (70, 64, 64), (4, 128, 80), (3, 200, 48)])
def test_tree_many_rows(dev, B, S, L):
    """The listing and batching paths by tree size: B*S*L = 135168 row ids
    (listing by 132 groups) and 286720 (more than 2^18: one group in
    passes); S = 128 (the most states batched by s*, positions up to 80) and
    S = 200 (one state per batch)."""
    say("tree many rows B", B, "S", S, "L", L, "V 7")
    x = workloads.tree_inputs(77 + B, B, S, L, 7, torch.bfloat16, sigma_node=0.5, temperature=1.0)
    g = dbv.verify_gumbel_tree(x["logits"].to(dev), x["parent"].to(dev), x["edge_pos"].to(dev),
                               x["edge_tok"].to(dev), masked=x["masked"].to(dev), gumbel=x["gumbel"].to(dev),
                               temperature=1.0, num_states=x["num_states"].to(dev))
    xn = _np_inputs(x)
    xn["masked"] = x["masked"].numpy()
    o = oracle.verify_gumbel_tree(xn["logits"], xn["masked"], xn["parent"], xn["edge_pos"], xn["edge_tok"],
                                  xn["num_states"], xn["gumbel"], 1.0)
    near = check_tree(g, xn, o, "bfloat16", 1.0)
    say("near", dict(near))


def test_tree_fixed_position(dev):
    say("tree fixed position")
    x = workloads.tree_inputs(61, 2, 10, 5, 4001, torch.bfloat16, sigma_node=0.05)
    g = torch.Generator().manual_seed(5)
    nxt = torch.randint(-1, 5, (2, 10), generator=g).to(torch.int32)
    r = dbv.verify_gumbel_tree(x["logits"].to(dev), x["parent"].to(dev), x["edge_pos"].to(dev),
                               x["edge_tok"].to(dev), gumbel=x["gumbel"].to(dev), temperature=1.0,
                               num_states=x["num_states"].to(dev), next_pos=nxt.to(dev),
                               mode=dbv.DBV_TREE_FIXED_POSITION)
    xn = _np_inputs(x)
    o = oracle.verify_gumbel_tree(xn["logits"], None, xn["parent"], xn["edge_pos"], xn["edge_tok"],
                                  xn["num_states"], xn["gumbel"], 1.0, oracle.TREE_FIXED_POSITION, npi(nxt))
    check_tree(r, xn, o, "bfloat16", 1.0)


def test_tree_orbit_and_edge_cases(dev):
    say("tree orbit / edge cases")
    # A chain tree that follows the oracle's own orbit is accepted to the end;
    # a bad parent index and a NaN row are reported per sequence.
    B, S, L, V = 3, 7, 6, 3000
    gen = torch.Generator().manual_seed(11)
    logits = (torch.randn(B, S, L, V, generator=gen) * 3).to(torch.bfloat16)
    G = workloads.gumbel_noise((B, L, V), gen)
    masked = torch.ones(B, S, L, dtype=torch.bool)
    parent = torch.full((B, S), -1, dtype=torch.int32)
    ep = torch.zeros(B, S, dtype=torch.int32)
    et = torch.zeros(B, S, dtype=torch.int32)
    ln = np64(logits)
    Gn = G.numpy().astype(np.float64)
    for b in range(B):
        for z in range(1, S):
            m = [s for s in range(L) if masked[b, z - 1, s]]
            t = oracle.state_transition(ln[b, z - 1], m, Gn[b], 1.0)
            parent[b, z] = z - 1
            ep[b, z], et[b, z] = t["pos"], t["tok"]
            masked[b, z] = masked[b, z - 1]
            masked[b, z, t["pos"]] = False
    parent[1, 3] = 5                       # child before parent: bad input
    logits[2, 2, int(ep[2, 3]), 17] = float("nan")
    ln = np64(logits)
    r = dbv.verify_gumbel_tree(logits.to(dev), parent.to(dev), ep.to(dev), et.to(dev),
                               masked=masked.to(dev), gumbel=G.to(dev), temperature=1.0)
    o = oracle.verify_gumbel_tree(ln, masked.numpy(), npi(parent), npi(ep), npi(et), None, Gn, 1.0)
    assert o["path_len"][0] == S - 1 and o["status"][1] == 1 and o["status"][2] == 2
    check_tree(r, dict(logits=ln, gumbel=Gn, parent=npi(parent), edge_pos=npi(ep), edge_tok=npi(et),
                       num_states=None), o, "bfloat16", 1.0)
