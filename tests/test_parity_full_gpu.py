"""Parity at the benchmark workloads' full sizes, in the launch configuration
the benchmark times (same entry points, shapes, dtypes and strides, so the
same launch plan).  Every sequence and every tree is compared with the
float64 oracle; the near-margin decisions met are recorded per workload
(tests.parity.record):

  * tiny rejection verify   B=1  K=4  V=1024   fp32
  * batch lossless verify   B=8  K=8  V=32000  bf16
  * lenient sweep           B=32 K=16 V=128256 bf16, sigma x T x lambda, with
    lambda = 0 (equal to the lossless entry point bit for bit), lambda = 1
    (every draft accepted) and a check that the accepted length does not
    fall as lambda rises under common uniforms
  * Cactus sweep            the same shape, sigma = 1, T = 1, budgets
    delta in {0, 0.25, 1, 4, 16} (delta = 0 equals the lossless entry point)
  * Gumbel tree verify      B=16 S=64 L=32 V=151936 bf16, the 16 trees in
    four groups (one tree at a time on the host)
  * packed greedy           B=64 K=31 W=32 V=131072 bf16, with and without
    the stopping rule
  * any-order greedy        B=64 U=32 V=131072 bf16, with and without EOS /
    end position
  * joint-space chain       B=16 K=8 V=151936 bf16, hybrid gate tau=0.6 and
    rejection sampling only
  * stored sparse Q         B=32 K=16 V=151936 bf16, top-k = 20
"""

import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as dbv
import oracle
import workloads
from tests.parity import (check_any_order, check_greedy, check_sampling, check_spot, check_tree, np64, npi,
                          record)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _take(res, seqs):
    """Rows `seqs` of every per-sequence output."""
    idx = torch.as_tensor(seqs, dtype=torch.long)
    return {k: v.detach().cpu()[idx] for k, v in res.items()}


def _chain_np(x, seqs=None):
    keys = ("tgt", "drf", "draft_tokens", "draft_len", "u_accept", "u_resample")
    out = {}
    for k in keys:
        v = x[k] if seqs is None else x[k][torch.as_tensor(seqs, dtype=torch.long)]
        out[k] = np64(v) if v.dtype.is_floating_point else npi(v)
    return out


def _sampling_call(x, dev, lam=None, T=1.0, **kw):
    args = (x["tgt"].to(dev), x["drf"].to(dev), x["draft_tokens"].to(dev), x["u_accept"].to(dev),
            x["u_resample"].to(dev))
    common = dict(draft_len=x["draft_len"].to(dev), temperature_target=T, temperature_draft=T, **kw)
    if lam is None:
        return dbv.verify_rejection(*args, **common)
    return dbv.verify_lenient(*args, lam, **common)


# ---------------------------------------------------------------- chains ---

def test_full_tiny_rejection_and_greedy(dev):
    say("full tiny B=1 K=4 V=1024 fp32")
    x = workloads.config1()
    xn = _chain_np(x)
    res = _sampling_call(x, dev)
    o = oracle.verify_rejection(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 1.0,
                                xn["u_accept"], xn["u_resample"])
    record("c1 tiny rejection B=1 K=4 V=1024 fp32", check_sampling(res, xn, o, 0.0, 1.0, 1.0, "float32"))
    for name, d in (("argmax drafts", x["greedy_tokens"]), ("sampled drafts", x["draft_tokens"])):
        say("greedy", name)
        g = dbv.verify_greedy(x["tgt"].to(dev), d.to(dev), x["draft_len"].to(dev), x["drf"].to(dev))
        og = oracle.verify_greedy(xn["tgt"], npi(d), xn["draft_len"], xn["drf"])
        check_greedy(g, og)


def test_full_batch_lossless(dev):
    say("full batch lossless B=8 K=8 V=32000 bf16")
    x = workloads.config2()
    xn = _chain_np(x)
    res = _sampling_call(x, dev)
    o = oracle.verify_rejection(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 1.0,
                                xn["u_accept"], xn["u_resample"])
    near = record("c2 batch lossless B=8 K=8 V=32000 bf16", check_sampling(res, xn, o, 0.0, 1.0, 1.0, "bfloat16"))
    say("near-margin", dict(near), "accept_len", list(o["accept_len"]))


@pytest.mark.parametrize("T", [0.7, 1.0])
@pytest.mark.parametrize("sigma", workloads.C3_SIGMAS)
def test_full_lenient_sweep(dev, sigma, T):
    say("full lenient B=32 K=16 V=128256 bf16 sigma", sigma, "T", T)
    x = workloads.config3(sigma, T)
    xn = _chain_np(x)
    n = npi(x["draft_len"])
    lossless = _sampling_call(x, dev, None, T)
    h_prev, flips_prev = None, 0
    for lam in (0.0,) + tuple(sorted(workloads.C3_LAMBDAS)):
        res = _sampling_call(x, dev, lam, T)
        if lam == 0.0:
            for k in lossless:
                assert torch.equal(lossless[k], res[k]), k
        h = npi(res["accept_len"])
        if lam == 1.0:
            np.testing.assert_array_equal(h, n)
        o = oracle.verify_lenient(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], T, T, lam,
                                  xn["u_accept"], xn["u_resample"])
        near = record(f"c3 lenient B=32 K=16 V=128256 bf16 sigma={sigma} T={T} lambda={lam}",
                      check_sampling(res, xn, o, lam, T, T, "bfloat16"))
        if h_prev is not None:
            # Under common uniforms alpha rises with lambda, so h cannot fall
            # except through a near-margin decision of either call (counted by
            # the checker).
            fell = [b for b in range(len(h)) if h[b] < h_prev[b]]
            assert len(fell) <= near["accept_flip"] + flips_prev, fell
        h_prev, flips_prev = h, near["accept_flip"]
        say(f"lambda={lam} mean accept length {h.mean():.3f} near-margin {dict(near)}")


C3_DELTAS = (0.25, 1.0, 4.0, 16.0)


def test_full_cactus_sweep(dev):
    say("full Cactus B=32 K=16 V=128256 bf16 sigma 1 T 1")
    x = workloads.config3(1.0, 1.0)
    xn = _chain_np(x)
    args = (x["tgt"].to(dev), x["drf"].to(dev), x["draft_tokens"].to(dev), x["u_accept"].to(dev),
            x["u_resample"].to(dev))
    common = dict(draft_len=x["draft_len"].to(dev))
    lossless = dbv.verify_rejection(*args, **common)
    h_prev, flips_prev = None, 0
    for delta in (0.0,) + C3_DELTAS:
        res = dbv.verify_cactus(*args, delta, **common)
        if delta == 0.0:
            for k in lossless:
                assert torch.equal(lossless[k], res[k]), k
        h = npi(res["accept_len"])
        o = oracle.verify_cactus(xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], 1.0, 1.0, delta,
                                 xn["u_accept"], xn["u_resample"])
        near = record(f"c3c Cactus B=32 K=16 V=128256 bf16 sigma=1 T=1 delta={delta}",
                      check_sampling(res, xn, o, 0.0, 1.0, 1.0, "bfloat16", delta=delta))
        if h_prev is not None:
            fell = [b for b in range(len(h)) if h[b] < h_prev[b]]
            assert len(fell) <= near["accept_flip"] + flips_prev, fell
        h_prev, flips_prev = h, near["accept_flip"]
        say(f"delta={delta} mean accept length {h.mean():.3f} near-margin {dict(near)}")


# ------------------------------------------------------------------ tree ---

@pytest.fixture(scope="module")
def tree_run(dev):
    """The tree workload on the device and the GPU's result, shared by the
    four groups of trees."""
    x = workloads.config4(device=dev)
    res = dbv.verify_gumbel_tree(x["logits"], x["parent"].to(dev), x["edge_pos"].to(dev),
                                 x["edge_tok"].to(dev), masked=x["masked"].to(dev), gumbel=x["gumbel"],
                                 temperature=1.0, num_states=x["num_states"].to(dev))
    r = {k: v.cpu() for k, v in res.items()}
    return x, r


@pytest.mark.parametrize("group", range(4))
def test_full_gumbel_tree(dev, tree_run, group):
    x, r = tree_run
    B = x["logits"].shape[0]
    assert int((r["status"] & dbv.SEQ_ERROR_MASK).sum()) == 0
    for b in range(group * B // 4, (group + 1) * B // 4):
        say("full tree B=16 S=64 L=32 V=151936 bf16: oracle tree", b)
        # float32 holds the bf16 logits exactly; the oracle upcasts each row
        # to float64 itself.
        xb = dict(logits=x["logits"][b:b + 1].float().cpu().numpy(), gumbel=x["gumbel"][b:b + 1].cpu().numpy(),
                  parent=npi(x["parent"][b:b + 1]), edge_pos=npi(x["edge_pos"][b:b + 1]),
                  edge_tok=npi(x["edge_tok"][b:b + 1]), num_states=npi(x["num_states"][b:b + 1]))
        o = oracle.verify_gumbel_tree(xb["logits"], x["masked"][b:b + 1].cpu().numpy(), xb["parent"],
                                      xb["edge_pos"], xb["edge_tok"], xb["num_states"], xb["gumbel"], 1.0)
        near = record("c4 Gumbel tree B=16 S=64 L=32 V=151936 bf16 T=1",
                      check_tree({k: v[b:b + 1] for k, v in r.items()}, xb, o, "bfloat16", 1.0))
        say("path", int(r["path_len"][b]), "near", dict(near))
        del xb, o


# ---------------------------------------------------------------- greedy ---

@pytest.mark.parametrize("stopping", [False, True])
def test_full_packed_greedy(dev, stopping):
    say("full packed greedy B=64 K=31 W=32 V=131072 bf16, stopping", stopping)
    x = workloads.config5()
    K = x["K"]
    p = x["packed"].to(dev)
    B = p.shape[0]
    kw = {}
    if stopping:
        # EOS = the verifier argmax of one seeded row; budgets over [0, K+1].
        g = torch.Generator().manual_seed(55)
        b0 = int(torch.randint(0, B, (1,), generator=g))
        kw["eos_id"] = int(torch.argmax(x["packed"][b0, 0].float()))
        kw["len_budget"] = torch.randint(0, K + 2, (B,), generator=g).to(torch.int32)
    res = dbv.verify_greedy(p[:, :K + 1], x["draft_tokens"].to(dev), x["draft_len"].to(dev), p[:, K + 1:],
                            **{k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in kw.items()})
    r = {k: v.cpu() for k, v in res.items()}
    for b in range(B):
        o = oracle.verify_greedy(np64(x["packed"][b:b + 1, :K + 1]), npi(x["draft_tokens"][b:b + 1]),
                                 npi(x["draft_len"][b:b + 1]), np64(x["packed"][b:b + 1, K + 1:]),
                                 eos_id=kw.get("eos_id", -1),
                                 len_budget=None if not stopping else npi(kw["len_budget"][b:b + 1]))
        check_greedy(_take(r, [b]), o)
    record(f"c5 packed greedy B=64 K=31 W=32 V=131072 bf16 stopping={stopping}", {"sequences": B})
    say("mean accept length", float(r["accept_len"].float().mean()), "mean emitted", float(r["num_out"].float().mean()))


# -------------------------------------------------------------- any-order ---

def test_full_any_order(dev):
    say("full any-order B=64 U=32 V=131072 bf16")
    x = workloads.config5_any_order()
    xd = {k: v.to(dev) for k, v in x.items()}
    for eos, end in ((-1, None), (int(x["draft_tokens"][x["draft_tokens"] >= 0][0]), x["positions"][:, 20].clone())):
        g = dbv.verify_greedy_any_order(xd["tgt"], xd["order"], xd["draft_tokens"], num_active=xd["num_active"],
                                        positions=xd["positions"], draft_rows=xd["draft_rows"], eos_id=eos,
                                        end_pos=None if end is None else end.to(dev))
        for b0 in range(0, 64, 8):
            sl = slice(b0, b0 + 8)
            o = oracle.verify_greedy_any_order(
                np64(x["tgt"][sl]), npi(x["order"][sl]), npi(x["num_active"][sl]), npi(x["positions"][sl]),
                npi(x["draft_tokens"][sl]), np64(x["draft_rows"][sl]), eos, None if end is None else npi(end[sl]))
            check_any_order({k: v[sl] for k, v in g.items()}, o)
        record(f"c5ao any-order greedy B=64 U=32 V=131072 bf16 eos={eos >= 0}", {"sequences": 64})
        say("eos", eos, "mean accepted", float(g["num_accepted"].float().mean()))


# ------------------------------------------------------- joint-space chain ---

def test_full_spot_chain(dev):
    say("full joint-space chain B=16 K=8 V=151936 bf16")
    x = workloads.config4_spot_chain()
    xd = {k: v.to(dev) if torch.is_tensor(v) else v for k, v in x.items()}
    for G in (xd["gumbel"], None):
        g = dbv.verify_spot_chain(xd["tgt"], xd["drf"], xd["pos_star"], xd["prop_pos"], xd["prop_tok"],
                                  xd["q_pos_star"], xd["u_accept"], xd["u_resample"], gumbel=G, tau=0.6,
                                  draft_len=xd["draft_len"])
        xn = {k: (np64(v) if v.is_floating_point() else npi(v)) if torch.is_tensor(v) else v for k, v in x.items()}
        if G is None:
            xn["gumbel"] = None
        o = oracle.verify_spot_chain(xn["tgt"], xn["drf"], xn["pos_star"], xn["prop_pos"], xn["prop_tok"],
                                     xn["q_pos_star"], xn["draft_len"], 1.0, 1.0, xn["u_accept"],
                                     xn["u_resample"], gumbel=xn["gumbel"], tau=0.6)
        near = record(f"c4s joint-space chain B=16 K=8 V=151936 bf16 gumbel={G is not None}",
                      check_spot(g, xn, o, 1.0, 1.0, 0.6, "bfloat16"))
        say("gumbel", G is not None, "mean h", float(o["accept_len"].mean()), "near", dict(near))


# ---------------------------------------------------------------- sparse Q ---

def test_full_sparse(dev):
    say("full sparse Q B=32 K=16 V=151936 bf16 top-k 20")
    x = workloads.config3_sparse()
    g = dbv.verify_sparse(x["tgt"].to(dev), x["q_idx"].to(dev), x["q_prob"].to(dev), x["q_nnz"].to(dev),
                          x["draft_tokens"].to(dev), x["u_accept"].to(dev), x["u_resample"].to(dev),
                          draft_len=x["draft_len"].to(dev))
    qi, qp, qn = npi(x["q_idx"]), np64(x["q_prob"]), npi(x["q_nnz"])
    xn = dict(tgt=np64(x["tgt"]), draft_tokens=npi(x["draft_tokens"]), draft_len=npi(x["draft_len"]),
              u_accept=np64(x["u_accept"]), u_resample=np64(x["u_resample"]))
    V = x["tgt"].shape[-1]
    for b0 in range(0, 32, 8):
        sl = list(range(b0, b0 + 8))
        o = oracle.verify_sparse(xn["tgt"][sl], qi[sl], qp[sl], qn[sl], xn["draft_tokens"][sl],
                                 xn["draft_len"][sl], 1.0, xn["u_accept"][sl], xn["u_resample"][sl])
        near = record("c3q stored sparse Q B=32 K=16 V=151936 bf16 top-k 20",
                      check_sampling(g, xn, o, 0.0, 1.0, 1.0, "bfloat16", seqs=sl,
                                     qfun=lambda b, i: oracle.dense_q(qi[b, i], qp[b, i], qn[b, i], V)))
        say("seqs", b0, "h", list(o["accept_len"]), "near", dict(near))
