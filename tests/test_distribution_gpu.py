"""Output laws of the HIP path over many seeds, batched on B.

  * chain verifiers: one target row p and one drafter row q shared by
    B = 100000 sequences of one draft each (stride-0 batch views), the draft
    token drawn from q and the two uniforms fresh per sequence.  The first
    emitted token must follow p under the lossless rule (with q close to p
    and with a miscalibrated q) and the modified target
    p~ = (1 - lambda) p + lambda q under the lenient rule ("Speculative
    Diffusion is a Tale of Two Tradeoffs", Sec. 2 and Theorem 1; "One Call
    Ahead", App. B.2): a chi-square test at V = 16 and V = 1024, which must
    also reject the drafter's own law q (the test has power).
  * coupled-noise commit: a one-state tree at every sequence, fresh Gumbel
    noise per sequence; the committed token must follow softmax(z / T)
    (the Gumbel-max law; "On the SPOT...", App. A.1).
  * lenient sweep: the mean accepted length of the B=32 K=16 V=128256 bf16
    workload for every (sigma, T, lambda) setting and the lossless control,
    over R = 64 seeds of draft tokens and uniforms, against the expected
    length sum_n prod_{i<=n} (1 - (1 - lambda) TV_i) of the rows' own
    acceptance rates (Two Tradeoffs Sec. 3.3 Eq. 6 and App. C, Eq. 10-11),
    TV_i from the oracle.  The table goes to $DBV_SWEEP_REPORT when set.
"""

import json
import os
import sys

import numpy as np
import pytest
import torch
from scipy.stats import chi2

import draft_block_verification_amd as dbv
import oracle
import workloads
from tests.parity import npi

pytestmark = pytest.mark.gpu

NSEQ = 100_000
P_MIN = 1e-5       # smallest p-value a correct law may give (19+ tests)


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def chi_square(counts, probs, min_expected=20.0):
    """Pearson chi-square of counts against a law, cells merged in order of
    rising expected count until each bin expects at least `min_expected`.
    Returns (statistic, degrees of freedom, p-value)."""
    counts = np.asarray(counts, np.float64)
    e = counts.sum() * np.asarray(probs, np.float64)
    order = np.argsort(e)
    bins_o, bins_e = [], []
    acc_o = acc_e = 0.0
    for i in order:
        acc_o += counts[i]
        acc_e += e[i]
        if acc_e >= min_expected:
            bins_o.append(acc_o)
            bins_e.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0.0 or acc_o > 0.0:
        if bins_e:
            bins_o[-1] += acc_o
            bins_e[-1] += acc_e
        else:
            bins_o.append(acc_o)
            bins_e.append(acc_e)
    o = np.array(bins_o)
    ee = np.array(bins_e)
    stat = float(np.sum((o - ee) ** 2 / ee))
    dof = len(ee) - 1
    return stat, dof, float(chi2.sf(stat, dof)) if dof > 0 else 1.0


def test_chi_square_helper():
    rng = np.random.default_rng(3)
    p = rng.dirichlet(np.ones(50))
    c = rng.multinomial(100000, p)
    assert chi_square(c, p)[2] > 1e-4
    q = rng.dirichlet(np.ones(50))
    assert chi_square(c, q)[2] < 1e-12


def _law_inputs(V, kind, seed):
    """z (target logits), y (drafter logits), float32 [V]."""
    g = np.random.default_rng(seed)
    z = g.normal(0.0, 1.5, V)
    if kind == "close":
        y = z + g.normal(0.0, 0.7, V)
    else:   # miscalibrated: a drafter that ignores the target
        y = g.normal(0.0, 2.0, V)
    return z.astype(np.float32), y.astype(np.float32)


def _unit(g, shape):
    """float32 uniforms in [0, 1) (float64 draws rounded, kept below 1)."""
    return np.minimum(g.random(shape), 1.0 - 2.0 ** -24).astype(np.float32)


def _draw(probs, u):
    """Inverse-CDF draws from a float64 law (host side, for the inputs)."""
    c = np.cumsum(probs)
    return np.minimum(np.searchsorted(c, u * c[-1], side="right"), len(probs) - 1)


@pytest.mark.parametrize("V", [16, 1024])
@pytest.mark.parametrize("rule,kind", [("rejection", "close"), ("rejection", "miscalibrated"),
                                       ("lenient", "close")])
def test_chain_output_law(dev, V, rule, kind):
    say("output law", rule, kind, "V", V, "B", NSEQ)
    z, y = _law_inputs(V, kind, 100 + V + len(kind))
    p = oracle.tempered_softmax(z.astype(np.float64), 1.0)
    q = oracle.tempered_softmax(y.astype(np.float64), 1.0)
    g = np.random.default_rng(7 + V)
    d = _draw(q, g.random(NSEQ)).astype(np.int32)
    zt = torch.tensor(np.stack([z, z]), device=dev).view(1, 2, V).expand(NSEQ, 2, V)
    yt = torch.tensor(y, device=dev).view(1, 1, V).expand(NSEQ, 1, V)
    dt = torch.tensor(d, device=dev).view(NSEQ, 1)
    ua = torch.tensor(_unit(g, (NSEQ, 1)), device=dev)
    ur = torch.tensor(_unit(g, (NSEQ, 2)), device=dev)
    if rule == "rejection":
        r = dbv.verify_rejection(zt, yt, dt, ua, ur)
        law = p
    else:
        lam = 0.5
        r = dbv.verify_lenient(zt, yt, dt, ua, ur, lam)
        law = (1.0 - lam) * p + lam * q
    assert int(npi(r["status"]).max()) == 0
    tok = npi(r["out_tokens"])[:, 0]
    assert tok.min() >= 0 and tok.max() < V
    counts = np.bincount(tok, minlength=V)
    stat, dof, pv = chi_square(counts, law)
    _, _, pq = chi_square(counts, q)
    acc = float(np.mean(npi(r["accept_len"])))
    say(f"chi2 {stat:.1f} dof {dof} p-value {pv:.3g}; against q {pq:.3g}; acceptance {acc:.4f}")
    assert pv > P_MIN, (stat, dof, pv)
    assert pq < 1e-12
    # the acceptance rate is 1 - TV(p~, q) (Two Tradeoffs Sec. 2, Eq. 1-2)
    beta = 1.0 - oracle.total_variation(law, q)
    assert abs(acc - beta) < 5.0 * np.sqrt(beta * (1.0 - beta) / NSEQ) + 1e-12


@pytest.mark.parametrize("V", [16, 1024])
@pytest.mark.parametrize("T", [0.7, 1.0])
def test_gumbel_commit_law(dev, V, T):
    say("coupled-noise commit law V", V, "T", T, "B", NSEQ)
    g = np.random.default_rng(11 + V)
    z = g.normal(0.0, 1.5, V).astype(np.float32)
    law = oracle.tempered_softmax(z.astype(np.float64), T)
    logits = torch.tensor(z, device=dev).view(1, 1, 1, V).expand(NSEQ, 1, 1, V)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234 + V)
    gum = workloads.gumbel_noise((NSEQ, 1, V), gen, device=dev)
    minus = torch.full((NSEQ, 1), -1, dtype=torch.int32, device=dev)
    r = dbv.verify_gumbel_tree(logits, minus, minus, minus, masked=torch.ones(NSEQ, 1, 1, dtype=torch.uint8,
                                                                                device=dev),
                               gumbel=gum, temperature=T)
    assert int(npi(r["status"]).max()) == 0
    nc = npi(r["num_commits"])
    assert (nc == 1).all()
    assert (npi(r["commit_pos"])[:, 0] == 0).all()
    tok = npi(r["commit_tok"])[:, 0]
    counts = np.bincount(tok, minlength=V)
    stat, dof, pv = chi_square(counts, law)
    _, _, pu = chi_square(counts, np.full(V, 1.0 / V))
    say(f"chi2 {stat:.1f} dof {dof} p-value {pv:.3g}; against uniform {pu:.3g}")
    assert pv > P_MIN, (stat, dof, pv)
    assert pu < 1e-12


SWEEP_R = 64


def _expected_length(tv, lam):
    """sum_n prod_{i<=n} beta_i with beta_i = 1 - (1 - lambda) TV_i, per
    sequence (rows [B, K])."""
    beta = 1.0 - (1.0 - lam) * tv
    return np.cumprod(beta, axis=1).sum(axis=1)


SWEEP = []


@pytest.mark.parametrize("T", workloads.C3_TEMPS)
@pytest.mark.parametrize("sigma", workloads.C3_SIGMAS)
def test_lenient_sweep_mean_length(dev, sigma, T):
    say("lenient sweep B=32 K=16 V=128256 bf16 sigma", sigma, "T", T, "R", SWEEP_R)
    x = workloads.config3(sigma, T)
    B, K = x["draft_tokens"].shape
    V = x["tgt"].shape[-1]
    tgt, drf = x["tgt"].to(dev), x["drf"].to(dev)
    tgt64 = x["tgt"].double().numpy()
    drf64 = x["drf"].double().numpy()
    tv = np.array([[oracle.total_variation(oracle.tempered_softmax(tgt64[b, i], T),
                                           oracle.tempered_softmax(drf64[b, i], T)) for i in range(K)]
                   for b in range(B)])
    q = torch.softmax(drf.float().reshape(B * K, V) / T, -1)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(sigma * 1000 + T * 10))
    n = torch.full((B,), K, dtype=torch.int32, device=dev)
    hs = {lam: [] for lam in (0.0,) + workloads.C3_LAMBDAS}
    for r in range(SWEEP_R):
        d = torch.multinomial(q, 1, generator=gen).reshape(B, K).to(torch.int32)
        ua = torch.rand(B, K, generator=gen, device=dev)
        ur = torch.rand(B, K + 1, generator=gen, device=dev)
        for lam in hs:
            res = dbv.verify_lenient(tgt, drf, d, ua, ur, lam, draft_len=n, temperature_target=T,
                                     temperature_draft=T)
            hs[lam].append(npi(res["accept_len"]))
    for lam, hl in hs.items():
        h = np.stack(hl, axis=1).astype(np.float64)          # [B, R]
        mean = float(h.mean())
        se = float(np.sqrt(h.var(axis=1, ddof=1).mean() / (B * SWEEP_R)))
        exact = float(_expected_length(tv, lam).mean())
        mu = float(1.0 - (1.0 - lam) * tv.mean())
        prop1 = float(sum(mu ** m for m in range(1, K + 1)))
        SWEEP.append(dict(sigma=sigma, T=T, lam=lam, mean_accept_len=mean, stderr=se, expected=exact,
                          expected_iid=prop1, mean_tv=float(tv.mean())))
        say(f"lambda {lam}: mean accepted {mean:.3f} +- {se:.3f}, expected {exact:.3f} "
            f"(i.i.d. rates {prop1:.3f}), mean TV {tv.mean():.4f}")
        if lam == 1.0:
            assert mean == K
        else:
            assert abs(mean - exact) <= 5.0 * se + 1e-9, (lam, mean, exact, se)
    path = os.environ.get("DBV_SWEEP_REPORT")
    if path:
        with open(path, "w") as fh:
            json.dump(dict(workload="lenient B=32 K=16 V=128256 bf16", seeds=SWEEP_R, rows=SWEEP), fh, indent=1)
